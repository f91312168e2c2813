"""Edge sizes of the HIP path at full model dimensions, against the oracle.

* Batch sizes around the implementation's switches at the V3 layer shape
  (d = 7168, 256 routed top-8 + 1 shared): T = 1 (one token, thin tiles
  everywhere), 128 / 129 (the shared group's down pass folds its bf16 pair
  into one tile up to 128 rows, and runs in fp16 beyond), 4095 / 4096 /
  4097 (the select kernel takes two tokens per wave from 4096 on, and the
  router's d split and the row-tile counts change with T).
* The largest batch the API takes: T K' = 2^22 pairs (T = 524,288, K' = 8,
  d = 256), the permutation's largest chunks and ~16k row tiles per GEMM.
* Node-limited routing at the full V4 shape on the V4 book's layout (384
  experts on 32 nodes of 12, at most M = 4 nodes per token).
* One GPU's share of the V3 layer under 8-way expert parallelism: 32
  resident experts at full width on received rows that name 1 to 8 of them
  (the other slots empty), about 2,300 rows per expert.
Routing is checked bit-exactly on identical logits for every token; the
layer output on the first and last row of every row tile of every group
(a seeded subset of them for the largest batch)."""
import numpy as np
import pytest
import torch

from fine_grained_moe_router_amd import binding as B
from fine_grained_moe_router_amd.configs import CONFIGS, scaled
from fine_grained_moe_router_amd.synth import make_inputs, make_share_routing, to_numpy
from oracle import oracle as O

from parity import (compare_h, gpu_h_as_f64, gpu_layer, host, oracle_h, oracle_route_tokens,
                    row_tile_tokens)

pytestmark = pytest.mark.gpu


def check_routing(cfg, inp, r):
    lg = to_numpy(r["logits"])
    idx, gate, _, _ = O.route(lg, cfg.n_routed, cfg.top_k, cfg.scoring, cfg.renorm,
                              offset=host(inp.offset), bias=host(inp.bias),
                              n_groups=cfg.n_groups, topk_groups=cfg.topk_groups)
    np.testing.assert_array_equal(to_numpy(r["idx"]), idx)
    np.testing.assert_array_equal(to_numpy(r["counts"]), O.counts(idx, cfg.n_routed))
    ulps = np.abs(to_numpy(r["w"]) - gate) / np.spacing(np.abs(gate))
    assert ulps.max() <= 1.0
    return idx


def check_layer(cfg, inp, r, tokens):
    """h on the listed tokens against the oracle's routing and layer."""
    x_h = host(inp.x)
    _, idx, gate, _, gap = oracle_route_tokens(cfg, inp, tokens, x_h=x_h)
    h_ref = oracle_h(cfg, inp, tokens, idx, gate, x_h=x_h)
    res = compare_h(cfg, gpu_h_as_f64(r["h"])[tokens], h_ref, gap)
    print(f"[edges] {cfg.name}: tokens {len(tokens)} max_abs {res[0]:.4g} rel_l2 {res[1]:.4g}",
          flush=True)


@pytest.mark.parametrize("T", [1, 128, 129, 4095, 4096, 4097])
def test_v3_batch_size_edges(T):
    cfg = CONFIGS["v3_prefill"].with_(name=f"v3_T{T}", T=T)
    print(f"[edges] {cfg.name}", flush=True)
    inp = make_inputs(cfg, "cuda")
    r = gpu_layer(cfg, inp)
    idx = check_routing(cfg, inp, r)
    tokens = np.arange(T) if T <= 64 else row_tile_tokens(idx, T, cfg.n_routed, True)
    check_layer(cfg, inp, r, tokens)


def test_largest_batch():
    cfg = scaled(CONFIGS["v3_prefill"], T=1 << 19, d_model=256, d_ff=128, name="max_pairs")
    assert cfg.T * cfg.top_k == 1 << 22
    print(f"[edges] {cfg.name}", flush=True)
    inp = make_inputs(cfg, "cuda")
    r = gpu_layer(cfg, inp)
    idx = check_routing(cfg, inp, r)
    tiles = row_tile_tokens(idx, cfg.T, cfg.n_routed, True)
    rng = np.random.default_rng(11)
    tokens = np.unique(np.concatenate([tiles[:64], tiles[-64:],
                                       rng.choice(tiles, 512, replace=False)]))
    check_layer(cfg, inp, r, tokens)


def test_v4_book_node_layout_full_size():
    """384 experts on 32 nodes of 12, at most 4 nodes per token, at the V4
    shape with its Zipf-skewed router: the GPU's routing equals the
    oracle's, no token spans more than 4 nodes, and (with these logits) the
    limit replaces a large share of the unrestricted choices."""
    cfg = CONFIGS["v4_skew"].with_(n_groups=32, topk_groups=4)
    inp = make_inputs(cfg, "cuda", experts=False)
    r = B.route(cfg, x=inp.x, w_gate=inp.w_gate, offset=inp.offset, bias=inp.bias,
                logits_out=True)
    plain = B.route(CONFIGS["v4_skew"], x=inp.x, w_gate=inp.w_gate, offset=inp.offset,
                    bias=inp.bias)
    torch.cuda.synchronize()
    idx = check_routing(cfg, inp, r)
    nodes = idx // (cfg.n_routed // cfg.n_groups)
    assert max(len(set(row)) for row in nodes) <= 4
    p = to_numpy(plain["idx"])
    replaced = np.mean([len(set(a) - set(b)) for a, b in zip(p, idx)]) / cfg.top_k
    print(f"[edges] v4 node limit: replaced share {replaced:.3f}", flush=True)
    assert replaced > 0.05


def test_ep_share_shape():
    """The routed part of one GPU's share under 8-way expert parallelism at
    the V3 width: 16,384 received rows over 32 resident experts, each row
    naming 1..8 of them in random slots (the rest -1), no shared expert;
    the first and last row of every row tile against the oracle."""
    cfg = CONFIGS["v3_prefill"].with_(name="v3_ep8_routed", T=16384, n_routed=32, n_shared=0)
    print(f"[edges] {cfg.name}", flush=True)
    inp = make_inputs(cfg, "cuda")
    idx, gate = make_share_routing(cfg.T, cfg.n_routed, cfg.top_k, seed=3)
    h = B.forward(cfg, inp.x, idx.cuda(), gate.cuda(), inp.w13, inp.w2)
    torch.cuda.synchronize()
    idx_np, gate_np = idx.numpy(), gate.numpy()
    tokens = row_tile_tokens(idx_np, cfg.T, cfg.n_routed, False)
    valid = idx_np[tokens] >= 0
    h_ref = oracle_h(cfg, inp, tokens, np.where(valid, idx_np[tokens], 0),
                     np.where(valid, gate_np[tokens], 0))
    res = compare_h(cfg, gpu_h_as_f64(h)[tokens], h_ref, np.full(len(tokens), np.inf))
    print(f"[edges] {cfg.name}: tokens {len(tokens)} max_abs {res[0]:.4g} rel_l2 {res[1]:.4g}",
          flush=True)
