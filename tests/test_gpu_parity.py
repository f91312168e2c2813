"""HIP path (through the C ABI) against the CPU oracle, on the same seeded
input bytes.

* Routing given identical fp32 logits: indices and counts bit-exact, gates
  within one fp32 ulp, in both directions (GPU logits fed to the oracle, and
  oracle logits fed to the GPU through MOE_LOGITS_IN).
* Layer output: each side routes from its own logits; bf16 within max-abs
  2e-2 / rel-L2 5e-3, fp32 within 1e-4 / 1e-5, near-tie tokens excluded.
* Balance statistics: f bit-exact, P and the loss to 1e-6 relative.
"""
import numpy as np
import pytest
import torch

from fine_grained_moe_router_amd import binding as B
from fine_grained_moe_router_amd.configs import CONFIGS, scaled
from fine_grained_moe_router_amd.synth import make_inputs, to_numpy
from oracle import oracle as O

from parity import (ROW_TILE, check_routing_identical_logits, compare_h, gpu_h_as_f64,
                    gpu_layer, host, oracle_h, oracle_route_tokens, row_tile_tokens)

pytestmark = pytest.mark.gpu

SMALL = {
    "toy_fp32": CONFIGS["toy_fp32"],
    "mid_ragged": scaled(CONFIGS["mid"], T=333, d_model=320, d_ff=192),
    "v3_ragged": scaled(CONFIGS["v3_prefill"], T=700, d_model=512, d_ff=128),
    "v4_skew_ragged": scaled(CONFIGS["v4_skew"], T=500, d_model=384, d_ff=128),
    "v4_hash_ragged": scaled(CONFIGS["v4_hash"], T=2000, d_model=256, d_ff=64),
    "no_shared": scaled(CONFIGS["v3_prefill"], T=257, d_model=256, d_ff=128).with_(n_shared=0),
    "one_token": scaled(CONFIGS["v3_prefill"], T=1, d_model=256, d_ff=128),
    "dense_mixture": scaled(CONFIGS["mid"], T=130, d_model=128, d_ff=64).with_(
        n_routed=8, top_k=8, n_shared=1, d_ff_shared=64),
    "f32_sigmoid": CONFIGS["toy_fp32"].with_(name="f32_sigmoid", T=200, scoring="sigmoid",
                                             renorm=True, bias=True),
    # ~250 rows per routed expert (as at V3 prefill): experts spanning
    # several row tiles, with ragged d (320) and d_ff (192)
    "many_rows_ragged": scaled(CONFIGS["v3_prefill"], T=1000, d_model=320, d_ff=192).with_(
        n_routed=16, top_k=4),
    # the smallest sizes the API takes (d = d_ff = 64): one k-tile per K loop
    "d64": scaled(CONFIGS["v3_prefill"], T=100, d_model=64, d_ff=64),
    # the largest K' the API takes (16): the select kernel's and the
    # combine's per-token bounds
    "top16": scaled(CONFIGS["mid"], T=300, d_model=256, d_ff=64).with_(top_k=16),
    # ~375 rows per routed expert and two 64-wide shared experts side by side
    "many_rows_two_shared": scaled(CONFIGS["mid"], T=1500, d_model=256, d_ff=128).with_(
        n_routed=8, top_k=2, n_shared=2, d_ff_shared=64),
    # hash routing over 12 experts, ~240 rows each: routed (hi, lo) tiles of
    # more than 128 rows take the unfolded pass, over one or two row tiles.
    # At T = 3000 one output reaches |h| = 8.27, where bf16's half-ulp alone
    # (0.031) exceeds the 2e-2 bar; T = 2900 keeps every |h| below 8 (6.76).
    "hash_many_rows": scaled(CONFIGS["v4_hash"], T=2900, d_model=256, d_ff=128).with_(
        n_routed=12),
}


def small_inputs(cfg):
    inp = make_inputs(cfg, "cpu")
    for k in ("x", "w_gate", "w13", "w2", "w13s", "w2s", "bias", "offset", "token_ids"):
        v = getattr(inp, k)
        if v is not None:
            setattr(inp, k, v.cuda())
    return inp


@pytest.mark.parametrize("name", list(SMALL))
def test_small_layer_end_to_end(name):
    cfg = SMALL[name]
    torch.manual_seed(0)
    inp = small_inputs(cfg)
    r = gpu_layer(cfg, inp)
    check_routing_identical_logits(cfg, inp, r)
    tokens = np.arange(cfg.T)
    _, idx, gate, _, gap = oracle_route_tokens(cfg, inp, tokens)
    h_ref = oracle_h(cfg, inp, tokens, idx, gate)
    compare_h(cfg, gpu_h_as_f64(r["h"]), h_ref, gap)


@pytest.mark.parametrize("name", ["toy_fp32", "v3_ragged", "v4_skew_ragged", "mid_ragged"])
def test_routing_from_oracle_logits(name):
    """Oracle logits fed to the GPU (MOE_LOGITS_IN): identical selection."""
    cfg = SMALL[name]
    inp = small_inputs(cfg)
    lg, idx, gate, _, _ = oracle_route_tokens(cfg, inp, np.arange(cfg.T))
    r = B.route(cfg, logits_in=torch.from_numpy(lg).cuda(), offset=inp.offset, bias=inp.bias)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_numpy(r["idx"]), idx)
    np.testing.assert_array_equal(to_numpy(r["counts"]), O.counts(idx, cfg.n_routed))
    ulps = np.abs(to_numpy(r["w"]) - gate) / np.spacing(np.abs(gate))
    assert ulps.max() <= 1.0


def test_forward_is_bitwise_deterministic():
    cfg = SMALL["v3_ragged"]
    inp = small_inputs(cfg)
    r = gpu_layer(cfg, inp)
    h2 = B.forward(cfg, inp.x, r["idx"], r["w"], inp.w13, inp.w2, inp.w13s, inp.w2s)
    torch.cuda.synchronize()
    assert torch.equal(r["h"].view(torch.int16), h2.view(torch.int16))


def caller_routing_case(cfg, idx_np, gate_np):
    inp = small_inputs(cfg)
    idx = torch.from_numpy(idx_np).cuda()
    w = torch.from_numpy(gate_np).cuda()
    h = B.forward(cfg, inp.x, idx, w, inp.w13, inp.w2, inp.w13s, inp.w2s)
    torch.cuda.synchronize()
    tokens = np.arange(cfg.T)
    valid = (idx_np >= 0) & (idx_np < cfg.n_routed)
    h_ref = oracle_h(cfg, inp, tokens, np.where(valid, idx_np, 0), np.where(valid, gate_np, 0))
    compare_h(cfg, gpu_h_as_f64(h), h_ref, np.full(cfg.T, np.inf))


def test_skewed_and_empty_experts():
    """Every token on expert 5 (several row tiles), a third also on expert 0,
    all other experts empty; an out-of-range index contributes nothing."""
    cfg = scaled(CONFIGS["v3_prefill"], T=300, d_model=256, d_ff=128).with_(top_k=3)
    rng = np.random.default_rng(1)
    idx = np.full((cfg.T, 3), -1, np.int32)
    idx[:, 0] = 5
    idx[::3, 1] = 0
    idx[1::7, 2] = cfg.n_routed + 3       # out of range
    idx[2::5, 2] = 200
    gate = rng.random((cfg.T, 3)).astype(np.float32)
    caller_routing_case(cfg, idx, gate)


def test_outputs_beyond_fp16_range():
    """bf16 layers stage the gate-scaled expert outputs as fp16 and keep fp32
    where fp16 overflows.  W2 and the shared W2 scaled by 2^16 (exact in bf16,
    so every expert output scales exactly): about a tenth of the outputs now
    exceed fp16's range, the rest do not.  h must equal x + 2^16 Y to the
    usual error of Y (scaled) plus h's own bf16 rounding."""
    cfg = scaled(CONFIGS["v3_prefill"], T=300, d_model=256, d_ff=128)
    inp = small_inputs(cfg)
    scale = 2.0 ** 16
    inp.w2 = (inp.w2.float() * scale).to(torch.bfloat16)
    inp.w2s = (inp.w2s.float() * scale).to(torch.bfloat16)
    r = gpu_layer(cfg, inp)
    idx, gate = check_routing_identical_logits(cfg, inp, r)
    tokens = np.arange(cfg.T)
    h_ref = oracle_h(cfg, inp, tokens, idx, gate)
    h_gpu = gpu_h_as_f64(r["h"])
    assert np.isfinite(h_gpu).all()
    assert (np.abs(h_ref) > 65520).mean() > 0.02          # the fp32 path is exercised
    err = np.abs(h_gpu - h_ref)
    assert (err <= scale * 6e-3 + 2.0 ** -8 * np.abs(h_ref)).all(), err.max()
    assert np.linalg.norm(h_gpu - h_ref) <= 5e-3 * np.linalg.norm(h_ref)


def test_one_hot_expert_stealing_and_column_order():
    """Every token on expert 7 and half of them also on expert 3: expert 7
    spans 8 row tiles (listed column tile fastest), the other XCDs have no
    work of their own and take items from the busy XCD's queue.  Repeated
    calls are bitwise identical whatever the pull order."""
    cfg = scaled(CONFIGS["v3_prefill"], T=2000, d_model=256, d_ff=128).with_(top_k=2)
    idx = np.full((cfg.T, 2), -1, np.int32)
    idx[:, 0] = 7
    idx[::2, 1] = 3
    gate = np.random.default_rng(3).random((cfg.T, 2)).astype(np.float32)
    caller_routing_case(cfg, idx, gate)
    inp = small_inputs(cfg)
    i_t, w_t = torch.from_numpy(idx).cuda(), torch.from_numpy(gate).cuda()
    outs = [B.forward(cfg, inp.x, i_t, w_t, inp.w13, inp.w2, inp.w13s, inp.w2s) for _ in range(3)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(outs[0].view(torch.int16), o.view(torch.int16))


def test_one_hot_expert_few_experts():
    """As above with 16 routed experts and 128-wide experts: expert 7 spans 8
    row tiles, expert 3 four; the other 14 are empty."""
    cfg = scaled(CONFIGS["v3_prefill"], T=2000, d_model=256, d_ff=128).with_(
        n_routed=16, top_k=2)
    idx = np.full((cfg.T, 2), -1, np.int32)
    idx[:, 0] = 7
    idx[::2, 1] = 3
    gate = np.random.default_rng(4).random((cfg.T, 2)).astype(np.float32)
    caller_routing_case(cfg, idx, gate)


def test_many_experts_select_path():
    """N' = 1024 routed experts (16 per lane in the select kernel), top-8."""
    cfg = scaled(CONFIGS["v3_prefill"], T=300, d_model=256, d_ff=64).with_(
        name="n1024", n_routed=1024)
    inp = small_inputs(cfg)
    r = gpu_layer(cfg, inp)
    idx, gate = check_routing_identical_logits(cfg, inp, r)
    tokens = np.arange(cfg.T)
    _, _, _, gap = O.route(to_numpy(r["logits"]), cfg.n_routed, cfg.top_k, cfg.scoring,
                           cfg.renorm, bias=host(inp.bias))
    compare_h(cfg, gpu_h_as_f64(r["h"]), oracle_h(cfg, inp, tokens, idx, gate), gap)


def test_segmentation_identity_on_gpu():
    """m fine experts (column slices) with the coarse gate reproduce the
    coarse expert: the GPU layer agrees with itself across the split."""
    base = scaled(CONFIGS["mid"], T=200, d_model=256, d_ff=256).with_(
        n_routed=8, top_k=2, n_shared=1, d_ff_shared=64)
    m = 4
    fine = base.with_(name="fine", n_routed=32, top_k=8, d_ff=64)
    inp = small_inputs(base)
    rng = np.random.default_rng(2)
    idx = np.stack([rng.choice(8, 2, replace=False) for _ in range(base.T)]).astype(np.int32)
    gate = rng.random((base.T, 2)).astype(np.float32)
    hc = B.forward(base, inp.x, torch.from_numpy(idx).cuda(), torch.from_numpy(gate).cuda(),
                   inp.w13, inp.w2, inp.w13s, inp.w2s)
    f, fm = base.d_ff, base.d_ff // m
    w13f = torch.empty((32, 2 * fm, base.d_model), dtype=inp.w13.dtype, device="cuda")
    w2f = torch.empty((32, base.d_model, fm), dtype=inp.w2.dtype, device="cuda")
    for e in range(8):
        for j in range(m):
            w13f[e * m + j, :fm] = inp.w13[e, j * fm:(j + 1) * fm]
            w13f[e * m + j, fm:] = inp.w13[e, f + j * fm:f + (j + 1) * fm]
            w2f[e * m + j] = inp.w2[e, :, j * fm:(j + 1) * fm]
    idxf = np.array([[e * m + j for e in row for j in range(m)] for row in idx], np.int32)
    gatef = np.repeat(gate, m, axis=1)
    hf = B.forward(fine, inp.x, torch.from_numpy(idxf).cuda(), torch.from_numpy(gatef).cuda(),
                   w13f.contiguous(), w2f.contiguous(), inp.w13s, inp.w2s)
    torch.cuda.synchronize()
    h_ref = oracle_h(base, inp, np.arange(base.T), idx, gate)
    compare_h(base, gpu_h_as_f64(hc), h_ref, np.full(base.T, np.inf))
    compare_h(base, gpu_h_as_f64(hf), h_ref, np.full(base.T, np.inf))


# ---------------------------------------------------------------- full sizes
#
# The benchmark's workloads at full size, launched as the benchmark launches
# them.  Routing of every token is checked bit-exactly on identical logits.
# The layer output is checked against the oracle on every token of the V3
# prefill batch (in four chunks of 2048 tokens, one test each) and, for the
# other workloads, on tokens chosen so that every row tile of every group of
# the expert GEMMs is hit at its first and at its last row (the tile
# boundaries the GEMMs' work lists draw), plus the first and last token of
# each 256-token slice of the shared group.

FULL = ["v3_decode", "mid", "v3_prefill", "v4_skew", "v4_hash"]
_STATE = {}             # the one full-size workload kept between tests


def full_state(cfg):
    """GPU inputs, the GPU layer's outputs and the host copies the oracle
    reads, for one full-size workload (kept until another is asked for)."""
    if cfg.name in _STATE:
        return _STATE[cfg.name]
    _STATE.clear()
    torch.cuda.empty_cache()
    print(f"[full-size] {cfg.name}: generating inputs", flush=True)
    inp = make_inputs(cfg, "cuda")
    print(f"[full-size] {cfg.name}: GPU layer", flush=True)
    r = gpu_layer(cfg, inp)
    print(f"[full-size] {cfg.name}: routing parity", flush=True)
    check_routing_identical_logits(cfg, inp, r)
    st = {"inp": inp, "r": r, "x_h": host(inp.x), "h_gpu": gpu_h_as_f64(r["h"]),
          "idx": to_numpy(r["idx"])}
    _STATE[cfg.name] = st
    return st


def check_tokens(cfg, st, tokens):
    inp, x_h = st["inp"], st["x_h"]
    print(f"[full-size] {cfg.name}: oracle on {len(tokens)} tokens", flush=True)
    _, idx, gate, _, gap = oracle_route_tokens(cfg, inp, tokens, x_h=x_h)
    h_ref = oracle_h(cfg, inp, tokens, idx, gate, x_h=x_h)
    res = compare_h(cfg, st["h_gpu"][tokens], h_ref, gap)
    print(f"[full-size] {cfg.name}: tokens {len(tokens)} max_abs {res[0]:.4g} "
          f"rel_l2 {res[1]:.4g} near-tie excluded {res[2]}", flush=True)
    return res


@pytest.mark.parametrize("chunk", range(4))
def test_v3_prefill_every_token(chunk):
    """Every token of the V3 prefill batch (8192) against the oracle, 2048
    per test."""
    cfg = CONFIGS["v3_prefill"]
    st = full_state(cfg)
    n = cfg.T // 4
    check_tokens(cfg, st, np.arange(chunk * n, (chunk + 1) * n))


@pytest.mark.parametrize("name", ["v3_decode", "mid", "v4_skew", "v4_hash"])
def test_full_size_workload(name):
    """Routing of every token bit-exact on identical logits; the layer
    output on every row tile's first and last row (every token of the
    64-token decode batch)."""
    cfg = CONFIGS[name]
    st = full_state(cfg)
    if cfg.T <= 64:
        tokens = np.arange(cfg.T)
    else:
        tokens = row_tile_tokens(st["idx"], cfg.T, cfg.n_routed, cfg.n_shared > 0)
    check_tokens(cfg, st, tokens)


def test_large_batch():
    """The V3 layer at T = 65536: 524,288 pairs (8 times the benchmark's
    batch), about 2,300 row tiles per GEMM and 2,048-pair permutation
    chunks; every row tile's first and last row against the oracle."""
    cfg = CONFIGS["v3_prefill"].with_(name="v3_T65536", T=65536)
    st = full_state(cfg)
    check_tokens(cfg, st, row_tile_tokens(st["idx"], cfg.T, cfg.n_routed, cfg.n_shared > 0))


@pytest.mark.parametrize("name", ["v3_prefill", "v4_skew"])
def test_full_size_forward_is_bitwise_repeatable(name):
    """At full size the order in which blocks pull and steal work items
    differs from run to run; the output may not: h of two more forward
    passes over the same routing equals the first bit for bit."""
    cfg = CONFIGS[name]
    st = full_state(cfg)
    inp, r = st["inp"], st["r"]
    ws = B.alloc_workspace(B.make_config(cfg), B.WS_FORWARD, "cuda")
    for _ in range(2):
        h2 = B.forward(cfg, inp.x, r["idx"], r["w"], inp.w13, inp.w2, inp.w13s, inp.w2s,
                       workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(r["h"].view(torch.int16), h2.view(torch.int16))
    del ws
