"""HIP path against the CPU oracle for the rows beyond the layer forward:
node-limited routing, in-sequence and device-level balance statistics, and
the aux-loss-free bias update.  Same bar as the layer: integer results
(indices, counts, f) bit-exact; values computed in double and rounded once
bit-exact when both sides add in the same order (device statistics, bias
update), else within 2 fp32 ulps (p^seq) or 1e-6 relative (losses)."""
import numpy as np
import pytest
import torch

from fine_grained_moe_router_amd import binding as B
from fine_grained_moe_router_amd.configs import CONFIGS, scaled
from fine_grained_moe_router_amd.synth import make_inputs, to_numpy
from oracle import oracle as O

from parity import compare_h, gpu_h_as_f64, gpu_layer, host, oracle_h

pytestmark = pytest.mark.gpu

GROUPED = {
    # V3: 256 experts on 8 nodes, at most 4 nodes per token
    "v3_node4": scaled(CONFIGS["v3_prefill"], T=1500, d_model=512, d_ff=128).with_(
        n_groups=8, topk_groups=4),
    # the V4 book's example layout: 384 experts on 32 nodes of 12, M = 4
    "v4_node4": scaled(CONFIGS["v4_skew"], T=1200, d_model=384, d_ff=128).with_(
        n_groups=32, topk_groups=4),
    "softmax_groups": scaled(CONFIGS["mid"], T=600, d_model=256, d_ff=64).with_(
        n_groups=8, topk_groups=3),
    "one_expert_groups": scaled(CONFIGS["mid"], T=300, d_model=256, d_ff=64).with_(
        n_groups=64, topk_groups=6),
}


def to_gpu(inp):
    for k in ("x", "w_gate", "w13", "w2", "w13s", "w2s", "bias", "offset", "token_ids"):
        v = getattr(inp, k)
        if v is not None:
            setattr(inp, k, v.cuda())
    return inp


def f32(v):
    """A value both sides see identically (the GPU takes fp32 scalars)."""
    return float(np.float32(v))


def check_grouped_routing(cfg, inp, r):
    lg = to_numpy(r["logits"])
    idx, gate, s32, _ = O.route(lg, cfg.n_routed, cfg.top_k, cfg.scoring, cfg.renorm,
                                offset=host(inp.offset), bias=host(inp.bias),
                                n_groups=cfg.n_groups, topk_groups=cfg.topk_groups)
    np.testing.assert_array_equal(to_numpy(r["idx"]), idx)
    np.testing.assert_array_equal(to_numpy(r["counts"]), O.counts(idx, cfg.n_routed))
    gw = to_numpy(r["w"])
    assert (np.abs(gw - gate) / np.spacing(np.abs(gate))).max() <= 1.0
    gsz = cfg.n_routed // cfg.n_groups
    groups = to_numpy(r["idx"]) // gsz
    assert max(len(set(row)) for row in groups) <= cfg.topk_groups
    return idx, gate, s32


@pytest.mark.parametrize("name", list(GROUPED))
def test_grouped_routing_identical_logits(name):
    cfg = GROUPED[name]
    inp = to_gpu(make_inputs(cfg, "cpu", experts=False))
    r = B.route(cfg, x=inp.x, w_gate=inp.w_gate, offset=inp.offset, bias=inp.bias,
                logits_out=True)
    torch.cuda.synchronize()
    check_grouped_routing(cfg, inp, r)


def test_grouped_layer_end_to_end():
    cfg = GROUPED["v3_node4"]
    inp = to_gpu(make_inputs(cfg, "cpu"))
    r = gpu_layer(cfg, inp)
    idx, gate, _ = check_grouped_routing(cfg, inp, r)
    tokens = np.arange(cfg.T)
    _, _, _, gap = O.route(to_numpy(r["logits"]), cfg.n_routed, cfg.top_k, cfg.scoring,
                           cfg.renorm, offset=host(inp.offset), bias=host(inp.bias),
                           n_groups=cfg.n_groups, topk_groups=cfg.topk_groups)
    h_ref = oracle_h(cfg, inp, tokens, idx, gate)
    compare_h(cfg, gpu_h_as_f64(r["h"]), h_ref, gap)


def test_grouped_routing_full_size():
    """V3 prefill shape (T = 8192, d = 7168, 256 experts), 8 nodes, M = 4."""
    cfg = CONFIGS["v3_prefill"].with_(n_groups=8, topk_groups=4)
    inp = make_inputs(cfg, "cuda", experts=False)
    r = B.route(cfg, x=inp.x, w_gate=inp.w_gate, bias=inp.bias, logits_out=True)
    torch.cuda.synchronize()
    check_grouped_routing(cfg, inp, r)


SEQ_CASES = {
    "v3_small": (scaled(CONFIGS["v3_prefill"], T=700, d_model=512, d_ff=128),
                 [0, 1, 1, 300, 699, 700]),
    "softmax_small": (scaled(CONFIGS["mid"], T=333, d_model=256, d_ff=64), [0, 333]),
    "v4_small": (scaled(CONFIGS["v4_skew"], T=500, d_model=384, d_ff=128), [0, 64, 128, 500]),
    "v3_prefill": (CONFIGS["v3_prefill"], [0, 1000, 1000, 4096, 8000, 8192]),
}


@pytest.mark.parametrize("name", list(SEQ_CASES))
def test_seq_balance_stats(name):
    cfg, off = SEQ_CASES[name]
    dev = "cuda" if cfg.T * cfg.d_model > 10 ** 7 else "cpu"
    inp = make_inputs(cfg, dev, experts=False)
    if dev == "cpu":
        inp = to_gpu(inp)
    r = B.route(cfg, x=inp.x, w_gate=inp.w_gate, offset=inp.offset, bias=inp.bias,
                logits_out=True)
    beta = f32(1e-4)
    segs = torch.tensor(off, dtype=torch.int32, device="cuda")
    f, p, loss = B.seq_balance_stats(cfg, r["logits"], r["idx"], segs, beta, offset=inp.offset)
    torch.cuda.synchronize()
    lg = to_numpy(r["logits"])
    idx, _, s32, _ = O.route(lg, cfg.n_routed, cfg.top_k, cfg.scoring, cfg.renorm,
                             offset=host(inp.offset), bias=host(inp.bias))
    np.testing.assert_array_equal(to_numpy(r["idx"]), idx)
    fo, po, lo = O.seq_balance_stats(idx, s32, off, beta)
    np.testing.assert_array_equal(to_numpy(f), fo.astype(np.float32))
    pg = to_numpy(p).astype(np.float64)
    po32 = po.astype(np.float32).astype(np.float64)
    ulps = np.abs(pg - po32) / np.maximum(np.spacing(np.abs(po.astype(np.float32))), 1e-45)
    assert ulps.max() <= 2.0, ulps.max()
    np.testing.assert_allclose(to_numpy(loss), lo, rtol=1e-6, atol=1e-30)


@pytest.mark.parametrize("n_dev", [1, 8, 32, 256])
def test_device_balance_stats(n_dev):
    cfg = scaled(CONFIGS["v3_prefill"], T=900, d_model=256, d_ff=64)
    inp = to_gpu(make_inputs(cfg, "cpu", experts=False))
    r = B.route(cfg, x=inp.x, w_gate=inp.w_gate, bias=inp.bias)
    f, P, _ = B.balance_stats(cfg, r["counts"], r["pstat"])
    a2 = f32(0.05)
    fd, pd, loss = B.device_balance_stats(cfg, f, P, n_dev, a2)
    torch.cuda.synchronize()
    fo, po, lo = O.device_balance_stats(to_numpy(f), to_numpy(P), n_dev, a2)
    np.testing.assert_array_equal(to_numpy(fd), fo.astype(np.float32))
    np.testing.assert_array_equal(to_numpy(pd), po.astype(np.float32))
    assert to_numpy(loss)[0] == np.float32(lo)


def test_bias_update_matches_oracle_and_balances_load():
    """One update bit-exact against the oracle; then a closed loop on a
    Zipf-skewed router (route with the live bias, update from its counts)
    lowers max/mean load."""
    cfg = scaled(CONFIGS["v4_skew"], T=2048, d_model=384, d_ff=128).with_(bias=True)
    inp = to_gpu(make_inputs(cfg, "cpu", experts=False))
    alpha = f32(0.05)
    bias = torch.zeros(cfg.n_routed, dtype=torch.float32, device="cuda")

    def route(b):
        return B.route(cfg, x=inp.x, w_gate=inp.w_gate, offset=inp.offset, bias=b,
                       want_pstat=False)

    r0 = route(bias)
    c0 = to_numpy(r0["counts"])
    b_host = to_numpy(bias).copy()
    B.bias_update(cfg, r0["counts"], cfg.T, alpha, bias)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_numpy(bias), O.bias_update(c0, cfg.T, cfg.top_k, alpha, b_host))
    skew0 = c0.max() / c0.mean()
    for _ in range(80):
        r = route(bias)
        B.bias_update(cfg, r["counts"], cfg.T, alpha, bias)
    c1 = to_numpy(route(bias)["counts"])
    skew1 = c1.max() / c1.mean()
    assert skew0 > 3.0, skew0
    assert skew1 < 0.3 * skew0, (skew0, skew1)
