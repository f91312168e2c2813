"""Router GEMM (the linear gating network, freedeepseekapi.com blog sec. 2)
against the CPU oracle, element by element.

bf16 x bf16 products are exact in fp32, so an fp32 sum of d of them, added
in any order (including the split-K partials and their sum), is within
gamma_n * sum_k |x_k w_k| of the exact value, gamma_n = n u / (1 - n u),
u = 2^-24, n = d + 16 (at most 16 partial sums).  The oracle sums in double
and rounds once, adding u |l|.  Full-size batches are checked on sampled
tokens (the first, the last, and a seeded sample), small ones on all."""
import numpy as np
import pytest
import torch

from fine_grained_moe_router_amd import binding as B
from fine_grained_moe_router_amd.configs import CONFIGS, scaled
from fine_grained_moe_router_amd.synth import make_inputs, to_numpy
from oracle import oracle as O

pytestmark = pytest.mark.gpu

CASES = {
    # one 256-expert column tile, 128-token row blocks, d split 4 ways on 256 CUs
    "v3_prefill": CONFIGS["v3_prefill"],
    # one partial 256-row tile (64 tokens), d split to fill the device
    "v3_decode": CONFIGS["v3_decode"],
    # 384 experts: a second, half-empty column tile; 256-token row tiles
    "v4_skew": CONFIGS["v4_skew"],
    # 64 experts (softmax, one per lane): a mostly empty column tile; 128-token row blocks
    "mid": CONFIGS["mid"],
    # 385 experts: a second column tile with 129 valid rows
    "n385": scaled(CONFIGS["v3_prefill"], T=4096, d_model=512, d_ff=128).with_(n_routed=385),
    # ragged row blocks (333 = 128 + 128 + 77 tokens), two d ranges
    "ragged": scaled(CONFIGS["v3_prefill"], T=333, d_model=1024, d_ff=128),
    # d of 4 k-tiles: no split
    "narrow": scaled(CONFIGS["mid"], T=700, d_model=256, d_ff=64),
}


def f64(t):
    return to_numpy(t.float()).astype(np.float64)


@pytest.mark.parametrize("name", list(CASES))
def test_router_logits_match_oracle(name):
    cfg = CASES[name]
    inp = make_inputs(cfg, "cuda", experts=False)
    r1 = B.route(cfg, x=inp.x, w_gate=inp.w_gate, offset=inp.offset, bias=inp.bias,
                 logits_out=True)
    r2 = B.route(cfg, x=inp.x, w_gate=inp.w_gate, offset=inp.offset, bias=inp.bias,
                 logits_out=True)
    torch.cuda.synchronize()
    lg = to_numpy(r1["logits"])
    # bitwise reproducible: the split partials are added in a fixed order
    assert np.array_equal(lg.view(np.uint32), to_numpy(r2["logits"]).view(np.uint32))
    T = cfg.T
    if T <= 1024:
        tok = np.arange(T)
    else:
        rng = np.random.default_rng(7)
        tok = np.unique(np.concatenate([[0, T - 1], rng.choice(T, 190, replace=False)]))
    x = to_numpy(inp.x.cpu())
    wg = to_numpy(inp.w_gate.cpu())
    ref = O.router_logits(x, wg, tokens=tok)
    got = lg[tok]
    assert got.shape == ref.shape and np.isfinite(got).all()
    xa = np.abs(f64(inp.x.cpu())[tok])
    wa = np.abs(f64(inp.w_gate.cpu()))
    mag = xa @ wa.T                                     # sum_k |x_k w_k|
    n = cfg.d_model + 16
    u = 2.0 ** -24
    bound = n * u / (1 - n * u) * mag + u * np.abs(ref.astype(np.float64))
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    assert (err <= bound).all(), (name, float((err / np.maximum(bound, 1e-30)).max()))
    # and the typical error is far below the worst case
    assert float(np.median(err)) <= 0.05 * float(np.median(bound)) + 1e-7


@pytest.mark.parametrize("name", list(CASES))
def test_routing_without_logits_out_is_identical(name):
    """The select kernel adds the router's split partials itself.  Whether
    or not the caller asks for the summed logits (MOE_LOGITS_OUT), the
    routing, counts and score partial sums are the same bits."""
    cfg = CASES[name]
    inp = make_inputs(cfg, "cuda", experts=False)
    a = B.route(cfg, x=inp.x, w_gate=inp.w_gate, offset=inp.offset, bias=inp.bias,
                logits_out=True)
    b = B.route(cfg, x=inp.x, w_gate=inp.w_gate, offset=inp.offset, bias=inp.bias,
                logits_out=False)
    torch.cuda.synchronize()
    for k in ("idx", "w", "counts", "pstat"):
        assert torch.equal(a[k].view(torch.uint8), b[k].view(torch.uint8)), k
