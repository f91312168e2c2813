"""The shared experts' fp16 down pass and its fallback.

Where the shared group has more than 128 rows, the down projection runs it
in fp16: z rounded once to fp16 against the shared W2 converted to fp16.
A value fp16 cannot hold (in z, or in the shared W2) sets a flag, and the
down launch then runs the (hi, lo) bf16 pair instead.  These tests read the
flag back from the forward workspace (parity.forward_workspace_layout) and
hold h to the oracle in every case: within the end-to-end tolerance for
ordinary weights, and within the same error relative to the output's scale
where weights are scaled up."""
import numpy as np
import pytest
import torch

from fine_grained_moe_router_amd import binding as B
from fine_grained_moe_router_amd.configs import CONFIGS, scaled
from fine_grained_moe_router_amd.synth import make_inputs

from parity import (check_routing_identical_logits, compare_h, forward_workspace_layout,
                    gpu_h_as_f64, oracle_h)

pytestmark = pytest.mark.gpu

CFG = scaled(CONFIGS["v3_prefill"], T=300, d_model=256, d_ff=128)


def inputs(cfg, w13s_scale=1.0, w2s_scale=1.0):
    inp = make_inputs(cfg, "cpu")
    # powers of two: exact in bf16, so the scaled layer is the same layer
    inp.w13s = (inp.w13s.float() * w13s_scale).to(torch.bfloat16)
    inp.w2s = (inp.w2s.float() * w2s_scale).to(torch.bfloat16)
    for k in ("x", "w_gate", "w13", "w2", "w13s", "w2s", "bias", "offset"):
        v = getattr(inp, k)
        if v is not None:
            setattr(inp, k, v.cuda())
    return inp


def layer_and_flag(cfg, inp):
    r = B.route(cfg, x=inp.x, w_gate=inp.w_gate, offset=inp.offset, bias=inp.bias,
                logits_out=True)
    ws = B.alloc_workspace(B.make_config(cfg), B.WS_FORWARD, "cuda")
    h = B.forward(cfg, inp.x, r["idx"], r["w"], inp.w13, inp.w2, inp.w13s, inp.w2s, workspace=ws)
    f, P, loss = B.balance_stats(cfg, r["counts"], r["pstat"])
    torch.cuda.synchronize()
    r.update(h=h, f=f, P=P, loss=loss)
    _, _, off_meta, _, _ = forward_workspace_layout(cfg.T, cfg.top_k, cfg.n_routed,
                                                    cfg.n_shared)
    G = cfg.n_routed + 1
    at = off_meta + 4 * (5 * G + 40)
    flag = int(ws[at:at + 4].cpu().view(torch.int32)[0])
    return r, flag


def oracle_on_gpu_routing(cfg, inp, r):
    idx, gate = check_routing_identical_logits(cfg, inp, r)
    tokens = np.arange(cfg.T)
    return gpu_h_as_f64(r["h"]), oracle_h(cfg, inp, tokens, idx, gate)


def test_fp16_pass_runs_and_meets_the_tolerance():
    inp = inputs(CFG)
    r, flag = layer_and_flag(CFG, inp)
    assert flag == 0
    h, h_ref = oracle_on_gpu_routing(CFG, inp, r)
    compare_h(CFG, h, h_ref, np.full(CFG.T, np.inf))


@pytest.mark.parametrize("what", ["w2s", "z"])
def test_values_beyond_fp16_fall_back_to_the_bf16_pair(what):
    """The shared W2 scaled by 2^20 (entries far beyond 65504), or the shared
    W13 by 2^9 (z ~ 2^18 beyond 65504): the flag is set, and h still matches
    the oracle to the tolerance's relative size."""
    if what == "w2s":
        inp = inputs(CFG, w2s_scale=2.0 ** 20)
    else:
        inp = inputs(CFG, w13s_scale=2.0 ** 9)
    r, flag = layer_and_flag(CFG, inp)
    assert flag == 1
    h, h_ref = oracle_on_gpu_routing(CFG, inp, r)
    assert np.isfinite(h).all()
    scale = np.abs(h_ref).max()
    assert scale > 1e5                                   # the shared term dominates
    err = np.abs(h - h_ref)
    assert err.max() <= 1e-2 * scale, err.max() / scale
    assert np.linalg.norm(err) <= 5e-3 * np.linalg.norm(h_ref)
