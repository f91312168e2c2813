"""The whole layer driven from C.  The C program of tests/c_caller (built
beside libmoe.so) reads a config and the layer's inputs from a file, runs
moe_route (logits written out), moe_forward and moe_balance_stats through
include/moe.h alone, on its own HIP stream, and writes the outputs back.
They are held to the same bar as the Python binding's: routing bit-exact
against the oracle on the program's logits, gates within 1 ulp, f
bit-exact, P and the loss to 1e-6, and h within the end-to-end tolerance
of the oracle's layer on the program's routing."""
import subprocess

import numpy as np
import pytest
import torch

from fine_grained_moe_router_amd import binding as B
from fine_grained_moe_router_amd import build as hipbuild
from fine_grained_moe_router_amd.configs import CONFIGS, scaled
from fine_grained_moe_router_amd.synth import make_inputs, to_numpy

from parity import check_routing_identical_logits, compare_h, gpu_h_as_f64, host, oracle_h

pytestmark = pytest.mark.gpu

MAGIC = 0x4D4F4531
CASES = {
    # bf16, sigmoid + renormalisation + selection bias, one shared expert
    "v3_small": scaled(CONFIGS["v3_prefill"], T=300, d_model=512, d_ff=128),
    # fp32, softmax, 64 experts from 16 split m = 4
    "toy_fp32": CONFIGS["toy_fp32"],
    # bf16, sqrt(softplus) with a Zipf logit offset, 32 node groups, M = 4
    "v4_nodes": scaled(CONFIGS["v4_skew"], T=200, d_model=384, d_ff=128).with_(n_groups=32,
                                                                              topk_groups=4),
}


def write_input(path, cfg, inp):
    mc = B.make_config(cfg)
    hdr = np.array([MAGIC] + [getattr(mc, f) for f, _ in B.MoeConfig._fields_], np.int32)
    parts = [hdr.tobytes(), np.float32(cfg.alpha1).tobytes(),
             np.int32(inp.offset is not None).tobytes(), np.int32(inp.bias is not None).tobytes()]
    for t in (inp.x, inp.w_gate, inp.offset, inp.bias, inp.w13, inp.w2, inp.w13s, inp.w2s):
        if t is not None:
            parts.append(np.ascontiguousarray(to_numpy(t)).tobytes())
    path.write_bytes(b"".join(parts))


def read_output(path, cfg):
    T, d, N, K = cfg.T, cfg.d_model, cfg.n_routed, cfg.top_k
    hdt = np.uint16 if cfg.dtype == "bf16" else np.float32
    spec = [("logits", np.float32, T * N, (T, N)), ("idx", np.int32, T * K, (T, K)),
            ("w", np.float32, T * K, (T, K)), ("counts", np.int32, N, (N,)),
            ("h", hdt, T * d, (T, d)), ("f", np.float32, N, (N,)), ("P", np.float32, N, (N,)),
            ("loss", np.float32, 2, (2,))]
    raw = path.read_bytes()
    out, off = {}, 0
    for name, dt, n, shape in spec:
        a = np.frombuffer(raw, dt, n, off).reshape(shape)
        off += a.nbytes
        out[name] = a
    assert off == len(raw)
    return out


@pytest.mark.parametrize("name", list(CASES))
def test_layer_from_c(tmp_path, name):
    cfg = CASES[name]
    assert hipbuild.CALLER.exists(), "the C caller is not built (run __graft_entry__.build())"
    inp = make_inputs(cfg, "cpu")
    fin, fout = tmp_path / "in.bin", tmp_path / "out.bin"
    write_input(fin, cfg, inp)
    print(f"[c-caller] {name}", flush=True)
    r = subprocess.run([str(hipbuild.CALLER), str(fin), str(fout)], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, (r.stdout, r.stderr)
    o = read_output(fout, cfg)
    res = {k: torch.from_numpy(np.array(v)) for k, v in o.items() if k != "h"}
    idx, gate = check_routing_identical_logits(cfg, inp, res)
    if cfg.dtype == "bf16":
        h = torch.from_numpy(o["h"].view(np.int16).copy()).view(torch.bfloat16)
    else:
        h = torch.from_numpy(o["h"].copy())
    tokens = np.arange(cfg.T)
    h_ref = oracle_h(cfg, inp, tokens, idx, gate, x_h=host(inp.x))
    res_h = compare_h(cfg, gpu_h_as_f64(h), h_ref, np.full(cfg.T, np.inf))
    print(f"[c-caller] {name}: max_abs {res_h[0]:.4g} rel_l2 {res_h[1]:.4g}", flush=True)
