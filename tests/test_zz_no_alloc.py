"""moe_forward_static (the entry point that allocates nothing: its scratch is
a library-owned device array) against moe_forward on the same inputs,
through the C ABI.  Two calls in a row, the second with a smaller batch, so
the second runs on scratch the first left behind; then a config too large
for the scratch is refused.  The two entry points run the same kernels and
the layer output is bitwise reproducible, so the outputs must be the same
bits."""
import pytest
import torch

from fine_grained_moe_router_amd import binding as B
from fine_grained_moe_router_amd.configs import CONFIGS, scaled
from fine_grained_moe_router_amd.synth import make_inputs

pytestmark = pytest.mark.gpu


def route_and_compare(cfg, inp, T):
    c = cfg.with_(T=T)
    x = inp.x[:T].contiguous()
    tid = None if inp.token_ids is None else inp.token_ids[:T].contiguous()
    r = B.route(c, x=x, w_gate=inp.w_gate, offset=inp.offset, bias=inp.bias, token_ids=tid,
                want_pstat=False)
    ref = B.forward(c, x, r["idx"], r["w"], inp.w13, inp.w2, inp.w13s, inp.w2s)
    got = torch.full_like(ref, 7)   # every element must be overwritten
    B.forward_static(c, x, r["idx"], r["w"], inp.w13, inp.w2, inp.w13s, inp.w2s, h=got)
    torch.cuda.synchronize()
    print(f"[no-alloc] {cfg.name} T={T}: compared", flush=True)
    assert torch.equal(ref.view(torch.uint8), got.view(torch.uint8)), (cfg.name, T)


@pytest.mark.parametrize("name", ["v3_decode", "v3_128", "toy_fp32", "hash_small"])
def test_forward_static_matches_forward(name):
    if name == "hash_small":
        cfg = scaled(CONFIGS["v4_hash"], T=256, d_model=512, d_ff=256)
    elif name == "v3_128":   # the largest V3 batch the scratch holds
        cfg = CONFIGS["v3_decode"].with_(name="v3_128", T=128)
    else:
        cfg = CONFIGS[name]
    inp = make_inputs(cfg, "cuda")
    route_and_compare(cfg, inp, cfg.T)
    route_and_compare(cfg, inp, max(1, cfg.T // 3))


def test_forward_static_refuses_configs_beyond_its_scratch():
    cfg = CONFIGS["v3_decode"].with_(T=4096)
    c = B.make_config(cfg)
    assert B.workspace_bytes(c, B.WS_FORWARD) > 64 << 20
    p = [torch.empty(256, dtype=torch.uint8, device="cuda") for _ in range(8)]
    import ctypes
    rc = B.lib().moe_forward_static(ctypes.byref(c), *[ctypes.c_void_p(t.data_ptr()) for t in p],
                                    None)
    assert rc == B.MOE_ERR_UNSUPPORTED
