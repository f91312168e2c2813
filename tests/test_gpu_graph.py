"""The layer step (moe_route + moe_forward + moe_balance_stats) captured in a
HIP graph, for callers that replay it (serving loops).  The library issues
no host synchronisation, allocation or memset inside these calls, so the
step captures as it stands.  Each replay, after eager work that overwrites
every output, must reproduce the eager step bit for bit; the eager step
itself is checked against the oracle by test_gpu_parity.py."""
import pytest
import torch

from fine_grained_moe_router_amd import binding as B
from fine_grained_moe_router_amd.configs import CONFIGS, scaled
from fine_grained_moe_router_amd.synth import make_inputs

pytestmark = pytest.mark.gpu

CASES = {
    "v3_ragged": scaled(CONFIGS["v3_prefill"], T=700, d_model=512, d_ff=128),
    "v4_hash_ragged": scaled(CONFIGS["v4_hash"], T=2000, d_model=256, d_ff=64),
}


@pytest.mark.parametrize("name", list(CASES))
def test_layer_step_replays_in_a_graph(name):
    cfg = CASES[name]
    hashed = cfg.scoring == "hash"
    inp = make_inputs(cfg, "cuda")
    c = B.make_config(cfg)
    T, N, K = cfg.T, cfg.n_routed, cfg.top_k
    dev = "cuda"
    out = {"idx": torch.empty((T, K), dtype=torch.int32, device=dev),
           "w": torch.empty((T, K), dtype=torch.float32, device=dev),
           "counts": torch.empty(N, dtype=torch.int32, device=dev),
           "pstat": None if hashed else torch.empty(B.workspace_bytes(c, B.WS_PSTAT),
                                                     dtype=torch.uint8, device=dev)}
    st = {"f": torch.empty(N, dtype=torch.float32, device=dev),
          "P": torch.empty(N, dtype=torch.float32, device=dev),
          "loss": torch.empty(2, dtype=torch.float32, device=dev)}
    h = torch.empty_like(inp.x)
    ws_r = B.alloc_workspace(c, B.WS_ROUTE, dev)
    ws_f = B.alloc_workspace(c, B.WS_FORWARD, dev)

    def step():
        B.route(cfg, x=inp.x, w_gate=inp.w_gate, offset=inp.offset, bias=inp.bias,
                token_ids=inp.token_ids, want_pstat=not hashed, out=out, workspace=ws_r)
        B.forward(cfg, inp.x, out["idx"], out["w"], inp.w13, inp.w2, inp.w13s, inp.w2s, h=h,
                  workspace=ws_f)
        B.balance_stats(cfg, out["counts"], out["pstat"], want_P=not hashed,
                        want_loss=not hashed, out=st)

    outputs = [out["idx"], out["w"], out["counts"], h, st["f"]]
    if not hashed:
        outputs += [st["P"], st["loss"]]
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outputs]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outputs:                       # eager work between replays
            t.view(torch.uint8).fill_(0xA5 if rep % 2 else 0x5A)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t, r in zip(outputs, ref):
            assert torch.equal(t.view(torch.uint8), r.view(torch.uint8)), (name, rep)
