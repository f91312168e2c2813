"""The stable permutation of moe_forward, read back from its workspace.

moe_forward's first step sorts the (token, slot) pairs p = t K' + k by the
expert they chose, keeping pair order within an expert (a stable counting
sort of topk_idx), and carries each pair's gate along; pairs with an
out-of-range expert are dropped.  This is integer work, so it must equal
numpy's stable argsort exactly: the pair id at every expert-ordered row,
the gate beside it, and every expert's row count and first row.

The arrays live in the forward workspace; their offsets below restate the
library's workspace layout (per-chunk counts, the metadata block, then the
pair ids and the gates, each 256-byte aligned), so a change of that layout
must be made here too.  Routings are seeded numpy draws; the GEMMs run at
d = d_ff = 64, since the permutation does not depend on the widths."""
import numpy as np
import pytest
import torch

from fine_grained_moe_router_amd import binding as B
from fine_grained_moe_router_amd.configs import CONFIGS, scaled
from fine_grained_moe_router_amd.synth import make_inputs, make_share_routing

from parity import forward_workspace_layout as layout

pytestmark = pytest.mark.gpu


def distinct_rows(rng, T, K, N):
    """T rows of K distinct experts, skewed towards low ids."""
    keys = rng.random((T, N)) * (1.0 + np.arange(N) / N) ** 2
    return np.argsort(keys, axis=1)[:, :K].astype(np.int32)


def case(name):
    rng = np.random.default_rng(len(name) * 7919)
    if name == "v3_batch":
        T, K, N, S = 8192, 8, 256, 1
        idx = distinct_rows(rng, T, K, N)
    elif name == "ep_share":
        T, K, N, S = 16384, 8, 32, 0
        idx = make_share_routing(T, N, K, seed=5)[0].numpy()
    elif name == "wide_with_dropped":
        T, K, N, S = 1000, 16, 1024, 2
        idx = distinct_rows(rng, T, K, N)
        idx[::5, 3] = -1
        idx[1::7, 9] = N + 11
    elif name == "largest_batch":
        T, K, N, S = 1 << 19, 8, 256, 1
        idx = distinct_rows(rng, T, K, N)
    elif name == "one_token":
        T, K, N, S = 1, 8, 256, 1
        idx = distinct_rows(rng, T, K, N)
    elif name == "one_expert":
        T, K, N, S = 300, 1, 1, 0
        idx = np.zeros((T, K), np.int32)
    else:
        raise KeyError(name)
    gate = rng.random((T, K)).astype(np.float32)
    cfg = scaled(CONFIGS["v3_prefill"], T=T, d_model=64, d_ff=64, name=name).with_(
        top_k=K, n_routed=N, n_shared=S, d_ff_shared=64)
    return cfg, idx, gate


@pytest.mark.parametrize("name", ["v3_batch", "ep_share", "wide_with_dropped", "largest_batch",
                                  "one_token", "one_expert"])
def test_permutation_is_the_stable_sort(name):
    cfg, idx, gate = case(name)
    T, K, N = cfg.T, cfg.top_k, cfg.n_routed
    print(f"[permute] {name}: T {T} K' {K} N' {N}", flush=True)
    inp = make_inputs(cfg, "cuda")
    ws = B.alloc_workspace(B.make_config(cfg), B.WS_FORWARD, "cuda")
    B.forward(cfg, inp.x, torch.from_numpy(idx).cuda(), torch.from_numpy(gate).cuda(),
              inp.w13, inp.w2, inp.w13s, inp.w2s, workspace=ws)
    torch.cuda.synchronize()
    _, _, off_meta, off_perm, off_gsort = layout(T, K, N, cfg.n_shared)
    P = T * K
    w = ws.cpu().numpy()
    perm = w[off_perm:off_perm + 4 * P].view(np.int32)
    gsort = w[off_gsort:off_gsort + 4 * P].view(np.uint32)
    G = N + (1 if cfg.n_shared else 0)
    meta = w[off_meta:off_meta + 4 * (5 * G + 41)].view(np.int32)

    ids = idx.ravel()
    valid = (ids >= 0) & (ids < N)
    n = int(valid.sum())
    order = np.argsort(np.where(valid, ids, N), kind="stable")[:n]
    counts = np.bincount(ids[valid], minlength=N)
    np.testing.assert_array_equal(perm[:n], order)
    np.testing.assert_array_equal(gsort[:n], gate.ravel().view(np.uint32)[order])
    np.testing.assert_array_equal(meta[G + 1:G + 1 + N], counts)                   # rows per expert
    np.testing.assert_array_equal(meta[:N], np.concatenate([[0], np.cumsum(counts)[:-1]]))
