"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI,
run the CPU oracle on the very same input bytes, compare."""
from __future__ import annotations

import numpy as np
import torch

from fine_grained_moe_router_amd import binding as B
from fine_grained_moe_router_amd.configs import LayerConfig
from fine_grained_moe_router_amd.synth import LayerInputs, to_numpy
from oracle import oracle as O

# End-to-end tolerances.  bf16: max-abs 2e-2 and relative L2 5e-3, tokens
# whose oracle gap between the K'-th and (K'+1)-th selection score is below
# 1e-4 excluded.  fp32: max-abs 1e-4, rel-L2 1e-5, gap threshold 1e-6.
TOL = {"bf16": dict(max_abs=2e-2, rel_l2=5e-3, gap=1e-4),
       "f32": dict(max_abs=1e-4, rel_l2=1e-5, gap=1e-6)}
ROW_TILE = 256          # rows per row tile of the bf16 expert GEMMs


def gpu_layer(cfg: LayerConfig, inp: LayerInputs, logits_out: bool = True):
    """moe_route + moe_forward + moe_balance_stats on the current stream."""
    hashed = cfg.scoring == "hash"
    r = B.route(cfg, x=inp.x, w_gate=inp.w_gate, offset=inp.offset, bias=inp.bias,
                token_ids=inp.token_ids, logits_out=logits_out and not hashed,
                want_pstat=not hashed)
    h = B.forward(cfg, inp.x, r["idx"], r["w"], inp.w13, inp.w2, inp.w13s, inp.w2s)
    f, P, loss = B.balance_stats(cfg, r["counts"], r["pstat"], want_P=not hashed,
                                 want_loss=not hashed)
    torch.cuda.synchronize()
    r.update(h=h, f=f, P=P, loss=loss)
    return r


def host(t):
    return None if t is None else to_numpy(t)


def host_experts(w: torch.Tensor, needed) -> np.ndarray:
    """A host copy of a [N][...] weight tensor holding only the listed
    experts (the rest stays as untouched zero pages)."""
    dt = np.uint16 if w.dtype == torch.bfloat16 else np.float32
    out = np.zeros(tuple(w.shape), dt)
    for e in sorted(set(int(v) for v in needed)):
        out[e] = to_numpy(w[e])
    return out


def oracle_route_tokens(cfg: LayerConfig, inp: LayerInputs, tokens, x_h=None):
    """Oracle logits (its own GEMM, double accumulation) and routing for the
    listed tokens."""
    if cfg.scoring == "hash":
        tid = to_numpy(inp.token_ids).view(np.uint32)[tokens]
        idx, gate, s32, gap = O.route(None, cfg.n_routed, cfg.top_k, "hash", False, token_ids=tid)
        return None, idx, gate, s32, gap
    x_h = host(inp.x) if x_h is None else x_h
    lg = O.router_logits(x_h, host(inp.w_gate), tokens=tokens)
    idx, gate, s32, gap = O.route(lg, cfg.n_routed, cfg.top_k, cfg.scoring, cfg.renorm,
                                  offset=host(inp.offset), bias=host(inp.bias),
                                  n_groups=cfg.n_groups, topk_groups=cfg.topk_groups)
    return lg, idx, gate, s32, gap


def oracle_h(cfg: LayerConfig, inp: LayerInputs, tokens, idx_t, gate_t, x_h=None):
    """Oracle layer output (double) for the listed tokens given their routing
    (idx_t/gate_t rows aligned with `tokens`)."""
    x_h = host(inp.x) if x_h is None else x_h
    T = x_h.shape[0]
    idx_full = np.full((T, cfg.top_k), -1, np.int32)
    gate_full = np.zeros((T, cfg.top_k), np.float32)
    idx_full[tokens] = idx_t
    gate_full[tokens] = gate_t
    w13 = host_experts(inp.w13, idx_t.ravel())
    w2 = host_experts(inp.w2, idx_t.ravel())
    return O.forward(x_h, idx_full, gate_full, w13, w2, host(inp.w13s), host(inp.w2s), tokens=tokens)


def compare_h(cfg: LayerConfig, h_gpu: np.ndarray, h_ref: np.ndarray, gap: np.ndarray):
    """Assert the end-to-end tolerance on tokens whose gap is not a near tie.
    Returns (max_abs, rel_l2, n_excluded)."""
    tol = TOL[cfg.dtype]
    keep = gap >= tol["gap"]
    assert keep.sum() >= max(1, int(0.5 * len(keep))), "too many near-tie tokens"
    a = h_gpu[keep].astype(np.float64)
    b = h_ref[keep]
    diff = a - b
    max_abs = float(np.abs(diff).max())
    rel = float(np.linalg.norm(diff) / max(np.linalg.norm(b), 1e-30))
    assert max_abs <= tol["max_abs"], (max_abs, rel)
    assert rel <= tol["rel_l2"], (max_abs, rel)
    return max_abs, rel, int((~keep).sum())


def gpu_h_as_f64(h: torch.Tensor) -> np.ndarray:
    return h.detach().float().cpu().numpy().astype(np.float64)


def row_tile_tokens(idx: np.ndarray, T: int, n_routed: int, has_shared: bool) -> np.ndarray:
    """Tokens at the first and the last row of every row tile of every group:
    a routed expert's rows are its (token, slot) pairs in pair order, dealt
    over R = ceil(rows / 256) row tiles in whole 32-row fragments (32
    ceil(rows / (32 R)) rows per tile, the rest in the last); the shared
    group's rows are the tokens in order, 256 per tile."""
    K = idx.shape[1]
    pairs = np.argsort(idx.ravel(), kind="stable")
    ids = idx.ravel()[pairs]
    out = set()
    for e in range(n_routed):
        lo, hi = np.searchsorted(ids, [e, e + 1])
        cnt = hi - lo
        if cnt == 0:
            continue
        R = -(-cnt // ROW_TILE)
        rpt = min(ROW_TILE, 32 * (-(-cnt // (32 * R))))
        for i in range(R):
            a, b = i * rpt, min(cnt, (i + 1) * rpt) - 1
            if a > b:
                continue
            out.add(int(pairs[lo + a]) // K)
            out.add(int(pairs[lo + b]) // K)
    if has_shared:
        for t0 in range(0, T, ROW_TILE):
            out.update((t0, min(T, t0 + ROW_TILE) - 1))
    return np.array(sorted(out), np.int64)


def check_routing_identical_logits(cfg, inp, r):
    """GPU logits -> oracle: same indices, counts, gates (<= 1 ulp), stats."""
    hashed = cfg.scoring == "hash"
    if hashed:
        tid = to_numpy(inp.token_ids).view(np.uint32)
        idx, gate, s32, _ = O.route(None, cfg.n_routed, 1, "hash", False, token_ids=tid)
    else:
        lg = to_numpy(r["logits"])
        idx, gate, s32, _ = O.route(lg, cfg.n_routed, cfg.top_k, cfg.scoring, cfg.renorm,
                                    offset=host(inp.offset), bias=host(inp.bias),
                                    n_groups=cfg.n_groups, topk_groups=cfg.topk_groups)
    gidx = to_numpy(r["idx"])
    np.testing.assert_array_equal(gidx, idx)
    cnt = O.counts(idx, cfg.n_routed)
    np.testing.assert_array_equal(to_numpy(r["counts"]), cnt)
    gw = to_numpy(r["w"])
    ulps = np.abs(gw - gate) / np.spacing(np.abs(gate))
    assert ulps.max() <= 1.0, ulps.max()
    a1 = float(np.float32(cfg.alpha1))
    f, P, loss = O.balance_stats(cnt, s32, cfg.T, cfg.top_k, a1)
    np.testing.assert_array_equal(to_numpy(r["f"]), f.astype(np.float32))
    if not hashed:
        np.testing.assert_allclose(to_numpy(r["P"]), P, rtol=1e-6, atol=1e-12)
        np.testing.assert_allclose(to_numpy(r["loss"]), loss, rtol=1e-6)
    return idx, gate


def align256(v):
    return (v + 255) & ~255


def forward_workspace_layout(T, K, N, n_shared):
    """Offsets into moe_forward's workspace, restating the library's layout
    (per-chunk counts, the metadata block of 5 G + 41 ints, then the pair ids
    and the gates, each 256-byte aligned): (pair chunk, chunks, offset of the
    metadata, of the pair ids, of the gates).  A change of that layout must
    be made here too."""
    P = T * K
    chunk = max(64, -(-(-(-P // 256)) // 64) * 64)
    n_chunks = -(-P // chunk)
    G = N + (1 if n_shared else 0)
    off_meta = align256(n_chunks * N * 4)
    off_perm = align256(off_meta + (5 * G + 41) * 4)
    off_gsort = align256(off_perm + P * 4)
    return chunk, n_chunks, off_meta, off_perm, off_gsort
