"""ctypes binding of libmoe.so: the same entry points as include/moe.h.

Argument marshalling only -- shapes, dtypes and device pointers of torch
tensors go in, status codes come out (non-zero raises MoeError).  Every step
of the layer runs in the library's HIP kernels; there is no fallback: if the
library has not been built, ``lib()`` raises.
"""
from __future__ import annotations

import ctypes
from pathlib import Path
from typing import Optional

import torch

from .configs import LayerConfig

import os

# The in-tree library, or (MOE_LIB) another build of the same sources, such
# as the host-sanitised one the CPU sanitizer test makes.
LIB_PATH = Path(os.environ.get("MOE_LIB", Path(__file__).resolve().parent / "libmoe.so"))

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4
SCORING = {"softmax": 0, "sigmoid": 1, "sqrt_softplus": 2, "hash": 3}
DTYPE = {"f32": 0, "bf16": 1}
LOGITS_IN, LOGITS_OUT = 1, 2
WS_ROUTE, WS_FORWARD, WS_PSTAT, WS_SEQSTAT = 0, 1, 2, 3
STAGES = ("router_gemm", "select", "permute", "gate_up", "down", "combine", "stats")

EXPORTS = ("moe_workspace_bytes", "moe_route", "moe_forward", "moe_forward_static",
           "moe_balance_stats",
           "moe_seq_balance_stats", "moe_device_balance_stats", "moe_bias_update",
           "moe_status_string", "moe_profile_enable", "moe_profile_collect")


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


class MoeConfig(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("n_routed", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("n_shared", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("d_ff_shared", ctypes.c_int32), ("scoring", ctypes.c_int32),
                ("renorm", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("flags", ctypes.c_uint32), ("n_groups", ctypes.c_int32),
                ("topk_groups", ctypes.c_int32)]


class StageTimes(ctypes.Structure):
    _fields_ = [("launches", ctypes.c_int32 * 7), ("ms", ctypes.c_double * 7)]


_lib = None


def lib():
    """Load libmoe.so (raises if it is missing: there is no other path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not LIB_PATH.exists():
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m fine_grained_moe_router_amd.build`")
    L = ctypes.CDLL(str(LIB_PATH))
    vp, sz, i32, f32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_float
    cfgp = ctypes.POINTER(MoeConfig)
    L.moe_workspace_bytes.argtypes = [cfgp, i32]
    L.moe_workspace_bytes.restype = sz
    L.moe_route.argtypes = [cfgp] + [vp] * 10 + [vp, sz, vp]
    L.moe_route.restype = i32
    L.moe_forward.argtypes = [cfgp] + [vp] * 9 + [sz, vp]
    L.moe_forward.restype = i32
    L.moe_forward_static.argtypes = [cfgp] + [vp] * 9
    L.moe_forward_static.restype = i32
    L.moe_balance_stats.argtypes = [cfgp, vp, vp, f32, vp, vp, vp, vp]
    L.moe_balance_stats.restype = i32
    L.moe_seq_balance_stats.argtypes = [cfgp, vp, vp, vp, vp, i32, f32, vp, vp, vp, vp, sz, vp]
    L.moe_seq_balance_stats.restype = i32
    L.moe_device_balance_stats.argtypes = [cfgp, vp, vp, i32, f32, vp, vp, vp, vp]
    L.moe_device_balance_stats.restype = i32
    L.moe_bias_update.argtypes = [cfgp, vp, ctypes.c_int64, f32, vp, vp]
    L.moe_bias_update.restype = i32
    L.moe_status_string.argtypes = [i32]
    L.moe_status_string.restype = ctypes.c_char_p
    L.moe_profile_enable.argtypes = [i32]
    L.moe_profile_enable.restype = i32
    L.moe_profile_collect.argtypes = [ctypes.POINTER(StageTimes)]
    L.moe_profile_collect.restype = i32
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def make_config(cfg: LayerConfig, flags: int = 0, T: Optional[int] = None) -> MoeConfig:
    return MoeConfig(cfg.T if T is None else T, cfg.d_model, cfg.n_routed, cfg.top_k,
                     cfg.n_shared, cfg.d_ff, cfg.d_ff_shared, SCORING[cfg.scoring],
                     int(cfg.renorm), DTYPE[cfg.dtype], flags, cfg.n_groups, cfg.topk_groups)


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(rc: int, what: str):
    if rc != MOE_OK:
        raise MoeError(rc, what)


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, shape, dtype, name):
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)} on the GPU, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")
    return t


def _elem(cfg: LayerConfig):
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def workspace_bytes(cfg: MoeConfig, which: int) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(cfg), which))


def alloc_workspace(cfg: MoeConfig, which: int, device) -> torch.Tensor:
    n = workspace_bytes(cfg, which)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def route(cfg: LayerConfig, x=None, w_gate=None, offset=None, bias=None, token_ids=None,
          logits_in: Optional[torch.Tensor] = None, logits_out: bool = False,
          want_pstat: bool = True, out=None, workspace=None, stream=None):
    """moe_route.  Returns dict(idx, w, counts, pstat, logits)."""
    flags = LOGITS_IN if logits_in is not None else (LOGITS_OUT if logits_out else 0)
    c = make_config(cfg, flags)
    dev = next(t.device for t in (x, logits_in, token_ids) if t is not None)
    T, N, K = cfg.T, cfg.n_routed, cfg.top_k
    o = out or {}
    idx = o.get("idx") if o.get("idx") is not None else torch.empty((T, K), dtype=torch.int32, device=dev)
    w = o.get("w") if o.get("w") is not None else torch.empty((T, K), dtype=torch.float32, device=dev)
    counts = o.get("counts") if o.get("counts") is not None else torch.empty(N, dtype=torch.int32, device=dev)
    pstat = None
    if want_pstat and cfg.scoring != "hash":
        pstat = o.get("pstat")
        if pstat is None:
            pstat = torch.empty(workspace_bytes(c, WS_PSTAT), dtype=torch.uint8, device=dev)
    logits = None
    if logits_in is not None:
        logits = _need(logits_in, (T, N), torch.float32, "logits_in")
    elif logits_out:
        logits = o.get("logits") if o.get("logits") is not None else torch.empty((T, N), dtype=torch.float32, device=dev)
    if cfg.scoring == "hash":
        _need(token_ids, (T,), torch.int32, "token_ids")
    elif logits_in is None:
        _need(x, (T, cfg.d_model), _elem(cfg), "x")
        _need(w_gate, (N, cfg.d_model), _elem(cfg), "w_gate")
    if offset is not None:
        _need(offset, (N,), torch.float32, "offset")
    if bias is not None:
        _need(bias, (N,), torch.float32, "bias")
    if workspace is None:
        workspace = alloc_workspace(c, WS_ROUTE, dev)
    rc = lib().moe_route(ctypes.byref(c), _p(x), _p(w_gate), _p(offset), _p(bias), _p(token_ids),
                         _p(logits), _p(idx), _p(w), _p(counts), _p(pstat), _p(workspace),
                         workspace.numel(), _stream(stream))
    _check(rc, "moe_route")
    return {"idx": idx, "w": w, "counts": counts, "pstat": pstat, "logits": logits}


def forward(cfg: LayerConfig, x, idx, w, w13, w2, w13s=None, w2s=None, h=None, workspace=None,
            stream=None) -> torch.Tensor:
    """moe_forward.  Returns h [T][d]."""
    c = make_config(cfg)
    T, d, N, K, f = cfg.T, cfg.d_model, cfg.n_routed, cfg.top_k, cfg.d_ff
    et = _elem(cfg)
    _need(x, (T, d), et, "x")
    _need(idx, (T, K), torch.int32, "idx")
    _need(w, (T, K), torch.float32, "w")
    _need(w13, (N, 2 * f, d), et, "w13")
    _need(w2, (N, d, f), et, "w2")
    if cfg.n_shared > 0:
        fs = cfg.d_ff_shared
        _need(w13s, (cfg.n_shared, 2 * fs, d), et, "w13s")
        _need(w2s, (cfg.n_shared, d, fs), et, "w2s")
    else:
        w13s = w2s = None
    if h is None:
        h = torch.empty((T, d), dtype=et, device=x.device)
    else:
        _need(h, (T, d), et, "h")
    if workspace is None:
        workspace = alloc_workspace(c, WS_FORWARD, x.device)
    rc = lib().moe_forward(ctypes.byref(c), _p(x), _p(idx), _p(w), _p(w13), _p(w2), _p(w13s),
                           _p(w2s), _p(h), _p(workspace), workspace.numel(), _stream(stream))
    _check(rc, "moe_forward")
    return h


def forward_static(cfg: LayerConfig, x, idx, w, w13, w2, w13s=None, w2s=None, h=None,
                   stream=None) -> torch.Tensor:
    """moe_forward_static: moe_forward on the library's own device scratch
    (no workspace argument; the library allocates nothing).  Returns h."""
    c = make_config(cfg)
    T, d, N, K, f = cfg.T, cfg.d_model, cfg.n_routed, cfg.top_k, cfg.d_ff
    et = _elem(cfg)
    _need(x, (T, d), et, "x")
    _need(idx, (T, K), torch.int32, "idx")
    _need(w, (T, K), torch.float32, "w")
    _need(w13, (N, 2 * f, d), et, "w13")
    _need(w2, (N, d, f), et, "w2")
    if cfg.n_shared > 0:
        fs = cfg.d_ff_shared
        _need(w13s, (cfg.n_shared, 2 * fs, d), et, "w13s")
        _need(w2s, (cfg.n_shared, d, fs), et, "w2s")
    else:
        w13s = w2s = None
    if h is None:
        h = torch.empty((T, d), dtype=et, device=x.device)
    else:
        _need(h, (T, d), et, "h")
    rc = lib().moe_forward_static(ctypes.byref(c), _p(x), _p(idx), _p(w), _p(w13), _p(w2),
                                  _p(w13s), _p(w2s), _p(h), _stream(stream))
    _check(rc, "moe_forward_static")
    return h


def balance_stats(cfg: LayerConfig, counts, pstat, alpha1: Optional[float] = None,
                  want_P: bool = True, want_loss: bool = True, out=None, stream=None):
    """moe_balance_stats.  Returns (f, P or None, loss[2] or None)."""
    c = make_config(cfg)
    N = cfg.n_routed
    dev = counts.device
    _need(counts, (N,), torch.int32, "counts")
    o = out or {}
    f = o.get("f") if o.get("f") is not None else torch.empty(N, dtype=torch.float32, device=dev)
    P = (o.get("P") if o.get("P") is not None else torch.empty(N, dtype=torch.float32, device=dev)) if want_P else None
    loss = (o.get("loss") if o.get("loss") is not None else torch.empty(2, dtype=torch.float32, device=dev)) if want_loss else None
    a1 = cfg.alpha1 if alpha1 is None else alpha1
    rc = lib().moe_balance_stats(ctypes.byref(c), _p(counts), _p(pstat), ctypes.c_float(a1),
                                 _p(f), _p(P), _p(loss), _stream(stream))
    _check(rc, "moe_balance_stats")
    return f, P, loss


def seq_balance_stats(cfg: LayerConfig, logits, idx, seg_offsets, beta: float, offset=None,
                      out=None, workspace=None, stream=None):
    """moe_seq_balance_stats.  seg_offsets: int32 [S+1] on the GPU.
    Returns (f_seq [S][N'], p_seq [S][N'], loss [S])."""
    c = make_config(cfg)
    T, N, K = cfg.T, cfg.n_routed, cfg.top_k
    _need(logits, (T, N), torch.float32, "logits")
    _need(idx, (T, K), torch.int32, "idx")
    S = seg_offsets.numel() - 1
    _need(seg_offsets, (S + 1,), torch.int32, "seg_offsets")
    if offset is not None:
        _need(offset, (N,), torch.float32, "offset")
    dev = logits.device
    o = out or {}
    f = o.get("f_seq") if o.get("f_seq") is not None else torch.empty((S, N), dtype=torch.float32, device=dev)
    p = o.get("p_seq") if o.get("p_seq") is not None else torch.empty((S, N), dtype=torch.float32, device=dev)
    loss = o.get("loss") if o.get("loss") is not None else torch.empty(S, dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = alloc_workspace(c, WS_SEQSTAT, dev)
    rc = lib().moe_seq_balance_stats(ctypes.byref(c), _p(logits), _p(offset), _p(idx),
                                     _p(seg_offsets), S, ctypes.c_float(beta), _p(f), _p(p),
                                     _p(loss), _p(workspace), workspace.numel(), _stream(stream))
    _check(rc, "moe_seq_balance_stats")
    return f, p, loss


def device_balance_stats(cfg: LayerConfig, f, P, n_dev: int, alpha2: float, want_loss=True,
                         stream=None):
    """moe_device_balance_stats.  Returns (f_dev [n_dev], P_dev [n_dev], loss [1] or None)."""
    c = make_config(cfg)
    N = cfg.n_routed
    _need(f, (N,), torch.float32, "f")
    _need(P, (N,), torch.float32, "P")
    dev = f.device
    fd = torch.empty(n_dev, dtype=torch.float32, device=dev)
    pd = torch.empty(n_dev, dtype=torch.float32, device=dev)
    loss = torch.empty(1, dtype=torch.float32, device=dev) if want_loss else None
    rc = lib().moe_device_balance_stats(ctypes.byref(c), _p(f), _p(P), n_dev,
                                        ctypes.c_float(alpha2), _p(fd), _p(pd), _p(loss),
                                        _stream(stream))
    _check(rc, "moe_device_balance_stats")
    return fd, pd, loss


def bias_update(cfg: LayerConfig, counts, n_tokens: int, alpha: float, bias, stream=None):
    """moe_bias_update: updates `bias` ([N'] fp32 on the GPU) in place and returns it."""
    c = make_config(cfg)
    N = cfg.n_routed
    _need(counts, (N,), torch.int32, "counts")
    _need(bias, (N,), torch.float32, "bias")
    rc = lib().moe_bias_update(ctypes.byref(c), _p(counts), int(n_tokens), ctypes.c_float(alpha),
                               _p(bias), _stream(stream))
    _check(rc, "moe_bias_update")
    return bias


def profile_enable(max_records: int):
    _check(lib().moe_profile_enable(max_records), "moe_profile_enable")


def profile_collect() -> dict:
    st = StageTimes()
    _check(lib().moe_profile_collect(ctypes.byref(st)), "moe_profile_collect")
    return {name: {"launches": st.launches[i], "ms": st.ms[i]} for i, name in enumerate(STAGES)}
