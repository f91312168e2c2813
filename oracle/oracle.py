"""CPU oracle for the DeepSeekMoE layer forward -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The product path (the HIP library and its
binding) never imports, links or calls it, and the two share no code.

This is a thin ctypes wrapper over ``oracle.c`` (plain C, double-precision
accumulation, OpenMP over tokens).  Arrays are numpy; bf16 tensors travel as
their raw 16-bit patterns (``numpy.uint16``).

Every function names the passage of the pages it follows:
  * DeepSeekMoE reading notes (heloowird.com): background equation for h_t,
    "core design 1" top-k gate equation, "core design 2" shared-expert
    equation, expert-level balance loss with f_i and P_i, worked example.
  * "MoE architecture" blog (freedeepseekapi.com), sec. 2: G(x)=Softmax(W_g x).
  * DeepSeek-V4 book, ch. 02 (igloomatics.github.io): sec. 1 sigmoid and
    renormalisation, sec. 2 sqrt(Softplus) score, sec. 3 selection bias,
    sec. 5 hash routing.
  * MoE tutorial (ai.clawlihai.cn): the bias affects selection only.

Parity pins for every function live in ``tests/test_oracle_pins.py``; the header
of ``oracle.c`` lists the readings taken where the pages are silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

HERE = Path(__file__).resolve().parent
SRC = HERE / "oracle.c"
LIB = HERE / "liboracle.so"
# A prebuilt copy of this oracle to load instead (the sanitizer test builds
# one with AddressSanitizer and UndefinedBehaviorSanitizer); not rebuilt here.
LIB_OVERRIDE = os.environ.get("MOE_ORACLE_LIB")

SCORING = {"softmax": 0, "sigmoid": 1, "sqrt_softplus": 2, "hash": 3}
DTYPES = {"f32": 0, "bf16": 1}

_lib = None


def build(force: bool = True) -> Path:
    """Compile oracle.c into liboracle.so with gcc (plain -O2, no fast-math,
    no FMA contraction, OpenMP)."""
    if not force and LIB.exists() and LIB.stat().st_mtime >= SRC.stat().st_mtime:
        return LIB
    tmp = LIB.with_suffix(".so.tmp")
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-fno-fast-math", "-ffp-contract=off", str(SRC), "-o", str(tmp), "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if LIB_OVERRIDE:
        lib = ctypes.CDLL(LIB_OVERRIDE)
    else:
        if not LIB.exists() or LIB.stat().st_mtime < SRC.stat().st_mtime:
            build()
        lib = ctypes.CDLL(str(LIB))
    i64, i32, dbl, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
    lib.oracle_router_logits.argtypes = [i64, vp, i64, i64, i32, vp, vp, vp]
    lib.oracle_router_logits.restype = None
    lib.oracle_threads.argtypes = []
    lib.oracle_threads.restype = i32
    lib.oracle_fmix32.argtypes = [ctypes.c_uint32]
    lib.oracle_fmix32.restype = ctypes.c_uint32
    lib.oracle_route.argtypes = [i64, i64, i64, i32, i32, vp, vp, vp, vp, i64, i64,
                                 vp, vp, vp, vp]
    lib.oracle_route.restype = i32
    lib.oracle_counts.argtypes = [i64, i64, i64, vp, vp]
    lib.oracle_counts.restype = None
    lib.oracle_balance_stats.argtypes = [i64, i64, i64, vp, vp, dbl, vp, vp, vp]
    lib.oracle_balance_stats.restype = None
    lib.oracle_seq_balance_stats.argtypes = [i64, i64, i64, i64, vp, vp, vp, dbl, vp, vp, vp]
    lib.oracle_seq_balance_stats.restype = None
    lib.oracle_device_balance_stats.argtypes = [i64, i64, vp, vp, dbl, vp, vp, vp]
    lib.oracle_device_balance_stats.restype = None
    lib.oracle_bias_update.argtypes = [i64, i64, i64, vp, dbl, vp, vp]
    lib.oracle_bias_update.restype = None
    lib.oracle_forward.argtypes = [i64, vp, i64, i64, i64, i64, i64, i64, i32,
                                   vp, vp, vp, vp, vp, vp, vp, vp]
    lib.oracle_forward.restype = None
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return DTYPES["f32"]
    if a.dtype == np.uint16:
        return DTYPES["bf16"]
    raise TypeError(f"oracle takes float32 or bf16 bit patterns (uint16), got {a.dtype}")


def _c(a, dtype=None):
    if a is None:
        return None
    a = np.ascontiguousarray(a if dtype is None else a.astype(dtype, copy=False))
    return a


def threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().oracle_threads())


def fmix32(v: int) -> int:
    """MurmurHash3's 32-bit finaliser, the hash used for token-id routing."""
    return int(_load().oracle_fmix32(ctypes.c_uint32(v & 0xFFFFFFFF)))


def router_logits(x: np.ndarray, w_gate: np.ndarray, tokens=None) -> np.ndarray:
    """l[t][i] = sum_k x[t][k] W_g[i][k] in double, rounded to fp32
    (freedeepseekapi.com blog sec. 2, the linear gating network)."""
    x, w_gate = _c(x), _c(w_gate)
    if x.dtype != w_gate.dtype:
        raise TypeError("x and w_gate must share a dtype")
    T, d = x.shape
    n_routed = w_gate.shape[0]
    tok = None if tokens is None else _c(np.asarray(tokens), np.int64)
    n = T if tok is None else len(tok)
    out = np.empty((n, n_routed), np.float32)
    _load().oracle_router_logits(n, _ptr(tok), d, n_routed, _dtype_code(x),
                                 _ptr(x), _ptr(w_gate), _ptr(out))
    return out


def route(logits, n_routed: int, top_k: int, scoring: str, renorm: bool,
          offset=None, bias=None, token_ids=None, n_groups: int = 0, topk_groups: int = 0):
    """Scores, selection and gates for every row.

    Follows the top-k gate equation of the DeepSeekMoE notes ("core design 1"),
    the V4 book ch. 02 sec. 1 (sigmoid, renormalisation), sec. 2 (sqrt of
    softplus), sec. 3 (selection score s + b) and sec. 5 (hash routing).
    With n_groups > 0, node-limited routing (V4 book ch. 02 sec. 4, V3's
    limit of M nodes per token): the experts form n_groups contiguous equal
    groups, the topk_groups groups with the largest best selection key are
    kept (ties: lower group index), and top-K' runs over their experts.
    Returns (idx int32 [n][K'], gate fp32 [n][K'], s32 fp32 [n][N'] or None,
    gap fp64 [n]); with groups the gap is the smaller of the expert gap
    within the kept groups and the gap between the last kept and the best
    dropped group (best score of a group in score units).
    """
    code = SCORING[scoring]
    if code == SCORING["hash"]:
        token_ids = _c(token_ids, np.uint32)
        n = len(token_ids)
        lg = None
    else:
        lg = _c(logits, np.float32)
        n = lg.shape[0]
        assert lg.shape[1] == n_routed
    idx = np.empty((n, top_k), np.int32)
    gate = np.empty((n, top_k), np.float32)
    s32 = None if code == SCORING["hash"] else np.empty((n, n_routed), np.float32)
    gap = np.empty(n, np.float64)
    rc = _load().oracle_route(n, n_routed, top_k, code, int(bool(renorm)), _ptr(lg),
                              _ptr(_c(offset, np.float32)), _ptr(_c(bias, np.float32)),
                              _ptr(token_ids if code == SCORING["hash"] else None),
                              int(n_groups), int(topk_groups),
                              _ptr(idx), _ptr(gate), _ptr(s32), _ptr(gap))
    if rc != 0:
        raise ValueError("oracle_route rejected its arguments")
    return idx, gate, s32, gap


def counts(idx: np.ndarray, n_routed: int) -> np.ndarray:
    """c_i = #{(t, k) : idx[t][k] == i}."""
    idx = _c(idx, np.int32)
    n, k = idx.shape
    out = np.empty(n_routed, np.int32)
    _load().oracle_counts(n, n_routed, k, _ptr(idx), _ptr(out))
    return out


def balance_stats(cnt: np.ndarray, s32, n_tok: int, top_k: int, alpha1: float):
    """f_i, P_i and (L_ExpBal, sum f_i P_i) per the expert-level balance loss
    of the DeepSeekMoE notes.  s32 may be None (hash routing): then only f."""
    cnt = _c(cnt, np.int32)
    n_routed = len(cnt)
    f = np.empty(n_routed, np.float64)
    P = np.empty(n_routed, np.float64)
    loss = np.empty(2, np.float64)
    s = None if s32 is None else _c(s32, np.float32)
    if s is not None:
        assert s.shape == (n_tok, n_routed)
    _load().oracle_balance_stats(n_tok, n_routed, top_k, _ptr(cnt), _ptr(s),
                                 float(alpha1), _ptr(f), _ptr(P), _ptr(loss))
    if s is None:
        return f, None, None
    return f, P, loss


def seq_balance_stats(idx, s32, seg_off, beta: float):
    """In-sequence balance statistics (V4 book ch. 02 sec. 3, change 2):
    per segment s (tokens seg_off[s] .. seg_off[s+1]-1) f_i^seq (normalised
    like the notes' f_i), p_i^seq (mean raw score) and
    L_seq = beta * sum_i f_i^seq p_i^seq.  Empty segments give zeros.
    Returns (f_seq [S][N'], p_seq [S][N'], loss [S]), all fp64."""
    idx, s32 = _c(idx, np.int32), _c(s32, np.float32)
    off = _c(np.asarray(seg_off), np.int64)
    T, K = idx.shape
    N = s32.shape[1]
    S = len(off) - 1
    assert s32.shape == (T, N) and off[0] >= 0 and off[-1] <= T and np.all(np.diff(off) >= 0)
    f = np.empty((S, N), np.float64)
    p = np.empty((S, N), np.float64)
    loss = np.empty(S, np.float64)
    _load().oracle_seq_balance_stats(T, N, K, S, _ptr(off), _ptr(idx), _ptr(s32), float(beta),
                                     _ptr(f), _ptr(p), _ptr(loss))
    return f, p, loss


def device_balance_stats(f, P, n_dev: int, alpha2: float):
    """Device-level balance loss of the DeepSeekMoE notes over n_dev contiguous
    groups of experts: f'_d (mean f), P'_d (sum P), L_DevBal.  f, P are the
    fp32 expert-level statistics.  Returns (f_dev, P_dev, loss) in fp64."""
    f, P = _c(f, np.float32), _c(P, np.float32)
    N = len(f)
    assert len(P) == N and n_dev >= 1 and N % n_dev == 0
    fd = np.empty(n_dev, np.float64)
    pd = np.empty(n_dev, np.float64)
    loss = np.empty(1, np.float64)
    _load().oracle_device_balance_stats(N, n_dev, _ptr(f), _ptr(P), float(alpha2), _ptr(fd),
                                        _ptr(pd), _ptr(loss))
    return fd, pd, float(loss[0])


def bias_update(cnt, n_tok: int, top_k: int, alpha: float, bias) -> np.ndarray:
    """Aux-loss-free bias update (V4 book ch. 02 sec. 3, V3):
    b_i + alpha (K'/N' - c_i / n_tok), in double, rounded to fp32."""
    cnt, b = _c(cnt, np.int32), _c(bias, np.float32)
    N = len(cnt)
    out = np.empty(N, np.float32)
    _load().oracle_bias_update(N, top_k, n_tok, _ptr(cnt), float(alpha), _ptr(b), _ptr(out))
    return out


def forward(x, idx, gate, w13, w2, w13s, w2s, tokens=None) -> np.ndarray:
    """h_t = u_t + sum_shared FFN(u_t) + sum_k g_{t,k} FFN_{idx}(u_t), double
    precision, SwiGLU experts (DeepSeekMoE notes, "core design 2" equation).

    x [T][d]; idx, gate [T][K']; w13 [N'][2f][d]; w2 [N'][d][f];
    w13s [K_s][2fs][d]; w2s [K_s][d][fs] (K_s may be 0).  Returns [n][d] fp64
    for the listed tokens (all tokens when ``tokens`` is None).
    """
    x, w13, w2 = _c(x), _c(w13), _c(w2)
    idx, gate = _c(idx, np.int32), _c(gate, np.float32)
    T, d = x.shape
    n_routed, two_f, d2 = w13.shape
    assert d2 == d and w2.shape == (n_routed, d, two_f // 2)
    f = two_f // 2
    if w13s is None or w13s.size == 0:
        n_shared, fs, w13s, w2s = 0, 0, None, None
    else:
        w13s, w2s = _c(w13s), _c(w2s)
        n_shared, two_fs, _ = w13s.shape
        fs = two_fs // 2
        assert w2s.shape == (n_shared, d, fs) and w13s.dtype == x.dtype
    dt = _dtype_code(x)
    assert w13.dtype == x.dtype and w2.dtype == x.dtype
    top_k = idx.shape[1]
    assert idx.shape == (T, top_k) and gate.shape == (T, top_k)
    tok = None if tokens is None else _c(np.asarray(tokens), np.int64)
    n = T if tok is None else len(tok)
    h = np.empty((n, d), np.float64)
    _load().oracle_forward(n, _ptr(tok), d, n_routed, top_k, n_shared, f, fs, dt,
                           _ptr(x), _ptr(idx), _ptr(gate), _ptr(w13), _ptr(w2),
                           _ptr(w13s), _ptr(w2s), _ptr(h))
    return h
