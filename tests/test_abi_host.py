"""Host-side checks of libmoe.so that need no GPU: the library loads, exports
every entry point include/moe.h declares, sizes its workspaces, and rejects
bad arguments with the documented status codes before touching a device."""
import ctypes
import re
from pathlib import Path

import pytest

from fine_grained_moe_router_amd import binding as B
from fine_grained_moe_router_amd.configs import CONFIGS

HEADER = Path(__file__).resolve().parents[1] / "include" / "moe.h"


@pytest.fixture(scope="module")
def L():
    return B.lib()


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(B.EXPORTS)


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def cfg_of(name, **kw):
    return B.make_config(CONFIGS[name].with_(**kw) if kw else CONFIGS[name])


@pytest.mark.parametrize("name", list(CONFIGS))
def test_workspace_sizes(L, name):
    c = cfg_of(name)
    cfg = CONFIGS[name]
    fwd = B.workspace_bytes(c, B.WS_FORWARD)
    P = cfg.T * cfg.top_k
    # at least the routed hidden activations and the fp32 routed outputs
    eb = 2 if cfg.dtype == "bf16" else 4
    assert fwd >= P * cfg.d_ff * eb + P * cfg.d_model * 4
    if cfg.scoring == "hash":
        assert B.workspace_bytes(c, B.WS_ROUTE) == 0
        assert B.workspace_bytes(c, B.WS_PSTAT) == 0
    else:
        assert B.workspace_bytes(c, B.WS_ROUTE) >= cfg.T * cfg.n_routed * 4
        assert B.workspace_bytes(c, B.WS_PSTAT) >= cfg.n_routed * 8
    assert B.workspace_bytes(c, 99) == 0


BAD_CONFIGS = [
    (dict(T=0), B.MOE_ERR_INVALID_ARG),
    (dict(top_k=0), B.MOE_ERR_INVALID_ARG),
    (dict(top_k=65), B.MOE_ERR_INVALID_ARG),          # K' > N'
    (dict(top_k=17, n_routed=64), B.MOE_ERR_INVALID_ARG),
    (dict(n_routed=2000), B.MOE_ERR_INVALID_ARG),
    (dict(n_shared=-1), B.MOE_ERR_INVALID_ARG),
    (dict(d_model=100), B.MOE_ERR_UNSUPPORTED),
    (dict(d_ff=96), B.MOE_ERR_UNSUPPORTED),
    (dict(d_ff_shared=80), B.MOE_ERR_UNSUPPORTED),
    (dict(T=1 << 20, top_k=8), B.MOE_ERR_UNSUPPORTED),
    (dict(n_groups=3, topk_groups=1), B.MOE_ERR_INVALID_ARG),      # 64 % 3
    (dict(n_groups=8, topk_groups=0), B.MOE_ERR_INVALID_ARG),
    (dict(n_groups=8, topk_groups=9), B.MOE_ERR_INVALID_ARG),
    (dict(n_groups=16, topk_groups=1), B.MOE_ERR_INVALID_ARG),     # 1 * 4 < K' = 7
    (dict(n_groups=0, topk_groups=2), B.MOE_ERR_INVALID_ARG),
    (dict(n_groups=128, topk_groups=8, n_routed=128), B.MOE_ERR_INVALID_ARG),  # > 64 groups
]


@pytest.mark.parametrize("kw,status", BAD_CONFIGS)
def test_bad_configs_are_rejected(L, kw, status):
    c = cfg_of("toy_fp32", **kw)
    assert L.moe_workspace_bytes(ctypes.byref(c), B.WS_FORWARD) == 0
    rc = L.moe_forward(ctypes.byref(c), *([ctypes.c_void_p(256)] * 8), ctypes.c_void_p(256),
                       1 << 40, None)
    assert rc == status


def test_bad_modes_are_rejected(L):
    for field, val in (("scoring", 7), ("renorm", 2), ("dtype", 5), ("flags", 8),
                       ("flags", B.LOGITS_IN | B.LOGITS_OUT)):
        c = cfg_of("toy_fp32")
        setattr(c, field, val)
        assert L.moe_workspace_bytes(ctypes.byref(c), B.WS_FORWARD) == 0, field
    c = cfg_of("v4_hash")
    c.top_k = 2
    assert L.moe_workspace_bytes(ctypes.byref(c), B.WS_FORWARD) == 0
    assert L.moe_workspace_bytes(None, B.WS_FORWARD) == 0


P = ctypes.c_void_p(4096)  # never dereferenced: validation fails first


def route(L, c, x=P, wg=P, off=None, bias=None, tid=None, logits=None, idx=P, w=P, counts=P,
          pstat=None, ws=P, ws_bytes=1 << 40):
    return L.moe_route(ctypes.byref(c), x, wg, off, bias, tid, logits, idx, w, counts, pstat, ws,
                       ws_bytes, None)


def test_route_workspace_holds_split_partials():
    # The route workspace holds the select blocks' expert histograms (one
    # int32 row of N' per block, blocks of at least 8 tokens) and, when the
    # router GEMM runs, its output.  The GEMM splits d so that its 256 x 256
    # tiles cover the CUs: then it holds one [T][N'] partial per split (at
    # most 16 splits of at least 8 k-tiles each), which the select kernel
    # adds up; unsplit, the logits.  With d below 8 k-tiles of 64 it does not
    # split.  With MOE_LOGITS_IN only the histograms remain.
    for name in ("v3_decode", "v3_prefill"):
        cfg = CONFIGS[name]
        tn = cfg.T * cfg.n_routed * 4
        hist_max = -(-cfg.T // 8) * cfg.n_routed * 4 + 256
        ws = B.workspace_bytes(B.make_config(cfg), B.WS_ROUTE)
        assert 2 * tn <= ws <= 16 * tn + hist_max, name
        ws_in = B.workspace_bytes(B.make_config(cfg, flags=B.LOGITS_IN), B.WS_ROUTE)
        assert 0 < ws_in <= hist_max and (ws - ws_in) % tn == 0, name
    narrow = CONFIGS["toy_fp32"].with_(dtype="bf16", d_model=256)
    tn = narrow.T * narrow.n_routed * 4
    ws = B.workspace_bytes(B.make_config(narrow), B.WS_ROUTE)
    ws_in = B.workspace_bytes(B.make_config(narrow, flags=B.LOGITS_IN), B.WS_ROUTE)
    assert ws - ws_in == tn


def test_route_argument_errors(L):
    c = cfg_of("v3_decode")
    assert route(L, c, idx=None) == B.MOE_ERR_INVALID_ARG
    assert route(L, c, w=None) == B.MOE_ERR_INVALID_ARG
    assert route(L, c, counts=None) == B.MOE_ERR_INVALID_ARG
    assert route(L, c, x=None) == B.MOE_ERR_INVALID_ARG
    assert route(L, c, wg=None) == B.MOE_ERR_INVALID_ARG
    assert route(L, c, ws=None) == B.MOE_ERR_INVALID_ARG
    assert route(L, c, ws_bytes=16) == B.MOE_ERR_WORKSPACE
    assert route(L, c, x=ctypes.c_void_p(4096 + 8)) == B.MOE_ERR_UNSUPPORTED
    assert route(L, c, wg=ctypes.c_void_p(4096 + 2)) == B.MOE_ERR_UNSUPPORTED
    assert route(L, c, logits=P) == B.MOE_ERR_INVALID_ARG      # logits given but no flag
    cin = cfg_of("v3_decode")
    cin.flags = B.LOGITS_IN
    assert route(L, cin, logits=None) == B.MOE_ERR_INVALID_ARG
    assert route(L, cin, logits=P, ws=None) == B.MOE_ERR_INVALID_ARG   # histogram rows
    assert route(L, cin, logits=P, ws_bytes=16) == B.MOE_ERR_WORKSPACE
    cout = cfg_of("v3_decode")
    cout.flags = B.LOGITS_OUT
    assert route(L, cout, logits=None) == B.MOE_ERR_INVALID_ARG
    assert route(L, cout, logits=P, ws=None) == B.MOE_ERR_INVALID_ARG  # split partials need it
    # the router GEMM addresses W_g with 32-bit byte offsets: N' d < 2^31
    big = cfg_of("v3_decode", T=8, d_model=1 << 21, n_routed=1024, d_ff=64, n_shared=0)
    assert L.moe_workspace_bytes(ctypes.byref(big), B.WS_FORWARD) > 0   # the layer itself is valid
    assert route(L, big) == B.MOE_ERR_UNSUPPORTED
    h = cfg_of("v4_hash")
    assert route(L, h, tid=None) == B.MOE_ERR_INVALID_ARG       # hash needs token ids
    assert route(L, h, tid=P, pstat=P) == B.MOE_ERR_INVALID_ARG  # no P under hash


def test_forward_argument_errors(L):
    c = cfg_of("mid")
    args = [ctypes.c_void_p(4096 * (i + 1)) for i in range(8)]  # x..h
    for i in (0, 1, 2, 3, 4, 7):          # x, idx, w, w13, w2, h
        a = list(args)
        a[i] = None
        assert L.moe_forward(ctypes.byref(c), *a, P, 1 << 40, None) == B.MOE_ERR_INVALID_ARG, i
    for i in (5, 6):                       # shared weights required when K_s > 0
        a = list(args)
        a[i] = None
        assert L.moe_forward(ctypes.byref(c), *a, P, 1 << 40, None) == B.MOE_ERR_INVALID_ARG, i
    assert L.moe_forward(ctypes.byref(c), *args, None, 1 << 40, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_forward(ctypes.byref(c), *args, P, 1024, None) == B.MOE_ERR_WORKSPACE
    a = list(args)
    a[7] = a[0]                            # h aliases x
    assert L.moe_forward(ctypes.byref(c), *a, P, 1 << 40, None) == B.MOE_ERR_INVALID_ARG
    for i in (0, 3, 4, 5, 6, 7):          # matrices must be 16-byte aligned
        a = list(args)
        a[i] = ctypes.c_void_p(a[i].value + 8)
        assert L.moe_forward(ctypes.byref(c), *a, P, 1 << 40, None) == B.MOE_ERR_UNSUPPORTED, i


def test_stats_argument_errors(L):
    c = cfg_of("mid")
    st = L.moe_balance_stats
    assert st(ctypes.byref(c), None, P, 0.01, P, P, P, None) == B.MOE_ERR_INVALID_ARG
    assert st(ctypes.byref(c), P, P, 0.01, None, P, P, None) == B.MOE_ERR_INVALID_ARG
    assert st(ctypes.byref(c), P, None, 0.01, P, P, None, None) == B.MOE_ERR_INVALID_ARG
    assert st(ctypes.byref(c), P, None, 0.01, P, None, P, None) == B.MOE_ERR_INVALID_ARG
    h = cfg_of("v4_hash")
    assert st(ctypes.byref(h), P, P, 0.01, P, P, None, None) == B.MOE_ERR_INVALID_ARG


def test_status_strings(L):
    for s in (0, -1, -2, -3):
        assert B.status_string(s)
    assert "workspace" in B.status_string(B.MOE_ERR_WORKSPACE)
    assert B.status_string(12345) == "unknown status"
    with pytest.raises(B.MoeError):
        B._check(B.MOE_ERR_INVALID_ARG, "x")


def test_grouped_routing_config_is_accepted(L):
    c = cfg_of("v3_prefill", n_groups=8, topk_groups=4)
    assert L.moe_workspace_bytes(ctypes.byref(c), B.WS_ROUTE) > 0
    h = cfg_of("v4_hash", n_groups=32, topk_groups=4)
    assert L.moe_workspace_bytes(ctypes.byref(h), B.WS_ROUTE) == 0    # no groups under hash


def test_seq_stats_argument_errors(L):
    c = cfg_of("v3_prefill")
    f = L.moe_seq_balance_stats
    ok = [P, None, P, P, 2, ctypes.c_float(1e-4), P, P, P, P, 1 << 40, None]
    assert B.workspace_bytes(c, B.WS_SEQSTAT) >= CONFIGS["v3_prefill"].T * 256 * 4
    for i in (0, 2, 3, 6, 7, 8, 9):               # logits, idx, offsets, outputs, workspace
        a = list(ok)
        a[i] = None
        assert f(ctypes.byref(c), *a) == B.MOE_ERR_INVALID_ARG, i
    a = list(ok)
    a[4] = 0                                       # no segment
    assert f(ctypes.byref(c), *a) == B.MOE_ERR_INVALID_ARG
    a = list(ok)
    a[10] = 16
    assert f(ctypes.byref(c), *a) == B.MOE_ERR_WORKSPACE
    h = cfg_of("v4_hash")
    assert f(ctypes.byref(h), *ok) == B.MOE_ERR_INVALID_ARG    # no scores under hash


def test_device_stats_and_bias_update_argument_errors(L):
    c = cfg_of("v3_prefill")
    d = L.moe_device_balance_stats
    a2 = ctypes.c_float(0.05)
    assert d(ctypes.byref(c), None, P, 8, a2, P, P, P, None) == B.MOE_ERR_INVALID_ARG
    assert d(ctypes.byref(c), P, P, 0, a2, P, P, P, None) == B.MOE_ERR_INVALID_ARG
    assert d(ctypes.byref(c), P, P, 3, a2, P, P, P, None) == B.MOE_ERR_INVALID_ARG   # 256 % 3
    assert d(ctypes.byref(c), P, P, 8, a2, None, P, P, None) == B.MOE_ERR_INVALID_ARG
    u = L.moe_bias_update
    al = ctypes.c_float(1e-3)
    assert u(ctypes.byref(c), None, 8192, al, P, None) == B.MOE_ERR_INVALID_ARG
    assert u(ctypes.byref(c), P, 0, al, P, None) == B.MOE_ERR_INVALID_ARG
    assert u(ctypes.byref(c), P, 8192, al, None, None) == B.MOE_ERR_INVALID_ARG


def test_forward_static_refuses_configs_beyond_its_scratch(L):
    """moe_forward_static runs on a library-owned scratch of
    MOE_STATIC_SCRATCH_BYTES (64 MiB): a larger forward workspace is refused
    before anything touches a device; its other argument checks are
    moe_forward's."""
    big = cfg_of("v3_prefill")
    assert B.workspace_bytes(big, B.WS_FORWARD) > 64 << 20
    args = [ctypes.c_void_p(4096 * (i + 1)) for i in range(8)]
    assert L.moe_forward_static(ctypes.byref(big), *args, None) == B.MOE_ERR_UNSUPPORTED
    small = cfg_of("v3_decode")
    assert B.workspace_bytes(small, B.WS_FORWARD) <= 64 << 20
    a = list(args)
    a[0] = None
    assert L.moe_forward_static(ctypes.byref(small), *a, None) == B.MOE_ERR_INVALID_ARG
    a = list(args)
    a[7] = a[0]                                # h aliases x
    assert L.moe_forward_static(ctypes.byref(small), *a, None) == B.MOE_ERR_INVALID_ARG
