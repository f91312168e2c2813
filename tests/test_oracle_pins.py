"""Pins of the CPU oracle against what the pages and mathematics fix.

Each test checks the oracle against something other than itself: values the
pages print (tests/golden/*.json, each with its citation), closed forms,
invariants, special cases that reduce to a library routine (torch on the CPU,
in float64), and brute force on tiny inputs.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import oracle as o

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        return json.load(fh)


def rng(seed=0):
    return np.random.default_rng(seed)


def swiglu_torch(x, w13, w2):
    """Library reference of one SwiGLU expert (float64 torch on the CPU)."""
    f = w13.shape[0] // 2
    a = x @ w13[:f].T
    b = x @ w13[f:].T
    return (torch.nn.functional.silu(a) * b) @ w2.T


def rand_layer(r, T, d, N, f, Ks=0, fs=0, scale=1.0):
    x = r.standard_normal((T, d)).astype(np.float32)
    w13 = (r.standard_normal((N, 2 * f, d)) * scale / math.sqrt(d)).astype(np.float32)
    w2 = (r.standard_normal((N, d, f)) * scale / math.sqrt(f)).astype(np.float32)
    w13s = (r.standard_normal((Ks, 2 * fs, d)) / math.sqrt(d)).astype(np.float32)
    w2s = (r.standard_normal((Ks, d, fs)) / math.sqrt(max(fs, 1))).astype(np.float32)
    return x, w13, w2, w13s, w2s


# ---------------------------------------------------------------- balance stats

def test_worked_example_f():
    g = golden("worked_example_balance.json")
    N, K, T = g["n_routed"], g["top_k"], g["T"]
    idx = np.array(g["picks_one_based"], np.int32) - 1
    c = o.counts(idx, N)
    f, _, _ = o.balance_stats(c, None, T, K, 0.01)
    assert K * T / N == g["expected_uniform_load"]
    assert f[0] == g["expected_f1"]
    # remaining experts: picked once each, 1 / 1.5
    for i in range(1, N):
        assert f[i] == pytest.approx(1 / g["expected_uniform_load"], rel=0, abs=1e-15)


@pytest.mark.parametrize("N,K,T", [(16, 3, 97), (64, 7, 512), (384, 9, 33)])
def test_sum_f_is_n_routed(N, K, T):
    """f_i = N'/(K'T) c_i and sum_i c_i = K'T whenever each token picks K'
    distinct experts, so sum_i f_i = N' (uniform load gives f = 1)."""
    r = rng(N)
    idx = np.stack([r.choice(N, K, replace=False) for _ in range(T)]).astype(np.int32)
    c = o.counts(idx, N)
    assert c.sum() == K * T
    f, _, _ = o.balance_stats(c, None, T, K, 0.01)
    assert f.sum() == pytest.approx(N, rel=1e-13)


def test_counts_brute_force():
    r = rng(3)
    idx = r.integers(0, 11, size=(50, 3)).astype(np.int32)
    c = o.counts(idx, 11)
    for i in range(11):
        assert c[i] == sum(1 for t in range(50) for k in range(3) if idx[t, k] == i)


def test_softmax_P_sums_to_one_and_uniform_loss_closed_form():
    """Under softmax sum_i P_i = 1.  With exactly uniform loads (f = 1) the loss
    reduces to alpha1 / N' * sum P = alpha1 / N'."""
    r = rng(5)
    T, N, K = 96, 32, 4           # T*K divisible by N
    logits = r.standard_normal((T, N)).astype(np.float32)
    _, _, s32, _ = o.route(logits, N, K, "softmax", False)
    idx = np.array([[(t * K + k) % N for k in range(K)] for t in range(T)], np.int32)
    c = o.counts(idx, N)
    assert np.all(c == T * K // N)
    f, P, loss = o.balance_stats(c, s32, T, K, 0.01)
    assert np.all(f == 1.0)
    assert P.sum() == pytest.approx(1.0, abs=1e-6)
    assert loss[1] == pytest.approx(P.sum(), rel=1e-15)
    assert loss[0] == pytest.approx(0.01 / N * P.sum(), rel=1e-15)
    # P is a plain column mean
    np.testing.assert_allclose(P, s32.astype(np.float64).mean(axis=0), rtol=1e-12)


def test_loss_is_weighted_by_f():
    """Concentrating the load on one expert with a high mean score raises the
    loss: f_1 = 2 in the worked example, and f.P weights P accordingly."""
    N, K, T = 4, 2, 3
    idx = np.array([[0, 1], [0, 2], [0, 3]], np.int32)
    s32 = np.array([[0.5, 0.3, 0.1, 0.1], [0.5, 0.1, 0.3, 0.1], [0.5, 0.1, 0.1, 0.3]], np.float32)
    f, P, loss = o.balance_stats(o.counts(idx, N), s32, T, K, 1.0)
    exp_P = s32.astype(np.float64).mean(0)
    np.testing.assert_allclose(P, exp_P, rtol=1e-12)
    assert loss[1] == pytest.approx(2 * exp_P[0] + (2 / 3) * exp_P[1:].sum(), rel=1e-12)


# ---------------------------------------------------------------- scores

def test_score_readings_from_the_pages():
    g = golden("score_readings.json")
    for rd in g["readings"]:
        lg = np.array([[rd["logit"], 0.0]], np.float32)
        fn = rd["function"]
        if fn == "softplus":          # s^2 of the sqrt-softplus score
            _, _, s32, _ = o.route(lg, 2, 1, "sqrt_softplus", False)
            val = float(s32[0, 0]) ** 2
        else:
            _, _, s32, _ = o.route(lg, 2, 1, fn, False)
            val = float(s32[0, 0])
        assert f"{val:.{rd['decimals']}f}" == rd["printed"], rd


@pytest.mark.parametrize("scoring", ["softmax", "sigmoid", "sqrt_softplus"])
def test_scores_match_library(scoring):
    r = rng(11)
    lg = (r.standard_normal((64, 40)) * 6).astype(np.float32)
    lg[0, :5] = [30.0, -30.0, 0.0, 80.0, -80.0]
    _, _, s32, _ = o.route(lg, 40, 3, scoring, False)
    t = torch.from_numpy(lg).double()
    if scoring == "softmax":
        ref = torch.softmax(t, dim=1)
    elif scoring == "sigmoid":
        ref = torch.sigmoid(t)
    else:
        ref = torch.sqrt(torch.nn.functional.softplus(t, threshold=50.0))
    ref32 = ref.float().numpy()
    # one fp32 rounding of a double computed two different ways: equal up to 1 ulp
    ulp = np.spacing(np.abs(ref32))
    assert np.all(np.abs(s32 - ref32) <= ulp), np.max(np.abs(s32 - ref32) / ulp)


def test_softmax_rows_sum_to_one():
    r = rng(12)
    lg = (r.standard_normal((200, 256)) * 2).astype(np.float32)
    _, _, s32, _ = o.route(lg, 256, 8, "softmax", False)
    np.testing.assert_allclose(s32.astype(np.float64).sum(1), 1.0, atol=1e-6)


# ---------------------------------------------------------------- selection

def brute_topk(key, k):
    """The unique size-k subset whose members all beat every non-member under
    the order (key desc, index asc)."""
    n = len(key)
    rank = lambda i: (key[i], -i)
    found = []
    for S in itertools.combinations(range(n), k):
        rest = [j for j in range(n) if j not in S]
        if all(rank(i) > rank(j) for i in S for j in rest):
            found.append(S)
    assert len(found) == 1
    return set(found[0])


@pytest.mark.parametrize("scoring", ["softmax", "sigmoid", "sqrt_softplus"])
@pytest.mark.parametrize("with_bias", [False, True])
def test_topk_matches_brute_force(scoring, with_bias):
    r = rng(21)
    for N in range(1, 11):
        for K in range(1, N + 1):
            T = 6
            lg = (r.integers(-3, 4, size=(T, N)) * 0.5).astype(np.float32)  # many ties
            bias = (r.integers(-2, 3, size=N) * 0.05).astype(np.float32) if with_bias else None
            idx, gate, s32, _ = o.route(lg, N, K, scoring, False, bias=bias)
            for t in range(T):
                key = [float(np.float32(s32[t, i]) + np.float32(bias[i])) if with_bias
                       else float(lg[t, i]) for i in range(N)]
                assert set(idx[t].tolist()) == brute_topk(key, K)
                ranks = [(key[i], -i) for i in idx[t]]
                assert ranks == sorted(ranks, reverse=True)     # output order
                np.testing.assert_array_equal(gate[t], s32[t, idx[t]])  # g = s ([P1])


@pytest.mark.parametrize("scoring", ["softmax", "sigmoid", "sqrt_softplus"])
def test_zero_router_selects_lowest_indices(scoring):
    """W_g = 0 makes every logit 0: the tie rule picks experts 0..K'-1."""
    T, d, N, K = 17, 32, 24, 5
    x = rng(1).standard_normal((T, d)).astype(np.float32)
    lg = o.router_logits(x, np.zeros((N, d), np.float32))
    assert np.all(lg == 0)
    idx, _, _, _ = o.route(lg, N, K, scoring, True)
    assert np.all(idx == np.arange(K)[None, :])


def test_huge_bias_forces_selection():
    r = rng(4)
    T, N, K = 50, 16, 3
    lg = r.standard_normal((T, N)).astype(np.float32)
    bias = np.zeros(N, np.float32)
    bias[9] = 10.0
    idx, gate, s32, _ = o.route(lg, N, K, "sigmoid", True, bias=bias)
    assert o.counts(idx, N)[9] == T
    assert np.all(idx[:, 0] == 9)


def test_bias_only_changes_selection_not_gates():
    """V4 book ch. 02 sec. 3 and the tutorial's load-balancing section: the
    bias changes who is selected; gates use the unbiased score."""
    r = rng(8)
    T, N, K = 400, 32, 4
    lg = r.standard_normal((T, N)).astype(np.float32)
    b1 = (r.uniform(-0.05, 0.05, N)).astype(np.float32)
    b2 = (r.uniform(-0.05, 0.05, N)).astype(np.float32)
    for scoring in ("sigmoid", "sqrt_softplus"):
        i1, g1, s1, _ = o.route(lg, N, K, scoring, True, bias=b1)
        i2, g2, s2, _ = o.route(lg, N, K, scoring, True, bias=b2)
        np.testing.assert_array_equal(s1, s2)
        same = [t for t in range(T) if set(i1[t]) == set(i2[t])]
        diff = [t for t in range(T) if set(i1[t]) != set(i2[t])]
        assert len(same) > 50 and len(diff) > 10
        for t in same:
            m1 = dict(zip(i1[t].tolist(), g1[t].tolist()))
            m2 = dict(zip(i2[t].tolist(), g2[t].tolist()))
            assert m1 == m2


@pytest.mark.parametrize("scoring", ["sigmoid", "sqrt_softplus", "softmax"])
def test_renorm_gates_sum_to_one(scoring):
    r = rng(9)
    lg = (r.standard_normal((300, 64)) * 2).astype(np.float32)
    _, gate, _, _ = o.route(lg, 64, 6, scoring, True)
    np.testing.assert_allclose(gate.astype(np.float64).sum(1), 1.0, atol=4e-7)


def test_gap_is_score_difference():
    lg = np.array([[3.0, 1.0, 2.0, 0.0]], np.float32)
    idx, _, s32, gap = o.route(lg, 4, 2, "sigmoid", False)
    assert idx.tolist() == [[0, 2]]
    exact = 1 / (1 + math.exp(-2.0)) - 1 / (1 + math.exp(-1.0))
    assert gap[0] == pytest.approx(exact, rel=1e-12)
    _, _, _, gap_all = o.route(lg, 4, 4, "sigmoid", False)
    assert np.isinf(gap_all[0])


def test_logit_offset_is_added_before_scoring():
    r = rng(10)
    lg = r.standard_normal((20, 8)).astype(np.float32)
    off = r.standard_normal(8).astype(np.float32)
    i1, g1, s1, _ = o.route(lg, 8, 2, "sigmoid", True, offset=off)
    i2, g2, s2, _ = o.route((lg + off).astype(np.float32), 8, 2, "sigmoid", True)
    np.testing.assert_array_equal(i1, i2)
    np.testing.assert_array_equal(s1, s2)


def test_segmented_router_gates_are_one_mth():
    """Duplicating each coarse router row m times (fine-grained segmentation)
    makes the softmax give every copy exactly 1/m of the coarse score, and
    the top-mK selection take all m copies of each top-K coarse expert."""
    r = rng(13)
    T, d, N, K, m = 40, 16, 6, 2, 4
    x = r.standard_normal((T, d)).astype(np.float32)
    wg = r.standard_normal((N, d)).astype(np.float32)
    wg_fine = np.repeat(wg, m, axis=0)
    lc = o.router_logits(x, wg)
    lf = o.router_logits(x, wg_fine)
    ic, gc, _, _ = o.route(lc, N, K, "softmax", False)
    if_, gf, _, _ = o.route(lf, N * m, K * m, "softmax", False)
    for t in range(T):
        assert set((if_[t] // m).tolist()) == set(ic[t].tolist())
        for e, g in zip(ic[t], gc[t]):
            for j in range(m):
                pos = list(if_[t]).index(e * m + j)
                assert abs(gf[t, pos] - g / m) <= np.spacing(np.float32(g / m))


# ---------------------------------------------------------------- hash routing

def test_fmix32_published_vectors():
    g = golden("fmix32_vectors.json")
    for v in g["vectors"]:
        assert o.fmix32(v["seed"]) == int(v["fmix32"], 16)


def test_hash_routing_is_uniform():
    """Hash routing needs no balancing because hashing spreads tokens evenly
    (V4 book ch. 02 sec. 5).  Every id of the 129280-token vocabulary hashed
    once: chi-square over 384 experts.  A random token stream: mean load
    K'T/N' exactly."""
    N, V = 384, 129280
    vocab = np.arange(V, dtype=np.uint32)
    idx, gate, s32, gap = o.route(None, N, 1, "hash", False, token_ids=vocab)
    assert s32 is None and np.all(gate == 1.0) and np.all(np.isinf(gap))
    c = o.counts(idx, N)
    exp_ = V / N
    chi2 = float(((c - exp_) ** 2 / exp_).sum())
    # 383 degrees of freedom: mean 383, sd ~27.7; accept within 6 sd
    assert abs(chi2 - 383) < 6 * math.sqrt(2 * 383), chi2
    r = rng(14)
    T = 1 << 16
    tid = r.integers(0, V, size=T).astype(np.uint32)
    idx, _, _, _ = o.route(None, N, 1, "hash", False, token_ids=tid)
    c = o.counts(idx, N)
    assert c.sum() == T and c.mean() == T / N
    # a hash of the id alone: equal ids, equal experts
    idx2, _, _, _ = o.route(None, N, 1, "hash", False, token_ids=tid[::-1].copy())
    np.testing.assert_array_equal(idx2[::-1], idx)


def test_hash_rejects_bad_arguments():
    with pytest.raises(ValueError):
        o.route(None, 16, 2, "hash", False, token_ids=np.zeros(4, np.uint32))


# ---------------------------------------------------------------- router GEMM

def test_router_logits_match_library():
    r = rng(15)
    x = r.standard_normal((33, 72)).astype(np.float32)
    wg = (r.standard_normal((20, 72)) * 0.02).astype(np.float32)
    lg = o.router_logits(x, wg)
    ref = (torch.from_numpy(x).double() @ torch.from_numpy(wg).double().T).float().numpy()
    assert np.all(np.abs(lg - ref) <= np.spacing(np.abs(ref)))
    sub = o.router_logits(x, wg, tokens=[5, 0, 32])
    np.testing.assert_array_equal(sub, lg[[5, 0, 32]])


def test_router_logits_bf16_is_exact_widening():
    r = rng(16)
    x = torch.from_numpy(r.standard_normal((9, 64)).astype(np.float32)).bfloat16()
    wg = torch.from_numpy((r.standard_normal((12, 64)) * 0.02).astype(np.float32)).bfloat16()
    xb = x.view(torch.int16).numpy().view(np.uint16)
    wb = wg.view(torch.int16).numpy().view(np.uint16)
    lg = o.router_logits(xb, wb)
    ref = (x.double() @ wg.double().T).float().numpy()
    assert np.all(np.abs(lg - ref) <= np.spacing(np.abs(ref)))


# ---------------------------------------------------------------- experts + combine

def test_single_expert_is_plain_swiglu():
    """N' = K' = 1 with renormalisation gives g = 1: the layer is x plus the
    shared FFN plus one SwiGLU FFN ("core design 2" equation)."""
    r = rng(17)
    T, d, f, fs = 7, 24, 16, 12
    x, w13, w2, w13s, w2s = rand_layer(r, T, d, 1, f, Ks=1, fs=fs)
    lg = r.standard_normal((T, 1)).astype(np.float32)
    idx, gate, _, _ = o.route(lg, 1, 1, "sigmoid", True)
    assert np.all(gate == 1.0) and np.all(idx == 0)
    h = o.forward(x, idx, gate, w13, w2, w13s, w2s)
    X = torch.from_numpy(x).double()
    ref = X + swiglu_torch(X, torch.from_numpy(w13s[0]).double(), torch.from_numpy(w2s[0]).double()) \
        + swiglu_torch(X, torch.from_numpy(w13[0]).double(), torch.from_numpy(w2[0]).double())
    np.testing.assert_allclose(h, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_dense_mixture_when_all_experts_active():
    """K' = N' under softmax without renormalisation is the dense soft mixture
    h = x + sum_i s_i FFN_i(x) (the gating network of the freedeepseekapi.com
    blog, sec. 2, with every expert kept)."""
    r = rng(18)
    T, d, N, f = 9, 16, 5, 8
    x, w13, w2, w13s, w2s = rand_layer(r, T, d, N, f)
    wg = (r.standard_normal((N, d)) * 0.5).astype(np.float32)
    lg = o.router_logits(x, wg)
    idx, gate, _, _ = o.route(lg, N, N, "softmax", False)
    h = o.forward(x, idx, gate, w13, w2, w13s, w2s)
    X = torch.from_numpy(x).double()
    s = torch.softmax(X @ torch.from_numpy(wg).double().T, dim=1)
    ref = X.clone()
    for i in range(N):
        ref += s[:, i:i + 1] * swiglu_torch(X, torch.from_numpy(w13[i]).double(),
                                            torch.from_numpy(w2[i]).double())
    np.testing.assert_allclose(h, ref.numpy(), rtol=1e-6, atol=1e-6)


def test_segmentation_identity():
    """Fine-grained segmentation ("core design 1"; airsota.com card sec. 3):
    splitting an expert of width f into m experts of width f/m (column slices
    of W1/W3 rows and W2 columns) and giving every slice the coarse gate
    reproduces the coarse expert exactly (to double round-off)."""
    r = rng(19)
    T, d, N, K, f, m = 11, 20, 4, 2, 24, 4
    x, w13, w2, w13s, w2s = rand_layer(r, T, d, N, f, Ks=1, fs=8)
    lg = r.standard_normal((T, N)).astype(np.float32)
    idx, gate, _, _ = o.route(lg, N, K, "softmax", False)
    h_coarse = o.forward(x, idx, gate, w13, w2, w13s, w2s)
    fm = f // m
    w13f = np.empty((N * m, 2 * fm, d), np.float32)
    w2f = np.empty((N * m, d, fm), np.float32)
    for e in range(N):
        for j in range(m):
            sl = slice(j * fm, (j + 1) * fm)
            w13f[e * m + j, :fm] = w13[e, :f][sl]
            w13f[e * m + j, fm:] = w13[e, f:][sl]
            w2f[e * m + j] = w2[e][:, sl]
    idxf = np.array([[e * m + j for e in idx[t] for j in range(m)] for t in range(T)], np.int32)
    gatef = np.repeat(gate, m, axis=1)
    h_fine = o.forward(x, idxf, gatef, w13f, w2f, w13s, w2s)
    np.testing.assert_allclose(h_fine, h_coarse, rtol=1e-12, atol=1e-12)


def test_shared_experts_concatenate():
    """K_s shared experts of width f act as one shared expert of width K_s f."""
    r = rng(20)
    T, d, f, Ks = 6, 16, 8, 3
    x, w13, w2, w13s, w2s = rand_layer(r, T, d, 2, f, Ks=Ks, fs=f)
    idx = np.zeros((T, 1), np.int32)
    gate = np.zeros((T, 1), np.float32)
    h = o.forward(x, idx, gate, w13, w2, w13s, w2s)
    w13c = np.concatenate([np.concatenate([w13s[j, :f] for j in range(Ks)]),
                           np.concatenate([w13s[j, f:] for j in range(Ks)])])[None]
    w2c = np.concatenate([w2s[j] for j in range(Ks)], axis=1)[None]
    h1 = o.forward(x, idx, gate, w13, w2, w13c, w2c)
    np.testing.assert_allclose(h, h1, rtol=1e-12, atol=1e-12)


def test_forward_token_subset_and_invalid_index():
    r = rng(22)
    T, d, N, f = 10, 16, 6, 8
    x, w13, w2, w13s, w2s = rand_layer(r, T, d, N, f, Ks=1, fs=8)
    idx = r.integers(0, N, size=(T, 2)).astype(np.int32)
    gate = r.random((T, 2)).astype(np.float32)
    full = o.forward(x, idx, gate, w13, w2, w13s, w2s)
    sub = o.forward(x, idx, gate, w13, w2, w13s, w2s, tokens=[7, 2])
    np.testing.assert_array_equal(sub, full[[7, 2]])
    # an out-of-range routed index contributes nothing
    idx2 = idx.copy()
    idx2[3, 1] = N + 5
    gate2 = gate.copy()
    gate2[3, 1] = 0.0
    idx3 = idx.copy()
    idx3[3, 1] = 0
    a = o.forward(x, idx2, gate, w13, w2, w13s, w2s, tokens=[3])
    b = o.forward(x, idx3, gate2, w13, w2, w13s, w2s, tokens=[3])
    np.testing.assert_allclose(a, b, rtol=1e-14, atol=1e-14)


def test_residual_and_zero_gate():
    """With every gate zero and no shared expert, h = u (the residual term)."""
    r = rng(23)
    x, w13, w2, w13s, w2s = rand_layer(r, 5, 8, 3, 4)
    idx = np.array([[0, 1]] * 5, np.int32)
    gate = np.zeros((5, 2), np.float32)
    h = o.forward(x, idx, gate, w13, w2, w13s, w2s)
    np.testing.assert_array_equal(h, x.astype(np.float64))
