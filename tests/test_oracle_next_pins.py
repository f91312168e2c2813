"""Pins of the oracle's extensions beyond the layer forward: node-limited
routing, in-sequence and device-level balance statistics, and the
aux-loss-free bias update.  Each is checked against what the pages or the
mathematics fix -- values the pages print (tests/golden/), closed forms,
invariants, reductions to already pinned functions, brute force on tiny
inputs -- never against a retyped copy of its own formula."""
from __future__ import annotations

import json
import os
from itertools import combinations

import numpy as np
import pytest

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        return json.load(fh)


def rand_logits(T, N, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal((T, N)) * scale).astype(np.float32)


def worked_example_idx():
    g = golden("worked_example_balance.json")
    return np.asarray(g["picks_one_based"], np.int32) - 1, g


# ------------------------------------------------------------ grouped routing

@pytest.mark.parametrize("scoring,bias", [("softmax", False), ("sigmoid", True),
                                          ("sqrt_softplus", False)])
def test_groups_of_one_expert_equal_plain_topk(scoring, bias):
    """Node limit with one expert per group and M = K' groups is plain top-K'
    (V4 book ch. 02 sec. 4: the limit only removes experts)."""
    T, N, K = 64, 16, 4
    lg = rand_logits(T, N, 1)
    b = np.random.default_rng(2).uniform(-0.05, 0.05, N).astype(np.float32) if bias else None
    a = O.route(lg, N, K, scoring, True, bias=b)
    g = O.route(lg, N, K, scoring, True, bias=b, n_groups=N, topk_groups=K)
    np.testing.assert_array_equal(a[0], g[0])
    np.testing.assert_array_equal(a[1], g[1])


def test_all_groups_kept_equal_plain_topk():
    T, N, K = 64, 32, 6
    lg = rand_logits(T, N, 3)
    a = O.route(lg, N, K, "sigmoid", True)
    g = O.route(lg, N, K, "sigmoid", True, n_groups=8, topk_groups=8)
    np.testing.assert_array_equal(a[0], g[0])
    np.testing.assert_array_equal(a[1], g[1])


@pytest.mark.parametrize("G,M,K", [(4, 2, 3), (4, 1, 2), (8, 5, 4), (2, 1, 4)])
def test_grouped_routing_brute_force(G, M, K):
    """Tiny cases against exhaustive search: over every set of M groups, the
    kept set is the one whose groups rank first by best key (ties: lower
    group index), and the selection is the K' best keys inside it."""
    T, N = 48, 8
    lg = rand_logits(T, N, 10 + G + M + K)
    lg[5, :] = 0.0                      # an all-tie row: lower indices win
    idx, gate, s32, _ = O.route(lg, N, K, "softmax", False, n_groups=G, topk_groups=M)
    gsz = N // G
    for t in range(T):
        key = lg[t]
        best = [max(key[g * gsz:(g + 1) * gsz]) for g in range(G)]
        # rank of each group: by (best key desc, group index asc)
        order = sorted(range(G), key=lambda g: (-best[g], g))
        want_groups = None
        for cand in combinations(range(G), M):
            if sorted(cand) == sorted(order[:M]):
                want_groups = set(cand)
        experts = [i for i in range(N) if i // gsz in want_groups]
        want = sorted(experts, key=lambda i: (-key[i], i))[:K]
        assert list(idx[t]) == want, t
        assert len({i // gsz for i in idx[t]}) <= M


def test_grouped_gates_renormalise_and_p_unaffected():
    T, N, K = 128, 64, 8
    lg = rand_logits(T, N, 7, 2.0)
    idx, gate, s32, gap = O.route(lg, N, K, "sigmoid", True, n_groups=8, topk_groups=4)
    np.testing.assert_allclose(gate.astype(np.float64).sum(1), 1.0, atol=1e-6)
    _, _, s_plain, _ = O.route(lg, N, K, "sigmoid", True)
    np.testing.assert_array_equal(s32, s_plain)       # scores (hence P) ignore the limit
    assert np.all(gap >= 0)


def test_grouped_routing_rejects_bad_shapes():
    lg = rand_logits(4, 12, 0)
    with pytest.raises(ValueError):
        O.route(lg, 12, 2, "softmax", False, n_groups=5, topk_groups=2)    # 12 % 5
    with pytest.raises(ValueError):
        O.route(lg, 12, 7, "softmax", False, n_groups=4, topk_groups=2)    # 2 * 3 < 7
    with pytest.raises(ValueError):
        O.route(lg, 12, 2, "softmax", False, n_groups=4, topk_groups=5)


# ------------------------------------------------------ in-sequence statistics

def test_seq_stats_worked_example_segment():
    """The notes' worked example as one segment of a two-segment batch gives
    f = [2, 2/3, 2/3, 2/3] exactly, whatever the other segment holds."""
    idx0, g = worked_example_idx()
    N, K = g["n_routed"], g["top_k"]
    idx1 = np.array([[3, 2], [0, 1]], np.int32)
    idx = np.concatenate([idx0, idx1])
    s32 = np.full((len(idx), N), 0.25, np.float32)
    f, p, loss = O.seq_balance_stats(idx, s32, [0, 3, 5], beta=1e-4)
    assert f[0, 0] == g["expected_f1"]
    np.testing.assert_allclose(f[0, 1:], 2.0 / 3.0, rtol=0, atol=1e-15)
    np.testing.assert_allclose(f[1], [1.0, 1.0, 1.0, 1.0], rtol=0, atol=1e-15)


def test_seq_stats_page_overload_ratio():
    """V4 book example: an expert holding 6x the ideal K' T / N' selections of
    a sequence has f^seq = 6 (scaled to T = 1024 so the ideal is 24)."""
    g = golden("seq_balance_example.json")
    N, K = g["n_routed"], g["top_k"]
    assert g["T"] * K / N == 6144                        # printed as "~6000"
    T = 1024
    ideal = T * K // N
    rng = np.random.default_rng(0)
    hot = list(range(g["printed_overloaded_experts"]))
    idx = np.empty((T, K), np.int32)
    for t in range(T):
        # every token takes a hot expert with probability 6 * ideal / T, the rest uniformly
        row = []
        if t < 6 * ideal * len(hot):
            row.append(hot[t % len(hot)])
        rest = [e for e in rng.permutation(N) if e not in hot and e not in row]
        row += rest[:K - len(row)]
        idx[t] = row
    s32 = np.zeros((T, N), np.float32)
    f, _, _ = O.seq_balance_stats(idx, s32, [0, T], beta=1e-4)
    for e in hot:
        assert f[0, e] == 6.0


def test_single_segment_equals_expert_level_stats():
    T, N, K = 96, 16, 3
    lg = rand_logits(T, N, 11)
    idx, _, s32, _ = O.route(lg, N, K, "softmax", False)
    beta = 3e-4
    f, p, loss = O.seq_balance_stats(idx, s32, [0, T], beta)
    fe, Pe, le = O.balance_stats(O.counts(idx, N), s32, T, K, 0.01)
    np.testing.assert_array_equal(f[0], fe)
    np.testing.assert_array_equal(p[0], Pe)
    np.testing.assert_allclose(loss[0], beta * le[1], rtol=1e-15)


def test_seq_stats_invariants():
    """Per non-empty segment sum_i f^seq = N' and, under softmax,
    sum_i p^seq = 1; token-weighted means over segments give back the
    batch's f and P; an empty segment gives zeros."""
    T, N, K = 200, 24, 5
    lg = rand_logits(T, N, 12, 2.0)
    idx, _, s32, _ = O.route(lg, N, K, "softmax", False)
    off = [0, 17, 17, 90, 91, 200]
    f, p, loss = O.seq_balance_stats(idx, s32, off, 1e-4)
    Ts = np.diff(off)
    for s in range(len(Ts)):
        if Ts[s] == 0:
            assert not f[s].any() and not p[s].any() and loss[s] == 0.0
            continue
        assert abs(f[s].sum() - N) < 1e-9
        assert abs(p[s].sum() - 1.0) < 1e-6
    fe, Pe, _ = O.balance_stats(O.counts(idx, N), s32, T, K, 0.01)
    np.testing.assert_allclose((Ts[:, None] * f).sum(0) / T, fe, rtol=1e-12)
    np.testing.assert_allclose((Ts[:, None] * p).sum(0) / T, Pe, rtol=1e-12)


# ---------------------------------------------------- device-level statistics

def test_device_stats_worked_example():
    """Worked example with two devices {E1, E2}, {E3, E4}: f' is the mean f
    of each group, (2 + 2/3)/2 and (2/3 + 2/3)/2."""
    idx, g = worked_example_idx()
    N, K, T = g["n_routed"], g["top_k"], g["T"]
    f, _, _ = O.balance_stats(O.counts(idx, N), None, T, K, 0.01)
    P = np.array([0.4, 0.3, 0.2, 0.1], np.float32)
    fd, pd, loss = O.device_balance_stats(f.astype(np.float32), P, 2, 0.05)
    np.testing.assert_allclose(fd, [4.0 / 3.0, 2.0 / 3.0], rtol=1e-7)
    np.testing.assert_allclose(pd, [0.7, 0.3], rtol=1e-7)
    np.testing.assert_allclose(loss, 0.05 * (4.0 / 3.0 * 0.7 + 2.0 / 3.0 * 0.3), rtol=1e-7)


def test_device_stats_limits():
    """One device per expert gives back f, P and alpha2 sum f P; a single
    device gives f' = 1 (sum f = N') and P' = sum P (= 1 under softmax)."""
    T, N, K = 128, 32, 4
    lg = rand_logits(T, N, 13)
    idx, _, s32, _ = O.route(lg, N, K, "softmax", False)
    f, P, le = O.balance_stats(O.counts(idx, N), s32, T, K, 0.01)
    f32, P32 = f.astype(np.float32), P.astype(np.float32)
    fd, pd, loss = O.device_balance_stats(f32, P32, N, 0.05)
    np.testing.assert_array_equal(fd, f32.astype(np.float64))
    np.testing.assert_array_equal(pd, P32.astype(np.float64))
    np.testing.assert_allclose(loss, 0.05 * le[1], rtol=1e-6)
    fd1, pd1, loss1 = O.device_balance_stats(f32, P32, 1, 0.05)
    np.testing.assert_allclose(fd1, [1.0], rtol=1e-6)
    np.testing.assert_allclose(pd1, [1.0], rtol=1e-6)
    np.testing.assert_allclose(loss1, 0.05, rtol=1e-5)


# ------------------------------------------------------------ bias update

def test_bias_update_directions_and_balance():
    """Worked-example loads: E1 is over-loaded (3 of 6 selections against a
    target share of K'/N' = 1/2 per token), the others under-loaded; the
    update lowers E1's bias, raises the others, and moves sum b by
    alpha (K' - sum c / T) = 0."""
    idx, g = worked_example_idx()
    N, K, T = g["n_routed"], g["top_k"], g["T"]
    c = O.counts(idx, N)
    b0 = np.zeros(N, np.float32)
    b1 = O.bias_update(c, T, K, 0.1, b0)
    assert b1[0] < 0 and np.all(b1[1:] > 0)
    assert abs(float(b1.astype(np.float64).sum())) < 1e-7
    # exactly balanced loads leave the bias bit-identical; alpha = 0 too
    bal = np.full(N, 4 * K // N, np.int32)        # T' K' / N' selections each, T' = 4
    b = np.random.default_rng(0).uniform(-0.05, 0.05, N).astype(np.float32)
    np.testing.assert_array_equal(O.bias_update(bal, 4, K, 0.1, b), b)
    np.testing.assert_array_equal(O.bias_update(c, T, K, 0.0, b), b)


def test_bias_update_closed_loop_reduces_skew():
    """Routing with the live bias on a Zipf-skewed router: repeated updates
    from each batch's counts pull the max/mean load down (the closed loop the
    V4 book describes for V3)."""
    T, N, K = 512, 32, 4
    rng = np.random.default_rng(5)
    ranks = rng.permutation(N) + 1
    off = (-1.1 * np.log(ranks)).astype(np.float32)
    off -= off.mean()
    b = np.zeros(N, np.float32)

    def load(bias, seed):
        lg = rand_logits(T, N, seed)
        idx, _, _, _ = O.route(lg, N, K, "sigmoid", True, offset=off, bias=bias)
        c = O.counts(idx, N)
        return c, c.max() / c.mean()

    _, skew0 = load(b, 100)
    for step in range(60):
        c, _ = load(b, 200 + step)
        b = O.bias_update(c, T, K, 0.01, b)
    _, skew1 = load(b, 100)
    assert skew0 > 2.0
    assert skew1 < 0.6 * skew0, (skew0, skew1)


def _runs(runs, dtype=np.int64):
    return np.concatenate([np.full(n, v, dtype) for n, v in runs])


@pytest.mark.parametrize("case", [c["name"] for c in golden("bias_update_examples.json")["cases"]])
def test_bias_update_step_size_worked_examples(case):
    """The step size of the update, pinned by hand-worked numbers of the
    pages' examples (tests/golden/bias_update_examples.json): the V4 book's
    256K-token sequence over 384 experts with top-9 (a hot expert at 36000
    selections moves by -15/128 alpha, the others at 5400 by +3/1280 alpha)
    and the DeepSeekMoE notes' worked routing ([-1/2, 1/6, 1/6, 1/6] alpha).
    The share fbar_i is selections per token (sum_i fbar_i = K'); a reading
    with the notes' f_i = N' c_i / (K' T) against a target of 1 moves the
    hot expert by -5 alpha and fails here."""
    from fractions import Fraction
    g = next(c for c in golden("bias_update_examples.json")["cases"] if c["name"] == case)
    N, K, T, alpha = g["n_routed"], g["top_k"], g["n_tok"], g["alpha"]
    cnt = _runs(g["counts_runs"], np.int32)
    assert len(cnt) == N
    b0 = np.full(N, g["bias_in"], np.float32)
    got = O.bias_update(cnt, T, K, alpha, b0)
    delta = [Fraction(v) for n, v in g["expected_delta_runs_over_alpha"] for _ in range(n)]
    want = np.array([float(g["bias_in"]) + alpha * float(d) for d in delta], np.float64)
    # one rounding of the exact value to fp32 (the oracle works in double)
    np.testing.assert_allclose(got.astype(np.float64), want, rtol=2 ** -23, atol=0)
    # the update conserves sum_i b_i when sum_i c_i = K' T (the notes' example)
    if int(cnt.sum()) == K * T:
        assert abs(float(np.sum(got.astype(np.float64) - b0))) < 1e-7


def test_node_limit_statistics_of_the_v4_book_exercise():
    """V4 book ch. 02 sec. 4 exercise: 384 experts on 32 nodes of 12, top-9,
    at most M = 4 nodes per token.  With independent random logits the
    unrestricted top-9 lies within 4 nodes for far fewer than 1% of tokens,
    and the limit replaces a large share of the chosen experts (the page:
    possibly 30% or more).  A limit that is not applied replaces nothing;
    one applied to the wrong groups keeps more than 4 nodes."""
    T, N, K, G, M = 4000, 384, 9, 32, 4
    lg = rand_logits(T, N, 21)
    plain = O.route(lg, N, K, "sigmoid", True)[0]
    lim = O.route(lg, N, K, "sigmoid", True, n_groups=G, topk_groups=M)[0]
    nodes = lim // (N // G)
    assert max(len(set(r)) for r in nodes) <= M
    same = np.mean([set(a) == set(b) for a, b in zip(plain, lim)])
    replaced = np.mean([len(set(a) - set(b)) for a, b in zip(plain, lim)]) / K
    within4 = np.mean([len(set(r // (N // G))) <= M for r in plain])
    assert within4 < 0.01 and same < 0.01, (within4, same)
    assert replaced > 0.30, replaced
