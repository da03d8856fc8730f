"""Pins of the fp64 oracle against facts the pages and the mathematics fix.

None of these tests touches the GPU.  The central pin is losslessness
([RheoSampling] section 6, Theorem 1; [Acceptance Is Not Speed] section 1):
the token sequence the verifier emits is distributed exactly as the target
model's own autoregressive samples.  It is checked by exhaustive enumeration
of the uniforms' cells on a tiny, prefix-dependent toy model, evaluating the
oracle function itself at every cell midpoint.  A dropped term, a wrong sign,
a shifted slot index or a transposed p/q in the oracle changes the emitted
distribution and fails it.
"""

from __future__ import annotations

import itertools
import math
import os
from collections import defaultdict

import numpy as np
import pytest

import oracle
from oracle import verify_row, tempered_softmax, topk_keep_mask, decode_logits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- helpers
def softmax_T(l, T):
    """The test's own tempered softmax (used to define the toy target)."""
    l = np.asarray(l, dtype=np.float64)
    finite = np.isfinite(l)
    e = np.zeros_like(l)
    e[finite] = np.exp((l[finite] - l[finite].max()) / T)
    return e / e.sum()


class ToyModel:
    """Prefix-dependent target and draft logits for every prefix of length <= K."""

    def __init__(self, V, K, T, k=0, seed=0, corr=0.6):
        self.V, self.K, self.T, self.k = V, K, T, k
        rng = np.random.default_rng(seed)
        self.lp, self.lq = {}, {}
        for L in range(K + 1):
            for pre in itertools.product(range(V), repeat=L):
                lp = rng.normal(0.0, 1.5, V)
                lq = corr * lp + rng.normal(0.0, 1.2, V)
                self.lp[pre] = lp
                self.lq[pre] = lq

    def p(self, pre):
        return softmax_T(self.lp[tuple(pre)], self.T)

    def q(self, pre):
        lq = self.lq[tuple(pre)]
        if 0 < self.k < self.V:
            # brute-force rank: count ids that beat this one (larger value, or
            # equal value and lower id); kept iff fewer than k beat it
            keep = np.array([
                sum((lq[j] > lq[x]) or (lq[j] == lq[x] and j < x) for j in range(self.V)) < self.k
                for x in range(self.V)])
            lq = np.where(keep, lq, -np.inf)
        return softmax_T(lq, self.T)

    def inputs(self, d):
        K = self.K
        tl = np.stack([self.lp[tuple(d[:i])] for i in range(K + 1)])
        dl = np.stack([self.lq[tuple(d[:i])] for i in range(K)]) if K else np.zeros((0, self.V))
        return tl, dl


def enumerate_verifier(model: ToyModel):
    """Exact output distribution of the oracle over drafts and uniforms.

    Drafts are drawn autoregressively from the (truncated, tempered) draft
    model; for each draft sequence the unit cube of uniforms splits into
    cells on which the output is constant: u_i below or above the acceptance
    probability min(1, p/q) at each reached position, and u_K in one interval
    per token of the normalised final distribution.  The oracle is evaluated
    at each cell's midpoint and the cell's measure is credited to its output.
    """
    V, K = model.V, model.K
    dist = defaultdict(float)
    exp_n = 0.0
    total = 0.0
    for d in itertools.product(range(V), repeat=K):
        wd = 1.0
        for i in range(K):
            wd *= model.q(d[:i])[d[i]]
        if wd == 0.0:
            continue
        tl, dl = model.inputs(d)
        P = [model.p(d[:i]) for i in range(K + 1)]
        Q = [model.q(d[:i]) for i in range(K)]
        a = [min(1.0, P[i][d[i]] / Q[i][d[i]]) for i in range(K)]
        for n in range(K + 1):
            meas = 1.0
            u = [0.5] * (K + 1)
            for i in range(n):
                meas *= a[i]
                u[i] = a[i] / 2.0
            if n < K:
                meas *= 1.0 - a[n]
                u[n] = (a[n] + 1.0) / 2.0
            if meas <= 0.0:
                continue
            w = np.maximum(0.0, P[n] - Q[n]) if n < K else P[K].copy()
            w = w / w.sum()
            cum = np.cumsum(w)
            for x in range(V):
                if w[x] <= 0.0:
                    continue
                lo = cum[x - 1] if x else 0.0
                u[K] = (lo + cum[x]) / 2.0
                r = verify_row(tl, dl, d, u, model.T, model.k)
                out = tuple(int(t) for t in r.tokens[: r.n + 1])
                m = wd * meas * w[x]
                dist[out] += m
                exp_n += m * r.n
                total += m
    return dist, exp_n, total


def check_lossless(model: ToyModel, dist, tol=1e-12):
    """P(len>=m, t_1..m = s) == P(len>=m, t_<m = s_<m) * p(s_m | s_<m) for all m, s."""
    K, V = model.K, model.V
    for m in range(1, K + 2):
        head = defaultdict(float)   # first m tokens of outputs with len >= m
        pre = defaultdict(float)    # first m-1 tokens of outputs with len >= m
        for out, mass in dist.items():
            if len(out) >= m:
                head[out[:m]] += mass
                pre[out[: m - 1]] += mass
        for s_prev, mass_prev in pre.items():
            p = model.p(s_prev)
            for x in range(V):
                lhs = head.get(s_prev + (x,), 0.0)
                assert abs(lhs - mass_prev * p[x]) < tol, (m, s_prev, x, lhs, mass_prev * p[x])


def expected_n_closed_form(model: ToyModel):
    """E[n] = sum_j sum_{s in V^j} prod_{i<=j} min(p_i(s_i|s_<i), q_i(s_i|s_<i)).

    Position j is reached and accepted with probability q*min(1, p/q) =
    min(p, q) at each step, so P(n >= j) is that product summed over s.
    """
    V, K = model.V, model.K
    total = 0.0
    for j in range(1, K + 1):
        for s in itertools.product(range(V), repeat=j):
            prod = 1.0
            for i in range(j):
                prod *= min(model.p(s[:i])[s[i]], model.q(s[:i])[s[i]])
            total += prod
    return total


# ----------------------------------------------------- losslessness (Theorem 1)
@pytest.mark.parametrize("V,K,T,k,seed", [
    (5, 3, 1.0, 0, 1),
    (4, 3, 0.7, 0, 2),
    (8, 2, 1.3, 0, 3),
    (6, 3, 0.8, 3, 4),     # sparse draft: q~ keeps the top 3 of 6
    (8, 2, 1.0, 1, 5),     # k = 1: the draft is one-hot
    (6, 0, 0.9, 0, 6),     # K = 0: plain sampling from p_0
])
def test_lossless_enumeration(V, K, T, k, seed):
    model = ToyModel(V, K, T, k, seed)
    dist, exp_n, total = enumerate_verifier(model)
    assert abs(total - 1.0) < 1e-12
    check_lossless(model, dist)
    assert abs(exp_n - expected_n_closed_form(model)) < 1e-12


def test_expected_n_prefix_independent_geometric():
    """With prefix-independent p and q, E[n] = alpha (1 - alpha^K) / (1 - alpha),
    alpha = sum_x min(p(x), q(x))."""
    V, K, T = 6, 3, 1.0
    model = ToyModel(V, K, T, 0, seed=7)
    lp, lq = model.lp[()], model.lq[()]
    for key in model.lp:
        model.lp[key] = lp
        model.lq[key] = lq
    alpha = float(np.minimum(softmax_T(lp, T), softmax_T(lq, T)).sum())
    dist, exp_n, total = enumerate_verifier(model)
    assert abs(exp_n - alpha * (1 - alpha ** K) / (1 - alpha)) < 1e-12
    check_lossless(model, dist)


# ------------------------------------------------------------------ greedy
@pytest.mark.parametrize("V,K,seed", [(5, 3, 11), (7, 2, 12), (3, 3, 13)])
def test_greedy_equals_greedy_decode_prefix(V, K, seed):
    """T = 0: the output is the greedy decode of the target up to and including
    the first position where the draft disagrees ([nalar] "Semantik ...")."""
    model = ToyModel(V, K, 1.0, 0, seed)
    g = []
    for i in range(K + 1):
        g.append(int(np.argmax(model.lp[tuple(g)])))
    for d in itertools.product(range(V), repeat=K):
        tl, dl = model.inputs(d)
        r = verify_row(tl, dl, d, np.full(K + 1, 0.5), 0.0)
        n = 0
        while n < K and d[n] == g[n]:
            n += 1
        assert r.n == n
        assert list(r.tokens[: n + 1]) == g[: n + 1]
        assert all(t == -1 for t in r.tokens[n + 1:])


def test_greedy_argmax_tie_lowest_id_and_ignores_uniforms():
    tl = np.array([[0.0, 2.0, 2.0, 1.0], [5.0, 5.0, 0.0, 0.0]])
    for u in ([0.0, 0.0], [0.999, 0.3]):
        r = verify_row(tl, None, [2], u, 0.0)        # draft 2 ties with 1 at the max
        assert r.n == 0 and list(r.tokens) == [1, -1]
        r = verify_row(tl, None, [1], u, -1.0)       # T < 0 is greedy too
        assert r.n == 1 and list(r.tokens) == [1, 0]


# ------------------------------------------------------------ worked example
def test_early_rejection_golden():
    """[nalar] "Penolakan ...": d1 d2 accepted, d3 rejected, d4 unused."""
    with open(os.path.join(GOLDEN, "early_rejection.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    status = [s for _, s in rows]
    K, V = len(rows), 8
    d = [1, 2, 3, 4]
    c = 6
    ninf = -np.inf
    tl = np.zeros((K + 1, V))
    dl = np.zeros((K, V))
    # positions 0, 1: draft equals target -> ratio 1 -> accepted for any u < 1
    tl[0] = dl[0] = np.linspace(-1, 1, V)
    tl[1] = dl[1] = np.linspace(1, -1, V)
    # position 2: the target gives d3 probability 0 and all mass to c; the
    # draft is one-hot at d3 -> rejected, residual is one-hot at c
    tl[2] = ninf
    tl[2, c] = 0.0
    dl[2] = ninf
    dl[2, d[2]] = 0.0
    tl[3] = dl[3] = 0.0
    u = [0.3, 0.9, 0.1, 0.5, 0.77]
    r = verify_row(tl, dl, d, u, 1.0)
    expected = []
    n_ok = 0
    for i, s in enumerate(status):
        if s == "ok":
            expected.append(d[i])
            n_ok += 1
        elif s == "reject":
            expected.append(c)
        else:
            expected.append(-1)
    expected.append(-1)  # bonus slot unused after a rejection
    assert status == ["ok", "ok", "reject", "unused"]
    assert r.n == n_ok == 2
    assert list(r.tokens) == expected == [1, 2, 6, -1, -1]


# -------------------------------------------------------------- softmax pins
def test_decode_bf16_exact():
    bits = np.array([0x3F80, 0xC000, 0xFF80, 0x7F80, 0x3F81, 0x0000, 0x8000, 0x4120], dtype=np.uint16)
    v = decode_logits(bits, oracle.BF16)
    assert v[0] == 1.0 and v[1] == -2.0 and v[2] == -np.inf and v[3] == np.inf
    assert v[4] == 1.0 + 2.0 ** -7 and v[5] == 0.0 and v[6] == 0.0 and v[7] == 10.0
    f = decode_logits(np.array([0.1], dtype=np.float32), oracle.F32)
    assert f[0] == float(np.float32(0.1))


def test_softmax_closed_forms():
    p = tempered_softmax(np.array([0.0, math.log(2), math.log(3)]), 1.0)
    np.testing.assert_allclose(p, [1 / 6, 2 / 6, 3 / 6], rtol=0, atol=1e-15)
    p2 = tempered_softmax(np.array([0.0, 2 * math.log(2), 2 * math.log(3)]), 2.0)
    np.testing.assert_allclose(p2, [1 / 6, 2 / 6, 3 / 6], rtol=0, atol=1e-15)
    assert np.all(tempered_softmax(np.full(7, 3.25), 0.6) == 1.0 / 7)
    oh = tempered_softmax(np.array([-np.inf, 4.0, -np.inf]), 0.5)
    assert list(oh) == [0.0, 1.0, 0.0]
    rng = np.random.default_rng(0)
    l = rng.normal(0, 3, 1000)
    p = tempered_softmax(l, 0.7)
    assert abs(p.sum() - 1.0) < 1e-12
    np.testing.assert_allclose(tempered_softmax(l + 123.0, 0.7), p, rtol=1e-12, atol=0)


# ----------------------------------------------------------------- top-k pins
@pytest.mark.parametrize("k", [1, 2, 5, 17, 64])
def test_topk_matches_brute_force_rank(k):
    rng = np.random.default_rng(k)
    l = rng.integers(-4, 5, size=97).astype(np.float64)   # many exact ties
    keep = topk_keep_mask(l, k)
    beats = np.array([np.sum((l > l[x]) | ((l == l[x]) & (np.arange(97) < x))) for x in range(97)])
    assert np.array_equal(keep, beats < k)
    assert keep.sum() == k


def test_topk_ties_lowest_id_and_degenerate_k():
    l = np.array([1.0, 3.0, 3.0, 2.0, 3.0, -np.inf])
    assert list(np.flatnonzero(topk_keep_mask(l, 2))) == [1, 2]
    assert list(np.flatnonzero(topk_keep_mask(l, 3))) == [1, 2, 4]
    assert list(np.flatnonzero(topk_keep_mask(l, 4))) == [1, 2, 3, 4]
    assert topk_keep_mask(l, 0).all() and topk_keep_mask(l, 6).all() and topk_keep_mask(l, 99).all()
    assert list(np.flatnonzero(topk_keep_mask(l, 1))) == [1]


def test_topk_k1_gives_one_hot_draft():
    rng = np.random.default_rng(3)
    tl = rng.normal(0, 1, (2, 9))
    dl = rng.normal(0, 1, (1, 9))
    top = int(np.argmax(dl[0]))
    r = verify_row(tl, dl, [top], [0.5, 0.5], 1.0, k=1)
    assert r.q_d[0] == 1.0
    other = (top + 1) % 9
    r = verify_row(tl, dl, [other], [0.0, 0.5], 1.0, k=1)
    assert r.q_d[0] == 0.0


# ------------------------------------------------------------ acceptance pins
def test_identical_distributions_accept_everything():
    rng = np.random.default_rng(5)
    K, V = 4, 50
    tl = rng.normal(0, 2, (K + 1, V))
    dl = tl[:K].copy()
    for _ in range(50):
        d = rng.integers(0, V, K)
        u = rng.random(K + 1)
        u[:K] = np.minimum(u[:K], 1 - 2.0 ** -24)
        r = verify_row(tl, dl, d, u, 0.9)
        assert r.n == K


def test_disjoint_supports_reject_first():
    V, K = 10, 3
    tl = np.full((K + 1, V), -np.inf)
    tl[:, :5] = 0.0
    dl = np.full((K, V), -np.inf)
    dl[:, 5:] = 0.0
    for d0 in range(5, 10):
        for u0 in (0.0, 0.5, 0.999):
            r = verify_row(tl, dl, [d0, 6, 7], [u0, 0.1, 0.1, 0.4], 1.0)
            assert r.n == 0
            assert 0 <= r.tokens[0] < 5        # the correction comes from the target's support


def test_confident_draft_does_not_force_acceptance():
    """[nalar] "Model target tetap menjadi otoritas distribusi": a one-hot draft
    at d is accepted with probability p(d), not 1."""
    V = 6
    tl = np.array([[0.0, math.log(3 / 7), math.log(2 / 7), -1.0, -2.0, -3.0], [0.0] * 6])
    p_d = softmax_T(tl[0], 1.0)[1]
    dl = np.full((1, V), -np.inf)
    dl[0, 1] = 0.0
    M = 20000
    acc = sum(verify_row(tl, dl, [1], [(j + 0.5) / M, 0.5], 1.0).n for j in range(M))
    assert abs(acc / M - p_d) <= 1.0 / M


def test_strict_branch_q_le_p_always_accepts():
    """[Acceptance Is Not Speed] section 6 harness, strict branch: q(d) <= p(d) accepts."""
    rng = np.random.default_rng(9)
    V = 12
    for _ in range(200):
        tl = rng.normal(0, 2, (2, V))
        dl = rng.normal(0, 2, (1, V))
        P = softmax_T(tl[0], 1.1)
        Q = softmax_T(dl[0], 1.1)
        for x in np.flatnonzero(Q <= P):
            for u in (0.0, 0.5, 1 - 2.0 ** -24):
                assert verify_row(tl, dl, [x], [u, 0.5], 1.1).n == 1


def test_out_of_range_draft_token_rejected():
    tl = np.zeros((3, 4))
    dl = np.zeros((2, 4))
    for bad in (-1, 4, 1 << 30):
        r = verify_row(tl, dl, [0, bad], [0.0, 0.0, 0.5], 1.0)
        assert r.n == 1 and r.p_d[1] == 0.0 and r.q_d[1] == 0.0
        assert r.tokens[0] == 0 and 0 <= r.tokens[1] < 4 and r.tokens[2] == -1


# -------------------------------------------------------------- residual pins
def test_residual_mass_is_total_variation():
    """S = sum max(0, p - q) = 1 - sum min(p, q) after a rejection."""
    rng = np.random.default_rng(21)
    V = 40
    hits = 0
    for _ in range(200):
        tl = rng.normal(0, 2, (2, V))
        dl = rng.normal(0, 2, (1, V))
        P = softmax_T(tl[0], 0.8)
        Q = softmax_T(dl[0], 0.8)
        x = int(np.argmax(Q / np.maximum(P, 1e-300)))   # a draft with q > p
        r = verify_row(tl, dl, [x], [0.999999, 0.5], 0.8)
        if r.n == 0:
            hits += 1
            assert abs(r.S - (1.0 - np.minimum(P, Q).sum())) < 1e-12
    assert hits > 100


def test_residual_never_picks_token_where_p_le_q():
    rng = np.random.default_rng(22)
    V = 30
    tl = rng.normal(0, 2, (2, V))
    dl = rng.normal(0, 2, (1, V))
    P, Q = softmax_T(tl[0], 1.0), softmax_T(dl[0], 1.0)
    x = int(np.argmax(Q - P))
    for j in range(2000):
        r = verify_row(tl, dl, [x], [0.9999999, (j + 0.5) / 2000], 1.0)
        assert r.n == 0
        y = r.tokens[0]
        assert P[y] > Q[y]


def test_zero_residual_falls_back_to_target():
    """u = 1 (outside [0, 1)) with p == q forces a rejection with zero residual."""
    tl = np.array([[0.0, math.log(3.0)], [0.0, 0.0]])
    dl = tl[:1].copy()
    r = verify_row(tl, dl, [0], [1.0, 0.3], 1.0)
    assert r.n == 0 and r.fallback and r.S == 1.0
    assert r.tokens[0] == 1          # p = [1/4, 3/4]: t = 0.3 falls in token 1's interval


# --------------------------------------------------------------- sampler pins
def test_k0_is_textbook_inverse_cdf():
    rng = np.random.default_rng(31)
    V = 25
    tl = rng.normal(0, 2, (1, V))
    P = softmax_T(tl[0], 0.9)
    for u in rng.random(300):
        r = verify_row(tl, np.zeros((0, V)), [], [u], 0.9)
        assert r.n == 0
        assert r.tokens[0] == np.searchsorted(np.cumsum(P), u, side="right")


def test_zero_weight_token_never_emitted_at_u_zero():
    tl = np.array([[-np.inf, 0.0, 0.0]])
    r = verify_row(tl, np.zeros((0, 3)), [], [0.0], 1.0)
    assert r.tokens[0] == 1


def test_bonus_after_all_accepted_uses_last_position():
    V = 4
    tl = np.zeros((3, V))
    tl[2] = [-np.inf, -np.inf, -np.inf, 0.0]     # bonus position is one-hot at 3
    dl = np.zeros((2, V))
    r = verify_row(tl, dl, [1, 2], [0.5, 0.5, 0.5], 1.0)
    assert r.n == 2 and list(r.tokens) == [1, 2, 3]


def test_margins_and_gap_reported():
    tl = np.array([[0.0, 0.0], [0.0, 0.0]])
    dl = np.array([[0.0, -np.inf]])
    r = verify_row(tl, dl, [0], [0.25, 0.5], 1.0)   # p = 0.5, q = 1
    assert r.n == 1 and abs(r.margins[0] - 0.25) < 1e-15
    assert abs(r.gap - 0.0) < 1e-15                  # t = 0.5 sits on the edge between 0 and 1
    assert r.tokens[1] == 1


# ------------------------------------------------ relaxed (lossy) acceptance
# [Acceptance Is Not Speed] sections 1, 6 and 7: relaxed verification accepts
# d with probability min(1, gamma(p)/q), gamma = min(p + sqrt(2 alpha p (1-p)), 1),
# behind a support guard on the target rank and probability of d.
def _two_token_logits(p0, T):
    """Logits of two tokens whose tempered softmax gives token 0 probability p0."""
    return np.array([0.0, T * math.log((1.0 - p0) / p0)])


def _accept_threshold(tl, dl, tok, T, relaxed, lo=0.0, hi=1.0, iters=60):
    """sup{u : the oracle accepts d at u}, by bisection (acceptance is an
    interval [0, u*) in u)."""
    if verify_row(tl, dl, [tok], [hi * (1 - 1e-15), 0.5], T, 0, relaxed).n == 1:
        return 1.0
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if verify_row(tl, dl, [tok], [mid, 0.5], T, 0, relaxed).n == 1:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


@pytest.mark.parametrize("alpha,p,q,expected", [
    (0.5, 0.2, 0.8, 0.75),     # gamma = 0.2 + sqrt(2*0.5*0.2*0.8) = 0.6; 0.6/0.8
    (0.125, 0.5, 0.9, 0.75 / 0.9),  # gamma = 0.5 + sqrt(0.0625) = 0.75
    (0.0, 0.2, 0.8, 0.25),     # alpha = 0: the lossless ratio p/q
    (2.0, 0.5, 0.6, 1.0),      # gamma clipped at 1 > q: always accepted
])
def test_relaxed_acceptance_probability(alpha, p, q, expected):
    T = 0.7
    tl = np.stack([_two_token_logits(p, T), np.zeros(2)])
    dl = _two_token_logits(q, T)[None, :]
    thr = _accept_threshold(tl, dl, 0, T, oracle.Relaxed(alpha=alpha))
    assert abs(thr - expected) < 1e-9, (thr, expected)


def test_relaxed_zero_alpha_without_guard_is_lossless():
    rng = np.random.default_rng(5)
    for trial in range(40):
        V, K = 9, 3
        tl = rng.normal(0, 2, (K + 1, V))
        dl = tl[:K] + rng.normal(0, 1, (K, V))
        d = rng.integers(0, V, K)
        u = rng.random(K + 1)
        k = [0, 4][trial % 2]
        a = verify_row(tl, dl, d, u, 0.9, k)
        b = verify_row(tl, dl, d, u, 0.9, k, oracle.Relaxed())
        assert a.n == b.n and list(a.tokens) == list(b.tokens)


def test_relaxed_never_accepts_less_than_lossless():
    rng = np.random.default_rng(6)
    for _ in range(60):
        V, K = 7, 4
        tl = rng.normal(0, 2, (K + 1, V))
        dl = tl[:K] + rng.normal(0, 1.5, (K, V))
        d = rng.integers(0, V, K)
        u = rng.random(K + 1)
        a = verify_row(tl, dl, d, u, 1.0)
        b = verify_row(tl, dl, d, u, 1.0, 0, oracle.Relaxed(alpha=0.3))
        assert b.n >= a.n


def test_target_rank_brute_force():
    rng = np.random.default_rng(7)
    for _ in range(50):
        l = np.round(rng.normal(0, 1, 40), 1)   # many ties
        tok = int(rng.integers(0, 40))
        better = sum(1 for x in range(40) if l[x] > l[tok])
        assert oracle.target_rank(l, tok) == better + 1
    # through the verifier's diagnostics
    tl = np.array([[3.0, 2.0, 2.0, 1.0, 0.0], [0.0] * 5])
    dl = np.array([[3.0, 2.0, 2.0, 1.0, 0.0]])
    r = verify_row(tl, dl, [3], [0.0, 0.5], 1.0, 0, oracle.Relaxed(max_rank=10))
    assert r.ranks[0] == 4


def test_support_guard():
    T = 1.0
    tl = np.array([[3.0, 2.0, 1.0, 0.0, -1.0], [0.0] * 5])
    dl = np.array([[0.0, 0.0, -4.0, 0.0, 0.0]])   # q(2) < p(2): the strict branch would accept
    p2 = softmax_T(tl[0], T)[2]
    assert verify_row(tl, dl, [2], [0.0, 0.5], T).n == 1
    assert verify_row(tl, dl, [2], [0.0, 0.5], T, 0, oracle.Relaxed(max_rank=2)).n == 0
    assert verify_row(tl, dl, [2], [0.0, 0.5], T, 0, oracle.Relaxed(max_rank=3)).n == 1
    assert verify_row(tl, dl, [2], [0.0, 0.5], T, 0, oracle.Relaxed(min_prob=p2 * 1.01)).n == 0
    assert verify_row(tl, dl, [2], [0.0, 0.5], T, 0, oracle.Relaxed(min_prob=p2 * 0.99)).n == 1
    # a token outside [0, V) is rejected whatever the budget
    assert verify_row(tl, dl, [7], [0.0, 0.5], T, 0, oracle.Relaxed(alpha=5.0)).n == 0


def test_relaxed_rejection_draws_the_lossless_residual():
    rng = np.random.default_rng(8)
    for _ in range(30):
        V, K = 8, 2
        tl = rng.normal(0, 2, (K + 1, V))
        dl = tl[:K] + rng.normal(0, 2, (K, V))
        d = [int(np.argmax(dl[0])), 0]
        u = np.array([0.999999, 0.5, rng.random()])
        a = verify_row(tl, dl, d, u, 1.0)
        b = verify_row(tl, dl, d, u, 1.0, 0, oracle.Relaxed(alpha=0.05))
        if a.n == 0 and b.n == 0:
            assert a.tokens[0] == b.tokens[0] and abs(a.S - b.S) < 1e-15


# ---------------------------------------------- KL(p || q) per position
# gist.science summary of 2605.09329, section 2: the distillation signal is
# KL(p || q) over the verified positions.
def test_kl_two_token_closed_form():
    # p = (1/2, 1/2), q = (1/4, 3/4): KL = 1/2 ln 2 + 1/2 ln(2/3) = 1/2 ln(4/3)
    T = 1.3
    tl = _two_token_logits(0.5, T)
    dl = _two_token_logits(0.25, T)
    assert abs(oracle.kl_divergence(tl, dl, T) - 0.5 * math.log(4.0 / 3.0)) < 1e-14
    # p = (0.2, 0.8), q = (0.5, 0.5): 0.2 ln 0.4 + 0.8 ln 1.6
    tl = _two_token_logits(0.2, T)
    dl = _two_token_logits(0.5, T)
    assert abs(oracle.kl_divergence(tl, dl, T) - (0.2 * math.log(0.4) + 0.8 * math.log(1.6))) < 1e-14


def test_kl_properties():
    rng = np.random.default_rng(9)
    for _ in range(30):
        l = rng.normal(0, 2, 50)
        m = l + rng.normal(0, 1, 50)
        T = float(rng.uniform(0.3, 2.0))
        assert oracle.kl_divergence(l, l, T) == 0.0
        kl = oracle.kl_divergence(l, m, T)
        assert kl > 0
        # invariant to shifting either set of logits
        assert abs(oracle.kl_divergence(l + 3.0, m - 2.0, T) - kl) < 1e-12
        # temperature T on l equals temperature 1 on l / T
        assert abs(oracle.kl_divergence(l / T, m / T, 1.0) - kl) < 1e-12
    # a token the draft cannot produce while the target can: +inf
    assert oracle.kl_divergence([0.0, 0.0], [0.0, -np.inf], 1.0) == float("inf")
    # the target's zero-probability tokens contribute nothing
    assert abs(oracle.kl_divergence([0.0, -np.inf], [0.0, 0.0], 1.0) - math.log(2.0)) < 1e-15


def test_kl_rows_greedy_rows_are_nan():
    tr = np.zeros((2, 3, 4), dtype=np.float32)
    dr = np.zeros((2, 2, 4), dtype=np.float32)
    out = oracle.kl_rows(tr, dr, np.array([1.0, 0.0]), "f32")
    assert out.shape == (2, 2) and (out[0] == 0).all() and np.isnan(out[1]).all()


# ------------------------------------------------------ tree verification
# [RheoSampling] section 4 (RheoVerification): siblings tested in turn, each
# rejection replacing the target by the residual norm(max(0, r - q)); an
# accepted node is descended into.  Section 6 (Theorem 1): lossless.
TREES = {
    "fan2": [-1, 0, 0],                      # root with two children
    "fan3-deep": [-1, 0, 0, 0, 1, 3],        # three children; two of them have a child
    "binary2": [-1, 0, 0, 1, 1],             # root -> 2 children, the first has 2 children
    "chain3": [-1, 0, 1, 2],                 # a chain: the linear verifier
}


def _depths(parent):
    dep = [0] * len(parent)
    for c in range(1, len(parent)):
        dep[c] = dep[parent[c]] + 1
    return dep


def _prefix(parent, tok, v):
    out = []
    while v > 0:
        out.append(int(tok[v]))
        v = parent[v]
    return tuple(reversed(out))


def enumerate_tree_verifier(model, parent):
    """Exact output distribution of the tree oracle over draft trees (each
    node's token drawn independently from the draft at its parent) and the
    uniforms (a depth-first split of each tested node's uniform at its
    acceptance threshold; the final draw is credited with final_w)."""
    N, V = len(parent), model.V
    dist = defaultdict(float)
    for toks in itertools.product(range(V), repeat=N - 1):
        tok = (0,) + toks
        wt = 1.0
        for c in range(1, N):
            wt *= model.q(_prefix(parent, tok, parent[c]))[tok[c]]
        if wt == 0.0:
            continue
        tl = np.stack([model.lp[_prefix(parent, tok, v)] for v in range(N)])
        dl = np.stack([model.lq[_prefix(parent, tok, v)] for v in range(N)])

        def explore(fixed, meas):
            u = np.full(N, 0.5)
            for node, val in fixed.items():
                u[node] = val
            r = oracle.verify_tree_row(tl, dl, tok, parent, u, model.T, model.k)
            nxt = next(((node, thr) for node, _, _, _, thr in r.tested if node not in fixed), None)
            if nxt is None:
                for x in range(V):
                    if r.final_w[x] > 0:
                        out = tuple(int(t) for t in r.tokens[: r.n]) + (x,)
                        dist[out] += wt * meas * r.final_w[x]
                return
            node, thr = nxt
            a = min(1.0, thr)
            if a > 0:
                explore({**fixed, node: a / 2.0}, meas * a)
            if a < 1:
                explore({**fixed, node: (1.0 + a) / 2.0}, meas * (1.0 - a))

        explore({}, 1.0)
    return dist


@pytest.mark.parametrize("tree,V,T,k,seed", [
    ("fan2", 4, 1.0, 0, 41),
    ("fan3-deep", 4, 0.8, 0, 42),
    ("binary2", 4, 1.2, 0, 43),
    ("binary2", 5, 1.0, 3, 44),     # sparse draft at every node
    ("chain3", 3, 0.9, 0, 45),
])
def test_tree_lossless_enumeration(tree, V, T, k, seed):
    parent = TREES[tree]
    model = ToyModel(V, max(_depths(parent)), T, k, seed)
    dist = enumerate_tree_verifier(model, parent)
    assert abs(sum(dist.values()) - 1.0) < 1e-12
    check_lossless(model, dist)


def test_tree_chain_equals_linear_verifier():
    rng = np.random.default_rng(46)
    for trial in range(40):
        K, V = 4, 12
        tl = rng.normal(0, 2, (K + 1, V))
        dl = tl + rng.normal(0, 1, (K + 1, V))
        d = rng.integers(0, V, K)
        u_lin = rng.random(K + 1)
        parent = [-1] + list(range(K))
        tok = np.concatenate([[0], d])
        u_tree = np.concatenate([[u_lin[K]], u_lin[:K]])
        T = [0.8, 0.0][trial % 2]
        a = oracle.verify_row(tl, dl[:K], d, u_lin, T)
        b = oracle.verify_tree_row(tl, dl, tok, parent, u_tree, T)
        assert a.n == b.n and list(a.tokens) == list(b.tokens)
        if T > 0:
            assert abs(a.S - b.S) < 1e-15


def test_tree_greedy_is_greedy_decode():
    model = ToyModel(4, 2, 1.0, 0, 47)
    parent = TREES["binary2"]
    for toks in itertools.product(range(4), repeat=4):
        tok = (0,) + toks
        tl = np.stack([model.lp[_prefix(parent, tok, v)] for v in range(5)])
        r = oracle.verify_tree_row(tl, None, tok, parent, np.full(5, 0.5), 0.0)
        # brute force: the greedy decode of the toy target, and the longest
        # prefix of it that is a path of the tree (first matching child)
        s = ()
        for _ in range(3):
            s = s + (int(np.argmax(model.lp[s])),)
        v, n = 0, 0
        for depth in range(2):
            nxt = [c for c in range(1, 5) if parent[c] == v and tok[c] == s[depth]]
            if not nxt:
                break
            v, n = nxt[0], n + 1
        assert r.n == n and list(r.tokens[: n + 1]) == list(s[: n + 1])


def test_tree_residual_recursion_closed_form():
    """The closed form the GPU walk evaluates -- r_j = max(0, p - c_j q) / W_j
    with c_0 = 0, W_0 = 1, c_{j+1} = c_j + W_j, W_j = sum max(0, p - c_j q) --
    equals the page's recursion r_{j+1} = norm(max(0, r_j - q)), which the
    oracle takes ([RheoSampling] section 4), and W_j equals the product of the
    recursion's normalisers (the oracle's S, the mass the GPU reports)."""
    rng = np.random.default_rng(48)
    p = softmax_T(rng.normal(0, 2, 9), 1.0)
    q = softmax_T(rng.normal(0, 2, 9), 1.0)
    r, c, W, prod = p.copy(), 0.0, 1.0, 1.0
    for _ in range(4):
        nxt = np.maximum(0.0, r - q)
        if nxt.sum() == 0:
            break
        prod *= nxt.sum()
        r = nxt / nxt.sum()
        c = c + W
        W = np.maximum(0.0, p - c * q).sum()
        assert np.allclose(r, np.maximum(0.0, p - c * q) / W, atol=1e-14)
        assert abs(prod - W) < 1e-14
    # and the oracle tests the second sibling against r_1 = norm(max(0, p - q))
    tl = np.stack([np.log(p), np.zeros(9), np.zeros(9)])
    dl = np.stack([np.log(q), np.zeros(9), np.zeros(9)])
    x = int(np.argmax(np.maximum(0.0, p - q)))
    res = oracle.verify_tree_row(tl, dl, [0, int(np.argmax(q - p)), x], [-1, 0, 0], [0.5, 0.999999, 0.3], 1.0)
    r1 = np.maximum(0.0, p - q) / np.maximum(0.0, p - q).sum()
    assert res.tested[1][0] == 2 and abs(res.tested[1][3] - r1[x]) < 1e-14


# ------------------------------------------- batch wrappers and margins
# verify() and verify_tree() decode each row's stored logits (bf16 bit
# patterns widen exactly), read a row's draft only when it samples (greedy
# verification needs the target's argmax alone, [nalar] "Semantik penerimaan
# ..."), and return one result per requested row, in the requested order.
class _RowReads:
    """Stored logits that record which rows are read."""

    def __init__(self, a):
        self.a, self.read = a, []

    @property
    def shape(self):
        return self.a.shape

    def __getitem__(self, b):
        self.read.append(int(b))
        return self.a[b]


def _bf16(x):
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def _batch(seed=50, B=3, K=3, V=37):
    rng = np.random.default_rng(seed)
    tgt = _bf16(rng.normal(0, 2, (B, K + 1, V)))
    dft = _bf16(decode_logits(tgt[:, :K], "bf16") + rng.normal(0, 0.7, (B, K, V)))
    dft[1] = 0x7FC0                       # the greedy row's draft: NaN bits, never to be read
    tok = rng.integers(0, V, (B, K)).astype(np.int32)
    uni = rng.random((B, K + 1)).astype(np.float32)
    temp = np.array([0.7, 0.0, 1.3], dtype=np.float32)[:B]
    return tgt, dft, tok, uni, temp


def _same_row(a, b):
    assert a.n == b.n and list(a.tokens) == list(b.tokens) and a.greedy == b.greedy
    if not a.greedy:
        assert np.array_equal(a.p_d, b.p_d) and np.array_equal(a.q_d, b.q_d) and a.S == b.S


@pytest.mark.parametrize("topk", [0, 5])
def test_verify_batch_equals_rows_and_skips_greedy_drafts(topk):
    tgt, dft, tok, uni, temp = _batch()
    reads = _RowReads(dft)
    got = oracle.verify(tgt, reads, tok, uni, temp, topk, "bf16")
    assert 1 not in reads.read, "a greedy row's draft was read"
    assert len(got) == 3
    for b in range(3):
        dl = decode_logits(dft[b], "bf16") if temp[b] > 0 else None
        _same_row(got[b], oracle.verify_row(decode_logits(tgt[b], "bf16"), dl, tok[b], uni[b], float(temp[b]),
                                            topk))
    sub = oracle.verify(tgt, dft, tok, uni, temp, topk, "bf16", rows=[2, 0])
    _same_row(sub[0], got[2])
    _same_row(sub[1], got[0])


def test_verify_tree_batch_equals_rows_and_skips_greedy_drafts():
    rng = np.random.default_rng(51)
    B, N, V = 3, 5, 23
    tgt = _bf16(rng.normal(0, 2, (B, N, V)))
    dft = _bf16(decode_logits(tgt, "bf16") + rng.normal(0, 0.8, (B, N, V)))
    dft[1] = 0x7FC0
    par = np.array([[-1, 0, 0, 1, 1]] * B, dtype=np.int32)
    tok = rng.integers(0, V, (B, N)).astype(np.int32)
    uni = rng.random((B, N)).astype(np.float32)
    temp = np.array([0.9, 0.0, 1.4], dtype=np.float32)
    reads = _RowReads(dft)
    got = oracle.verify_tree(tgt, reads, tok, par, uni, temp, 0, "bf16")
    assert 1 not in reads.read, "a greedy row's draft was read"
    for b, rows in ((0, None), (1, None), (2, None)):
        dl = decode_logits(dft[b], "bf16") if temp[b] > 0 else None
        want = oracle.verify_tree_row(decode_logits(tgt[b], "bf16"), dl, tok[b], par[b], uni[b], float(temp[b]))
        assert got[b].path == want.path and list(got[b].tokens) == list(want.tokens)
        assert got[b].greedy == want.greedy and (want.greedy or got[b].S == want.S)
    sub = oracle.verify_tree(tgt, dft, tok, par, uni, temp, 0, "bf16", rows=[2, 1])
    assert list(sub[0].tokens) == list(got[2].tokens) and list(sub[1].tokens) == list(got[1].tokens)


def _two_token_row(p, q):
    """Target / draft logits over two ids with softmax (p, 1-p) and (q, 1-q) at T = 1."""
    return np.log([p, 1.0 - p]), np.log([q, 1.0 - q])


def test_min_margin_takes_reached_decisions_and_the_draw():
    # Position 0: p(0) = 0.3, q(0) = 0.6, u = 0.9 -> 0.54 >= 0.3, rejected
    # with margin 0.24.  Position 1 is never reached; its test sits exactly on
    # the threshold (u q = p, margin 0).  The residual max(0, p - q) = (0, 0.3)
    # has S = 0.3; u_K = 0.5 gives t = 0.15 inside id 1's interval [0, 0.3],
    # gap 0.15.  So the smallest margin of the decisions taken is 0.15.
    lp, lq = _two_token_row(0.3, 0.6)
    tl = np.stack([lp, lp, lp])
    dl = np.stack([lq, lq])
    r = verify_row(tl, dl, [0, 0], [0.9, 0.5, 0.5], 1.0)
    assert r.n == 0 and list(r.tokens) == [1, -1, -1]
    assert abs(r.margins[0] - 0.24) < 1e-12 and abs(r.margins[1]) < 1e-12
    assert abs(r.gap - 0.15) < 1e-12 and abs(r.min_margin() - 0.15) < 1e-12
    # Both accepted (u q < p at each position: 0.1*0.6 < 0.3), bonus draw from
    # p = (0.3, 0.7) at t = 0.31: id 1, gap 0.01; the margins are 0.24 each.
    r = verify_row(tl, dl, [0, 0], [0.1, 0.1, 0.31], 1.0)
    assert r.n == 2 and abs(r.min_margin() - 0.01) < 1e-12
    # A draw far from every edge: the smallest acceptance margin decides.
    r = verify_row(tl, dl, [0, 0], [0.1, 0.45, 0.65], 1.0)   # margins 0.24, 0.03; gap 0.35
    assert r.n == 2 and abs(r.min_margin() - 0.03) < 1e-12
    g = verify_row(tl, dl, [0, 0], [0.9, 0.5, 0.5], 0.0)
    assert g.min_margin() == float("inf")


def test_tree_min_margin_takes_tested_nodes_and_the_draw():
    # Root with two children, both with token 0: p = (0.3, 0.7), q = (0.6, 0.4).
    # Child 1: u = 0.9 -> 0.54 >= 0.3, rejected, margin 0.24.  The residual
    # norm(max(0, p - q)) = (0, 1), so child 2 (token 0, r = 0) is rejected with
    # margin |0.2 * 0.6 - 0| = 0.12; its residual max(0, (0, 1) - q) = (0, 0.6)
    # normalises to (0, 1) again, so S = 0.3 * 0.6 = 0.18 (in units of p:
    # max(0, p - 1.3 q) = (0, 0.18)).  The final draw from (0, 1) at
    # t = u_0 = 0.995 has gap 0.005.
    lp, lq = _two_token_row(0.3, 0.6)
    z = np.zeros(2)
    tl = np.stack([lp, z, z])
    dl = np.stack([lq, z, z])
    r = oracle.verify_tree_row(tl, dl, [0, 0, 0], [-1, 0, 0], [0.995, 0.9, 0.2], 1.0)
    assert r.n == 0 and [c for c, *_ in r.tested] == [1, 2] and r.tokens[0] == 1
    assert abs(r.margins[0] - 0.24) < 1e-12 and abs(r.margins[1] - 0.12) < 1e-12
    assert abs(r.S - 0.18) < 1e-12 and abs(r.gap - 0.005) < 1e-12
    assert abs(r.min_margin() - 0.005) < 1e-12
    r = oracle.verify_tree_row(tl, dl, [0, 0, 0], [-1, 0, 0], [0.5, 0.9, 0.2], 1.0)
    assert abs(r.min_margin() - 0.12) < 1e-12


def test_forced_outcome_follows_the_other_path():
    # The same two-token row: position 0 rejects (0.54 >= 0.3).  Forcing it to
    # accept continues at position 1 under the rule, without changing the
    # recorded outcome; forcing position 1 to reject ends the scan there.
    lp, lq = _two_token_row(0.3, 0.6)
    tl = np.stack([lp, lp, lp])
    dl = np.stack([lq, lq])
    u = [0.9, 0.1, 0.5]
    r = verify_row(tl, dl, [0, 0], u, 1.0)
    assert r.n == 0 and list(r.accept) == [False, True]
    f = verify_row(tl, dl, [0, 0], u, 1.0, force={0: True})
    assert f.n == 2 and list(f.accept) == [False, True] and list(f.tokens[:2]) == [0, 0]
    f = verify_row(tl, dl, [0, 0], u, 1.0, force={0: True, 1: False})
    assert f.n == 1 and f.tokens[1] == 1 and abs(f.S - 0.3) < 1e-12
    # Tree: forcing the first child to be accepted descends into it (a leaf:
    # bonus draw from its target, uniform over 2 ids at t = 0.995 -> id 1).
    z = np.zeros(2)
    t = oracle.verify_tree_row(np.stack([lp, z, z]), np.stack([lq, z, z]), [0, 0, 0], [-1, 0, 0],
                               [0.995, 0.9, 0.2], 1.0, force={1: True})
    assert t.path == [1] and list(t.tokens[:2]) == [0, 1] and t.accepts == [False] and t.S == 1.0


def test_near_ids_are_the_neighbours_of_t():
    # K = 0, four equally likely ids: the intervals are [0, .25], [.25, .5],
    # [.5, .75], [.75, 1].  t just above 0.5 draws id 2 and is within 1e-5 of
    # id 1's interval too; t = 0.6 is near id 2 only.  A zero-weight id (a
    # -inf logit) is never a neighbour, even when its empty interval sits at t.
    tl = np.zeros((1, 4))
    r = verify_row(tl, None, [], [0.5 + 1e-6], 1.0)
    assert r.tokens[0] == 2 and r.near_ids == (1, 2) and abs(r.t - (0.5 + 1e-6)) < 1e-15
    r = verify_row(tl, None, [], [0.6], 1.0)
    assert r.near_ids == (2,)
    tl = np.array([[0.0, -np.inf, 0.0, 0.0]])          # thirds; id 1 has weight 0
    r = verify_row(tl, None, [], [1.0 / 3.0 + 1e-7], 1.0)
    assert r.tokens[0] == 2 and r.near_ids == (0, 2)
