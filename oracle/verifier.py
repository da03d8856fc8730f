"""fp64 CPU oracle of the batched speculative-sampling verifier.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the product path.

Sources (cited by page title and section; no source code from the pages is
used, every step is restated from the mathematics):

* [nalar] "Speculative decoding: memverifikasi token draft sebelum diterima"
  (nalar.dev).  Subsections "Draft mengubah tebakan serial menjadi batch
  verifikasi" (one target pass gives the next-token distribution at every
  draft position, conditioned on the earlier drafts), "Semantik penerimaan
  bergantung pada algoritma decoding" (greedy: accept while the draft equals
  the target's greedy choice, the target's choice replaces the first mismatch;
  sampling: acceptance probability from p and q, then a correction
  distribution on rejection) and "Penolakan memendekkan pekerjaan speculative
  yang berguna" (nothing after the first rejection is committed).
* [RheoSampling] "RheoSampling 2026: Mengatasi Dilema One-Hot pada Stochastic
  Dynamic-Tree Speculative Decoding, ..." (newsaint.id).  Section 3 (the draft
  logits are cut to the 128 largest before the softmax, the rest set to -inf),
  section 4 (RheoVerification: a candidate is accepted with probability
  min(1, p/q~) where q~ is its true sampling probability; on rejection the
  residual norm(max(0, p - q~)) is the distribution sampled next), section 6
  (Theorem 1: the output distribution equals the target's) and section 7
  (temperature applies at the verification gate).
* [Acceptance Is Not Speed] newsaint.id article on arXiv:2610.23818, section 1
  (lossless speculative decoding keeps the target distribution) and the
  strict branch of the section 6 harness (q <= p always accepts).

Readings where the pages are silent:

* uniforms ``u[K+1]``: ``u[i]`` (i < K) drives the acceptance test at
  position i, ``u[K]`` drives the final (correction or bonus) sample;
* acceptance is the strict test ``u*q < p``;
* the final sample is the inverse CDF in ascending token id, taking the
  smallest x with ``C(x) > t`` (strict), ``t = u[K] * S``;
* a residual of total mass 0 (possible only through rounding) falls back to
  the target distribution at that position;
* ``T <= 0`` selects greedy verification; argmax ties go to the lowest id;
* top-k keeps exactly k ids, ties at the boundary go to the lowest id; it is
  applied to the draft only and only for ``T > 0`` rows; ``k <= 0`` or
  ``k >= V`` means no truncation;
* a draft token outside ``[0, V)`` has p = q = 0 and is rejected.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

BF16 = "bf16"
F32 = "f32"


def decode_logits(raw, dtype: str) -> np.ndarray:
    """Widen stored logits to float64 exactly.

    bf16 values arrive as their raw 16-bit patterns (uint16); a bf16 number
    is the upper half of the float32 with the same bits, so the widening is
    exact.  float32 values widen exactly to float64.
    """
    if dtype == BF16:
        u16 = np.asarray(raw, dtype=np.uint16)
        return (u16.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == F32:
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def tempered_softmax(logits: np.ndarray, T: float) -> np.ndarray:
    """softmax(logits / T) in float64; -inf logits get probability 0.

    Temperature is applied to the logits before the softmax at the
    verification gate ([RheoSampling] section 7).  The largest scaled logit is
    subtracted before exponentiation, which leaves the result unchanged.
    At least one logit must be finite.
    """
    z = np.asarray(logits, dtype=np.float64) / float(T)
    zmax = np.max(z)
    e = np.exp(z - zmax)
    return e / np.sum(e)


def topk_keep_mask(logits: np.ndarray, k: int) -> np.ndarray:
    """Boolean mask of the k largest logits, ties at the boundary to the lowest id.

    Sparse draft truncation ([RheoSampling] section 3): only the top
    candidates of the draft survive; every other logit becomes -inf before the
    softmax.  ``k <= 0`` or ``k >= V`` keeps everything.  A stable sort of the
    negated logits orders by value descending and, among equal values, by id
    ascending; the first k of that order are kept.
    """
    logits = np.asarray(logits, dtype=np.float64)
    V = logits.shape[0]
    keep = np.ones(V, dtype=bool)
    if k <= 0 or k >= V:
        return keep
    order = np.argsort(-logits, kind="stable")
    keep[:] = False
    keep[order[:k]] = True
    return keep


@dataclass(frozen=True)
class Relaxed:
    """Parameters of the lossy relaxed acceptance rule.

    [Acceptance Is Not Speed] section 1 describes relaxed verification that
    tolerates q > p within a divergence budget; its section 6 harness and
    section 7 recommendations add a support filter.  The rule, restated:

    * support guard: reject d if its target rank exceeds ``max_rank`` (rank 1
      is the most likely token; ``max_rank <= 0`` disables the check) or if
      p(d) < ``min_prob``;
    * strict branch: accept if q(d) <= p(d) (and p(d) > 0);
    * otherwise accept iff u * q(d) < gamma with
      gamma = min(p + sqrt(2 * alpha * p * (1 - p)), 1).

    With alpha = 0 and no guard this is the lossless rule.
    """

    alpha: float = 0.0
    max_rank: int = 0
    min_prob: float = 0.0


def relaxed_gamma(p: float, alpha: float) -> float:
    """gamma(p) = min(p + sqrt(2 alpha p (1 - p)), 1) ([Acceptance Is Not
    Speed] section 6: the reverse-KL budget expanded to second order)."""
    return min(p + float(np.sqrt(2.0 * alpha * p * (1.0 - p))), 1.0)


def target_rank(logits: np.ndarray, tok: int) -> int:
    """1 + the number of ids whose logit is strictly larger than tok's (equal
    logits share the better rank).  Order on logits equals order on p for
    T > 0."""
    logits = np.asarray(logits, dtype=np.float64)
    return 1 + int(np.count_nonzero(logits > logits[tok]))


@dataclass
class RowResult:
    """Outcome of verifying one row, with the diagnostics the parity tests use.

    tokens      int64 [K+1]: accepted drafts, then the final token, then -1.
    n           number of accepted drafts (0..K).
    greedy      True when the row was verified greedily (T <= 0).
    p_d, q_d    float64 [K]: target / draft probability of each draft token
                (all K positions, also those after the first rejection);
                NaN for greedy rows.
    margins     float64 [K]: |u_i*q_i - p_i| for each position (NaN greedy).
    S           total mass of the final distribution before normalisation
                (residual mass after a rejection, 1 for the bonus); NaN greedy.
    gap         distance from t = u_K*S to the nearer edge of the sampled
                token's CDF interval (probability units); inf for greedy.
    fallback    True when a zero residual fell back to the target row.
    ranks       int64 [K]: target rank of each draft token under the relaxed
                rule (0 when not computed or the token is out of range).
    accept      bool [K]: the rule's outcome at every position (also those
                after the first rejection); False for greedy rows.  A forced
                outcome (see verify_row) does not change it.
    t           u_K * S, the point of the final distribution's CDF that was
                sampled (NaN for greedy rows).
    near_ids    ids of positive weight whose CDF interval [C(x-1), C(x)]
                meets [t - draw_eps, t + draw_eps]: the draws a computation
                rounding differently could return (empty for greedy rows).
    """

    tokens: np.ndarray
    n: int
    greedy: bool
    p_d: np.ndarray
    q_d: np.ndarray
    margins: np.ndarray
    S: float
    gap: float
    fallback: bool
    ranks: np.ndarray = None
    accept: np.ndarray = None
    t: float = float("nan")
    near_ids: tuple = ()

    def min_margin(self) -> float:
        """Smallest margin over the decisions this row actually took.

        Those are the acceptance tests at positions 0..n (position n only if
        n < K, where it is the rejecting test) and the final inverse-CDF
        sample.  Greedy decisions compare exact values: margin inf.
        """
        if self.greedy:
            return float("inf")
        K = self.margins.shape[0]
        reached = self.margins[: min(self.n + 1, K)]
        m = float(np.min(reached)) if reached.size else float("inf")
        return min(m, self.gap)


def inverse_cdf(w: np.ndarray, t: float, draw_eps: float):
    """Inverse-CDF draw from the non-negative weights w at the point t.

    Ascending token id; the drawn token is the smallest x whose cumulative
    weight C(x) exceeds t (strict, so a zero-weight token is never drawn).
    If no C(x) exceeds t, which happens only when rounding lets t reach the
    total, the last id of positive weight is drawn.  Returns (x, gap,
    near_ids): gap is the distance from t to the nearer edge of x's interval
    [C(x-1), C(x)]; near_ids lists every id of positive weight whose interval
    meets [t - draw_eps, t + draw_eps].
    """
    C = np.cumsum(w)
    above = np.flatnonzero(C > t)
    if above.size:
        x = int(above[0])
    else:  # t reached the top only through rounding
        x = int(np.flatnonzero(w > 0)[-1])
    lo = C[x - 1] if x > 0 else 0.0
    gap = float(min(t - lo, C[x] - t))
    starts = np.concatenate(([0.0], C[:-1]))
    near = np.flatnonzero((w > 0) & (starts <= t + draw_eps) & (C >= t - draw_eps))
    return x, gap, tuple(int(i) for i in near)


def verify_row(tl, dl, d, u, T: float, k: int = 0, relaxed: Relaxed | None = None,
               force: dict | None = None, draw_eps: float = 1e-5) -> RowResult:
    """Verify one row of K draft tokens against K+1 target positions.

    tl  float64 [K+1, V] target logits; row i is the target's next-token
        logits after the accepted prefix plus drafts d_0..d_{i-1}
        ([nalar] "Draft mengubah tebakan serial menjadi batch verifikasi");
        row K is the bonus position.
    dl  float64 [K, V] draft logits; row i is the distribution d_i was drawn
        from (may be None when K == 0 or T <= 0).
    d   int [K] draft tokens.
    u   float [K+1] uniforms in [0, 1).
    T   temperature of this row; T <= 0 selects greedy verification.
    k   sparse draft truncation (0 = none).
    relaxed  optional lossy acceptance rule (see Relaxed); greedy rows and the
        final draw are unchanged by it (reading: a relaxed rejection is
        corrected from the same residual norm(max(0, p - q)), which the pages
        leave open).
    force   optional {position: accepted} overriding the rule's outcome at
        those positions of a sampling row.  The verifier itself never uses
        it; a test uses it to follow the other outcome of a decision that
        lies within rounding distance of its threshold, which a computation
        in another precision may take.
    draw_eps  half-width of the window around t that defines near_ids.
    """
    tl = np.asarray(tl, dtype=np.float64)
    Kp1, V = tl.shape
    K = Kp1 - 1
    d = np.asarray(d, dtype=np.int64).reshape(K)
    u = np.asarray(u, dtype=np.float64).reshape(K + 1)
    tokens = np.full(K + 1, -1, dtype=np.int64)
    nanK = np.full(K, np.nan)

    if not (T > 0):
        # Greedy verification ([nalar] "Semantik penerimaan ..."): a draft is
        # accepted while it equals the target's greedy choice at its position;
        # the target's greedy choice replaces the first mismatch, and after K
        # matches the greedy choice at the bonus position is emitted.
        # np.argmax returns the first (lowest) id among equal maxima.
        a = [int(np.argmax(tl[i])) for i in range(K + 1)]
        n = K
        for i in range(K):
            if int(d[i]) != a[i]:
                n = i
                break
        tokens[:n] = d[:n]
        tokens[n] = a[n]
        return RowResult(tokens, n, True, nanK, nanK.copy(), nanK.copy(),
                         float("nan"), float("inf"), False, np.zeros(K, dtype=np.int64),
                         np.zeros(K, dtype=bool))

    dl = np.zeros((0, V)) if K == 0 else np.asarray(dl, dtype=np.float64).reshape(K, V)
    P =[tempered_softmax(tl[i], T) for i in range(K + 1)]
    Q = []
    for i in range(K):
        keep = topk_keep_mask(dl[i], k)
        Q.append(tempered_softmax(np.where(keep, dl[i], -np.inf), T))

    # Acceptance scan ([RheoSampling] section 4, step 1): d_i is accepted
    # with probability min(1, p_i(d_i)/q_i(d_i)); with u_i uniform this is the
    # event u_i < p/q, written without a division as u_i*q < p (which also
    # gives the right limit q = 0).  The first rejection ends the committed
    # prefix ([nalar] "Penolakan memendekkan ...").
    p_d = np.zeros(K)
    q_d = np.zeros(K)
    margins = np.zeros(K)
    ranks = np.zeros(K, dtype=np.int64)
    accept = np.zeros(K, dtype=bool)
    for i in range(K):
        tok = int(d[i])
        if 0 <= tok < V:
            p_d[i] = P[i][tok]
            q_d[i] = Q[i][tok]
        if relaxed is None:
            accept[i] = u[i] * q_d[i] < p_d[i]
            margins[i] = abs(u[i] * q_d[i] - p_d[i])
            continue
        # Relaxed rule: the margin is the smallest distance of any comparison
        # the rule evaluates to its threshold.
        p, q = p_d[i], q_d[i]
        m = float("inf")
        ok = True
        if not (0 <= tok < V):
            ok = False  # p = q = 0: rejected, as under the lossless rule
        else:
            ranks[i] = target_rank(tl[i], tok)
            if relaxed.max_rank > 0 and ranks[i] > relaxed.max_rank:
                ok = False
        if ok and relaxed.min_prob > 0:
            m = min(m, abs(p - relaxed.min_prob))
            ok = p >= relaxed.min_prob
        if ok:
            m = min(m, abs(q - p))
            if p > 0 and q <= p:
                accept[i] = True
            else:
                g = relaxed_gamma(p, relaxed.alpha)
                m = min(m, abs(u[i] * q - g))
                accept[i] = u[i] * q < g
        margins[i] = m
    taken = accept.copy()
    for i, outcome in (force or {}).items():
        taken[int(i)] = bool(outcome)
    n = K
    for i in range(K):
        if not taken[i]:
            n = i
            break

    # Final distribution ([RheoSampling] section 4, step 3): after a rejection
    # at position n, the residual max(0, p_n - q_n) (normalised); when every
    # draft was accepted, the target at the bonus position.
    fallback = False
    if n < K:
        w = np.maximum(0.0, P[n] - Q[n])
        S = float(np.sum(w))
        if S == 0.0:
            w = P[n]
            S = float(np.sum(w))
            fallback = True
    else:
        w = P[K]
        S = float(np.sum(w))

    # Inverse-CDF sample with u_K: ascending token id, first x whose
    # cumulative weight exceeds t = u_K * S.
    t = u[K] * S
    x, gap, near_ids = inverse_cdf(w, t, draw_eps)

    tokens[:n] = d[:n]
    tokens[n] = x
    return RowResult(tokens, n, False, p_d, q_d, margins, S, gap, fallback, ranks, accept, float(t), near_ids)


def verify(target_raw, draft_raw, draft_tokens, uniforms, temperature,
           topk: int, dtype: str, rows=None, relaxed: Relaxed | None = None) -> list[RowResult]:
    """Verify a batch row by row.

    target_raw  [B, K+1, V] stored logits (uint16 bf16 patterns or float32)
    draft_raw   [B, K, V] stored logits (may be None if K == 0)
    draft_tokens int [B, K]; uniforms float [B, K+1]; temperature float [B]
    rows        optional iterable of row indices (default: all rows)
    relaxed     optional lossy acceptance rule (see Relaxed)
    """
    B = target_raw.shape[0]
    K = target_raw.shape[1] - 1
    out = []
    for b in (range(B) if rows is None else rows):
        tl = decode_logits(target_raw[b], dtype)
        T = float(temperature[b])
        dl = None
        if K > 0 and T > 0:
            dl = decode_logits(draft_raw[b], dtype)
        out.append(verify_row(tl, dl, draft_tokens[b], uniforms[b], T, topk, relaxed))
    return out


def kl_divergence(target_logits, draft_logits, T: float) -> float:
    """KL(p || q) = sum_x p(x) log(p(x) / q(x)) of the tempered softmaxes, in
    nats, in float64.

    The test-time speculation summary on gist.science (paper 2605.09329,
    section 2) distils the drafter with KL(p || q) between the target's and
    the drafter's distributions over the verified positions; this is that
    value, exactly, at one position.  Terms with p(x) = 0 contribute 0; a
    token with p(x) > 0 and q(x) = 0 makes it +inf.
    """
    P = tempered_softmax(target_logits, T)
    Q = tempered_softmax(draft_logits, T)
    m = P > 0
    if np.any(Q[m] == 0):
        return float("inf")
    return float(np.sum(P[m] * (np.log(P[m]) - np.log(Q[m]))))


def kl_rows(target_raw, draft_raw, temperature, dtype: str, rows=None) -> np.ndarray:
    """KL(p_i || q_i) for every draft position i of each row: float64 [n, K].
    Greedy rows (T <= 0) have no sampling distribution: NaN."""
    B = target_raw.shape[0]
    K = target_raw.shape[1] - 1
    rows = range(B) if rows is None else rows
    out = []
    for b in rows:
        T = float(temperature[b])
        if not (T > 0):
            out.append(np.full(K, np.nan))
            continue
        tl = decode_logits(target_raw[b], dtype)
        dl = decode_logits(draft_raw[b], dtype)
        out.append(np.array([kl_divergence(tl[i], dl[i], T) for i in range(K)]))
    return np.array(out).reshape(len(out), K)


# ---------------------------------------------------------------------------
# Tree verification ([RheoSampling] section 4, RheoVerification).
# ---------------------------------------------------------------------------
@dataclass
class TreeResult:
    """Outcome of verifying one row's draft tree.

    path        accepted node ids, root-to-leaf order (node 0, the root, is
                not listed).
    tokens      int64 [N]: the accepted nodes' tokens, then the final token,
                then -1.
    n           len(path).
    greedy      True for a greedy row (T <= 0).
    final_w     float64 [V]: the normalised distribution the final token was
                drawn from (None for greedy rows).
    S           mass of that distribution in units of the node's target p:
                1 for a bonus draw at a leaf, else the product of the masses
                removed by normalisation at each rejection (the mass of
                max(0, p - c q) with c the accumulated draft weight).
    gap         distance of t = u_0 * sum(final_w) to the nearer edge of the
                drawn token's CDF interval (inf for greedy rows).
    fallback    True when a residual of mass 0 fell back to the node's target.
    tested      [(node, p(d), q(d), r(d), threshold)] for every sibling
                tested, in order; threshold = r(d) / q(d) (inf when q(d) = 0).
    margins     |u_node * q(d) - r(d)| for each tested node, in order.
    accepts     the rule's outcome for each tested node, in order (a forced
                outcome does not change it).
    t           the point of the final distribution's CDF that was sampled.
    near_ids    ids of positive weight whose CDF interval meets
                [t - draw_eps, t + draw_eps].
    """

    path: list
    tokens: np.ndarray
    n: int
    greedy: bool
    final_w: np.ndarray
    S: float
    gap: float
    fallback: bool
    tested: list
    margins: list
    accepts: list = None
    t: float = float("nan")
    near_ids: tuple = ()

    def min_margin(self) -> float:
        """Smallest margin over the decisions the walk took: every tested
        sibling and the final draw.  Greedy decisions compare exact values."""
        if self.greedy:
            return float("inf")
        return min(min(self.margins, default=float("inf")), self.gap)


def tree_children(parent, N: int) -> list:
    """children[v]: nodes c in 1..N-1 with parent[c] == v, ascending (the
    order in which siblings are tested).  A parent outside [0, c) makes c
    unreachable."""
    ch = [[] for _ in range(N)]
    for c in range(1, N):
        p = int(parent[c])
        if 0 <= p < c:
            ch[p].append(c)
    return ch


def verify_tree_row(tl, dl, tok, parent, u, T: float, k: int = 0, force: dict | None = None,
                    draw_eps: float = 1e-5) -> TreeResult:
    """Verify one row's draft tree against the target ([RheoSampling]
    section 4, RheoVerification).

    tl      float64 [N, V]: target logits at each node (the next-token
            distribution after the path to that node; node 0 is the root).
    dl      float64 [N, V]: draft logits at each node (the distribution the
            node's children were drawn from); read for nodes with children.
    tok     int [N]: token of each node (entry 0 unused).
    parent  int [N]: parent of each node (< the node; entry 0 unused).
    u       float [N]: u[c] drives the test of node c; u[0] the final draw.
    T       temperature; T <= 0 selects greedy verification.
    k       sparse draft truncation at every node (0 = none).
    force   optional {node: accepted} overriding the rule's outcome for those
            nodes (tests only: following the other outcome of a decision
            within rounding distance of its threshold).
    draw_eps  half-width of the window around t that defines near_ids.

    The walk, as the page states it: at node v the distribution the next
    candidate is tested against starts as v's target p.  A candidate with
    token d is accepted with probability min(1, r(d)/q(d)), i.e. iff
    u * q(d) < r(d), and the walk descends into it.  After a rejection r is
    replaced by norm(max(0, r - q)) and the next sibling is tested against
    it.  When every child is rejected the final token is drawn from the last
    r; at a leaf it is drawn from the leaf's target (the bonus token).

    Reading (the pages leave the sibling draw open): siblings are independent
    draws from the drafter's distribution at their parent, tested in id
    order.  A residual of mass 0 (reachable only through rounding) ends the
    walk with a draw from the node's target.
    """
    tl = np.asarray(tl, dtype=np.float64)
    N, V = tl.shape
    tok = np.asarray(tok, dtype=np.int64).reshape(N)
    u = np.asarray(u, dtype=np.float64).reshape(N)
    ch = tree_children(parent, N)
    tokens = np.full(N, -1, dtype=np.int64)
    path = []
    force = force or {}
    if not (T > 0):
        # Greedy: descend into the first child (in id order) equal to the
        # node's target argmax; when none is, emit the argmax.
        v = 0
        while True:
            a = int(np.argmax(tl[v]))
            nxt = next((c for c in ch[v] if int(tok[c]) == a), None)
            if nxt is None:
                break
            path.append(nxt)
            v = nxt
        tokens[: len(path)] = [int(tok[c]) for c in path]
        tokens[len(path)] = int(np.argmax(tl[v]))
        return TreeResult(path, tokens, len(path), True, None, float("nan"), float("inf"), False, [], [], [])
    dl = np.asarray(dl, dtype=np.float64).reshape(N, V)
    tested, margins, accepts = [], [], []
    fallback = False
    v = 0
    while True:
        P = tempered_softmax(tl[v], T)
        if not ch[v]:
            w, S = P, 1.0      # leaf: bonus token from the target
            break
        keep = topk_keep_mask(dl[v], k)
        Q = tempered_softmax(np.where(keep, dl[v], -np.inf), T)
        r = P                  # the distribution the next sibling is tested against
        S = 1.0                # mass of r in units of p
        accepted = None
        for child in ch[v]:
            d = int(tok[child])
            pd, qd, rd = (P[d], Q[d], r[d]) if 0 <= d < V else (0.0, 0.0, 0.0)
            ok = u[child] * qd < rd
            tested.append((child, pd, qd, rd, rd / qd if qd > 0 else float("inf")))
            margins.append(abs(u[child] * qd - rd))
            accepts.append(bool(ok))
            if force.get(child, ok):
                accepted = child
                break
            res = np.maximum(0.0, r - Q)   # rejected: r <- norm(max(0, r - q))
            m = float(np.sum(res))
            if m == 0.0:                   # only through rounding (c4)
                fallback = True
                break
            r = res / m
            S = S * m
        if accepted is not None:
            path.append(accepted)
            v = accepted
            continue
        if fallback:
            w, S = P, 1.0
        else:
            w = r
        break
    t = u[0] * float(np.sum(w))
    x, gap, near_ids = inverse_cdf(w, t, draw_eps)
    tokens[: len(path)] = [int(tok[c]) for c in path]
    tokens[len(path)] = x
    return TreeResult(path, tokens, len(path), False, w / np.sum(w), float(S), gap, fallback, tested, margins,
                      accepts, float(t), near_ids)


def verify_tree(target_raw, draft_raw, tokens, parents, uniforms, temperature, topk: int, dtype: str,
                rows=None) -> list:
    """verify_tree_row over a batch: target_raw / draft_raw [B, N, V] stored
    logits, tokens / parents int [B, N], uniforms [B, N], temperature [B]."""
    B = target_raw.shape[0]
    out = []
    for b in (range(B) if rows is None else rows):
        T = float(temperature[b])
        tl = decode_logits(target_raw[b], dtype)
        dl = decode_logits(draft_raw[b], dtype) if T > 0 else None
        out.append(verify_tree_row(tl, dl, tokens[b], parents[b], uniforms[b], T, topk))
    return out
