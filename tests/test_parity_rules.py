"""The GPU parity checkers themselves, exercised on the CPU.

The checkers in tests/parity.py decide what
"matches the oracle" means.  Here they are fed outputs built from the oracle
(no GPU): correct outputs must pass, outputs that take the other side of a
decision within rounding distance of its threshold must pass, and outputs
with a planted mistake -- a firm decision flipped, a wrong token after a
firm draw, a token outside the near set after a near draw, a wrong mass --
must fail.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads as W
from tests.parity import check_rows


def _outputs(d, results):
    """The four arrays the GPU returns, built from oracle results."""
    B, K = d["tokens"].shape
    out = np.stack([r.tokens for r in results]).astype(np.int32)
    nacc = np.array([r.n for r in results], dtype=np.int32)
    probs = np.zeros((B, K, 2), dtype=np.float32)
    mass = np.zeros(B, dtype=np.float32)
    for b, r in enumerate(results):
        if not r.greedy:
            probs[b, :, 0], probs[b, :, 1], mass[b] = r.p_d, r.q_d, r.S
    return out, nacc, probs, mass


def _small(seed=3, **kw):
    base = dict(B=6, K=4, V=300, dtype=W.F32, draft_sigma=0.6, temperature=0.9, greedy_rows=1, seed=seed)
    base.update(kw)
    return W.make(W.Case(**base))


def _ref(d, **kw):
    return oracle.verify(d["target"], d["draft"], d["tokens"], d["uniforms"], d["temperature"], d["topk"],
                         d["dtype"], **kw)


def test_oracle_outputs_pass():
    d = _small()
    st = {}
    check_rows(d, _outputs(d, _ref(d)), stats=st)
    assert st["rows"] == 6


def _row_with_threshold_at(d, b, i):
    """Put position i of row b exactly at its acceptance threshold from
    above (u q = p (1 + 2e-9)), positions before it accepted."""
    r = _ref(d, rows=[b])[0]
    d["uniforms"][b, :i] = 0.0
    d["uniforms"][b, i] = np.float32(r.p_d[i] / r.q_d[i] * (1 + 2e-9))
    return d


def test_other_side_of_a_near_acceptance_passes_and_a_firm_flip_fails():
    d = _small(seed=4, greedy_rows=0, draft_sigma=0.2)
    b, i = 2, 1
    d = _row_with_threshold_at(d, b, i)
    r = _ref(d, rows=[b])[0]
    assert r.margins[i] <= 1e-5 * max(r.p_d[i], 1e-30)
    ref = _ref(d)
    alt = list(ref)
    tl = oracle.decode_logits(d["target"][b], d["dtype"])
    dl = oracle.decode_logits(d["draft"][b], d["dtype"])
    alt[b] = oracle.verify_row(tl, dl, d["tokens"][b], d["uniforms"][b], float(d["temperature"][b]), 0,
                               force={i: not bool(r.accept[i])})
    assert alt[b].n != ref[b].n
    st = {}
    check_rows(d, _outputs(d, alt), stats=st)
    assert st["near_accept"] == 1
    # The same flip at a firm decision must fail.
    d2 = _small(seed=4, greedy_rows=0, draft_sigma=0.2)
    ref2 = _ref(d2)
    b2 = next(k for k, x in enumerate(ref2) if x.n < 4 and x.margins[x.n] > 1e-3)
    tl = oracle.decode_logits(d2["target"][b2], d2["dtype"])
    dl = oracle.decode_logits(d2["draft"][b2], d2["dtype"])
    bad = list(ref2)
    bad[b2] = oracle.verify_row(tl, dl, d2["tokens"][b2], d2["uniforms"][b2], float(d2["temperature"][b2]), 0,
                                force={ref2[b2].n: True})
    with pytest.raises(AssertionError, match="firm decision"):
        check_rows(d2, _outputs(d2, bad))


def test_near_draw_accepts_neighbours_only():
    # K = 0 over a flat distribution: t just above a CDF edge.
    d = _small(seed=5, K=0, greedy_rows=0, temperature=50.0)
    ref = _ref(d)
    b = 1
    w = oracle.tempered_softmax(oracle.decode_logits(d["target"][b, 0], d["dtype"]), 50.0)
    edge = float(np.cumsum(w)[99])
    d["uniforms"][b, 0] = np.float32(edge + 3e-7)
    ref = _ref(d)
    r = ref[b]
    assert r.gap <= 1e-5 and len(r.near_ids) >= 2
    out, nacc, probs, mass = _outputs(d, ref)
    for x in r.near_ids:
        out[b, 0] = x
        check_rows(d, (out, nacc, probs, mass))
    out[b, 0] = max(r.near_ids) + 2
    with pytest.raises(AssertionError):
        check_rows(d, (out, nacc, probs, mass))


def test_wrong_firm_token_or_mass_fails():
    d = _small(seed=6)
    ref = _ref(d)
    out, nacc, probs, mass = _outputs(d, ref)
    b = next(k for k, r in enumerate(ref) if not r.greedy and r.gap > 1e-4)
    n = ref[b].n
    o2 = out.copy()
    o2[b, n] = (o2[b, n] + 1) % d["target"].shape[2]
    with pytest.raises(AssertionError):
        check_rows(d, (o2, nacc, probs, mass))
    m2 = mass.copy()
    m2[b] += 3e-6
    with pytest.raises(AssertionError):
        check_rows(d, (out, nacc, probs, m2))
    p2 = probs.copy()
    p2[b, 0, 1] += 3e-6
    with pytest.raises(AssertionError):
        check_rows(d, (out, nacc, p2, mass))
    g = next(k for k, r in enumerate(ref) if r.greedy)
    o3 = out.copy()
    o3[g, ref[g].n] = (o3[g, ref[g].n] + 1) % d["target"].shape[2]
    with pytest.raises(AssertionError):
        check_rows(d, (o3, nacc, probs, mass))


# ---------------------------------------------------------------- draft trees
from tests.parity import check_tree_rows  # noqa: E402


def _tree_outputs(d, results):
    B, N = d["tokens"].shape
    out = np.stack([r.tokens for r in results]).astype(np.int32)
    nodes = np.full((B, N), -1, dtype=np.int32)
    nacc = np.array([r.n for r in results], dtype=np.int32)
    probs = np.full((B, N, 3), np.nan, dtype=np.float32)
    mass = np.zeros(B, dtype=np.float32)
    for b, r in enumerate(results):
        nodes[b, : r.n] = r.path
        if not r.greedy:
            for node, pd, qd, rd, _ in r.tested:
                probs[b, node] = (pd, qd, rd)
            mass[b] = r.S
    return out, nodes, nacc, probs, mass


def _tree(seed=7, **kw):
    base = dict(B=5, V=200, dtype=W.F32, parents=(-1, 0, 0, 0, 1, 1, 2), draft_sigma=1.5, greedy_rows=1, seed=seed)
    base.update(kw)
    return W.make_tree(W.TreeCase(**base))


def _tree_ref(d, b, force=None):
    T = float(d["temperature"][b])
    tl = oracle.decode_logits(d["target"][b], d["dtype"])
    dl = oracle.decode_logits(d["draft"][b], d["dtype"]) if T > 0 else None
    return oracle.verify_tree_row(tl, dl, d["tokens"][b], d["parents"][b], d["uniforms"][b], T, 0, force=force)


def test_tree_checker_passes_oracle_and_near_flips_and_catches_firm_flips():
    d = _tree()
    ref = [_tree_ref(d, b) for b in range(5)]
    check_tree_rows(d, _tree_outputs(d, ref))
    # Put the first tested node of a sampling row exactly at its threshold,
    # then take the other outcome: passes as a near decision.
    b = next(k for k, r in enumerate(ref) if not r.greedy and r.tested)
    node, pd, qd, rd, _ = ref[b].tested[0]
    d["uniforms"][b, node] = np.float32(rd / qd * (1 + 2e-9))
    r = _tree_ref(d, b)
    alt = [_tree_ref(d, k) for k in range(5)]
    alt[b] = _tree_ref(d, b, force={node: not r.accepts[0]})
    assert alt[b].path != r.path
    st = {}
    check_tree_rows(d, _tree_outputs(d, alt), stats=st)
    assert st["near_accept"] == 1
    # A firm flip fails.
    d2 = _tree(seed=8)
    ref2 = [_tree_ref(d2, k) for k in range(5)]
    b2 = next(k for k, r in enumerate(ref2) if not r.greedy and r.tested and r.margins[0] > 1e-3)
    node2 = ref2[b2].tested[0][0]
    bad = list(ref2)
    bad[b2] = _tree_ref(d2, b2, force={node2: not ref2[b2].accepts[0]})
    with pytest.raises(AssertionError):
        check_tree_rows(d2, _tree_outputs(d2, bad))
    # A wrong mass or a wrong r(d) fails.
    out, nodes, nacc, probs, mass = _tree_outputs(d2, ref2)
    m2 = mass.copy()
    m2[b2] += 3e-6
    with pytest.raises(AssertionError):
        check_tree_rows(d2, (out, nodes, nacc, probs, m2))
    p2 = probs.copy()
    p2[b2, node2, 2] += 3e-6
    with pytest.raises(AssertionError):
        check_tree_rows(d2, (out, nodes, nacc, p2, mass))
