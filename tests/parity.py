"""Helpers for GPU-vs-oracle parity tests.

Comparison rules, decision by decision:
* p_i(d_i), q_i(d_i) (every draft position of sampling rows) and the mass S of
  the final distribution: within 1e-6 absolute of the fp64 oracle.
* Each acceptance decision the GPU took (positions 0..num_accepted, the last
  one only if it is a rejection) must equal the oracle's outcome at that
  position, unless the decision is near its threshold: margin |u*q - p| at
  most 1e-5 and at most 1e-4 of max(p, u*q) (the GPU computes p and q to a
  few 1e-7 relative).  Where a near decision went the other way, the oracle
  is run again with that outcome forced, and the rest of the row is compared
  with that path.  So num_accepted and the accepted prefix are always
  compared, never skipped.
* The final token: bit-exact when the oracle's CDF gap exceeds 1e-5;
  otherwise it must be one of the ids whose CDF interval lies within 1e-5 of
  the sampled point (the oracle's near_ids), i.e. the oracle's token or a
  neighbour of positive weight.
* Greedy decisions compare exact values: always bit-exact.
* Tokens after the emitted one are -1.
"""

from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np
import torch

import oracle
from rejection_sampling_verifier_amd import verify_probe, verify_relaxed

ABS_MARGIN = 1e-5
REL_MARGIN = 1e-4
PROB_TOL = 1e-6
ORACLE_THREADS = min(16, os.cpu_count() or 1)


def to_device(d, dev="cuda"):
    tgt = torch.from_numpy(d["target"])
    dft = torch.from_numpy(d["draft"])
    if d["dtype"] == "bf16":
        tgt = tgt.view(torch.bfloat16)
        dft = dft.view(torch.bfloat16)
    return dict(
        target=tgt.to(dev), draft=dft.to(dev),
        tokens=torch.from_numpy(np.ascontiguousarray(d["tokens"], dtype=np.int32)).to(dev),
        uniforms=torch.from_numpy(np.ascontiguousarray(d["uniforms"], dtype=np.float32)).to(dev),
        temperature=torch.from_numpy(np.ascontiguousarray(d["temperature"], dtype=np.float32)).to(dev),
    )


def run_gpu(d, dev_inputs=None, relaxed: oracle.Relaxed | None = None):
    x = dev_inputs if dev_inputs is not None else to_device(d)
    if relaxed is None:
        out, nacc, probs, mass = verify_probe(x["target"], x["draft"], x["tokens"], x["uniforms"],
                                              x["temperature"], d["topk"])
    else:
        out, nacc, probs, mass = verify_relaxed(x["target"], x["draft"], x["tokens"], x["uniforms"],
                                                x["temperature"], d["topk"], alpha=relaxed.alpha,
                                                max_rank=relaxed.max_rank, min_prob=relaxed.min_prob,
                                                probes=True)
    torch.cuda.synchronize()
    return out.cpu().numpy(), nacc.cpu().numpy(), probs.cpu().numpy(), mass.cpu().numpy()


def near_decision(margin: float, scale: float) -> bool:
    """A decision within rounding distance of its threshold (see the module
    docstring)."""
    return margin <= ABS_MARGIN and margin <= REL_MARGIN * scale


def oracle_rows(d, rows, relaxed=None):
    """oracle.verify on `rows`, spread over threads (rows are independent)."""
    def one(b):
        return oracle.verify(d["target"], d["draft"], d["tokens"], d["uniforms"], d["temperature"],
                             d["topk"], d["dtype"], rows=[b], relaxed=relaxed)[0]

    if len(rows) <= 4:
        return [one(b) for b in rows]
    with ThreadPoolExecutor(ORACLE_THREADS) as ex:
        return list(ex.map(one, rows))


def check_well_formed(d, out, nacc, rows=None):
    K = d["tokens"].shape[1]
    V = d["target"].shape[2]
    rows = range(out.shape[0]) if rows is None else rows
    for b in rows:
        n = int(nacc[b])
        assert 0 <= n <= K, (b, n)
        assert list(out[b, :n]) == list(d["tokens"][b, :n]), (b, out[b], d["tokens"][b])
        assert 0 <= out[b, n] < V, (b, out[b])
        assert all(out[b, n + 1:] == -1), (b, out[b])


def check_row(d, b, r: oracle.RowResult, out, nacc, probs, mass, relaxed=None, counts=None,
              reached_only=False):
    """Compare GPU row b with the oracle's result r, decision by decision.
    With reached_only the GPU reports p and q only for the positions it
    tested (NaN after its first rejection)."""
    K = d["tokens"].shape[1]
    u = d["uniforms"][b]
    n = int(nacc[b])
    assert 0 <= n <= K, (b, n)
    if r.greedy:
        assert n == r.n and list(out[b]) == list(r.tokens), (b, out[b], r.tokens)
        return
    upto = min(n + 1, K) if reached_only else K
    np.testing.assert_allclose(probs[b, :upto, 0], r.p_d[:upto], rtol=0, atol=PROB_TOL, err_msg=f"p row {b}")
    np.testing.assert_allclose(probs[b, :upto, 1], r.q_d[:upto], rtol=0, atol=PROB_TOL, err_msg=f"q row {b}")
    if reached_only:
        assert np.isnan(probs[b, upto:]).all(), (b, probs[b])
    # The acceptance decisions the GPU took: positions 0..n-1 accepted, n rejected.
    force = {}
    for i in range(min(n + 1, K)):
        gpu_accepted = i < n
        if gpu_accepted != bool(r.accept[i]):
            scale = max(r.p_d[i], float(u[i]) * r.q_d[i])
            assert near_decision(r.margins[i], scale), (
                f"row {b}: firm decision at position {i} differs (gpu accepted={gpu_accepted}, "
                f"margin {r.margins[i]:.3e}, p {r.p_d[i]:.6e}, q {r.q_d[i]:.6e}, u {u[i]:.6e})")
            force[i] = gpu_accepted
    if force:
        dl = oracle.decode_logits(d["draft"][b], d["dtype"]) if K > 0 else None
        r = oracle.verify_row(oracle.decode_logits(d["target"][b], d["dtype"]), dl, d["tokens"][b], u,
                              float(d["temperature"][b]), d["topk"], relaxed, force=force)
        if counts is not None:
            counts["near_accept"] = counts.get("near_accept", 0) + 1
    assert r.n == n, (b, n, r.n)
    assert list(out[b, :n]) == list(d["tokens"][b, :n]), (b, out[b], d["tokens"][b])
    assert all(out[b, n + 1:] == -1), (b, out[b])
    assert abs(float(mass[b]) - r.S) <= PROB_TOL, (b, float(mass[b]), r.S)
    x = int(out[b, n])
    if r.gap > ABS_MARGIN:
        assert x == int(r.tokens[n]), (b, out[b], r.tokens, r.gap)
    else:
        assert x in r.near_ids, (b, x, r.tokens[n], r.near_ids, r.gap)
        if counts is not None:
            counts["near_draw"] = counts.get("near_draw", 0) + 1
            counts["near_draw_equal"] = counts.get("near_draw_equal", 0) + int(x == int(r.tokens[n]))


def check_rows(d, gpu, rows=None, stats=None, relaxed: oracle.Relaxed | None = None, reached_only=False):
    """Compare GPU results with the oracle on `rows` (all rows by default;
    under the relaxed rule when given; reached_only as for check_row).
    Returns the number of rows with a
    near decision (acceptance or draw), all of them still checked as above.

    If `stats` is a dict it receives 'rows', 'near_accept' (rows that took the
    other side of a near acceptance decision), 'near_draw' (rows whose final
    draw was near a CDF edge) and 'near_draw_equal' (of those, how many drew
    the oracle's own token)."""
    out, nacc, probs, mass = gpu
    B = out.shape[0]
    rows = list(range(B)) if rows is None else list(rows)
    ref = oracle_rows(d, rows, relaxed)
    counts = {}
    near_rows = 0
    for b, r in zip(rows, ref):
        before = counts.get("near_accept", 0) + counts.get("near_draw", 0)
        check_row(d, b, r, out, nacc, probs, mass, relaxed, counts, reached_only)
        near_rows += int(counts.get("near_accept", 0) + counts.get("near_draw", 0) > before)
    if stats is not None:
        stats.update(rows=len(rows), near_accept=counts.get("near_accept", 0),
                     near_draw=counts.get("near_draw", 0), near_draw_equal=counts.get("near_draw_equal", 0),
                     near=near_rows, near_equal=counts.get("near_draw_equal", 0))
    return near_rows


# ---------------------------------------------------------------- draft trees
def check_tree_well_formed(d, gpu, rows):
    out, nodes, nacc = gpu[:3]
    V = d["target"].shape[2]
    for b in rows:
        n = int(nacc[b])
        par, tok = d["parents"][b], d["tokens"][b]
        N = par.shape[0]
        assert 0 <= n < N, (b, n)
        v = 0
        for i in range(n):
            c = int(nodes[b, i])
            assert 0 < c < N and int(par[c]) == v, (b, nodes[b])
            assert int(out[b, i]) == int(tok[c]), (b, out[b], nodes[b])
            v = c
        assert 0 <= int(out[b, n]) < V, (b, out[b])
        assert (out[b, n + 1:] == -1).all() and (nodes[b, n:] == -1).all(), (b, out[b], nodes[b])


def _oracle_tree_row(d, b, force=None):
    T = float(d["temperature"][b])
    tl = oracle.decode_logits(d["target"][b], d["dtype"])
    dl = oracle.decode_logits(d["draft"][b], d["dtype"]) if T > 0 else None
    return oracle.verify_tree_row(tl, dl, d["tokens"][b], d["parents"][b], d["uniforms"][b], T, d.get("topk", 0),
                                  force=force)


def check_tree_row(d, b, gpu, counts):
    """Row b decision by decision: every tested sibling's outcome equals the
    oracle's unless it is near its threshold (then the oracle follows the
    GPU's outcome, forced); p(d), q(d), r(d) of every tested node and the
    final mass within 1e-6; the final token exact when its CDF gap exceeds
    1e-5, else one of the oracle's near_ids."""
    out, nodes, nacc, probs, mass = gpu
    N = out.shape[1]
    u = d["uniforms"][b]
    n = int(nacc[b])
    gpu_path = [int(c) for c in nodes[b, :n]]
    force = {}
    r = _oracle_tree_row(d, b)
    if r.greedy:
        assert n == r.n and gpu_path == r.path and list(out[b]) == list(r.tokens), (b, out[b], r.tokens)
        assert float(mass[b]) == 0.0
        return 0.0
    for _ in range(N):
        if r.path == gpu_path:
            break
        # The first tested node whose outcome differs: the walks agree before it.
        for (node, pd, qd, rd, _), m, acc in zip(r.tested, r.margins, r.accepts):
            gpu_acc = node in gpu_path
            if gpu_acc != (node in r.path):
                assert near_decision(m, max(rd, float(u[node]) * qd)), (
                    f"row {b}: firm decision at node {node} differs (gpu accepted={gpu_acc}, margin {m:.3e})")
                force[node] = gpu_acc
                break
        else:
            raise AssertionError(f"row {b}: gpu path {gpu_path} is not a walk of the tree ({r.path})")
        r = _oracle_tree_row(d, b, force)
        counts["near_accept"] = counts.get("near_accept", 0) + 1
    assert r.path == gpu_path, (b, gpu_path, r.path)
    worst = 0.0
    tested = {node: (pd, qd, rd) for node, pd, qd, rd, _ in r.tested}
    for c in range(N):
        if c in tested:
            err = np.abs(probs[b, c].astype(np.float64) - np.array(tested[c]))
            worst = max(worst, float(err.max()))
            assert (err <= PROB_TOL).all(), (b, c, probs[b, c], tested[c])
        else:
            assert np.isnan(probs[b, c]).all(), (b, c, probs[b, c])
    assert abs(float(mass[b]) - r.S) <= PROB_TOL, (b, float(mass[b]), r.S)
    assert list(out[b, :n]) == list(r.tokens[:n]) and (out[b, n + 1:] == -1).all(), (b, out[b], r.tokens)
    x = int(out[b, n])
    if r.gap > ABS_MARGIN:
        assert x == int(r.tokens[n]), (b, out[b], r.tokens, r.gap)
    else:
        assert x in r.near_ids, (b, x, r.tokens[n], r.near_ids)
        counts["near_draw"] = counts.get("near_draw", 0) + 1
        counts["near_draw_equal"] = counts.get("near_draw_equal", 0) + int(x == int(r.tokens[n]))
    return worst


def check_tree_rows(d, gpu, rows=None, stats=None):
    """Compare GPU results with the oracle on `rows` (all by default), decision
    by decision; return the number of rows with a near decision."""
    B = gpu[0].shape[0]
    rows = list(range(B)) if rows is None else list(rows)
    check_tree_well_formed(d, gpu, rows)
    counts = {}
    worst = 0.0
    near_rows = 0
    for b in rows:
        before = counts.get("near_accept", 0) + counts.get("near_draw", 0)
        worst = max(worst, check_tree_row(d, b, gpu, counts))
        near_rows += int(counts.get("near_accept", 0) + counts.get("near_draw", 0) > before)
    if stats is not None:
        stats.update(rows=len(rows), worst=worst, near=near_rows, near_accept=counts.get("near_accept", 0),
                     near_draw=counts.get("near_draw", 0), near_draw_equal=counts.get("near_draw_equal", 0))
    return near_rows
