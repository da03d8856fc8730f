"""Helpers for GPU-vs-oracle parity tests.

Comparison rules:
* p_i(d_i), q_i(d_i) (every draft position of sampling rows) and the mass S of
  the final distribution: within 1e-6 absolute of the fp64 oracle.
* num_accepted and all output tokens: bit-exact on every row whose decisions
  are all firm.  A decision is firm when its margin |u*q - p| (acceptance) or
  CDF gap (final draw) exceeds 1e-5; an acceptance decision is also firm when
  its margin exceeds 1e-4 of max(p, u*q), since the GPU computes p and q to a
  few 1e-7 relative.  Greedy decisions compare exact values and are always
  firm.
* Rows with a non-firm decision ("near-boundary") are counted and must still
  be well formed: the accepted prefix equals the drafts, the emitted token is
  a valid id, the rest is -1.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle
from rejection_sampling_verifier_amd import verify_probe, verify_relaxed

ABS_MARGIN = 1e-5
REL_MARGIN = 1e-4
PROB_TOL = 1e-6


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


def decisions_firm(r: oracle.RowResult, u) -> bool:
    if r.greedy:
        return True
    K = r.margins.shape[0]
    for i in range(min(r.n + 1, K)):
        m = r.margins[i]
        scale = max(r.p_d[i], float(u[i]) * r.q_d[i])
        if m <= ABS_MARGIN and m <= REL_MARGIN * scale:
            return False
    return r.gap > ABS_MARGIN


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


def check_rows(d, gpu, rows=None, stats=None, relaxed: oracle.Relaxed | None = None):
    """Compare GPU results with the oracle on `rows` (under the relaxed rule
    when given); return the near-boundary count.

    If `stats` is a dict it receives 'near' and 'near_equal' (near-boundary
    rows whose tokens match the oracle anyway)."""
    out, nacc, probs, mass = gpu
    B = out.shape[0]
    rows = list(range(B)) if rows is None else list(rows)
    ref = oracle.verify(d["target"], d["draft"], d["tokens"], d["uniforms"], d["temperature"],
                        d["topk"], d["dtype"], rows=rows, relaxed=relaxed)
    near = near_equal = 0
    for b, r in zip(rows, ref):
        if not r.greedy:
            np.testing.assert_allclose(probs[b, :, 0], r.p_d, rtol=0, atol=PROB_TOL, err_msg=f"p row {b}")
            np.testing.assert_allclose(probs[b, :, 1], r.q_d, rtol=0, atol=PROB_TOL, err_msg=f"q row {b}")
            assert abs(float(mass[b]) - r.S) <= PROB_TOL, (b, float(mass[b]), r.S)
        if decisions_firm(r, d["uniforms"][b]):
            assert int(nacc[b]) == r.n, (b, int(nacc[b]), r.n, out[b], r.tokens)
            assert list(out[b]) == list(r.tokens), (b, out[b], r.tokens)
        else:
            near += 1
            near_equal += int(int(nacc[b]) == r.n and list(out[b]) == list(r.tokens))
    check_well_formed(d, out, nacc, rows)
    if stats is not None:
        stats.update(near=near, near_equal=near_equal, rows=len(rows))
    return near
