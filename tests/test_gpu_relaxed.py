"""GPU parity of the lossy relaxed acceptance rule (spec_verify_relaxed)
against the fp64 oracle's relaxed rule, on the same seeded inputs.

The rule ([Acceptance Is Not Speed] sections 1, 6, 7): a support guard on the
target rank and probability of d_i, the strict branch q <= p, else
acceptance against gamma = min(p + sqrt(2 alpha p (1 - p)), 1).  Decisions are
compared with the same firm/near-boundary rule as the lossless tests; ranks are
exact integers on both sides.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from rejection_sampling_verifier_amd import verify, verify_relaxed
from tests.parity import check_rows, check_well_formed, run_gpu, to_device

pytestmark = pytest.mark.gpu

PAGES_RULE = oracle.Relaxed(alpha=0.5, max_rank=10, min_prob=0.1)   # the pages' support filter
RULES = {
    "pages": PAGES_RULE,
    "budget-only": oracle.Relaxed(alpha=0.2),
    "tight-rank": oracle.Relaxed(alpha=1.0, max_rank=3),
}


def _case(**kw):
    base = dict(B=8, K=4, V=40000, dtype=W.BF16, draft_sigma=1.5, temperature=0.9, seed=70)
    base.update(kw)
    return W.Case(**base)


CASES = {
    "bf16-3chunks": _case(),
    "f32-ragged": _case(dtype=W.F32, V=20001, seed=71),
    "topk128": _case(topk=128, seed=72),
    "mixed-greedy": _case(B=12, greedy_rows=5, seed=73),
    "K12": _case(K=12, V=5000, seed=74),
    "K64-top16": _case(B=4, K=64, V=5000, draft_sigma=0.3, topk=16, seed=77),
}


@pytest.mark.parametrize("rule", sorted(RULES))
@pytest.mark.parametrize("name", sorted(CASES))
def test_relaxed_matches_oracle(name, rule):
    d = W.make(CASES[name])
    st = {}
    check_rows(d, run_gpu(d, relaxed=RULES[rule]), stats=st, relaxed=RULES[rule])
    print(f"[relaxed] {name}/{rule}: near acceptance {st['near_accept']}, near draws {st['near_draw']} "
          f"of {st['rows']} rows", flush=True)


def test_relaxed_zero_budget_equals_lossless_bitwise():
    d = W.make(1)
    x = to_device(d)
    a_out, a_n = verify(x["target"], x["draft"], x["tokens"], x["uniforms"], x["temperature"], d["topk"])
    b_out, b_n = verify_relaxed(x["target"], x["draft"], x["tokens"], x["uniforms"], x["temperature"],
                                d["topk"])
    torch.cuda.synchronize()
    assert torch.equal(a_out, b_out) and torch.equal(a_n, b_n)


def test_relaxed_accepts_at_least_as_many_without_guard():
    d = W.make(_case(B=32, seed=75))
    x = to_device(d)
    _, a_n = verify(x["target"], x["draft"], x["tokens"], x["uniforms"], x["temperature"], 0)
    _, b_n = verify_relaxed(x["target"], x["draft"], x["tokens"], x["uniforms"], x["temperature"], 0,
                            alpha=0.5)
    torch.cuda.synchronize()
    a_n, b_n = a_n.cpu().numpy(), b_n.cpu().numpy()
    assert (b_n >= a_n).all() and (b_n > a_n).any()


def test_relaxed_out_of_range_tokens_rejected():
    d = W.make(_case(B=6, seed=76))
    d["tokens"] = d["tokens"].copy()
    d["tokens"][:, 1] = np.array([-1, 40000, 1 << 30, -(1 << 30), 39999, 0])[:6]
    check_rows(d, run_gpu(d, relaxed=PAGES_RULE), relaxed=PAGES_RULE)


@pytest.mark.parametrize("c", [1, 4])
def test_relaxed_full_config_every_row(c):
    d = W.make(c)
    x = to_device(d)
    gpu = run_gpu(d, x, relaxed=PAGES_RULE)
    st = {}
    check_rows(d, gpu, stats=st, relaxed=PAGES_RULE)
    print(f"[relaxed] config {c}: near acceptance {st['near_accept']}, near draws {st['near_draw']} "
          f"of {st['rows']} rows", flush=True)
