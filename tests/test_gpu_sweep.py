"""A seeded sweep of small random shapes: the GPU against the fp64 oracle
(spec_verify and spec_verify_tree) and early exit against spec_verify bit
for bit.

Shapes mix B, K (0 to 9), V (1 to 9,000, aligned and ragged), bf16 and
fp32, dense and top-k drafts (k from 1 to 1,024, and past V), greedy and
sampling rows, cold and hot temperatures and low and high draft agreement;
each case is drawn from its own seed, so a failure names a reproducible
shape.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from rejection_sampling_verifier_amd import verify_early_exit, verify_probe
from tests.parity import check_rows, check_well_formed, to_device

pytestmark = pytest.mark.gpu

N_CASES = 150


def _draw_case(i: int) -> W.Case:
    rng = np.random.default_rng(5000 + i)
    B = int(rng.integers(1, 13))
    K = int(rng.integers(0, 10))
    V = int(rng.choice([1, 2, 7, 8, 100, 1024, 4096, 4097, 8191, 9000]))
    dtype = W.BF16 if rng.random() < 0.6 else W.F32
    topk = 0
    if rng.random() < 0.5:
        # a truncation below V is supported up to SV_MAX_TOPK = 1024
        topk = int(rng.choice([1, 3, 16, 128, 300, max(1, min(V - 1, 1024)), V, V + 5]))
    return W.Case(B=B, K=K, V=V, dtype=dtype, target_sigma=float(rng.choice([0.5, 2.0, 3.0])),
                  peaks=int(rng.integers(0, 4)) if V >= 100 else 0,
                  draft_sigma=float(rng.choice([0.05, 0.8, 3.0])),
                  temperature=float(rng.choice([0.05, 0.3, 1.0, 2.5])),
                  greedy_rows=int(rng.integers(0, B + 1)), topk=max(0, topk), seed=6000 + i, name=f"sweep-{i}")


@pytest.mark.parametrize("i", range(N_CASES))
def test_sweep_case(i):
    case = _draw_case(i)
    print(f"[sweep] {i}: B={case.B} K={case.K} V={case.V} {case.dtype} topk={case.topk} "
          f"T={case.temperature} greedy={case.greedy_rows} sigma={case.draft_sigma}", flush=True)
    d = W.make(case)
    x = to_device(d)
    lin = verify_probe(x["target"], x["draft"], x["tokens"], x["uniforms"], x["temperature"], case.topk)
    ee = verify_early_exit(x["target"], x["draft"], x["tokens"], x["uniforms"], x["temperature"], case.topk)
    torch.cuda.synchronize()
    lin = tuple(t.cpu().numpy() for t in lin)
    e_out, e_n = (t.cpu().numpy() for t in ee)
    check_rows(d, lin)
    np.testing.assert_array_equal(e_n, lin[1])
    np.testing.assert_array_equal(e_out, lin[0])
    check_well_formed(d, e_out, e_n)


N_TREE_CASES = 60


def _draw_tree_case(i: int) -> W.TreeCase:
    rng = np.random.default_rng(7000 + i)
    B = int(rng.integers(1, 9))
    V = int(rng.choice([1, 8, 100, 1024, 4097, 9000]))
    topk = int(rng.choice([0, 0, 1, 16, 128, max(1, min(V - 1, 1024)), V])) if rng.random() < 0.5 else 0
    return W.TreeCase(B=B, V=V, parents=None, nodes=int(rng.integers(1, 65)),
                      dtype=W.BF16 if rng.random() < 0.6 else W.F32,
                      target_sigma=float(rng.choice([0.5, 2.0, 3.0])),
                      peaks=int(rng.integers(0, 4)) if V >= 100 else 0,
                      draft_sigma=float(rng.choice([0.05, 0.8, 3.0])),
                      temperature=float(rng.choice([0.05, 0.3, 1.0, 2.5])),
                      greedy_rows=int(rng.integers(0, B + 1)), topk=topk, seed=8000 + i, name=f"tree-sweep-{i}")


@pytest.mark.parametrize("i", range(N_TREE_CASES))
def test_tree_sweep_case(i):
    """Random trees of 1 to 64 nodes (one per row) against the fp64 tree walk."""
    from tests.test_gpu_tree import check_tree_rows, run_tree_gpu

    case = _draw_tree_case(i)
    print(f"[tree-sweep] {i}: B={case.B} nodes={case.nodes} V={case.V} {case.dtype} topk={case.topk} "
          f"T={case.temperature} greedy={case.greedy_rows} sigma={case.draft_sigma}", flush=True)
    d = W.make_tree(case)
    check_tree_rows(d, run_tree_gpu(d))


@pytest.mark.parametrize("i", range(0, N_CASES, 3))
def test_sweep_relaxed_and_kl(i):
    """The same shapes under a random relaxed rule (against the oracle's
    relaxed walk) and, for dense drafts, the per-position KL."""
    import oracle
    from tests.parity import run_gpu
    from tests.test_gpu_kl import _check_kl
    from rejection_sampling_verifier_amd import verify_kl

    case = _draw_case(i)
    rng = np.random.default_rng(9000 + i)
    rule = oracle.Relaxed(alpha=float(rng.choice([0.0, 0.2, 0.5, 1.0])),
                          max_rank=int(rng.choice([0, 1, 3, 10])), min_prob=float(rng.choice([0.0, 0.01, 0.1])))
    print(f"[sweep-relaxed] {i}: B={case.B} K={case.K} V={case.V} {case.dtype} topk={case.topk} {rule}", flush=True)
    d = W.make(case)
    check_rows(d, run_gpu(d, relaxed=rule), relaxed=rule)
    if case.topk == 0 or case.topk >= case.V:
        x = to_device(d)
        _, _, kl = verify_kl(x["target"], x["draft"], x["tokens"], x["uniforms"], x["temperature"])
        torch.cuda.synchronize()
        _check_kl(d, kl.cpu().numpy(), list(range(case.B)))
