"""GPU tests of early-exit verification (spec_verify_early_exit).

The call verifies a row's positions one after the other and stops reading
its logits at the first rejection ("Speculative decoding: memverifikasi token
draft sebelum diterima", subsection "Penolakan memendekkan pekerjaan
speculative yang berguna").  Every sum is formed as in spec_verify, so its
tokens, counts, tested probabilities and final mass must equal spec_verify's
bit for bit; spec_verify itself is held to the oracle in test_gpu_parity.py.
The oracle is also checked directly on a few cases.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from rejection_sampling_verifier_amd import (new_early_exit_workspace, verify_early_exit,
                                             verify_probe, SV_BF16, SV_F32)
from tests.parity import check_rows, check_well_formed, to_device

pytestmark = pytest.mark.gpu


def _case(**kw):
    base = dict(B=6, K=3, V=40000, dtype=W.BF16, draft_sigma=0.8, temperature=0.9, seed=7)
    base.update(kw)
    return W.Case(**base)


CASES = {
    "bf16-3chunks": _case(),
    "bf16-ragged-unaligned": _case(V=40001, seed=8),
    "f32-3chunks-ragged": _case(dtype=W.F32, V=20001, seed=10),
    "tiny-V": _case(V=100, peaks=3, seed=12),
    "V1": _case(V=1, peaks=0, seed=13),
    "K0": _case(K=0, seed=15),
    "B1-K1": _case(B=1, K=1, seed=16),
    "K12": _case(K=12, V=5000, seed=17),
    "mixed-greedy": _case(B=12, greedy_rows=6, seed=18),
    "all-greedy": _case(B=5, greedy_rows=5, seed=19),
    "hot-T": _case(B=32, temperature=4.0, seed=20),
    "cold-T": _case(temperature=0.05, seed=21),
    "low-agreement": _case(B=16, draft_sigma=3.0, seed=22),
    "high-agreement": _case(B=16, K=8, draft_sigma=0.05, seed=33),
    "K64-high-agreement": _case(B=4, K=64, V=3000, draft_sigma=0.02, seed=76),
    "V1M-ragged-unaligned": _case(B=2, K=2, V=(1 << 20) + 3, seed=78),
}


def _both(d, x=None, ws=None):
    x = x if x is not None else to_device(d)
    k = int(d["topk"])
    a = verify_probe(x["target"], x["draft"], x["tokens"], x["uniforms"], x["temperature"], k)
    e = verify_early_exit(x["target"], x["draft"], x["tokens"], x["uniforms"], x["temperature"], k, probes=True,
                          workspace=ws)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in a], [t.cpu().numpy() for t in e]


def _assert_equal(d, lin, ee):
    l_out, l_n, l_probs, l_mass = lin
    e_out, e_n, e_probs, e_mass = ee
    np.testing.assert_array_equal(e_n, l_n)
    np.testing.assert_array_equal(e_out, l_out)
    K = d["tokens"].shape[1]
    for b in range(e_out.shape[0]):
        if d["temperature"][b] > 0:
            n = int(l_n[b])
            tested = min(n + 1, K)
            np.testing.assert_array_equal(e_probs[b, :tested], l_probs[b, :tested])
            assert np.isnan(e_probs[b, tested:]).all(), (b, e_probs[b])
            assert e_mass[b] == l_mass[b], (b, e_mass[b], l_mass[b])
        else:
            assert np.isnan(e_probs[b]).all()
            assert e_mass[b] == 0.0


@pytest.mark.parametrize("name", sorted(CASES))
def test_equals_spec_verify_bitwise(name):
    d = W.make(CASES[name])
    lin, ee = _both(d)
    _assert_equal(d, lin, ee)
    check_well_formed(d, ee[0], ee[1])


@pytest.mark.parametrize("cfg", [0, 1, 2, 3])
def test_equals_spec_verify_on_the_workloads(cfg):
    d = W.make(cfg)
    lin, ee = _both(d)
    _assert_equal(d, lin, ee)
    print(f"[early-exit] config {cfg}: mean accepted {ee[1].mean():.3f} of {d['tokens'].shape[1]}", flush=True)


def test_matches_oracle_directly():
    d = W.make(_case(B=10, K=5, V=30000, draft_sigma=1.2, greedy_rows=3, seed=34))
    _, ee = _both(d)
    check_rows(d, tuple(ee), reached_only=True)


def test_workspace_is_left_clean_between_calls():
    a = W.make(_case(B=8, K=4, draft_sigma=2.0, seed=35))
    b = W.make(_case(B=8, K=4, draft_sigma=0.3, seed=36))
    ws = new_early_exit_workspace(8, 4, 40000, SV_BF16)
    xa, xb = to_device(a), to_device(b)
    la, ea = _both(a, xa, ws)
    lb, eb = _both(b, xb, ws)
    la2, ea2 = _both(a, xa, ws)
    _assert_equal(a, la, ea)
    _assert_equal(b, lb, eb)
    _assert_equal(a, la2, ea2)
    # the workspace must be all zero again
    torch.cuda.synchronize()
    assert int(ws.count_nonzero().item()) == 0


def test_out_of_range_draft_tokens_are_rejected():
    d = W.make(_case(B=6, K=3, seed=37))
    tok = d["tokens"].copy()
    tok[0, 0] = -1
    tok[1, 1] = 40000
    tok[2, 2] = 2 ** 31 - 1
    d["tokens"] = tok
    lin, ee = _both(d)
    _assert_equal(d, lin, ee)
    assert ee[1][0] == 0 and ee[1][1] <= 1 and ee[1][2] <= 2


SPARSE = {
    "top128": _case(B=8, topk=128, seed=50),
    "top1": _case(topk=1, seed=51),
    "top3-ragged": _case(V=40001, topk=3, seed=52),
    "top300-wide-fast-path": _case(topk=300, seed=53),
    "top600-exact-path": _case(B=4, topk=600, seed=81),
    "top1024-exact-path": _case(B=3, topk=1024, seed=54),
    "f32-top64": _case(dtype=W.F32, V=20001, topk=64, seed=55),
    "mixed-greedy-top128": _case(B=10, greedy_rows=4, topk=128, seed=56),
    "small-V-top128": _case(V=200, peaks=3, topk=128, seed=57),
    "K0-top16": _case(K=0, topk=16, seed=58),
    "high-agreement-top32": _case(B=16, K=8, draft_sigma=0.05, topk=32, seed=59),
    "K64-top16-high-agreement": _case(B=3, K=64, V=5000, draft_sigma=0.02, topk=16, seed=77),
    "topk-ge-V-is-dense": _case(V=3000, topk=3000, seed=79),
    "top1023-of-1024": _case(B=4, K=3, V=1024, topk=1023, seed=80),
}


@pytest.mark.parametrize("name", sorted(SPARSE))
def test_sparse_draft_equals_spec_verify_bitwise(name):
    """A truncated draft: each reached position's selection is made inside
    the call, from the same candidate lists and in the same order as
    spec_verify's, so the results are the same bits."""
    d = W.make(SPARSE[name])
    lin, ee = _both(d)
    _assert_equal(d, lin, ee)
    check_well_formed(d, ee[0], ee[1])


def test_sparse_draft_on_the_top128_workload():
    d = W.make(4)
    lin, ee = _both(d)
    _assert_equal(d, lin, ee)
    print(f"[early-exit] config 4: mean accepted {ee[1].mean():.3f} of {d['tokens'].shape[1]}", flush=True)


def test_sparse_draft_matches_oracle_directly():
    d = W.make(_case(B=8, K=4, V=30000, draft_sigma=1.2, greedy_rows=2, topk=64, seed=60))
    _, ee = _both(d)
    check_rows(d, tuple(ee), reached_only=True)


def test_sparse_workspace_is_reused_within_a_shape():
    """Calls of one shape reuse the workspace without clearing it: each row's
    last work-group clears the published words (also where a chunk's fast
    selection overflowed into the exact path), and the candidate lists and
    selections are rewritten by every call.  Another shape starts from a
    zero-filled workspace, as the header asks."""
    groups = [[_case(B=8, K=4, draft_sigma=2.0, topk=600, seed=61),
               _case(B=8, K=4, draft_sigma=0.3, topk=600, seed=62)],
              [_case(B=5, K=2, V=30000, topk=8, seed=63),
               _case(B=5, K=2, V=30000, draft_sigma=0.2, topk=8, seed=64)]]
    ws = new_early_exit_workspace(8, 4, 40000, SV_BF16, topk_draft=600)
    for group in groups:
        ws.zero_()
        for case in group + group[:1]:
            d = W.make(case)
            x = to_device(d)
            a = verify_probe(x["target"], x["draft"], x["tokens"], x["uniforms"], x["temperature"], case.topk)
            e = verify_early_exit(x["target"], x["draft"], x["tokens"], x["uniforms"], x["temperature"],
                                  case.topk, probes=True, workspace=ws)
            torch.cuda.synchronize()
            _assert_equal(d, [t.cpu().numpy() for t in a], [t.cpu().numpy() for t in e])


def test_f32_workspace_query_and_reuse_across_shapes():
    ws = new_early_exit_workspace(8, 6, 20001, SV_F32)
    for K, V, seed in [(6, 20001, 39), (2, 5000, 40), (6, 20001, 41)]:
        d = W.make(_case(B=8, K=K, V=V, dtype=W.F32, seed=seed))
        lin, ee = _both(d, ws=ws)
        _assert_equal(d, lin, ee)
