"""spec_verify_noalloc (static per-GPU scratch, no workspace) against
spec_verify with a workspace of its own, through the C ABI: tokens and
counts equal bit for bit, over consecutive calls whose shapes change (the
second smaller, then larger ones whose layouts put counters where the
previous call's partials were)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
import rejection_sampling_verifier_amd as rsv
from tests.parity import check_rows, to_device

pytestmark = pytest.mark.gpu


def _case(**kw):
    base = dict(B=6, K=3, V=40000, dtype=W.BF16, draft_sigma=0.8, temperature=0.9, seed=7)
    base.update(kw)
    return W.Case(**base)


def _compare(d, tag):
    x = to_device(d)
    ws = rsv.new_workspace(d["target"].shape[0], d["tokens"].shape[1], d["target"].shape[2], d["topk"],
                           rsv.SV_BF16 if d["dtype"] == "bf16" else rsv.SV_F32, "cuda")
    r_out, r_n = rsv.verify(x["target"], x["draft"], x["tokens"], x["uniforms"], x["temperature"], d["topk"],
                            workspace=ws)
    out = torch.full_like(r_out, 12345)
    nacc = torch.full_like(r_n, 777)
    rsv.verify_noalloc(x["target"], x["draft"], x["tokens"], x["uniforms"], x["temperature"], d["topk"],
                       out_tokens=out, num_accepted=nacc)
    torch.cuda.synchronize()
    assert torch.equal(out, r_out) and torch.equal(nacc, r_n), tag
    print(f"[no-alloc] {tag}: equal to spec_verify, mean accepted {nacc.float().mean().item():.3f}", flush=True)
    return out.cpu().numpy(), nacc.cpu().numpy()


def test_two_calls_second_smaller_equal_spec_verify():
    _compare(W.make(2), "config 2 (B256 K7 V201088)")
    _compare(W.make(_case(B=16, K=3, V=40000, seed=80)), "then B16 K3 V40000")


def test_shape_changes_and_sparse_drafts():
    for i, case in enumerate([_case(B=9, K=2, V=30000, seed=81),
                              _case(B=300, K=4, V=20000, greedy_rows=120, seed=82),
                              _case(B=8, K=3, V=40000, topk=128, seed=83),
                              _case(B=4, K=4, V=1024, dtype=W.F32, seed=84),
                              _case(B=300, K=4, V=20000, greedy_rows=120, seed=82)]):
        _compare(W.make(case), f"shape {i}: B{case.B} K{case.K} V{case.V} top{case.topk}")


def test_matches_the_oracle():
    d = W.make(_case(B=12, K=4, V=30001, greedy_rows=3, seed=85))
    x = to_device(d)
    out, nacc = rsv.verify_noalloc(x["target"], x["draft"], x["tokens"], x["uniforms"], x["temperature"], 0)
    torch.cuda.synchronize()
    ws = rsv.new_workspace(12, 4, 30001, 0, rsv.SV_BF16, "cuda")
    _, _, probs, mass = rsv.verify_probe(x["target"], x["draft"], x["tokens"], x["uniforms"], x["temperature"], 0,
                                         workspace=ws)
    torch.cuda.synchronize()
    check_rows(d, (out.cpu().numpy(), nacc.cpu().numpy(), probs.cpu().numpy(), mass.cpu().numpy()))


def test_oversized_shape_is_refused():
    t = torch.zeros((256, 9, 151936), dtype=torch.bfloat16, device="cuda")
    dft = torch.zeros((256, 8, 151936), dtype=torch.bfloat16, device="cuda")
    tok = torch.zeros((256, 8), dtype=torch.int32, device="cuda")
    u = torch.zeros((256, 9), dtype=torch.float32, device="cuda")
    T = torch.ones(256, dtype=torch.float32, device="cuda")
    with pytest.raises(rsv.SpecVerifyError) as e:
        rsv.verify_noalloc(t, dft, tok, u, T, 128)
    assert e.value.status == rsv.binding.SV_ERR_SCRATCH
