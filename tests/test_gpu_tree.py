"""GPU parity of draft-tree verification (spec_verify_tree) with the fp64
oracle's tree walk, on the same seeded inputs.

The method ([RheoSampling] section 4, RheoVerification): siblings are tested
in node order, an accepted node is descended into, after a rejection the next
sibling is tested against the residual norm(max(0, r - q)), and the final token
is drawn from the last residual (or, at a leaf, from the leaf's target).

Comparison rules (as for the linear verifier):
* p(d), q(d) and r(d) of every tested node, and the mass of the final draw's
  distribution: within 1e-6 absolute of the oracle;
* every sibling test the GPU took equals the oracle's outcome unless its
  margin |u q(d) - r(d)| is at most 1e-5 and at most 1e-4 of max(r, u q);
  where such a near test went the other way the oracle follows the GPU's
  outcome and the rest of the row is compared with that walk;
* the final token bit-exact when its CDF gap exceeds 1e-5, else one of the
  ids whose CDF interval lies within 1e-5 of the sampled point.
A chain tree must reproduce spec_verify bit for bit, and repeated calls must
give the same bits.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from rejection_sampling_verifier_amd import verify_probe, verify_tree
from tests.parity import check_tree_rows, to_device

pytestmark = pytest.mark.gpu

FAN_4x2 = (-1, 0, 0, 0, 0, 1, 1, 2, 2, 3, 3, 4, 4)           # root: 4 children, each with 2
WIDE_8 = (-1,) + (0,) * 8 + (1, 1, 1, 2, 2, 9, 9)              # root: 8 children


def tree_to_device(d, dev="cuda"):
    tgt = torch.from_numpy(d["target"])
    dft = torch.from_numpy(d["draft"])
    if d["dtype"] == "bf16":
        tgt = tgt.view(torch.bfloat16)
        dft = dft.view(torch.bfloat16)

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

    def f32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)

    return dict(target=tgt.to(dev), draft=dft.to(dev), tokens=i32(d["tokens"]), parents=i32(d["parents"]),
                uniforms=f32(d["uniforms"]), temperature=f32(d["temperature"]))


def run_tree_gpu(d, x=None, workspace=None):
    x = x if x is not None else tree_to_device(d)
    out, nodes, nacc, probs, mass = verify_tree(x["target"], x["draft"], x["tokens"], x["parents"], x["uniforms"],
                                                x["temperature"], d.get("topk", 0), probes=True,
                                                workspace=workspace)
    torch.cuda.synchronize()
    return tuple(t.cpu().numpy() for t in (out, nodes, nacc, probs, mass))


def _case(**kw):
    base = dict(B=8, V=40000, dtype=W.BF16, draft_sigma=1.5, temperature=1.0, seed=90)
    base.update(kw)
    return W.TreeCase(**base)


CASES = {
    "f32-V1024-fan": _case(V=1024, dtype=W.F32, target_sigma=2.0, peaks=0, draft_sigma=0.5, parents=FAN_4x2,
                           seed=91),
    "bf16-3chunks-level": _case(parents=W.level_tree((3, 4, 4, 3), seed=1), seed=92),
    "f32-ragged-random": _case(V=20001, dtype=W.F32, parents=None, nodes=12, seed=93),
    "wide-low-agreement": _case(V=9000, draft_sigma=3.0, parents=WIDE_8, seed=94),
    "mixed-greedy": _case(B=10, V=30000, parents=None, nodes=16, greedy_rows=4, seed=95),
    "61-node-tree": _case(B=4, V=17000, parents=W.TREE_60_DEPTH8, temperature=0.7, seed=96),
    "fp32-T0.3-chain-and-fan": _case(V=5000, dtype=W.F32, parents=(-1, 0, 1, 1, 2, 0, 5), temperature=0.3,
                                     seed=97),
    # sparse (top-k truncated) drafts at every node
    "top128-bf16-3chunks-level": _case(parents=W.level_tree((3, 4, 4, 3), seed=1), topk=128, seed=102),
    "top3-f32-V1024-fan": _case(V=1024, dtype=W.F32, target_sigma=2.0, peaks=0, draft_sigma=0.5,
                                parents=FAN_4x2, topk=3, seed=103),
    "top128-61-node-tree": _case(B=4, V=17000, parents=W.TREE_60_DEPTH8, temperature=0.7, topk=128, seed=104),
    "top128-wide-low-agreement": _case(V=9000, draft_sigma=3.0, parents=WIDE_8, topk=128, seed=105),
    "top300-random": _case(V=20001, parents=None, nodes=10, topk=300, seed=106),
    "top600-exact-path-random": _case(V=20001, parents=None, nodes=10, topk=600, seed=111),
    "top128-mixed-greedy": _case(B=10, V=30000, parents=None, nodes=16, greedy_rows=4, topk=128, seed=107),
    # the largest trees (SV_MAX_NODES = 64)
    "64-node-random": _case(B=4, V=5000, parents=None, nodes=64, seed=108),
    "64-node-chain-high-agreement": _case(B=3, V=3000, parents=tuple([-1] + list(range(63))), draft_sigma=0.02,
                                          seed=109),
    "top16-64-node-random": _case(B=3, V=5000, parents=None, nodes=64, topk=16, seed=110),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_tree_matches_oracle(name):
    d = W.make_tree(CASES[name])
    st = {}
    check_tree_rows(d, run_tree_gpu(d), stats=st)
    print(f"[tree] {name}: near acceptance {st['near_accept']}, near draws {st['near_draw']} of {st['rows']} "
          f"rows, worst prob error {st['worst']:.2e}", flush=True)


@pytest.mark.parametrize("name", ["wide-low-agreement", "mixed-greedy", "61-node-tree"])
def test_tree_result_is_reproducible(name):
    """The residual passes' chunks go to whichever work-group of the row asks
    first, so the assignment changes from call to call; every chunk's sums
    are computed the same way wherever they are computed, so the results
    are the same bits every time."""
    d = W.make_tree(CASES[name])
    x = tree_to_device(d)
    ref = run_tree_gpu(d, x)
    for _ in range(4):
        got = run_tree_gpu(d, x)
        for a, b in zip(ref, got):
            np.testing.assert_array_equal(a, b)


def _chain_from_linear(d):
    """The linear batch as chain trees: node i+1 holds draft d_i, its parent
    is node i; u[0] is the final-draw uniform."""
    B, K = d["tokens"].shape
    tgt = d["target"]
    dft = np.concatenate([d["draft"], tgt[:, K:K + 1]], axis=1)     # the leaf's draft is never read
    tok = np.concatenate([np.full((B, 1), -1, np.int32), d["tokens"]], axis=1)
    par = np.broadcast_to(np.arange(-1, K, dtype=np.int32), (B, K + 1)).copy()
    u = np.concatenate([d["uniforms"][:, K:], d["uniforms"][:, :K]], axis=1)
    return dict(target=tgt, draft=dft, tokens=tok, parents=par, uniforms=u, temperature=d["temperature"],
                topk=d["topk"], dtype=d["dtype"])


@pytest.mark.parametrize("cfg", [0, 1, 3, 4])
def test_chain_tree_equals_linear_verifier_bitwise(cfg):
    d = W.make(cfg)
    B, K = d["tokens"].shape
    x = to_device(d)
    l_out, l_n, l_probs, l_mass = verify_probe(x["target"], x["draft"], x["tokens"], x["uniforms"],
                                               x["temperature"], d["topk"])
    torch.cuda.synchronize()
    l_out, l_n, l_probs, l_mass = (t.cpu().numpy() for t in (l_out, l_n, l_probs, l_mass))
    del x
    t = _chain_from_linear(d)
    out, nodes, nacc, probs, mass = run_tree_gpu(t)
    np.testing.assert_array_equal(nacc, l_n)
    np.testing.assert_array_equal(out, l_out)
    for b in range(B):
        n = int(l_n[b])
        assert list(nodes[b, :n]) == list(range(1, n + 1))
        if d["temperature"][b] > 0:
            tested = min(n + 1, K)      # positions 0..n were tested
            np.testing.assert_array_equal(probs[b, 1:tested + 1, 0], l_probs[b, :tested, 0])
            np.testing.assert_array_equal(probs[b, 1:tested + 1, 1], l_probs[b, :tested, 1])
            assert mass[b] == l_mass[b], (b, mass[b], l_mass[b])


def test_single_node_tree_draws_the_bonus_token():
    d = W.make_tree(_case(B=6, V=3000, parents=(-1,), seed=98))
    st = {}
    check_tree_rows(d, run_tree_gpu(d), stats=st)
    # The same draw as the linear verifier with K = 0.
    x = tree_to_device(d)
    l_out, l_n, _, _ = verify_probe(x["target"], None, None, x["uniforms"], x["temperature"], 0)
    torch.cuda.synchronize()
    out, _, nacc, _, _ = run_tree_gpu(d, x)
    np.testing.assert_array_equal(out, l_out.cpu().numpy())
    assert (nacc == 0).all()


def test_out_of_range_tokens_are_rejected():
    d = W.make_tree(_case(B=6, V=7000, parents=FAN_4x2, draft_sigma=0.3, seed=99))
    tok = d["tokens"].copy()
    tok[:, 1] = -7                  # the first child of the root
    tok[1:3, 2] = 7000              # the second child, in two rows
    d["tokens"] = tok
    gpu = run_tree_gpu(d)
    check_tree_rows(d, gpu)
    out, nodes, nacc, probs, _ = gpu
    assert (nodes[:, 0] != 1).all()
    np.testing.assert_array_equal(probs[:, 1, :2], 0.0)


def test_workspace_is_left_clean_between_calls():
    """The walking kernel clears its published sums and counters, so one
    workspace serves consecutive calls of different inputs."""
    from rejection_sampling_verifier_amd import new_tree_workspace, SV_BF16
    a = W.make_tree(_case(B=8, V=40000, parents=WIDE_8, draft_sigma=2.5, seed=100))
    b = W.make_tree(_case(B=8, V=40000, parents=WIDE_8, draft_sigma=2.5, seed=101))
    ws = new_tree_workspace(8, len(WIDE_8), 40000, SV_BF16)
    xa, xb = tree_to_device(a), tree_to_device(b)
    ra = run_tree_gpu(a, xa, workspace=ws)
    rb = run_tree_gpu(b, xb, workspace=ws)
    ra2 = run_tree_gpu(a, xa, workspace=ws)
    for u, v in zip(ra, ra2):
        np.testing.assert_array_equal(u, v)
    for u, v in zip(rb, run_tree_gpu(b, xb)):
        np.testing.assert_array_equal(u, v)
    check_tree_rows(a, ra)
    check_tree_rows(b, rb)


@pytest.mark.parametrize("cfg", [0, 1])
def test_full_size_tree_workload_every_row(cfg):
    """The 61-node, depth-8 tree over 151,936 ids (B = 32; dense and top-128
    drafts): every row against the oracle, decision by decision."""
    d = W.make_tree(cfg)
    gpu = run_tree_gpu(d)
    st = {}
    check_tree_rows(d, gpu, stats=st)
    print(f"[tree] full size {cfg}: near acceptance {st['near_accept']}, near draws {st['near_draw']} of "
          f"{st['rows']} rows, mean accepted {gpu[2].mean():.2f}, worst prob error {st['worst']:.2e}", flush=True)
