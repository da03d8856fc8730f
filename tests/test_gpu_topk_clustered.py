"""Truncated drafts whose best logits crowd into a few vocabulary chunks.

Each chunk of a draft position lists only about one and a half times its
share of the top k (at least keep = min(k, ceil(1.5k/C) + 8) logits, all
those at or above a bound).  When one chunk holds more of the top k than that, the union of the
lists misses some of them; the merge kernel detects it (the union's k-th
largest lies below that chunk's bound) and selects again with the chunk's
logits read from the draft row.  These cases build such drafts, check on the
host that the re-read is needed (a model of the chunk bound, below), and
compare the GPU with the fp64 oracle, the early-exit path with spec_verify
bit for bit, and the tree path with the oracle's tree walk.
"""

from __future__ import annotations

import numpy as np
import pytest

import workloads as W
from rejection_sampling_verifier_amd import plan, SV_BF16, SV_F32
from tests.parity import check_rows, check_tree_rows, run_gpu
from tests.test_gpu_early_exit import _assert_equal, _both
from tests.test_gpu_tree import run_tree_gpu

pytestmark = pytest.mark.gpu

WG, NT, NWAVE = 256, 8, 4


def _case(**kw):
    base = dict(B=4, K=3, V=151936, dtype=W.BF16, draft_sigma=0.8, temperature=0.9, topk=128, seed=120)
    base.update(kw)
    return W.Case(**base)


def _values(arr, dtype):
    return W.bf16_to_f32(arr) if dtype == W.BF16 else arr.astype(np.float32)


def _store(vals, dtype):
    return W.bf16_bits(vals) if dtype == W.BF16 else vals.astype(np.float32)


def _layout(k, V, C):
    kk = min(k, V)
    keep = min(kk, (3 * kk + 2 * C - 1) // (2 * C) + 8)
    stride = -(-max(NWAVE * 64, kk, 3 * keep) // 64) * 64
    return kk, keep, stride


def _chunk_bounds(row, C, CS, k, vec):
    """Host model of a chunk's bound: in each wave, the ceil(keep/4)-th
    largest of its vector maxima; the smallest over the four waves.  -inf
    when the chunk's list holds its whole top k: keep covers it, or the list
    overflows (a wave's over 256 entries, the chunk's over its area) and the
    exact path runs."""
    V = row.shape[0]
    kk, keep, stride = _layout(k, V, C)
    m = -(-keep // NWAVE)
    bounds = []
    for c in range(C):
        seg = row[c * CS:min((c + 1) * CS, V)]
        tile = np.full(WG * NT * vec, -np.inf, np.float32)
        tile[:seg.shape[0]] = seg
        t3 = tile.reshape(NT, WG, vec)
        vm = t3.max(axis=2)
        b = min(np.sort(vm[:, 64 * w:64 * w + 64].ravel())[::-1][m - 1] for w in range(NWAVE))
        per_wave = [int((t3[:, 64 * w:64 * w + 64] >= b).sum()) for w in range(NWAVE)]
        exact = max(per_wave) > 256 or sum(per_wave) > stride
        bounds.append(b if keep < min(kk, seg.shape[0]) and not exact else -np.inf)
    return np.array(bounds, np.float32)


def _needs_reread(row, C, CS, k, vec):
    """Whether the union of the chunk lists misses some of the row's top k."""
    bounds = _chunk_bounds(row, C, CS, k, vec)
    listed = np.concatenate([row[c * CS:(c + 1) * CS][row[c * CS:(c + 1) * CS] >= bounds[c]]
                             for c in range(C)])
    kth = np.sort(listed)[::-1][min(k, row.shape[0]) - 1]
    return bool((bounds > kth).any())


def _clustered(case, shape):
    """The case's draft logits reshaped by shape(dv, CS, V, rng) (in place,
    float32 values).  The first draft token of each row is its draft's
    argmax (inside the kept set)."""
    d = W.make(case)
    dt = case.dtype
    C, CS = plan(case.B, case.K, case.V, case.topk, SV_BF16 if dt == W.BF16 else SV_F32)
    dv = _values(d["draft"], dt).copy()
    shape(dv, CS, case.V, np.random.default_rng(case.seed + 1))
    d["draft"] = _store(dv, dt)
    dv = _values(d["draft"], dt)
    d["tokens"][:, 0] = np.argmax(dv[:, 0], axis=1).astype(np.int32)
    vec = 8 if dt == W.BF16 else 4
    need = sum(_needs_reread(dv[b, i], C, CS, case.topk, vec) for b in range(case.B) for i in range(case.K))
    assert need > 0, "the construction must make the merge kernel read a chunk again"
    return d, need


def _one_chunk(dv, CS, V, rng):
    dv[..., 3 * CS:4 * CS] += np.float32(20.0)


def _two_chunks_with_ragged_tail(dv, CS, V, rng):
    dv[..., 0:CS] += np.float32(20.0)
    dv[..., 9 * CS:V] += np.float32(20.0)


def _run_in_one_chunk(dv, CS, V, rng):
    # 2048 consecutive ids: 64 vectors in each wave of the chunk's tile
    dv[..., 5 * CS + 1024:5 * CS + 3072] += np.float32(20.0)


def _ties_across_chunks(dv, CS, V, rng):
    # chunk 1: 60 logits at 30 and 200 at 29; chunk 6: 100 at 29.  The top
    # 128 are the 30s and the 68 lowest-id 29s, all in chunk 1, whose list
    # stops at 30.
    for i in np.ndindex(dv.shape[:-1]):
        ids = CS + rng.choice(CS, 260, replace=False)
        dv[i + (ids[:60],)] = 30.0
        dv[i + (ids[60:],)] = 29.0
        dv[i + (6 * CS + rng.choice(CS, 100, replace=False),)] = 29.0


SHAPES = {"one-chunk": _one_chunk, "two-chunks-with-ragged-tail": _two_chunks_with_ragged_tail,
          "run-in-one-chunk": _run_in_one_chunk, "ties-across-chunks": _ties_across_chunks}


@pytest.mark.parametrize("name", sorted(SHAPES))
def test_clustered_draft_matches_oracle(name):
    case = _case()
    d, need = _clustered(case, SHAPES[name])
    print(f"[clustered] {name}: {need} of {case.B * case.K} positions need a chunk read again", flush=True)
    check_rows(d, run_gpu(d))


def test_clustered_f32_draft_matches_oracle():
    case = _case(dtype=W.F32, V=60001, topk=64, seed=121)

    def shape(dv, CS, V, rng):
        dv[..., 2 * CS:2 * CS + 3000] += np.float32(20.0)

    d, need = _clustered(case, shape)
    print(f"[clustered] f32: {need} positions need a chunk read again", flush=True)
    check_rows(d, run_gpu(d))


@pytest.mark.parametrize("name", ["one-chunk", "ties-across-chunks"])
def test_clustered_early_exit_equals_spec_verify(name):
    case = _case(B=6, seed=122)
    d, _ = _clustered(case, SHAPES[name])
    lin, ee = _both(d)
    _assert_equal(d, lin, ee)


def test_clustered_tree_drafts_match_oracle():
    case = W.TreeCase(B=4, V=151936, dtype=W.BF16, draft_sigma=1.5, temperature=1.0, parents=None, nodes=8,
                      topk=128, seed=123)
    d = W.make_tree(case)
    C, CS = plan(case.B, 1, case.V, case.topk, SV_BF16)
    dv = W.bf16_to_f32(d["draft"]).copy()
    dv[:, :, 4 * CS:5 * CS] += np.float32(20.0)
    d["draft"] = W.bf16_bits(dv)
    dv = W.bf16_to_f32(d["draft"])
    need = sum(_needs_reread(dv[b, v], C, CS, case.topk, 8) for b in range(case.B) for v in range(case.nodes))
    assert need > 0
    st = {}
    check_tree_rows(d, run_tree_gpu(d), stats=st)
    print(f"[clustered] tree: {need} nodes need a chunk read again; near draws {st['near_draw']}", flush=True)
