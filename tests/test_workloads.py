"""Host-side checks of the seeded synthetic input generator."""

import numpy as np

import workloads as W


def test_bf16_rounding_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1e-40], dtype=np.float32)
    b = W.bf16_bits(x)
    assert list(b[:4]) == [0x3F80, 0x3F80, 0x3F82, 0xC020]
    assert W.bf16_to_f32(b)[0] == 1.0


def test_deterministic_and_thread_count_independent():
    case = W.replace(W.CONFIGS[1], B=3, V=4096)
    a = W.make(case, threads=1)
    b = W.make(case, threads=3)
    for key in ("target", "draft", "tokens", "uniforms", "temperature"):
        assert np.array_equal(a[key], b[key])
    assert a["target"].dtype == np.uint16 and a["target"].shape == (3, 6, 4096)
    assert a["uniforms"].min() >= 0.0 and a["uniforms"].max() < 1.0


def test_mixed_temperature_rows_and_greedy_drafts():
    case = W.replace(W.CONFIGS[3], B=16, V=2048, greedy_rows=8)
    d = W.make(case)
    T = d["temperature"]
    assert (T == 0).sum() == 8 and (T == np.float32(0.8)).sum() == 8
    dv = W.bf16_to_f32(d["draft"])
    for b in np.flatnonzero(T == 0):
        for i in range(case.K):
            assert d["tokens"][b, i] == int(np.argmax(dv[b, i]))


def test_topk_drafts_lie_in_the_kept_set():
    case = W.replace(W.CONFIGS[4], B=3, V=5000)
    d = W.make(case)
    dv = W.bf16_to_f32(d["draft"])
    for b in range(3):
        for i in range(case.K):
            row = dv[b, i]
            tok = d["tokens"][b, i]
            better = np.sum((row > row[tok]) | ((row == row[tok]) & (np.arange(row.size) < tok)))
            assert better < 128


def test_tree_topology_of_the_tree_workload():
    par = np.asarray(W.TREE_60_DEPTH8)
    assert par.shape == (61,) and par[0] == -1
    assert all(0 <= par[c] < c for c in range(1, 61))
    depth = np.zeros(61, dtype=int)
    for c in range(1, 61):
        depth[c] = depth[par[c]] + 1
    assert depth.max() == 8


def test_tree_batches_are_seeded_and_well_formed():
    case = W.TreeCase(B=5, V=3000, parents=None, nodes=14, greedy_rows=2, seed=12)
    a = W.make_tree(case, threads=1)
    b = W.make_tree(case, threads=4)
    for key in ("target", "draft", "tokens", "parents", "uniforms", "temperature"):
        assert np.array_equal(a[key], b[key])
    assert a["target"].shape == (5, 14, 3000) and a["draft"].shape == (5, 14, 3000)
    dv = W.bf16_to_f32(a["draft"])
    for r in range(5):
        par, tok = a["parents"][r], a["tokens"][r]
        assert par[0] == -1 and tok[0] == -1
        assert all(0 <= par[c] < c for c in range(1, 14))
        assert ((tok[1:] >= 0) & (tok[1:] < 3000)).all()
        if a["temperature"][r] == 0:
            # greedy rows: children take the parent's draft ids in decreasing logit order
            for v in set(par[1:].tolist()):
                kids = [c for c in range(1, 14) if par[c] == v]
                order = np.argsort(-dv[r, v], kind="stable")
                assert list(tok[kids]) == list(order[: len(kids)])
        leaves = set(range(14)) - set(par[1:].tolist())
        for v in leaves:                       # drafts at leaves hold the target (never read)
            assert np.array_equal(a["draft"][r, v], a["target"][r, v])
