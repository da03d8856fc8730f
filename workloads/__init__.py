"""Seeded synthetic inputs for the speculative-sampling verifier.

Shared by the tests, ``bench.py`` and ``smoke()``; holds none of the
verifier's arithmetic (no target/draft softmax, no acceptance test, no
residual).  What it does compute belongs to the *drafter* that produced the
inputs: draft tokens are drawn from the tempered (optionally top-k
truncated) draft distribution with the Gumbel-max trick, which is a different
sampling route from the verifier's inverse CDF.

The workload shapes stand in for the pages' models and datasets, which are
not available here: vocabularies of 151,936 / 201,088 / 128,256 ids are the
tokenizer sizes of the Qwen3, GPT-OSS and Llama-3.1 families the pages
evaluate, K = 4..8 drafts per row brackets the draft depths the pages use,
and the +8 peaks model the few dominant tokens that lossless verification
accepts most often.

Each row is generated from its own ``numpy.random.SeedSequence`` child, so
rows can be produced in parallel threads and the result does not depend on
the thread count.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

BF16 = "bf16"
F32 = "f32"


@dataclass(frozen=True)
class Case:
    """Recipe of one synthetic batch."""

    B: int
    K: int
    V: int
    dtype: str = BF16            # storage type of both logit tensors
    target_sigma: float = 3.0    # std of the N(0, sigma) base target logits
    peaks: int = 20              # distinct ids per target slot raised by peak_height
    peak_height: float = 8.0
    draft_sigma: float = 1.0     # draft = target + N(0, draft_sigma)
    temperature: float = 1.0     # T of the sampling rows
    greedy_rows: int = 0         # rows with T = 0, placed by a seeded permutation
    topk: int = 0                # sparse draft truncation (0 = dense)
    seed: int = 0
    name: str = ""


# The five workloads (seed 1000 + index).  Index 0 is the small float32 case
# the oracle finishes in milliseconds; 1 is the 151,936-id bf16 batch the
# throughput is quoted on; 2 is a low-agreement 201,088-id batch; 3 mixes
# greedy (T=0) and sampling rows; 4 truncates the draft to its top 128.
CONFIGS = [
    Case(B=4, K=4, V=1024, dtype=F32, target_sigma=2.0, peaks=0, draft_sigma=0.5,
         temperature=1.0, seed=1000, name="B4-K4-V1024-f32"),
    Case(B=64, K=5, V=151936, dtype=BF16, draft_sigma=1.0, temperature=0.6,
         seed=1001, name="B64-K5-V151936-bf16-T0.6"),
    Case(B=256, K=7, V=201088, dtype=BF16, draft_sigma=1.5, temperature=1.0,
         seed=1002, name="B256-K7-V201088-bf16-T1.0"),
    Case(B=512, K=4, V=128256, dtype=BF16, draft_sigma=0.7, temperature=0.8,
         greedy_rows=256, seed=1003, name="B512-K4-V128256-bf16-mixedT0/0.8"),
    Case(B=256, K=8, V=151936, dtype=BF16, draft_sigma=0.8, temperature=0.8,
         topk=128, seed=1004, name="B256-K8-V151936-bf16-T0.8-top128"),
]


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest even); return the bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _top_ids(row: np.ndarray, k: int) -> np.ndarray:
    """Ids of the k largest values of a float32 row; among equal values at the
    boundary the lowest ids are taken (drafter-side truncation)."""
    V = row.shape[0]
    if k <= 0 or k >= V:
        return np.arange(V)
    kth = np.partition(row, V - k)[V - k]          # k-th largest value
    above = np.flatnonzero(row > kth)
    ties = np.flatnonzero(row == kth)[: k - above.size]
    return np.concatenate([above, ties])


def _make_row(case: Case, seq: np.random.SeedSequence, T: float):
    rng = np.random.default_rng(seq)
    K, V = case.K, case.V
    tgt = rng.standard_normal((K + 1, V), dtype=np.float32)
    tgt *= np.float32(case.target_sigma)
    for i in range(K + 1):
        if case.peaks:
            ids = rng.choice(V, size=case.peaks, replace=False)
            tgt[i, ids] += np.float32(case.peak_height)
    if case.dtype == BF16:
        tgt_store = bf16_bits(tgt)
        tgt_val = bf16_to_f32(tgt_store)
    else:
        tgt_store = tgt
        tgt_val = tgt
    noise = rng.standard_normal((K, V), dtype=np.float32)
    noise *= np.float32(case.draft_sigma)
    dft = tgt_val[:K] + noise
    if case.dtype == BF16:
        dft_store = bf16_bits(dft)
        dft_val = bf16_to_f32(dft_store)
    else:
        dft_store = dft
        dft_val = dft
    toks = np.empty(K, dtype=np.int32)
    # Gumbel-max: argmax(l/T + G) with G = -log(E), E ~ Exp(1), draws an id
    # with probability softmax(l/T) restricted to the candidate set.
    expo = rng.standard_exponential((K, V), dtype=np.float32)
    for i in range(K):
        if T > 0:
            ids = _top_ids(dft_val[i], case.topk)
            with np.errstate(divide="ignore"):
                score = dft_val[i, ids] / np.float32(T) - np.log(expo[i, ids])
            toks[i] = ids[int(np.argmax(score))]
        else:
            toks[i] = int(np.argmax(dft_val[i]))
    uni = rng.random(K + 1, dtype=np.float32)
    return tgt_store, dft_store, toks, uni


def make(case: Case | int, threads: int | None = None) -> dict:
    """Generate one batch.  Returns a dict of host arrays:

    target  [B, K+1, V] uint16 (bf16 bits) or float32
    draft   [B, K, V]   same storage type
    tokens  [B, K] int32, uniforms [B, K+1] float32 in [0, 1),
    temperature [B] float32, plus 'topk', 'dtype', 'case'.
    """
    if isinstance(case, int):
        case = CONFIGS[case]
    B, K, V = case.B, case.K, case.V
    root = np.random.SeedSequence(case.seed)
    seqs = root.spawn(B + 1)
    T = np.full(B, case.temperature, dtype=np.float32)
    if case.greedy_rows:
        perm = np.random.default_rng(seqs[B]).permutation(B)
        T[perm[: case.greedy_rows]] = 0.0
    st = np.uint16 if case.dtype == BF16 else np.float32
    target = np.empty((B, K + 1, V), dtype=st)
    draft = np.empty((B, K, V), dtype=st)
    tokens = np.empty((B, K), dtype=np.int32)
    uniforms = np.empty((B, K + 1), dtype=np.float32)

    def work(b):
        t, d, tk, u = _make_row(case, seqs[b], float(T[b]))
        target[b] = t
        draft[b] = d
        tokens[b] = tk
        uniforms[b] = u

    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    if threads <= 1 or B == 1:
        for b in range(B):
            work(b)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(work, range(B)))
    return dict(target=target, draft=draft, tokens=tokens, uniforms=uniforms,
                temperature=T, topk=case.topk, dtype=case.dtype, case=case)


# ---------------------------------------------------------------- draft trees


def level_tree(widths, seed: int = 0) -> tuple:
    """Parents of a tree with widths[l] nodes at depth l + 1, in breadth-first
    order (node 0 is the root, every parent precedes its children).  Each node
    of a level picks its parent among the previous level's nodes with
    probability proportional to 1 / (rank + 1): like a dynamic draft tree,
    the best-ranked nodes are expanded most."""
    rng = np.random.default_rng(seed)
    parents = [-1]
    prev = [0]
    for w in widths:
        wts = 1.0 / np.arange(1, len(prev) + 1)
        pick = rng.choice(len(prev), size=w, p=wts / wts.sum())
        level = []
        for j in sorted(pick.tolist()):
            parents.append(prev[j])
            level.append(len(parents) - 1)
        prev = level
    return tuple(parents)


def random_tree(N: int, rng: np.random.Generator) -> np.ndarray:
    """A uniformly drawn recursive tree: node c's parent is uniform on [0, c)."""
    par = np.full(N, -1, dtype=np.int32)
    for c in range(1, N):
        par[c] = rng.integers(0, c)
    return par


# A 60-node draft tree of depth 8 (plus the root), the tree size and depth
# of the pages' dynamic-tree experiments.
TREE_60_DEPTH8 = level_tree((4, 8, 12, 12, 10, 7, 4, 3), seed=7)


@dataclass(frozen=True)
class TreeCase:
    """Recipe of one synthetic batch of draft trees.  Logits follow Case's
    recipe at every node (the target at a node is the distribution after the
    path to it; the draft there is target + noise); node c's token is drawn
    from the tempered draft at its parent, independently of its siblings
    (greedy rows: the parent's draft ids in decreasing logit order)."""

    B: int
    V: int
    parents: tuple | None = TREE_60_DEPTH8   # shared topology; None: a random tree per row
    nodes: int = 0                           # node count of the random trees
    dtype: str = BF16
    target_sigma: float = 3.0
    peaks: int = 20
    peak_height: float = 8.0
    draft_sigma: float = 1.0
    temperature: float = 1.0
    greedy_rows: int = 0
    topk: int = 0                            # sparse draft truncation at every node (0 = dense)
    seed: int = 0
    name: str = ""

    @property
    def N(self) -> int:
        return len(self.parents) if self.parents is not None else self.nodes


# The tree workloads: B = 32 rows of the 61-node tree over the 151,936-id
# vocabulary, bf16, T = 1.0 (the pages' temperature for the tree experiments),
# with dense drafts and with drafts truncated to their top 128.
TREE_CONFIGS = [
    TreeCase(B=32, V=151936, draft_sigma=1.0, temperature=1.0, seed=2001,
             name="B32-N61-depth8-V151936-bf16-T1.0"),
    # The same trees with every node's draft cut to its top 128 logits.
    TreeCase(B=32, V=151936, draft_sigma=1.0, temperature=1.0, topk=128, seed=2002,
             name="B32-N61-depth8-V151936-bf16-T1.0-top128"),
]


def _make_tree_row(case: TreeCase, seq: np.random.SeedSequence, T: float):
    rng = np.random.default_rng(seq)
    N, V = case.N, case.V
    par = np.asarray(case.parents, dtype=np.int32) if case.parents is not None else random_tree(N, rng)
    has_kids = np.zeros(N, dtype=bool)
    has_kids[par[1:]] = True
    tgt = rng.standard_normal((N, V), dtype=np.float32)
    tgt *= np.float32(case.target_sigma)
    for i in range(N):
        if case.peaks:
            ids = rng.choice(V, size=case.peaks, replace=False)
            tgt[i, ids] += np.float32(case.peak_height)
    if case.dtype == BF16:
        tgt_store = bf16_bits(tgt)
        tgt_val = bf16_to_f32(tgt_store)
    else:
        tgt_store = tgt
        tgt_val = tgt
    # Drafts at leaves are never read: they hold the target.
    dft_store = tgt_store.copy()
    dft_val = tgt_val.copy()
    for i in np.flatnonzero(has_kids):
        noise = rng.standard_normal(V, dtype=np.float32)
        noise *= np.float32(case.draft_sigma)
        d = tgt_val[i] + noise
        if case.dtype == BF16:
            dft_store[i] = bf16_bits(d)
            dft_val[i] = bf16_to_f32(dft_store[i])
        else:
            dft_store[i] = d
            dft_val[i] = d
    toks = np.full(N, -1, dtype=np.int32)
    for v in np.flatnonzero(has_kids):
        kids = np.flatnonzero(par == v)
        kids = kids[kids > v]
        if T > 0:
            # Gumbel-max over the (truncated) draft, one independent draw per child
            ids = _top_ids(dft_val[v], case.topk)
            for c in kids:
                with np.errstate(divide="ignore"):
                    score = dft_val[v, ids] / np.float32(T) - np.log(rng.standard_exponential(ids.size,
                                                                                          dtype=np.float32))
                toks[c] = int(ids[int(np.argmax(score))])
        else:
            order = np.argsort(-dft_val[v], kind="stable")
            toks[kids] = order[: kids.size]
    uni = rng.random(N, dtype=np.float32)
    return tgt_store, dft_store, toks, par, uni


def make_tree(case: TreeCase | int, threads: int | None = None) -> dict:
    """Generate one batch of draft trees.  Returns host arrays:

    target, draft [B, N, V] uint16 (bf16 bits) or float32
    tokens, parents [B, N] int32 (entry 0: -1), uniforms [B, N] float32 in
    [0, 1), temperature [B] float32, plus 'dtype' and 'case'.
    """
    if isinstance(case, int):
        case = TREE_CONFIGS[case]
    B, N, V = case.B, case.N, case.V
    seqs = np.random.SeedSequence(case.seed).spawn(B + 1)
    T = np.full(B, case.temperature, dtype=np.float32)
    if case.greedy_rows:
        perm = np.random.default_rng(seqs[B]).permutation(B)
        T[perm[: case.greedy_rows]] = 0.0
    st = np.uint16 if case.dtype == BF16 else np.float32
    target = np.empty((B, N, V), dtype=st)
    draft = np.empty((B, N, V), dtype=st)
    tokens = np.empty((B, N), dtype=np.int32)
    parents = np.empty((B, N), dtype=np.int32)
    uniforms = np.empty((B, N), dtype=np.float32)

    def work(b):
        t, d, tk, par, u = _make_tree_row(case, seqs[b], float(T[b]))
        target[b] = t
        draft[b] = d
        tokens[b] = tk
        parents[b] = par
        uniforms[b] = u

    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    if threads <= 1 or B == 1:
        for b in range(B):
            work(b)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(work, range(B)))
    return dict(target=target, draft=draft, tokens=tokens, parents=parents, uniforms=uniforms,
                temperature=T, topk=case.topk, dtype=case.dtype, case=case)


__all__ = ["BF16", "F32", "Case", "CONFIGS", "make", "bf16_bits", "bf16_to_f32", "replace",
           "TreeCase", "TREE_CONFIGS", "TREE_60_DEPTH8", "level_tree", "random_tree", "make_tree"]
