"""The calls enqueue kernels only (no allocation, no memset, no synchronization),
so a caller can capture them in a HIP graph.  Each graph is replayed several
times over inputs changed in place between the replays (eager copies, with
the stream synchronized), and every replay must equal an eager call on the
same inputs bit for bit.  Early exit's workspace must also be all zero after
every replay (its kernel clears what it used)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
import rejection_sampling_verifier_amd as rsv
from tests.parity import to_device
from tests.test_gpu_tree import tree_to_device

pytestmark = pytest.mark.gpu


def _linear_case(seed, topk=0):
    return W.Case(B=6, K=4, V=40000, dtype=W.BF16, draft_sigma=0.8, temperature=0.9, greedy_rows=1, topk=topk,
                  seed=seed)


def _tree_case(seed, topk=0):
    return W.TreeCase(B=4, V=20000, dtype=W.BF16, draft_sigma=1.0, temperature=1.0,
                      parents=W.level_tree((3, 4, 3)), topk=topk, seed=seed)


def _copy_into(static, x):
    for k, v in x.items():
        static[k].copy_(v)


KINDS = {
    # name: (call, top-k of the draft)
    "spec_verify": ("linear", 0),
    "spec_verify-top128": ("linear", 128),
    "early_exit": ("early", 0),
    "early_exit-top32": ("early", 32),
    "tree": ("tree", 0),
    "tree-top16": ("tree", 16),
}


def _setup(kind, topk, static):
    """Returns call(inputs, outputs, workspace) and factories of outputs and workspaces."""
    if kind == "tree":
        B, N, V = static["target"].shape

        def call(x, outs, ws):
            return rsv.verify_tree(x["target"], x["draft"], x["tokens"], x["parents"], x["uniforms"],
                                   x["temperature"], topk, out_tokens=outs[0], out_nodes=outs[1],
                                   num_accepted=outs[2], workspace=ws)

        def outputs():
            return (torch.empty((B, N), dtype=torch.int32, device="cuda"),
                    torch.empty((B, N), dtype=torch.int32, device="cuda"),
                    torch.empty((B,), dtype=torch.int32, device="cuda"))

        return call, outputs, lambda: rsv.new_tree_workspace(B, N, V, rsv.SV_BF16, "cuda", topk)
    B, Kp1, V = static["target"].shape
    K = Kp1 - 1
    fn = rsv.verify if kind == "linear" else rsv.verify_early_exit

    def call(x, outs, ws):
        return fn(x["target"], x["draft"], x["tokens"], x["uniforms"], x["temperature"], topk,
                  out_tokens=outs[0], num_accepted=outs[1], workspace=ws)

    def outputs():
        return (torch.empty((B, Kp1), dtype=torch.int32, device="cuda"),
                torch.empty((B,), dtype=torch.int32, device="cuda"))

    if kind == "linear":
        return call, outputs, lambda: rsv.new_workspace(B, K, V, topk, rsv.SV_BF16, "cuda")
    return call, outputs, lambda: rsv.new_early_exit_workspace(B, K, V, rsv.SV_BF16, "cuda", topk)


@pytest.mark.parametrize("name", sorted(KINDS))
def test_graph_replays_equal_eager_calls(name):
    kind, topk = KINDS[name]
    if kind == "tree":
        sets = [tree_to_device(W.make_tree(_tree_case(200 + i, topk))) for i in range(3)]
    else:
        sets = [to_device(W.make(_linear_case(210 + i, topk))) for i in range(3)]
    static = {k: v.clone() for k, v in sets[0].items()}
    call, outputs, workspace = _setup(kind, topk, static)
    g_outs, g_ws = outputs(), workspace()

    # warm-up on a side stream, then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(static, g_outs, g_ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(static, g_outs, g_ws)
    torch.cuda.synchronize()

    e_outs, e_ws = outputs(), workspace()
    for i in [1, 2, 0, 1, 1]:
        _copy_into(static, sets[i])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [t.cpu().numpy().copy() for t in g_outs]
        call(sets[i], e_outs, e_ws)
        torch.cuda.synchronize()
        want = [t.cpu().numpy() for t in e_outs]
        for a, b in zip(got, want):
            np.testing.assert_array_equal(a, b, err_msg=f"{name}: replay over input set {i}")
        if kind == "early" and topk == 0:  # all zero between calls (the others keep plain data)
            assert int(g_ws.count_nonzero().item()) == 0, "graph workspace left dirty"
