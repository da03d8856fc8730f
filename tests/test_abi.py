"""Host-side checks of the C ABI: symbols, plan, workspace query, error codes.

Nothing here launches a kernel: every call returns before the first launch.
"""

from __future__ import annotations

import ctypes
import os
import re

import pytest

from rejection_sampling_verifier_amd import binding as B

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "spec_verify.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\**\s*(spec_verify\w*)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_function():
    lib = B.load_library()
    names = declared_functions()
    assert {"spec_verify", "spec_verify_probe", "spec_verify_timed", "spec_verify_plan",
            "spec_verify_status_string"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    lib = B.load_library()
    for code in range(6):
        assert lib.spec_verify_status_string(code)
    assert lib.spec_verify_status_string(B.SV_OK) == b"ok"


@pytest.mark.parametrize("V", [1, 7, 100, 1000, 1001, 16384, 16385, 40001, 128256, 151936, 201088])
@pytest.mark.parametrize("dtype", [B.SV_BF16, B.SV_F32])
def test_plan_covers_vocabulary(V, dtype):
    C, L = B.plan(4, 3, V, 0, dtype)
    vec = 8 if dtype == B.SV_BF16 else 4
    assert L % vec == 0 and C >= 1
    assert (C - 1) * L < V <= C * L
    assert L <= 256 * 8 * vec


def test_workspace_query_grows_with_shape():
    small = B.workspace_bytes(4, 4, 1024, 0, B.SV_F32)
    big = B.workspace_bytes(256, 7, 201088, 0, B.SV_BF16)
    assert 0 < small < big
    assert small % 256 == 0 and big % 256 == 0


def _call(lib, B_=4, K=3, V=1000, topk=0, dtype=B.SV_BF16, ptrs=True, ws=None, ws_n=None):
    p = ctypes.c_void_p(0x100000) if ptrs else None
    n = None if ws_n is None else ctypes.byref(ctypes.c_size_t(ws_n))
    return lib.spec_verify(p, p, p, p, p, B_, K, V, topk, dtype, p, p, ws, n, None)


def test_argument_errors_without_launch():
    lib = B.load_library()
    need = B.workspace_bytes(4, 3, 1000, 0, B.SV_BF16)
    ws = ctypes.c_void_p(0x200000)
    assert _call(lib, B_=0, ws=ws, ws_n=need) == B.SV_ERR_ARG
    assert _call(lib, K=-1, ws=ws, ws_n=need) == B.SV_ERR_ARG
    assert _call(lib, V=0, ws=ws, ws_n=need) == B.SV_ERR_ARG
    assert _call(lib, topk=-3, ws=ws, ws_n=need) == B.SV_ERR_ARG
    assert _call(lib, dtype=7, ws=ws, ws_n=need) == B.SV_ERR_ARG
    assert _call(lib, ws=ws, ws_n=None) == B.SV_ERR_ARG                     # no size pointer
    assert _call(lib, ws=ws, ws_n=need - 1) == B.SV_ERR_WORKSPACE
    assert _call(lib, ptrs=False, ws=ws, ws_n=need) == B.SV_ERR_ARG         # NULL tensors
    assert _call(lib, ws=ctypes.c_void_p(0x200010), ws_n=need) == B.SV_ERR_ARG  # misaligned
    assert _call(lib, K=B.SV_MAX_K + 1, ws=ws, ws_n=1 << 40) == B.SV_ERR_UNSUPPORTED


def test_size_query_launches_nothing_and_accepts_null_tensors():
    lib = B.load_library()
    n = ctypes.c_size_t(0)
    rc = lib.spec_verify(None, None, None, None, None, 64, 5, 151936, 0, B.SV_BF16,
                         None, None, None, ctypes.byref(n), None)
    assert rc == B.SV_OK and n.value > 0


def test_topk_at_or_above_vocab_is_dense():
    assert B.workspace_bytes(4, 3, 500, 500, B.SV_BF16) == B.workspace_bytes(4, 3, 500, 0, B.SV_BF16)
    assert B.workspace_bytes(4, 3, 500, 10**6, B.SV_BF16) == B.workspace_bytes(4, 3, 500, 0, B.SV_BF16)


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="no fallback"):
        B.load_library(str(tmp_path / "absent.so"))


def test_relaxed_rule_argument_errors_without_launch():
    lib = B.load_library()
    p = ctypes.c_void_p(0x100000)
    need = B.workspace_bytes(4, 3, 1000, 0, B.SV_BF16)
    ws = ctypes.c_void_p(0x200000)

    def call(alpha, max_rank, min_prob):
        n = ctypes.c_size_t(need)
        return lib.spec_verify_relaxed(p, p, p, p, p, 4, 3, 1000, 0, B.SV_BF16, ctypes.c_float(alpha),
                                       max_rank, ctypes.c_float(min_prob), p, p, ws, ctypes.byref(n),
                                       None, None, None)

    assert call(-0.5, 0, 0.0) == B.SV_ERR_ARG
    assert call(float("nan"), 0, 0.0) == B.SV_ERR_ARG
    assert call(0.5, -1, 0.0) == B.SV_ERR_ARG
    assert call(0.5, 10, 1.5) == B.SV_ERR_ARG
    assert call(0.5, 10, -0.1) == B.SV_ERR_ARG
    # a valid rule still runs the usual checks first: a short workspace
    n = ctypes.c_size_t(need - 1)
    assert lib.spec_verify_relaxed(p, p, p, p, p, 4, 3, 1000, 0, B.SV_BF16, ctypes.c_float(0.5), 10,
                                   ctypes.c_float(0.1), p, p, ws, ctypes.byref(n), None, None,
                                   None) == B.SV_ERR_WORKSPACE


def test_timed_call_needs_six_events():
    lib = B.load_library()
    p = ctypes.c_void_p(0x100000)
    need = B.workspace_bytes(4, 3, 1000, 0, B.SV_BF16)
    evs = (ctypes.c_void_p * 6)()
    n = ctypes.c_size_t(need)
    assert lib.spec_verify_timed(p, p, p, p, p, 4, 3, 1000, 0, B.SV_BF16, p, p, ctypes.c_void_p(0x200000),
                                 ctypes.byref(n), None, evs, 5) == B.SV_ERR_ARG


def test_kl_argument_errors_without_launch():
    lib = B.load_library()
    p = ctypes.c_void_p(0x100000)
    need = B.workspace_bytes(4, 3, 1000, 0, B.SV_BF16)

    def call(topk, kl):
        n = ctypes.c_size_t(need)
        return lib.spec_verify_kl(p, p, p, p, p, 4, 3, 1000, topk, B.SV_BF16, p, p, ctypes.c_void_p(0x200000),
                                  ctypes.byref(n), None, kl)

    assert call(128, p) == B.SV_ERR_UNSUPPORTED      # KL against a truncated draft
    assert call(0, None) == B.SV_ERR_ARG             # no output for the KL values


def _tree_call(lib, B_=4, N=7, V=1000, topk=0, dtype=B.SV_BF16, ptrs=True, ws=None, ws_n=None,
               events=None, n_events=0):
    p = ctypes.c_void_p(0x100000) if ptrs else None
    n = None if ws_n is None else ctypes.byref(ctypes.c_size_t(ws_n))
    if events is not None:
        return lib.spec_verify_tree_timed(p, p, p, p, p, p, B_, N, V, topk, dtype, p, p, p, ws, n, None,
                                          events, n_events)
    return lib.spec_verify_tree(p, p, p, p, p, p, B_, N, V, topk, dtype, p, p, p, ws, n, None, None, None)


def test_tree_argument_errors_without_launch():
    lib = B.load_library()
    need = B.tree_workspace_bytes(4, 7, 1000, B.SV_BF16)
    assert need % 256 == 0 and need > 0
    assert B.tree_workspace_bytes(64, 61, 151936, B.SV_BF16) > need
    ws = ctypes.c_void_p(0x200000)
    assert _tree_call(lib, B_=0, ws=ws, ws_n=need) == B.SV_ERR_ARG
    assert _tree_call(lib, N=0, ws=ws, ws_n=need) == B.SV_ERR_ARG
    assert _tree_call(lib, V=0, ws=ws, ws_n=need) == B.SV_ERR_ARG
    assert _tree_call(lib, dtype=9, ws=ws, ws_n=need) == B.SV_ERR_ARG
    assert _tree_call(lib, topk=-1, ws=ws, ws_n=need) == B.SV_ERR_ARG
    assert _tree_call(lib, ws=ws, ws_n=None) == B.SV_ERR_ARG
    assert _tree_call(lib, ws=ws, ws_n=need - 1) == B.SV_ERR_WORKSPACE
    assert _tree_call(lib, ptrs=False, ws=ws, ws_n=need) == B.SV_ERR_ARG
    assert _tree_call(lib, ws=ctypes.c_void_p(0x200040), ws_n=need) == B.SV_ERR_ARG
    assert _tree_call(lib, V=5000, topk=B.SV_MAX_TOPK + 1, ws=ws, ws_n=1 << 40) == B.SV_ERR_UNSUPPORTED
    assert B.tree_workspace_bytes(4, 7, 1000, B.SV_BF16) == need                    # dense
    n = ctypes.c_size_t(0)
    assert lib.spec_verify_tree(None, None, None, None, None, None, 4, 7, 1000, 128, B.SV_BF16, None, None, None,
                                None, ctypes.byref(n), None, None, None) == B.SV_OK
    assert n.value > need                                                           # sparse: candidate areas
    assert _tree_call(lib, N=B.SV_MAX_NODES + 1, ws=ws, ws_n=1 << 40) == B.SV_ERR_UNSUPPORTED
    # the row's chunk statistics must fit the walking kernel's LDS
    assert _tree_call(lib, N=64, V=1 << 20, dtype=B.SV_F32, ws=ws, ws_n=1 << 40) == B.SV_ERR_UNSUPPORTED
    # topk at or above V is a dense draft
    assert _tree_call(lib, topk=1000, ws=None, ws_n=0) == B.SV_OK
    evs = (ctypes.c_void_p * 4)()
    assert _tree_call(lib, ws=ws, ws_n=need, events=evs, n_events=3) == B.SV_ERR_ARG


def test_tree_single_node_needs_no_tree_inputs():
    lib = B.load_library()
    need = B.tree_workspace_bytes(2, 1, 500, B.SV_F32)
    p = ctypes.c_void_p(0x100000)
    n = ctypes.c_size_t(need - 1)
    # N == 1: draft logits, tokens and parents may be NULL (only the size check fails here)
    assert lib.spec_verify_tree(p, None, None, None, p, p, 2, 1, 500, 0, B.SV_F32, p, p, p,
                                ctypes.c_void_p(0x200000), ctypes.byref(n), None, None, None) == B.SV_ERR_WORKSPACE


def test_early_exit_argument_errors_without_launch():
    lib = B.load_library()
    p = ctypes.c_void_p(0x100000)
    need = B.early_exit_workspace_bytes(4, 3, 1000, B.SV_BF16)
    assert need > 0 and need % 256 == 0

    def call(B_=4, K=3, V=1000, topk=0, dtype=B.SV_BF16, ws=0x200000, n=None, ptrs=True):
        q = p if ptrs else None
        size = ctypes.c_size_t(need if n is None else n)
        return lib.spec_verify_early_exit(q, q, q, q, q, B_, K, V, topk, dtype, q, q,
                                          ctypes.c_void_p(ws) if ws else None, ctypes.byref(size), None, None, None)

    assert call(B_=0) == B.SV_ERR_ARG
    assert call(K=-1) == B.SV_ERR_ARG
    assert call(V=0) == B.SV_ERR_ARG
    assert call(dtype=5) == B.SV_ERR_ARG
    assert call(topk=-2) == B.SV_ERR_ARG
    assert call(topk=B.SV_MAX_TOPK + 1, V=5000, n=1 << 40) == B.SV_ERR_UNSUPPORTED
    # a truncated draft needs room for its candidate lists and selections;
    # without drafts (K = 0) there is nothing to truncate
    sparse = B.early_exit_workspace_bytes(4, 3, 5000, B.SV_BF16, 10)
    assert sparse > B.early_exit_workspace_bytes(4, 3, 5000, B.SV_BF16) and sparse % 256 == 0
    assert B.early_exit_workspace_bytes(4, 0, 5000, B.SV_BF16, 10) == B.early_exit_workspace_bytes(4, 0, 5000, B.SV_BF16)
    assert call(topk=10, V=5000, n=sparse - 1) == B.SV_ERR_WORKSPACE
    assert call(topk=1000, ws=0) == B.SV_OK               # topk >= V is dense (size query only)
    assert B.early_exit_workspace_bytes(4, 3, 1000, B.SV_BF16, 1000) == need
    assert call(n=need - 1) == B.SV_ERR_WORKSPACE
    assert call(ptrs=False) == B.SV_ERR_ARG
    assert call(ws=0x200080) == B.SV_ERR_ARG              # misaligned
    assert call(K=B.SV_MAX_K + 1, n=1 << 40) == B.SV_ERR_UNSUPPORTED
    # the row's statistics must fit the kernel's LDS
    assert call(K=64, V=1 << 22, dtype=B.SV_F32, n=1 << 40) == B.SV_ERR_UNSUPPORTED


def test_noalloc_errors_before_any_launch():
    """spec_verify_noalloc rejects a shape whose workspace exceeds the static
    scratch (SV_ERR_SCRATCH) and bad arguments before touching the GPU."""
    lib = B.load_library()
    src = open(HEADER).read()
    m = re.search(r"#define\s+SV_SCRATCH_BYTES\s+\((\d+)u\s*<<\s*(\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == B.SV_SCRATCH_BYTES
    p = ctypes.c_void_p(0x100000)
    # a top-128 draft batch of 256 rows x 8 positions needs ~170 MB of candidate lists
    assert B.workspace_bytes(256, 8, 151936, 128, B.SV_BF16) > B.SV_SCRATCH_BYTES
    assert lib.spec_verify_noalloc(p, p, p, p, p, 256, 8, 151936, 128, B.SV_BF16, p, p, None) == B.SV_ERR_SCRATCH
    # the dense 201,088-id batch fits
    assert B.workspace_bytes(256, 7, 201088, 0, B.SV_BF16) <= B.SV_SCRATCH_BYTES
    assert lib.spec_verify_noalloc(None, p, p, p, p, 4, 3, 1000, 0, B.SV_BF16, p, p, None) == B.SV_ERR_ARG
    assert lib.spec_verify_noalloc(p, None, p, p, p, 4, 3, 1000, 0, B.SV_BF16, p, p, None) == B.SV_ERR_ARG
    assert lib.spec_verify_noalloc(p, p, p, p, p, 0, 3, 1000, 0, B.SV_BF16, p, p, None) == B.SV_ERR_ARG
    assert lib.spec_verify_noalloc(p, p, p, p, p, 4, 3, 1000, -1, B.SV_BF16, p, p, None) == B.SV_ERR_ARG
    assert lib.spec_verify_noalloc(p, p, p, p, p, 4, 3, 1000, 0, 9, p, p, None) == B.SV_ERR_ARG
    assert lib.spec_verify_status_string(B.SV_ERR_SCRATCH).startswith(b"shape needs more")


def test_launch_count_query():
    assert B.launches(256, 7, 201088, 0, B.SV_BF16) == 2
    assert B.launches(256, 8, 151936, 128, B.SV_BF16) == 3
    assert B.launches(4, 0, 1000, 16, B.SV_BF16) == 2          # no draft positions: no selection
    assert B.launches(4, 3, 500, 500, B.SV_BF16) == 2           # top-k >= V is dense
    lib = B.load_library()
    assert lib.spec_verify_launches(0, 3, 1000, 0, B.SV_BF16) == -B.SV_ERR_ARG
    assert lib.spec_verify_launches(4, B.SV_MAX_K + 1, 1000, 0, B.SV_BF16) == -B.SV_ERR_UNSUPPORTED
