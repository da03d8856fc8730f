"""Batched speculative-sampling verifier for AMD MI355X (gfx950).

The work happens in ``libspecverify.so`` (hand-written HIP kernels behind a C
ABI, declared in ``include/spec_verify.h``).  ``binding`` marshals torch
tensors to that ABI; it never computes anything itself and fails loudly when
the library is missing.
"""

from .binding import (  # noqa: F401
    SV_BF16,
    SV_F32,
    SV_MAX_K,
    SV_MAX_NODES,
    SV_MAX_TOPK,
    SV_SCRATCH_BYTES,
    SpecVerifyError,
    StageTimer,
    TreeTimer,
    early_exit_workspace_bytes,
    launches,
    load_library,
    new_early_exit_workspace,
    new_tree_workspace,
    new_workspace,
    plan,
    tree_workspace_bytes,
    verify,
    verify_early_exit,
    verify_kl,
    verify_noalloc,
    verify_probe,
    verify_relaxed,
    verify_tree,
    workspace_bytes,
)
