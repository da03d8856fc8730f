"""fp64 CPU oracle of the batched speculative-sampling verifier.

TEST INFRASTRUCTURE ONLY. This package is the plain, slow reference that the
GPU path is checked against. Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import it. The product path
(``rejection_sampling_verifier_amd``) never imports, calls or falls back to it,
and this package imports nothing from the product path.

Every function here is pinned by ``-m "not gpu"`` tests against facts the
pages and the mathematics fix (losslessness by exhaustive enumeration, closed
forms, brute force, a worked example).  See ``oracle/verifier.py``.
"""

from .verifier import (  # noqa: F401
    BF16,
    F32,
    Relaxed,
    RowResult,
    TreeResult,
    decode_logits,
    kl_divergence,
    kl_rows,
    relaxed_gamma,
    target_rank,
    tempered_softmax,
    topk_keep_mask,
    verify_row,
    verify,
    tree_children,
    verify_tree,
    verify_tree_row,
)
