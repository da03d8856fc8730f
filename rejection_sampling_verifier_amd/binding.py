"""ctypes binding of libspecverify.so: torch tensors in, device pointers out.

Argument marshalling only.  Every step of the verifier runs in the library's
HIP kernels; torch provides the device memory and the current HIP stream.
If the library has not been built the calls raise instead of computing
anything another way.

Workspaces.  A call given no ``workspace`` uses one cached per (call kind,
device, stream, shape): allocated and zero-filled on that stream the first
time and reused afterwards (the library leaves a workspace zeroed, for the
layout of the shape it ran, after every call).  Calls on one stream run in
order, so they can share it; calls on different streams get different
workspaces.  Each (kind, device, stream) keeps its most recently used
shapes only (WS_CACHE_SHAPES).  Outputs the binding allocates are allocated
on the stream the call runs on.
"""

from __future__ import annotations

import ctypes
import os
import re

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libspecverify.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "spec_verify.h")

SV_BF16, SV_F32 = 0, 1
SV_OK, SV_ERR_ARG, SV_ERR_WORKSPACE, SV_ERR_UNSUPPORTED, SV_ERR_HIP, SV_ERR_SCRATCH = 0, 1, 2, 3, 4, 5


def _header_define(name: str) -> int:
    with open(HEADER) as f:
        m = re.search(rf"#define\s+{name}\s+(\d+)", f.read())
    return int(m.group(1))


SV_MAX_TOPK = _header_define("SV_MAX_TOPK")
SV_MAX_K = _header_define("SV_MAX_K")
SV_MAX_NODES = _header_define("SV_MAX_NODES")
SV_SCRATCH_BYTES = 32 << 20  # spec_verify.h: (32u << 20)


class SpecVerifyError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"spec_verify failed: {msg} (status {status})")
        self.status = status


_lib = None
_vp, _i32, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)
_COMMON = [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _sz, _vp]


def load_library(path: str | None = None):
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(
            f"{p} is missing: build it with `python -m rejection_sampling_verifier_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(p)
    lib.spec_verify.argtypes = _COMMON
    lib.spec_verify.restype = _i32
    lib.spec_verify_noalloc.argtypes = _COMMON[:12] + [_vp]
    lib.spec_verify_noalloc.restype = _i32
    lib.spec_verify_probe.argtypes = _COMMON + [_vp, _vp]
    lib.spec_verify_probe.restype = _i32
    lib.spec_verify_relaxed.argtypes = ([_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                          ctypes.c_float, _i32, ctypes.c_float, _vp, _vp, _vp, _sz, _vp,
                                          _vp, _vp])
    lib.spec_verify_relaxed.restype = _i32
    lib.spec_verify_kl.argtypes = _COMMON + [_vp]
    lib.spec_verify_kl.restype = _i32
    lib.spec_verify_timed.argtypes = _COMMON + [ctypes.POINTER(_vp), _i32]
    lib.spec_verify_timed.restype = _i32
    lib.spec_verify_early_exit.argtypes = _COMMON + [_vp, _vp]
    lib.spec_verify_early_exit.restype = _i32
    _tree = [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _sz, _vp]
    lib.spec_verify_tree.argtypes = _tree + [_vp, _vp]
    lib.spec_verify_tree.restype = _i32
    lib.spec_verify_tree_timed.argtypes = _tree + [ctypes.POINTER(_vp), _i32]
    lib.spec_verify_tree_timed.restype = _i32
    lib.spec_verify_launches.argtypes = [_i32, _i32, _i32, _i32, _i32]
    lib.spec_verify_launches.restype = _i32
    lib.spec_verify_plan.argtypes = [_i32, _i32, _i32, _i32, _i32, ctypes.POINTER(_i32), ctypes.POINTER(_i32)]
    lib.spec_verify_plan.restype = _i32
    lib.spec_verify_status_string.argtypes = [_i32]
    lib.spec_verify_status_string.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def _check(status: int):
    if status != SV_OK:
        msg = load_library().spec_verify_status_string(status).decode()
        raise SpecVerifyError(status, msg)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SV_BF16
    if t.dtype == torch.float32:
        return SV_F32
    raise TypeError(f"logits must be bfloat16 or float32, got {t.dtype}")


def plan(B: int, K: int, V: int, topk_draft: int = 0, dtype: int = SV_BF16):
    """(chunks, chunk_len) of the vocabulary split used for this shape."""
    c, L = ctypes.c_int(0), ctypes.c_int(0)
    _check(load_library().spec_verify_plan(B, K, V, topk_draft, dtype, ctypes.byref(c), ctypes.byref(L)))
    return c.value, L.value


def launches(B: int, K: int, V: int, topk_draft: int = 0, dtype: int = SV_BF16) -> int:
    """Kernels a spec_verify call of this shape enqueues (1: the fused kernel)."""
    n = load_library().spec_verify_launches(B, K, V, topk_draft, dtype)
    if n < 0:
        _check(-n)
    return n


def workspace_bytes(B: int, K: int, V: int, topk_draft: int = 0, dtype: int = SV_BF16) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().spec_verify(None, None, None, None, None, B, K, V, topk_draft, dtype,
                                      None, None, None, ctypes.byref(n), None))
    return n.value


def new_workspace(B: int, K: int, V: int, topk_draft: int = 0, dtype: int = SV_BF16, device="cuda"):
    """A zero-filled workspace for this shape (reusable, without clearing,
    across calls of this shape on one stream)."""
    n = workspace_bytes(B, K, V, topk_draft, dtype)
    return torch.zeros(max(n, 256), dtype=torch.uint8, device=device)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


_WS_CACHE: dict = {}
_NO_WORKSPACE = torch.empty(0, dtype=torch.uint8)  # marks a call that takes no workspace
WS_CACHE_SHAPES = 4


def _stream_handle(dev, stream) -> int:
    return torch.cuda.current_stream(dev).cuda_stream if stream is None else int(stream)


class _OnStream:
    """Allocations inside belong to the stream with this handle (torch's
    caching allocator then reuses their blocks only in that stream's order)."""

    def __init__(self, dev, handle):
        self.ctx = None
        if handle != torch.cuda.current_stream(dev).cuda_stream:
            self.ctx = torch.cuda.stream(torch.cuda.ExternalStream(handle, device=dev))

    def __enter__(self):
        if self.ctx is not None:
            self.ctx.__enter__()

    def __exit__(self, *exc):
        if self.ctx is not None:
            self.ctx.__exit__(*exc)


def _empty_on(args, shape, dtype, dev):
    """torch.empty on the stream of the prepared call `args` (its last entry)."""
    with _OnStream(dev, args[-1].value or 0):
        return torch.empty(shape, dtype=dtype, device=dev)


def _cached_workspace(kind: str, shape: tuple, nbytes: int, dev, handle: int):
    """The zeroed workspace of this (kind, device, stream) for `shape`.  A
    workspace is reused only for the shape it was used with: the library
    keeps a shape's counter regions zero between calls, and another shape's
    layout puts other regions there."""
    key = (kind, dev.index if dev.index is not None else torch.cuda.current_device(), handle)
    per = _WS_CACHE.setdefault(key, {})
    ws = per.pop(shape, None)
    if ws is None:
        while len(per) >= WS_CACHE_SHAPES:
            per.pop(next(iter(per)))       # least recently used; freed in this stream's order
        with _OnStream(dev, handle):
            ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=dev)
    per[shape] = ws                         # most recently used last
    return ws


def release_workspaces():
    """Drop the cached workspaces (their memory returns to torch's allocator
    in the order of the streams they were used on)."""
    _WS_CACHE.clear()


def _prepare(target, draft, draft_tokens, uniforms, temperature, topk_draft, out_tokens,
             num_accepted, workspace, stream, ws_kind="linear"):
    if target.dim() != 3:
        raise ValueError("target_logits must be [B, K+1, V]")
    B, Kp1, V = target.shape
    K = Kp1 - 1
    dev = target.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    dt = _dtype_code(target)
    tensors = [("target_logits", target, (B, K + 1, V), target.dtype),
               ("uniforms", uniforms, (B, K + 1), torch.float32),
               ("temperature", temperature, (B,), torch.float32)]
    if K > 0:
        tensors += [("draft_logits", draft, (B, K, V), target.dtype),
                    ("draft_tokens", draft_tokens, (B, K), torch.int32)]
    for name, t, shape, dtype in tensors:
        if t is None or tuple(t.shape) != shape or t.dtype != dtype or t.device != dev or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {shape} on {dev}")
    stream = _stream_handle(dev, stream)
    with _OnStream(dev, stream):
        if out_tokens is None:
            out_tokens = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
        if num_accepted is None:
            num_accepted = torch.empty((B,), dtype=torch.int32, device=dev)
    if workspace is _NO_WORKSPACE:
        pass
    elif workspace is None:
        n = (early_exit_workspace_bytes(B, K, V, dt, topk_draft) if ws_kind == "early_exit"
             else workspace_bytes(B, K, V, topk_draft, dt))
        workspace = _cached_workspace(ws_kind, (B, K, V, topk_draft, dt), n, dev, stream)
    ws_n = ctypes.c_size_t(workspace.numel() * workspace.element_size())
    args = [_ptr(target), _ptr(draft) if K > 0 else None, _ptr(draft_tokens) if K > 0 else None,
            _ptr(uniforms), _ptr(temperature), B, K, V, topk_draft, dt, _ptr(out_tokens),
            _ptr(num_accepted), _ptr(workspace), ctypes.byref(ws_n), ctypes.c_void_p(stream)]
    keep = (target, draft, draft_tokens, uniforms, temperature, workspace)
    return args, out_tokens, num_accepted, keep


def verify(target, draft, draft_tokens, uniforms, temperature, topk_draft: int = 0, *,
           out_tokens=None, num_accepted=None, workspace=None, stream=None):
    """Enqueue spec_verify on the current (or given) stream.

    Returns (out_tokens [B, K+1] int32, num_accepted [B] int32); valid after
    the stream is synchronised.
    """
    args, out_tokens, num_accepted, _ = _prepare(target, draft, draft_tokens, uniforms, temperature,
                                                 topk_draft, out_tokens, num_accepted, workspace, stream)
    _check(load_library().spec_verify(*args))
    return out_tokens, num_accepted


def verify_noalloc(target, draft, draft_tokens, uniforms, temperature, topk_draft: int = 0, *,
                   out_tokens=None, num_accepted=None, stream=None):
    """spec_verify_noalloc: spec_verify without a workspace (the library's
    static per-GPU scratch; see the header).  Calls that overlap in time on
    one GPU race.  Returns (out_tokens, num_accepted)."""
    args, out_tokens, num_accepted, _ = _prepare(target, draft, draft_tokens, uniforms, temperature,
                                                 topk_draft, out_tokens, num_accepted, _NO_WORKSPACE, stream)
    _check(load_library().spec_verify_noalloc(*(args[:12] + [args[-1]])))
    return out_tokens, num_accepted


def verify_probe(target, draft, draft_tokens, uniforms, temperature, topk_draft: int = 0, *,
                 workspace=None, stream=None):
    """spec_verify_probe: also returns probs [B, K, 2] = (p_i(d_i), q_i(d_i))
    and mass [B] = weight of the distribution the final token was drawn from."""
    args, out_tokens, num_accepted, _ = _prepare(target, draft, draft_tokens, uniforms, temperature,
                                                 topk_draft, None, None, workspace, stream)
    B, Kp1 = out_tokens.shape
    probs = _empty_on(args, (B, Kp1 - 1, 2), torch.float32, target.device)
    mass = _empty_on(args, (B,), torch.float32, target.device)
    _check(load_library().spec_verify_probe(*args, _ptr(probs), _ptr(mass)))
    return out_tokens, num_accepted, probs, mass


def verify_relaxed(target, draft, draft_tokens, uniforms, temperature, topk_draft: int = 0, *,
                   alpha: float = 0.0, max_rank: int = 0, min_prob: float = 0.0, probes: bool = False,
                   out_tokens=None, num_accepted=None, workspace=None, stream=None):
    """spec_verify_relaxed: the lossy relaxed acceptance rule (see the header).

    Returns (out_tokens, num_accepted), plus (probs [B, K, 2], mass [B]) when
    ``probes`` is set.
    """
    args, out_tokens, num_accepted, _ = _prepare(target, draft, draft_tokens, uniforms, temperature,
                                                 topk_draft, out_tokens, num_accepted, workspace, stream)
    probs = mass = None
    if probes:
        B, Kp1 = out_tokens.shape
        probs = _empty_on(args, (B, Kp1 - 1, 2), torch.float32, target.device)
        mass = _empty_on(args, (B,), torch.float32, target.device)
    a = args[:10] + [ctypes.c_float(alpha), int(max_rank), ctypes.c_float(min_prob)] + args[10:] + \
        [_ptr(probs), _ptr(mass)]
    _check(load_library().spec_verify_relaxed(*a))
    if probes:
        return out_tokens, num_accepted, probs, mass
    return out_tokens, num_accepted


def verify_kl(target, draft, draft_tokens, uniforms, temperature, topk_draft: int = 0, *,
              out_tokens=None, num_accepted=None, kl=None, workspace=None, stream=None):
    """spec_verify_kl: verification plus KL(p_i || q_i) per draft position.

    Returns (out_tokens [B, K+1], num_accepted [B], kl [B, K] float32)."""
    args, out_tokens, num_accepted, _ = _prepare(target, draft, draft_tokens, uniforms, temperature,
                                                 topk_draft, out_tokens, num_accepted, workspace, stream)
    B, Kp1 = out_tokens.shape
    if kl is None:
        kl = _empty_on(args, (B, Kp1 - 1), torch.float32, target.device)
    _check(load_library().spec_verify_kl(*args, _ptr(kl)))
    return out_tokens, num_accepted, kl


def early_exit_workspace_bytes(B: int, K: int, V: int, dtype: int = SV_BF16, topk_draft: int = 0) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().spec_verify_early_exit(None, None, None, None, None, B, K, V, topk_draft, dtype, None,
                                                 None, None, ctypes.byref(n), None, None, None))
    return n.value


def new_early_exit_workspace(B: int, K: int, V: int, dtype: int = SV_BF16, device="cuda", topk_draft: int = 0):
    """A zero-filled workspace for spec_verify_early_exit at this shape (its
    own: not to be shared with the other calls)."""
    n = early_exit_workspace_bytes(B, K, V, dtype, topk_draft)
    return torch.zeros(max(n, 256), dtype=torch.uint8, device=device)


def verify_early_exit(target, draft, draft_tokens, uniforms, temperature, topk_draft: int = 0, *,
                      probes: bool = False, out_tokens=None, num_accepted=None, workspace=None, stream=None):
    """spec_verify_early_exit: the same results as ``verify``, reading each
    row's target logits (and a dense draft's) only up to its first rejection;
    a truncated draft is selected in full first.

    Returns (out_tokens, num_accepted), plus (probs [B, K, 2], mass [B]) when
    ``probes`` is set (probabilities past a row's first rejection are NaN).
    """
    args, out_tokens, num_accepted, _ = _prepare(target, draft, draft_tokens, uniforms, temperature,
                                                 topk_draft, out_tokens, num_accepted, workspace, stream,
                                                 ws_kind="early_exit")
    probs = mass = None
    if probes:
        B, Kp1 = out_tokens.shape
        probs = _empty_on(args, (B, Kp1 - 1, 2), torch.float32, target.device)
        mass = _empty_on(args, (B,), torch.float32, target.device)
    _check(load_library().spec_verify_early_exit(*args, _ptr(probs), _ptr(mass)))
    if probes:
        return out_tokens, num_accepted, probs, mass
    return out_tokens, num_accepted


def tree_workspace_bytes(B: int, N: int, V: int, dtype: int = SV_BF16, topk_draft: int = 0) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().spec_verify_tree(None, None, None, None, None, None, B, N, V, topk_draft, dtype,
                                           None, None, None, None, ctypes.byref(n), None, None, None))
    return n.value


def new_tree_workspace(B: int, N: int, V: int, dtype: int = SV_BF16, device="cuda", topk_draft: int = 0):
    """A zero-filled workspace for spec_verify_tree at this shape."""
    n = tree_workspace_bytes(B, N, V, dtype, topk_draft)
    return torch.zeros(max(n, 256), dtype=torch.uint8, device=device)


def _prepare_tree(target, draft, node_tokens, parents, uniforms, temperature, topk_draft,
                  out_tokens, out_nodes, num_accepted, workspace, stream):
    if target.dim() != 3:
        raise ValueError("target_logits must be [B, N, V]")
    B, N, V = target.shape
    dev = target.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    dt = _dtype_code(target)
    tensors = [("target_logits", target, (B, N, V), target.dtype),
               ("uniforms", uniforms, (B, N), torch.float32),
               ("temperature", temperature, (B,), torch.float32)]
    if N > 1:
        tensors += [("draft_logits", draft, (B, N, V), target.dtype),
                    ("node_tokens", node_tokens, (B, N), torch.int32),
                    ("parents", parents, (B, N), torch.int32)]
    for name, t, shape, dtype in tensors:
        if t is None or tuple(t.shape) != shape or t.dtype != dtype or t.device != dev or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {shape} on {dev}")
    stream = _stream_handle(dev, stream)
    with _OnStream(dev, stream):
        if out_tokens is None:
            out_tokens = torch.empty((B, N), dtype=torch.int32, device=dev)
        if out_nodes is None:
            out_nodes = torch.empty((B, N), dtype=torch.int32, device=dev)
        if num_accepted is None:
            num_accepted = torch.empty((B,), dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = _cached_workspace("tree", (B, N, V, topk_draft, dt), tree_workspace_bytes(B, N, V, dt, topk_draft),
                                      dev, stream)
    ws_n = ctypes.c_size_t(workspace.numel() * workspace.element_size())
    many = N > 1
    args = [_ptr(target), _ptr(draft) if many else None, _ptr(node_tokens) if many else None,
            _ptr(parents) if many else None, _ptr(uniforms), _ptr(temperature), B, N, V, topk_draft, dt,
            _ptr(out_tokens), _ptr(out_nodes), _ptr(num_accepted), _ptr(workspace), ctypes.byref(ws_n),
            ctypes.c_void_p(stream)]
    keep = (target, draft, node_tokens, parents, uniforms, temperature, workspace)
    return args, out_tokens, out_nodes, num_accepted, keep


def verify_tree(target, draft, node_tokens, parents, uniforms, temperature, topk_draft: int = 0, *,
                probes: bool = False, out_tokens=None, out_nodes=None, num_accepted=None, workspace=None,
                stream=None):
    """spec_verify_tree: verify one draft tree per row (see the header).

    Returns (out_tokens [B, N], out_nodes [B, N], num_accepted [B]), plus
    (probs [B, N, 3], mass [B]) when ``probes`` is set.
    """
    args, out_tokens, out_nodes, num_accepted, keep = _prepare_tree(
        target, draft, node_tokens, parents, uniforms, temperature, topk_draft, out_tokens, out_nodes,
        num_accepted, workspace, stream)
    probs = mass = None
    if probes:
        B, N = out_tokens.shape
        probs = _empty_on(args, (B, N, 3), torch.float32, target.device)
        mass = _empty_on(args, (B,), torch.float32, target.device)
    _check(load_library().spec_verify_tree(*args, _ptr(probs), _ptr(mass)))
    del keep
    if probes:
        return out_tokens, out_nodes, num_accepted, probs, mass
    return out_tokens, out_nodes, num_accepted


class _Events:
    def __init__(self, n: int):
        self.N = n
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(_vp)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), _vp, _vp]
        self.hip.hipEventDestroy.argtypes = [_vp]
        self.events = (_vp * n)()
        for i in range(n):
            ev = _vp()
            if self.hip.hipEventCreate(ctypes.byref(ev)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.events[i] = ev

    def stage_ms(self):
        out = []
        for i in range(0, self.N, 2):
            ms = ctypes.c_float(0.0)
            if self.hip.hipEventElapsedTime(ctypes.byref(ms), self.events[i], self.events[i + 1]) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            out.append(ms.value)
        return out

    def close(self):
        for i in range(self.N):
            if self.events[i]:
                self.hip.hipEventDestroy(self.events[i])
                self.events[i] = None


class TreeTimer(_Events):
    """Four HIP events taken by spec_verify_tree_timed: ``stage_ms()`` returns
    [statistics kernel, walking kernel] in ms."""

    def __init__(self):
        super().__init__(4)

    def run(self, target, draft, node_tokens, parents, uniforms, temperature, topk_draft=0, *,
            out_tokens=None, out_nodes=None, num_accepted=None, workspace=None, stream=None):
        args, out_tokens, out_nodes, num_accepted, keep = _prepare_tree(
            target, draft, node_tokens, parents, uniforms, temperature, topk_draft, out_tokens,
            out_nodes, num_accepted, workspace, stream)
        _check(load_library().spec_verify_tree_timed(*args, self.events, self.N))
        del keep
        return out_tokens, out_nodes, num_accepted


class StageTimer(_Events):
    """Six HIP events taken by spec_verify_timed: the start and end of each of
    its kernels (statistics, sparse-draft merge, finishing), from the
    dispatches' own timestamps.

    ``run(...)`` enqueues one verification; ``stage_ms()`` (after the stream is
    synchronised) returns each kernel's duration in milliseconds:
    [statistics, top-k merge (0 without a sparse draft), finishing].
    """

    def __init__(self):
        super().__init__(6)

    def run(self, target, draft, draft_tokens, uniforms, temperature, topk_draft=0, *,
            out_tokens=None, num_accepted=None, workspace=None, stream=None):
        args, out_tokens, num_accepted, _ = _prepare(target, draft, draft_tokens, uniforms, temperature,
                                                     topk_draft, out_tokens, num_accepted, workspace,
                                                     stream)
        _check(load_library().spec_verify_timed(*args, self.events, self.N))
        return out_tokens, num_accepted
