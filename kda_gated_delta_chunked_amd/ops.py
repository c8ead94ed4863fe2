"""Thin Python binding over libkda's C ABI (include/kda.h).

Argument marshalling only: tensors are checked for dtype, shape, contiguity
and device, their device pointers and the current HIP stream are handed to
``kda_prefill``, and every step of the computation runs in the library's HIP
kernels.  There is no fallback: if the library cannot be loaded, calls raise.
PyTorch provides device memory and streams.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

from . import build as _build

KDA_OK = 0
STATUS_NAMES = {0: "KDA_OK", -1: "KDA_ERR_INVALID_ARG", -2: "KDA_ERR_UNSUPPORTED",
                -3: "KDA_ERR_ALIGNMENT", -4: "KDA_ERR_OVERLAP",
                -5: "KDA_ERR_WORKSPACE_TOO_SMALL", -6: "KDA_ERR_TOO_LARGE", -7: "KDA_ERR_HIP",
                -8: "KDA_ERR_SCRATCH_TOO_SMALL"}
# bytes of the static device scratch kda_prefill_noalloc uses (KDA_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 128 << 20
VARIANTS = {"auto": 0, "decomp": 1, "fused": 2}
HEAD_DIM = 128

_lib = None


class KDAError(RuntimeError):
    """A libkda call returned a non-OK status."""

    def __init__(self, status: int, what: str = ""):
        self.status = status
        name = STATUS_NAMES.get(status, str(status))
        msg = _lib.kda_status_string(status).decode() if _lib is not None else name
        super().__init__(f"{what}: {name} ({msg})" if what else f"{name} ({msg})")


class Problem(ctypes.Structure):
    """Mirror of ``kda_problem``."""

    _fields_ = [("num_seqs", ctypes.c_int32), ("total_tokens", ctypes.c_int64),
                ("num_heads", ctypes.c_int32), ("head_dim_k", ctypes.c_int32),
                ("head_dim_v", ctypes.c_int32), ("scale", ctypes.c_float),
                ("gate_lower_bound", ctypes.c_float), ("variant", ctypes.c_int32),
                ("value_split", ctypes.c_int32), ("stages", ctypes.c_int32),
                ("ckpt_per_seq", ctypes.c_int32), ("state_dtype", ctypes.c_int32),
                ("prologue", ctypes.c_int32), ("cu_seqlens_int64", ctypes.c_int32),
                ("seq_order", ctypes.c_void_p), ("chain_parts", ctypes.c_int32)]


STAGES = {"both": 0, "prepare": 1, "recurrence": 2}
STATE_DTYPES = {"fp32": 0, "bf16": 1}


class DecodeProblem(ctypes.Structure):
    """Mirror of ``kda_decode_problem``."""

    _fields_ = [("num_seqs", ctypes.c_int32), ("tokens_per_seq", ctypes.c_int32),
                ("num_heads", ctypes.c_int32), ("head_dim_k", ctypes.c_int32),
                ("head_dim_v", ctypes.c_int32), ("scale", ctypes.c_float),
                ("gate_lower_bound", ctypes.c_float), ("pool_size", ctypes.c_int64),
                ("prologue", ctypes.c_int32), ("state_dtype", ctypes.c_int32)]


def make_decode_problem(num_seqs: int, tokens_per_seq: int, num_heads: int, pool_size: int, *,
                        scale: float, gate_lower_bound: float = -5.0,
                        head_dim_k: int = HEAD_DIM, head_dim_v: int = HEAD_DIM,
                        qk_l2norm: bool = False, beta_logit: bool = False,
                        state_dtype: str = "fp32") -> DecodeProblem:
    return DecodeProblem(int(num_seqs), int(tokens_per_seq), int(num_heads), int(head_dim_k),
                         int(head_dim_v), float(scale), float(gate_lower_bound), int(pool_size),
                         (1 if qk_l2norm else 0) | (2 if beta_logit else 0), STATE_DTYPES[state_dtype])


def make_problem(num_seqs: int, total_tokens: int, num_heads: int, *, scale: float,
                 gate_lower_bound: float = -5.0, variant: str | int = "auto",
                 value_split: int = 0, head_dim_k: int = HEAD_DIM,
                 head_dim_v: int = HEAD_DIM, stages: str | int = "both",
                 ckpt_per_seq: int = 0, state_dtype: str = "fp32", qk_l2norm: bool = False,
                 beta_logit: bool = False, cu_seqlens_int64: bool = False,
                 seq_order: int = 0, chain_parts: int = 0) -> Problem:
    """Mirror of kda_problem; seq_order is a raw device pointer (0 = none)."""
    v = VARIANTS[variant] if isinstance(variant, str) else int(variant)
    st = STAGES[stages] if isinstance(stages, str) else int(stages)
    return Problem(int(num_seqs), int(total_tokens), int(num_heads), int(head_dim_k),
                   int(head_dim_v), float(scale), float(gate_lower_bound), v, int(value_split), st,
                   int(ckpt_per_seq), STATE_DTYPES[state_dtype],
                   (1 if qk_l2norm else 0) | (2 if beta_logit else 0),
                   1 if cu_seqlens_int64 else 0, int(seq_order) or None, int(chain_parts))


def periodic_offsets(seq_lens, every: int):
    """Checkpoint offsets [N, C] (int32 numpy) for a checkpoint every `every`
    tokens of each sequence (every, 2 every, ... <= L_n), padded with -1 (an
    offset that exports nothing) up to the longest list; C >= 1."""
    import numpy as np
    if every < 1:
        raise ValueError("every must be >= 1")
    lens = [int(x) for x in seq_lens]
    C = max([1] + [L // every for L in lens])
    offs = np.full((len(lens), C), -1, np.int32)
    for n, L in enumerate(lens):
        m = L // every
        offs[n, :m] = np.arange(1, m + 1, dtype=np.int64) * every
    return offs


def library_path() -> str:
    """The libkda.so to load: $KDA_LIBRARY when set (another build of the same
    sources, such as one with host sanitizers), else the in-tree build."""
    return os.environ.get("KDA_LIBRARY") or _build.LIB_PATH


def load_library(path: Optional[str] = None):
    """Load libkda.so (building it first if it is absent)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or library_path()
    if not os.path.exists(p):
        if p != _build.LIB_PATH:
            raise OSError(f"libkda not found at {p}")
        _build.build()
    lib = ctypes.CDLL(p)
    P = ctypes.c_void_p
    PP = ctypes.POINTER(Problem)
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_prefill_workspace_size.argtypes = [PP, ctypes.POINTER(ctypes.c_size_t)]
    lib.kda_prefill_workspace_size.restype = ctypes.c_int
    lib.kda_validate.argtypes = [PP, P, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t]
    lib.kda_validate.restype = ctypes.c_int
    lib.kda_prefill.argtypes = [PP, P, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.kda_prefill.restype = ctypes.c_int
    lib.kda_prefill_noalloc.argtypes = [PP, P, P, P, P, P, P, P, P, P, P, P, P]
    lib.kda_prefill_noalloc.restype = ctypes.c_int
    lib.kda_plan.argtypes = [PP, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32),
                             ctypes.POINTER(ctypes.c_int32)]
    lib.kda_plan.restype = ctypes.c_int
    DP = ctypes.POINTER(DecodeProblem)
    lib.kda_decode_validate.argtypes = [DP, P, P, P, P, P, P, P, P]
    lib.kda_decode_validate.restype = ctypes.c_int
    lib.kda_decode.argtypes = [DP, P, P, P, P, P, P, P, P, P]
    lib.kda_decode.restype = ctypes.c_int
    lib.kda_decode_verify.argtypes = [DP, P, P, P, P, P, P, P, P, P, P]
    lib.kda_decode_verify.restype = ctypes.c_int
    lib.kda_decode_commit.argtypes = [DP, P, P, P, P, P]
    lib.kda_decode_commit.restype = ctypes.c_int
    lib.kda_decode_advance.argtypes = [DP, P, P, P, P, P, P, P, P, P]
    lib.kda_decode_advance.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def _check(status: int, what: str):
    if status != KDA_OK:
        raise KDAError(status, what)


def workspace_size(problem: Problem) -> int:
    lib = load_library()
    n = ctypes.c_size_t(0)
    _check(lib.kda_prefill_workspace_size(ctypes.byref(problem), ctypes.byref(n)),
           "kda_prefill_workspace_size")
    return int(n.value)


def plan(problem: Problem) -> Tuple[str, int, int]:
    """(schedule, workgroups per pair, chain pieces) kda_prefill would use on
    the current device."""
    lib = load_library()
    var, vs, parts = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int32(0)
    _check(lib.kda_plan(ctypes.byref(problem), ctypes.byref(var), ctypes.byref(vs),
                        ctypes.byref(parts)), "kda_plan")
    name = {v: k for k, v in VARIANTS.items()}.get(var.value, str(var.value))
    return name, int(vs.value), int(parts.value)


def prefill_raw(problem: Problem, q, k, v, g, beta, cu_seqlens, initial_state, out, final_state,
                ckpt_offsets, ckpt_state, workspace, workspace_bytes: int, stream) -> int:
    """Call ``kda_prefill`` with raw integer pointers (0 for NULL); returns the status."""
    lib = load_library()
    return lib.kda_prefill(ctypes.byref(problem), q or None, k or None, v or None, g or None,
                           beta or None, cu_seqlens or None, initial_state or None, out or None,
                           final_state or None, ckpt_offsets or None, ckpt_state or None,
                           workspace or None, int(workspace_bytes), stream or None)


def prefill_noalloc_raw(problem: Problem, q, k, v, g, beta, cu_seqlens, initial_state, out,
                        final_state, ckpt_offsets, ckpt_state, stream) -> int:
    """Call ``kda_prefill_noalloc`` (the workspace is the library's static
    device scratch) with raw integer pointers (0 for NULL); returns the status."""
    lib = load_library()
    return lib.kda_prefill_noalloc(ctypes.byref(problem), q or None, k or None, v or None,
                                   g or None, beta or None, cu_seqlens or None,
                                   initial_state or None, out or None, final_state or None,
                                   ckpt_offsets or None, ckpt_state or None, stream or None)


def validate_raw(problem: Problem, q, k, v, g, beta, cu_seqlens, initial_state, out, final_state,
                 ckpt_offsets, ckpt_state, workspace, workspace_bytes: int) -> int:
    """Call ``kda_validate`` with raw integer pointers; returns the status (host only)."""
    lib = load_library()
    return lib.kda_validate(ctypes.byref(problem), q or None, k or None, v or None, g or None,
                            beta or None, cu_seqlens or None, initial_state or None, out or None,
                            final_state or None, ckpt_offsets or None, ckpt_state or None,
                            workspace or None, int(workspace_bytes))


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def prefill(q, k, v, g, beta, *, cu_seqlens=None, initial_state=None, scale: Optional[float] = None,
            out=None, final_state=None, output_final_state: bool = True, ckpt_offsets=None,
            ckpt_state=None, gate_lower_bound: float = -5.0, variant: str = "auto",
            value_split: int = 0, workspace=None, stream=None, state_dtype=None,
            qk_l2norm: bool = False, beta_logit: bool = False, seq_order=None,
            chain_parts: int = 0):
    """KDA multi-token recurrent prefill on the GPU.

    q, k, v: bf16 [T, H, 128] (packed, with cu_seqlens int32 [N+1]) or
    [B, T, H, 128] (fixed layout).  g: fp32 like q (log-decay, >= the gate
    lower bound, <= 0).  beta: fp32 [T, H] or [B, T, H].  initial_state:
    fp32 [N, H, 128, 128] or None; bf16 states (initial, final and
    checkpoint alike, or state_dtype=torch.bfloat16) are widened on load and
    rounded on store.  Returns (out, final_state); out has q's
    shape, final_state is None when output_final_state is False.  Pass
    ``final_state=initial_state`` for an in-place update and ``out=v`` to
    overwrite v.  ckpt_offsets int32 [N] / ckpt_state fp32 [N, H, 128, 128]
    export the state after ckpt_offsets[n] tokens of sequence n; with
    ckpt_offsets [N, C] and ckpt_state [N, C, H, 128, 128], C states per
    sequence (``periodic_offsets`` builds a checkpoint every n tokens).
    workspace: a device buffer of at least ``workspace_size`` bytes; when None
    and the schedule may use one, a buffer is taken from torch's allocator.
    cu_seqlens may be int32 or int64.  seq_order: optional int32 [N], the
    order in which the recurrence takes packed sequences (a permutation; see
    kda_problem.seq_order).  chain_parts: pieces each (sequence, head)'s
    recurrence is split into (0 = the library's choice, 1 = none; see
    kda_problem.chain_parts).
    """
    import torch

    fixed = q.dim() == 4
    if fixed:
        B, T, H, D = q.shape
        N, T_total = B, B * T
        if cu_seqlens is not None:
            raise ValueError("cu_seqlens is for packed [T, H, 128] inputs")
    elif q.dim() == 3:
        T_total, H, D = q.shape
        if cu_seqlens is None:
            N = 1
        else:
            N = int(cu_seqlens.numel()) - 1
    else:
        raise ValueError("q must be [T, H, 128] or [B, T, H, 128]")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("libkda runs on the GPU: tensors must be on a cuda (HIP) device")
    for name, t, dt in (("q", q, torch.bfloat16), ("k", k, torch.bfloat16), ("v", v, torch.bfloat16),
                        ("g", g, torch.float32), ("beta", beta, torch.float32)):
        if t.dtype != dt:
            raise TypeError(f"{name} must be {dt}, got {t.dtype}")
        if t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if k.shape != q.shape or v.shape != q.shape or g.shape != q.shape:
        raise ValueError("q, k, v and g must have the same shape")
    if beta.shape != q.shape[:-1]:
        raise ValueError("beta must be q.shape[:-1]")
    # states: fp32, or bf16 (all of them alike); taken from the given state
    # tensors unless state_dtype names it
    if state_dtype is None:
        given = [t for t in (initial_state, final_state, ckpt_state) if t is not None]
        state_dtype = torch.bfloat16 if given and given[0].dtype == torch.bfloat16 else torch.float32
    if state_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("states must be float32 or bfloat16")
    cu64 = cu_seqlens is not None and cu_seqlens.dtype == torch.int64
    for name, t, dt in (("cu_seqlens", cu_seqlens, torch.int64 if cu64 else torch.int32),
                        ("seq_order", seq_order, torch.int32), ("initial_state", initial_state,
                        state_dtype), ("ckpt_offsets", ckpt_offsets, torch.int32),
                        ("ckpt_state", ckpt_state, state_dtype), ("out", out, torch.bfloat16),
                        ("final_state", final_state, state_dtype)):
        if t is None:
            continue
        if t.dtype != dt:
            raise TypeError(f"{name} must be {dt}, got {t.dtype}")
        if t.device != dev or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous on {dev}")
    state_shape = (N, H, D, D)
    for name, t in (("initial_state", initial_state), ("final_state", final_state)):
        if t is not None and tuple(t.shape) != state_shape:
            raise ValueError(f"{name} must have shape {state_shape}")
    C = 1
    if ckpt_offsets is not None:
        if ckpt_offsets.dim() == 2:
            C = int(ckpt_offsets.shape[1])
        if tuple(ckpt_offsets.shape) not in ((N,), (N, C)) or ckpt_state is None:
            raise ValueError("ckpt_offsets must be [N] or [N, C], with ckpt_state")
        want = (N, H, D, D) if ckpt_offsets.dim() == 1 else (N, C, H, D, D)
        if tuple(ckpt_state.shape) != want:
            raise ValueError(f"ckpt_state must have shape {want}")
    if scale is None:
        scale = D ** -0.5
    prob = make_problem(N, T_total, H, scale=scale, gate_lower_bound=gate_lower_bound,
                        variant=variant, value_split=value_split, head_dim_k=D, head_dim_v=D,
                        ckpt_per_seq=C,
                        state_dtype="bf16" if state_dtype == torch.bfloat16 else "fp32",
                        qk_l2norm=qk_l2norm, beta_logit=beta_logit, cu_seqlens_int64=cu64,
                        seq_order=_ptr(seq_order), chain_parts=chain_parts)
    if seq_order is not None and tuple(seq_order.shape) != (N,):
        raise ValueError(f"seq_order must be [{N}]")
    out_given, final_given = out, final_state
    if out is None:
        out = torch.empty_like(v)
    elif out.shape != q.shape:
        raise ValueError("out must have q's shape")
    if final_state is None and output_final_state:
        final_state = torch.empty(state_shape, dtype=state_dtype, device=dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    own_ws = False
    with torch.cuda.device(dev):
        if workspace is None:
            # a workspace only for the two-launch schedule (AUTO: when the
            # library's table picks it on this device)
            need = workspace_size(prob)
            if need and variant != "fused" and (variant != "auto" or plan(prob)[0] == "decomp"):
                workspace = torch.empty(need, dtype=torch.uint8, device=dev)
                own_ws = True
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        st = prefill_raw(prob, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens),
                         _ptr(initial_state), _ptr(out), _ptr(final_state), _ptr(ckpt_offsets),
                         _ptr(ckpt_state), _ptr(workspace), ws_bytes, int(stream.cuda_stream))
        # Blocks allocated here belong to the current stream in torch's caching
        # allocator.  When the call runs on another stream, tell the allocator
        # that stream uses them, so that a block (above all the workspace,
        # dropped on return) is not handed to a new allocation on the current
        # stream while the kernels still read or write it.
        if stream != torch.cuda.current_stream(dev):
            for t, mine in ((workspace, own_ws), (out, out_given is None),
                            (final_state, final_given is None)):
                if mine and t is not None:
                    t.record_stream(stream)
    _check(st, "kda_prefill")
    return out, final_state


def decode_raw(problem: DecodeProblem, q, k, v, g, beta, state_pool, state_indices, out,
               stream) -> int:
    """Call ``kda_decode`` with raw integer pointers (0 for NULL); returns the status."""
    lib = load_library()
    return lib.kda_decode(ctypes.byref(problem), q or None, k or None, v or None, g or None,
                          beta or None, state_pool or None, state_indices or None, out or None,
                          stream or None)


def decode_verify_raw(problem: DecodeProblem, q, k, v, g, beta, state_pool, state_indices, out,
                      state_trace, stream) -> int:
    """Call ``kda_decode_verify`` with raw integer pointers (0 for NULL); returns the status."""
    lib = load_library()
    return lib.kda_decode_verify(ctypes.byref(problem), q or None, k or None, v or None, g or None,
                                 beta or None, state_pool or None, state_indices or None, out or None,
                                 state_trace or None, stream or None)


def decode_commit_raw(problem: DecodeProblem, state_pool, state_indices, state_trace, accepted,
                      stream) -> int:
    """Call ``kda_decode_commit`` with raw integer pointers (0 for NULL); returns the status."""
    lib = load_library()
    return lib.kda_decode_commit(ctypes.byref(problem), state_pool or None, state_indices or None,
                                 state_trace or None, accepted or None, stream or None)


def decode_advance_raw(problem: DecodeProblem, q, k, v, g, beta, state_pool, state_indices, accepted,
                       stream) -> int:
    """Call ``kda_decode_advance`` with raw integer pointers (0 for NULL); returns the status."""
    lib = load_library()
    return lib.kda_decode_advance(ctypes.byref(problem), q or None, k or None, v or None, g or None,
                                  beta or None, state_pool or None, state_indices or None,
                                  accepted or None, stream or None)


def decode_validate_raw(problem: DecodeProblem, q, k, v, g, beta, state_pool, state_indices,
                        out) -> int:
    """Call ``kda_decode_validate`` with raw integer pointers; returns the status (host only)."""
    lib = load_library()
    return lib.kda_decode_validate(ctypes.byref(problem), q or None, k or None, v or None,
                                   g or None, beta or None, state_pool or None,
                                   state_indices or None, out or None)


def _decode_setup(q, k, v, g, beta, state_pool, state_indices, scale, gate_lower_bound, qk_l2norm,
                  beta_logit):
    """Shape, dtype and device checks shared by decode and decode_verify;
    returns the problem struct."""
    import torch

    if q.dim() != 4:
        raise ValueError("q must be [N, T, H, 128]")
    N, T, H, D = q.shape
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("libkda runs on the GPU: tensors must be on a cuda (HIP) device")
    if state_pool.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"state_pool must be float32 or bfloat16, got {state_pool.dtype}")
    for name, t, dt in (("q", q, torch.bfloat16), ("k", k, torch.bfloat16), ("v", v, torch.bfloat16),
                        ("g", g, torch.float32), ("beta", beta, torch.float32),
                        ("state_pool", state_pool, state_pool.dtype),
                        ("state_indices", state_indices, torch.int32)):
        if t.dtype != dt:
            raise TypeError(f"{name} must be {dt}, got {t.dtype}")
        if t.device != dev or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous on {dev}")
    if k.shape != q.shape or v.shape != q.shape or g.shape != q.shape:
        raise ValueError("q, k, v and g must have the same shape")
    if beta.shape != q.shape[:-1]:
        raise ValueError("beta must be q.shape[:-1]")
    if state_pool.dim() != 4 or tuple(state_pool.shape[1:]) != (H, D, D):
        raise ValueError(f"state_pool must be [P, {H}, {D}, {D}]")
    if tuple(state_indices.shape) != (N,):
        raise ValueError(f"state_indices must be [{N}]")
    if scale is None:
        scale = D ** -0.5
    return make_decode_problem(N, T, H, state_pool.shape[0], scale=scale,
                               gate_lower_bound=gate_lower_bound, head_dim_k=D, head_dim_v=D,
                               qk_l2norm=qk_l2norm, beta_logit=beta_logit,
                               state_dtype="bf16" if state_pool.dtype == torch.bfloat16 else "fp32")


def _decode_out(q, v, out):
    import torch

    if out is None:
        return torch.empty_like(v)
    if out.shape != q.shape or out.dtype != torch.bfloat16:
        raise ValueError("out must be bf16 with q's shape")
    return out


def decode(q, k, v, g, beta, state_pool, state_indices, *, scale: Optional[float] = None,
           out=None, gate_lower_bound: float = -5.0, stream=None, qk_l2norm: bool = False,
           beta_logit: bool = False):
    """One state-pool decode step on the GPU.

    q, k, v: bf16 [N, T, H, 128] (T tokens per request; T = 1 for decode).
    g: fp32 like q; beta: fp32 [N, T, H].  state_pool: fp32 or bf16 [P, H, 128, 128],
    updated in place (bf16: widened on load, rounded to nearest even on store).  state_indices: int32 [N]; entries outside [0, P) mark
    empty request slots (zero outputs, no state touched).  Returns out, with
    q's shape (``out=v`` overwrites v)."""
    import torch

    prob = _decode_setup(q, k, v, g, beta, state_pool, state_indices, scale, gate_lower_bound,
                         qk_l2norm, beta_logit)
    out = _decode_out(q, v, out)
    dev = q.device
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        st = decode_raw(prob, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_pool),
                        _ptr(state_indices), _ptr(out), int(stream.cuda_stream))
    _check(st, "kda_decode")
    return out


def decode_verify(q, k, v, g, beta, state_pool, state_indices, *, scale: Optional[float] = None,
                  out=None, state_trace=None, gate_lower_bound: float = -5.0, stream=None,
                  qk_l2norm: bool = False, beta_logit: bool = False):
    """Speculative verify: decode's update over the T draft tokens of every
    request, with state_pool only read.  state_trace: None allocates the trace
    of the state after each token (fp32 [N, T, H, 128, 128]), False stores no
    trace, or a tensor of that shape.  Returns (out, state_trace or None);
    decode_commit (with a trace) or decode_advance (without) then keeps the
    accepted prefix."""
    import torch

    prob = _decode_setup(q, k, v, g, beta, state_pool, state_indices, scale, gate_lower_bound,
                         qk_l2norm, beta_logit)
    out = _decode_out(q, v, out)
    N, T, H, D = q.shape
    dev = q.device
    sdt = state_pool.dtype
    if state_trace is None:
        state_trace = torch.empty((N, T, H, D, D), dtype=sdt, device=dev)
    elif state_trace is False:
        state_trace = None
    elif (tuple(state_trace.shape) != (N, T, H, D, D) or state_trace.dtype != sdt
          or state_trace.device != dev or not state_trace.is_contiguous()):
        raise ValueError(f"state_trace must be contiguous {sdt} [{N}, {T}, {H}, {D}, {D}] on {dev}")
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        st = decode_verify_raw(prob, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                               _ptr(state_pool), _ptr(state_indices), _ptr(out),
                               0 if state_trace is None else _ptr(state_trace), int(stream.cuda_stream))
    _check(st, "kda_decode_verify")
    return out, state_trace


def decode_advance(q, k, v, g, beta, state_pool, state_indices, accepted, *,
                   scale: Optional[float] = None, gate_lower_bound: float = -5.0, stream=None,
                   qk_l2norm: bool = False, beta_logit: bool = False):
    """After a verify without a trace: each request's pool state advances by
    its first accepted[n] tokens of the same drafts (int32 [N] on the device;
    0 or out of range leaves it as it is), recomputed, with no outputs."""
    import torch

    prob = _decode_setup(q, k, v, g, beta, state_pool, state_indices, scale, gate_lower_bound,
                         qk_l2norm, beta_logit)
    N = q.shape[0]
    dev = q.device
    if accepted.dtype != torch.int32 or tuple(accepted.shape) != (N,) or accepted.device != dev \
            or not accepted.is_contiguous():
        raise ValueError(f"accepted must be contiguous int32 [{N}] on {dev}")
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        st = decode_advance_raw(prob, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_pool),
                                _ptr(state_indices), _ptr(accepted), int(stream.cuda_stream))
    _check(st, "kda_decode_advance")


def decode_commit(state_pool, state_indices, state_trace, accepted, *, stream=None):
    """After decode_verify: pool[state_indices[n]] <- state_trace[n, accepted[n] - 1]
    for the requests with a pool index and 1 <= accepted[n] <= T (int32 [N] on
    the device); the others keep their pool state."""
    import torch

    if state_trace.dim() != 5:
        raise ValueError("state_trace must be [N, T, H, 128, 128]")
    N, T, H, D, _ = state_trace.shape
    dev = state_trace.device
    if state_pool.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"state_pool must be float32 or bfloat16, got {state_pool.dtype}")
    for name, t, dt in (("state_pool", state_pool, state_pool.dtype),
                        ("state_indices", state_indices, torch.int32),
                        ("state_trace", state_trace, state_pool.dtype),
                        ("accepted", accepted, torch.int32)):
        if t.dtype != dt:
            raise TypeError(f"{name} must be {dt}, got {t.dtype}")
        if t.device != dev or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous on {dev}")
    if dev.type != "cuda":
        raise ValueError("libkda runs on the GPU: tensors must be on a cuda (HIP) device")
    if state_pool.dim() != 4 or tuple(state_pool.shape[1:]) != (H, D, D):
        raise ValueError(f"state_pool must be [P, {H}, {D}, {D}]")
    if tuple(state_indices.shape) != (N,) or tuple(accepted.shape) != (N,):
        raise ValueError(f"state_indices and accepted must be [{N}]")
    prob = make_decode_problem(N, T, H, state_pool.shape[0], scale=1.0, head_dim_k=D, head_dim_v=D,
                               state_dtype="bf16" if state_pool.dtype == torch.bfloat16 else "fp32")
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        st = decode_commit_raw(prob, _ptr(state_pool), _ptr(state_indices), _ptr(state_trace),
                               _ptr(accepted), int(stream.cuda_stream))
    _check(st, "kda_decode_commit")
