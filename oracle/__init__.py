"""fp64 CPU oracle for KDA multi-token recurrent prefill -- TEST INFRASTRUCTURE.

Only the test suite, the package smoke check and the CPU-baseline leg of the
benchmark may import this package.  The product path (the HIP library and its
Python binding) never imports, links or calls anything here, and this package
shares no code with it.  The arithmetic lives in ``kda_oracle.c`` (plain C,
fp64, token by token); this module only builds it with gcc and marshals numpy
arrays into it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libkda_oracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile kda_oracle.c with gcc (strict IEEE fp64: no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-fPIC", "-shared", "-pthread",
                               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _open(path: str):
    lib = ctypes.CDLL(path)
    f = lib.kda_oracle_prefill_f64
    P = ctypes.c_void_p
    f.argtypes = [ctypes.c_int, ctypes.c_long, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                  ctypes.c_double, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_int, ctypes.c_int]
    f.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        build()
        _lib = _open(_LIB_PATH)
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def prefill(q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray, g: np.ndarray,
            beta: np.ndarray, *, scale: float, num_seqs: int,
            cu_seqlens: Optional[np.ndarray] = None,
            initial_state: Optional[np.ndarray] = None,
            ckpt_offsets: Optional[np.ndarray] = None,
            threads: Optional[int] = None, qk_l2norm: bool = False, beta_logit: bool = False,
            _library=None) -> dict:
    """Run the token-by-token fp64 recurrence.

    q_bits, k_bits: [T, H, K] uint16 bf16 patterns; v_bits [T, H, V]; g [T, H, K]
    fp32; beta [T, H] fp32; cu_seqlens [N+1] int32 or None (N equal
    sequences); initial_state [N, H, K, V] fp32 or None; ckpt_offsets [N] int32
    or None.  Returns dict(out [T,H,V], final [N,H,K,V], ckpt [N,H,K,V] or
    None), all fp64.  Checkpoint slots whose offset is outside [0, L] stay NaN.
    qk_l2norm / beta_logit: the input prologue of kda_oracle.c (q and k divided
    by their L2 norms per token and head; beta given as a logit).
    """
    lib = _library if _library is not None else _load()
    q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
    k_bits = np.ascontiguousarray(k_bits, dtype=np.uint16)
    v_bits = np.ascontiguousarray(v_bits, dtype=np.uint16)
    g = np.ascontiguousarray(g, dtype=np.float32)
    beta = np.ascontiguousarray(beta, dtype=np.float32)
    T, H, K = q_bits.shape
    V = v_bits.shape[2]
    if k_bits.shape != (T, H, K) or v_bits.shape[:2] != (T, H) or g.shape != (T, H, K) \
            or beta.shape != (T, H):
        raise ValueError("inconsistent input shapes")
    N = int(num_seqs)
    cu = None if cu_seqlens is None else np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    s0 = None if initial_state is None else np.ascontiguousarray(initial_state, dtype=np.float32)
    if s0 is not None and s0.shape != (N, H, K, V):
        raise ValueError("initial_state shape")
    offs = None if ckpt_offsets is None else np.ascontiguousarray(ckpt_offsets, dtype=np.int32)
    out = np.empty((T, H, V), dtype=np.float64)
    final = np.empty((N, H, K, V), dtype=np.float64)
    ck = None
    if offs is not None:
        ck = np.full((N, H, K, V), np.nan, dtype=np.float64)
    rc = lib.kda_oracle_prefill_f64(N, T, H, K, V, float(scale), _ptr(q_bits), _ptr(k_bits),
                                    _ptr(v_bits), _ptr(g), _ptr(beta), _ptr(cu), _ptr(s0),
                                    _ptr(offs), _ptr(out), _ptr(final), _ptr(ck),
                                    (1 if qk_l2norm else 0) | (2 if beta_logit else 0),
                                    int(threads if threads is not None else default_threads()))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return {"out": out, "final": final, "ckpt": ck}


def prefill_problem(p, *, threads: Optional[int] = None, qk_l2norm: bool = False,
                    beta_logit: bool = False) -> dict:
    """Run the oracle on a ``synth.Problem``."""
    return prefill(p.q, p.k, p.v, p.g, p.beta, scale=p.scale, num_seqs=p.N,
                   cu_seqlens=None if p.fixed else p.cu_seqlens,
                   initial_state=p.initial_state, ckpt_offsets=p.ckpt_offsets, threads=threads,
                   qk_l2norm=qk_l2norm, beta_logit=beta_logit)


def decode(q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray, g: np.ndarray,
           beta: np.ndarray, *, scale: float, num_seqs: int, tokens_per_seq: int,
           state_pool: np.ndarray, state_indices: np.ndarray,
           threads: Optional[int] = None, qk_l2norm: bool = False,
           beta_logit: bool = False) -> dict:
    """State-pool decode: request n advances by tokens_per_seq tokens from
    state_pool[state_indices[n]] and the result replaces that pool entry.

    This is the serving step of the sglang KDA decode backend (the state pool
    and its ssm_state_indices, FlashInferKDAKernel page; FlashInfer PR #4262,
    Description, names decode and state-pool features).  The pages give no
    formula for it beyond the recurrence itself, so the reading is: the same
    token recurrence as ``prefill`` (decay, delta-rule correction, read-out),
    run from the pool entry; an index outside [0, pool_size) means an empty
    request slot: zero outputs, pool untouched.

    Inputs are request-major [N * T, H, ...] arrays as in ``prefill``'s fixed
    layout; state_pool [P, H, K, V] fp32; state_indices [N] int.  Returns
    dict(out [N*T, H, V] fp64, pool [P, H, K, V] fp64 after the step)."""
    N, T = int(num_seqs), int(tokens_per_seq)
    idx = np.asarray(state_indices, np.int64)
    P, H = state_pool.shape[0], state_pool.shape[1]
    pool = state_pool.astype(np.float64)
    out = np.zeros((N * T, H, v_bits.shape[2]), np.float64)
    live = [n for n in range(N) if 0 <= idx[n] < P]
    if live:
        rows = np.concatenate([np.arange(n * T, (n + 1) * T) for n in live])
        res = prefill(q_bits[rows], k_bits[rows], v_bits[rows], g[rows], beta[rows], scale=scale,
                      num_seqs=len(live), initial_state=state_pool[idx[live]], threads=threads,
                      qk_l2norm=qk_l2norm, beta_logit=beta_logit)
        out[rows] = res["out"]
        pool[idx[live]] = res["final"]
    return {"out": out, "pool": pool}


def prefill_with_library(path: str):
    """Return a ``prefill`` bound to another build of kda_oracle.c (used by the
    tests that plant mistakes in a copy of the oracle and check that the pins
    catch them)."""
    lib = _open(path)

    def run(*args, **kwargs):
        kwargs["_library"] = lib
        return prefill(*args, **kwargs)

    return run
