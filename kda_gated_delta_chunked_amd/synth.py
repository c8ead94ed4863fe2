"""Seeded synthetic KDA prefill inputs, shared by the tests and the benchmark.

This module only draws random numbers and lays them out.  It holds none of the
recurrence's arithmetic, so the fp64 oracle and the HIP path can both be fed
from it without sharing any of the method.

Value recipe (the workloads the FlashInfer KDA prefill pages benchmark at
H = 12, K = V = 128, BF16; "cake_kda" PR #4262, Performance, and the SM120
CuTe DSL PR #4633, Performance):

* q, k: N(0, 1) in fp32, L2-normalised over the 128 channels of each
  (token, head), then rounded to bf16 (round to nearest even).  The kernel
  contract takes already normalised keys and queries.
* v: N(0, 1) rounded to bf16 (not normalised).
* beta: sigmoid(N(0, 1)) in fp32, shape [T, H] (already activated).
* g: -5 * sigmoid(N(0, 1)) in fp32, one value per key channel, shape
  [T, H, 128]; a natural-log decay inside the gate lower bound [-5, 0].
* initial state (when used): N(0, 0.02^2) in fp32, shape [N, H, 128, 128].

Every array is produced on the host with ``numpy.random.default_rng(seed)``
and bf16 rounding is done bitwise here, so the oracle and the GPU see the same
bf16 values.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

HEAD_DIM = 128


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); return bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    out = ((u + rounding) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def f32_from_bf16_bits(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Problem:
    """One KDA prefill call's host inputs.

    Layouts: q/k/v bits [T_total, H, 128] uint16 (bf16), g [T_total, H, 128]
    fp32, beta [T_total, H] fp32, cu_seqlens [N+1] int32 (always filled, also
    for fixed layout), initial_state [N, H, 128, 128] fp32 or None,
    ckpt_offsets [N] int32 or None.  ``fixed`` marks a fixed-length batch (the
    device call then passes no cu_seqlens).
    """

    name: str
    seq_lens: np.ndarray
    H: int
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta: np.ndarray
    cu_seqlens: np.ndarray
    fixed: bool
    initial_state: Optional[np.ndarray]
    ckpt_offsets: Optional[np.ndarray]
    scale: float
    seed: int

    @property
    def N(self) -> int:
        return int(len(self.seq_lens))

    @property
    def T_total(self) -> int:
        return int(self.cu_seqlens[-1])


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


def _unit_rows(rng: np.random.Generator, shape) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    nrm = np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=-1, keepdims=True))
    nrm = np.maximum(nrm, 1e-30)
    return (x / nrm).astype(np.float32)


def make_problem(seq_lens: Sequence[int], H: int, *, seed: int, fixed: bool = False,
                 init_state: bool = False, ckpt: str | Sequence[int] | None = None,
                 gate: str = "random", beta_mode: str = "random", name: str = "",
                 K: int = HEAD_DIM, V: int = HEAD_DIM) -> Problem:
    """Draw one problem.

    ckpt: None (no export), "inside" (one offset per sequence, uniform in
    [1, L-1], or 0 when L < 2), or an explicit sequence of offsets.
    gate: "random" (-5 sigmoid(N(0,1))), "zero" (g = 0), "min" (g = -5).
    beta_mode: "random" (sigmoid(N(0,1))), "zero", "one".
    """
    seq_lens = np.asarray(list(seq_lens), dtype=np.int64)
    if fixed and len(set(seq_lens.tolist())) > 1:
        raise ValueError("fixed layout needs equal sequence lengths")
    rng = np.random.default_rng(seed)
    T = int(seq_lens.sum())
    N = len(seq_lens)
    cu = np.zeros(N + 1, dtype=np.int64)
    cu[1:] = np.cumsum(seq_lens)
    if cu[-1] > np.iinfo(np.int32).max:
        raise ValueError("too many tokens for int32 offsets")
    q = bf16_bits_from_f32(_unit_rows(rng, (T, H, K)))
    k = bf16_bits_from_f32(_unit_rows(rng, (T, H, K)))
    v = bf16_bits_from_f32(rng.standard_normal((T, H, V), dtype=np.float32))
    if beta_mode == "random":
        beta = _sigmoid(rng.standard_normal((T, H), dtype=np.float32))
    elif beta_mode == "zero":
        beta = np.zeros((T, H), dtype=np.float32)
    elif beta_mode == "one":
        beta = np.ones((T, H), dtype=np.float32)
    else:
        raise ValueError(beta_mode)
    if gate == "random":
        g = (-5.0 * _sigmoid(rng.standard_normal((T, H, K), dtype=np.float32))).astype(np.float32)
    elif gate == "zero":
        g = np.zeros((T, H, K), dtype=np.float32)
    elif gate == "min":
        g = np.full((T, H, K), -5.0, dtype=np.float32)
    else:
        raise ValueError(gate)
    s0 = None
    if init_state:
        s0 = (0.02 * rng.standard_normal((N, H, K, V), dtype=np.float32)).astype(np.float32)
    offs = None
    if ckpt is not None:
        if isinstance(ckpt, str):
            if ckpt != "inside":
                raise ValueError(ckpt)
            offs = np.array([rng.integers(1, L) if L >= 2 else 0 for L in seq_lens], dtype=np.int32)
        else:
            offs = np.asarray(list(ckpt), dtype=np.int32)
            if offs.shape != (N,):
                raise ValueError("one checkpoint offset per sequence")
    return Problem(name=name or f"N{N}_T{T}_H{H}", seq_lens=seq_lens, H=H, q=q, k=k, v=v, g=g,
                   beta=beta, cu_seqlens=cu.astype(np.int32), fixed=fixed, initial_state=s0,
                   ckpt_offsets=offs, scale=float(1.0 / np.sqrt(K)), seed=seed)


def uniform_lengths(rng_seed: int, count: int, lo: int, hi: int) -> list[int]:
    """Sequence lengths uniform in [lo, hi] from their own seeded stream."""
    rng = np.random.default_rng(rng_seed)
    return [int(x) for x in rng.integers(lo, hi + 1, size=count)]


# Named workloads: (B, T) fixed batches at H = 12, and packed batches.
# Seeds are 1000 + the workload's index in this table.
def workload(name: str, *, H: int = 12) -> Problem:
    """Build one of the named workloads at full size.

    b1_t64_h1      one chunk, H = 1, zero initial state
    b1_t8192       fixed B1 T8192, zero initial state       (also b1_t512)
    b8_t8192       fixed B8 T8192, initial state N(0,0.02^2) (also b8_t1024,
                   b32_t512, b6_t8192)
    packed_8x1024  8 sequences of 1024 tokens, per-sequence initial states
    packed_32_rand 32 sequences, lengths uniform in [1, 4096]
    ckpt_16_rand   16 sequences, lengths uniform in [512, 8192], one
                   checkpoint offset per sequence inside it
    packed_512x32, packed_128x8, mixed_6
                   the packed shapes of FlashInfer PR #4262's B200 table
                   (32 x 512, 8 x 128, and six lengths 1300, 547, 2048,
                   963, 271, 3063), per-sequence initial states
    """
    table = {
        "b1_t64_h1": dict(lens=[64], H=1, fixed=True, init=False, seed=1000),
        "b1_t8192": dict(lens=[8192], H=H, fixed=True, init=False, seed=1001),
        "b1_t512": dict(lens=[512], H=H, fixed=True, init=False, seed=1001),
        "b8_t8192": dict(lens=[8192] * 8, H=H, fixed=True, init=True, seed=1002),
        "b8_t1024": dict(lens=[1024] * 8, H=H, fixed=True, init=True, seed=1002),
        "b32_t512": dict(lens=[512] * 32, H=H, fixed=True, init=True, seed=1002),
        "b6_t8192": dict(lens=[8192] * 6, H=H, fixed=True, init=True, seed=1002),
        "packed_8x1024": dict(lens=[1024] * 8, H=H, fixed=False, init=True, seed=1003),
        "packed_32_rand": dict(lens=uniform_lengths(2003, 32, 1, 4096), H=H, fixed=False,
                               init=True, seed=1003),
        "ckpt_16_rand": dict(lens=uniform_lengths(2004, 16, 512, 8192), H=H, fixed=False,
                             init=True, seed=1004, ckpt="inside"),
        "packed_512x32": dict(lens=[512] * 32, H=H, fixed=False, init=True, seed=1005),
        "packed_128x8": dict(lens=[128] * 8, H=H, fixed=False, init=True, seed=1005),
        "mixed_6": dict(lens=[1300, 547, 2048, 963, 271, 3063], H=H, fixed=False, init=True,
                        seed=1005),
    }
    if name not in table:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(table)}")
    w = table[name]
    return make_problem(w["lens"], w["H"], seed=w["seed"], fixed=w["fixed"], init_state=w["init"],
                        ckpt=w.get("ckpt"), name=name)
