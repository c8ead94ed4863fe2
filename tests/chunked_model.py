"""Chunk-parallel form of the KDA recurrence, in numpy, for checking the maths.

This is not the oracle and not the GPU code.  It restates the chunked algebra
the HIP kernels implement, so a CPU test can show that (a) in fp64 the chunked
form reproduces the token recurrence to rounding (any chunk size, any tail),
and (b) with bf16 rounding placed where the kernels feed the matrix cores,
the result still meets the parity tolerances.

Within a chunk of c <= C rows that starts from state S0 (rows r = 0..c-1):

  G_r   = g_0 + ... + g_r                       (per key channel)
  A[r,s] = sum_d k_rd k_sd exp(G_rd - G_sd)      s < r
  M[r,s] = sum_d q_rd k_sd exp(G_rd - G_sd)      s <= r
  T     = (I + diag(beta) A)^-1,  N = T - I      (unit lower triangular)
  X     = V - (K * exp(G)) S0                    (what the state mispredicts)
  Y     = diag(beta) X,   U = Y + N Y            (the delta-rule writes)
  O     = scale ((Q * exp(G)) S0 + M U)
  S     = diag(exp(G_{c-1})) S0 + (K * exp(G_{c-1} - G))^T U

The gated products are formed the way the kernels form them: rows are grouped
in 16-row blocks, block i has reference point ref_i = G_{16i-1} (ref_0 = 0),
and exp(G_r - G_s) = exp(G_r - ref_i) * exp(ref_i - G_s) with r in block i.
For s in an earlier block both factors are <= 1; within the block the right
factor is at most exp(5 * 16) when g >= -5, which fp32 holds.
"""
from __future__ import annotations

import numpy as np

from kda_gated_delta_chunked_amd.synth import bf16_bits_from_f32, f32_from_bf16_bits

SUB = 16


def bf16(x):
    """Round to bf16 (nearest even) and return as float32."""
    return f32_from_bf16_bits(bf16_bits_from_f32(np.asarray(x, dtype=np.float32)))


def split_hi_lo(x):
    hi = bf16(x)
    lo = bf16(np.asarray(x, np.float32) - hi)
    return hi, lo


# Where bf16 rounding is injected in "emulate" mode.
DEFAULT_RECIPE = {
    "gate_operands": True,   # exp-scaled operands of A and M
    "k_q_tilde": True,       # K*exp(G), Q*exp(G) as matrix operands
    "state_operand": True,   # S0 as matrix operand (X and O)
    "n_matrix": True,        # N = T - I
    "y_operand": True,       # Y in N Y (identity part stays fp32)
    "m_matrix": True,        # M
    "u_operand_out": True,   # U in M U
    "khat": "hilo",          # "hilo" | "bf16" | "exact": K*exp(G_c - G) in the state update
    "u_state": "hilo",       # "hilo" | "bf16" | "exact": U in the state update
}


def _op(x, on, dt):
    return bf16(x) if on else x.astype(dt)


def _mm_split(a, b, mode_a, mode_b, dt):
    """a @ b with a / b given as hi+lo bf16 pairs, plain bf16, or exact."""
    def parts(x, mode):
        if mode == "hilo":
            return list(split_hi_lo(x))
        if mode == "bf16":
            return [bf16(x)]
        return [x.astype(dt)]
    pa, pb = parts(a, mode_a), parts(b, mode_b)
    out = pa[0] @ pb[0]
    if len(pb) > 1:
        out = out + pa[0] @ pb[1]
    if len(pa) > 1:
        out = out + pa[1] @ pb[0]
    return out


def _state_update(khat, U, rc, dt):
    """khat^T U with the recipe's rounding; "hilo_lastN" splits only the last N
    rows of khat (the least-decayed ones) into hi+lo."""
    mode = rc["khat"]
    if isinstance(mode, str) and mode.startswith("hilo_last"):
        n = int(mode[len("hilo_last"):])
        c = khat.shape[0]
        lo_rows = max(c - n, 0)
        hi, lo = split_hi_lo(khat)
        lo[:lo_rows] = 0
        return _mm_split(hi.T, U, "exact", rc["u_state"], dt) + _mm_split(lo.T, U, "exact", "bf16", dt)
    return _mm_split(khat.T, U, mode, rc["u_state"], dt)


def chunk_step(S, q, k, v, g, beta, scale, C_end=None, *, emulate=False, recipe=None):
    """One chunk from state S.  q,k [c,K] v [c,V] g [c,K] beta [c].

    Returns (O [c,V], S_new, U).  With C_end = p < c also returns the state
    after the first p rows as a fourth value (the masked partial update).
    """
    rc = recipe or DEFAULT_RECIPE
    dt = np.float32 if emulate else np.float64
    c, K = k.shape
    S = S.astype(dt)
    q = q.astype(dt); k = k.astype(dt); v = v.astype(dt)
    g = g.astype(dt); beta = beta.astype(dt)
    G = np.cumsum(g, axis=0, dtype=dt)
    nb = (c + SUB - 1) // SUB
    refs = [np.zeros(K, dt)] + [G[SUB * i - 1] for i in range(1, nb)]
    A = np.zeros((c, c), dt)
    M = np.zeros((c, c), dt)
    for i in range(nb):
        r0, r1 = SUB * i, min(SUB * (i + 1), c)
        lf = np.exp(G[r0:r1] - refs[i])
        rf = np.exp(refs[i] - G[:r1])
        kl, ql, kr = k[r0:r1] * lf, q[r0:r1] * lf, k[:r1] * rf
        gm = rc["gate_operands"] if emulate else False
        if gm is True or gm == "bf16":
            A[r0:r1, :r1] = bf16(kl) @ bf16(kr).T
            M[r0:r1, :r1] = bf16(ql) @ bf16(kr).T
        elif gm == "diag_hilo":
            # earlier blocks: plain bf16; the block's own rows: hi+lo
            A[r0:r1, :r1] = bf16(kl) @ bf16(kr).T
            M[r0:r1, :r0] = bf16(ql) @ bf16(kr[:r0]).T
            M[r0:r1, r0:r1] = _mm_split(ql, kr[r0:r1].T, "hilo", "hilo", dt)
        elif gm == "hilo":
            A[r0:r1, :r1] = bf16(kl) @ bf16(kr).T
            M[r0:r1, :r1] = _mm_split(ql, kr.T, "hilo", "hilo", dt)
        else:
            A[r0:r1, :r1] = kl @ kr.T
            M[r0:r1, :r1] = ql @ kr.T
    A = np.tril(A, -1)
    M = np.tril(M, 0)
    Lm = beta[:, None] * A
    T = np.linalg.inv(np.eye(c, dtype=dt) + Lm) if not emulate else \
        np.linalg.inv((np.eye(c) + Lm.astype(np.float64))).astype(dt)
    Nm = np.tril(T, -1)
    eG = np.exp(G)
    kt, qt = k * eG, q * eG
    khat = k * np.exp(G[c - 1] - G)
    gam = np.exp(G[c - 1])
    if emulate:
        S_op = _op(S, rc["state_operand"], dt)
        X = v - _op(kt, rc["k_q_tilde"], dt) @ S_op
        Y = beta[:, None] * X
        U = Y + _op(Nm, rc["n_matrix"], dt) @ _op(Y, rc["y_operand"], dt)
        mu_m = rc["m_matrix"] if isinstance(rc["m_matrix"], str) else ("bf16" if rc["m_matrix"] else "exact")
        mu_u = rc["u_operand_out"] if isinstance(rc["u_operand_out"], str) else \
            ("bf16" if rc["u_operand_out"] else "exact")
        O = scale * (_op(qt, rc["k_q_tilde"], dt) @ S_op + _mm_split(M, U, mu_m, mu_u, dt))
        S_new = gam[:, None] * S + _state_update(khat, U, rc, dt)
    else:
        X = v - kt @ S
        Y = beta[:, None] * X
        U = Y + Nm @ Y
        O = scale * (qt @ S + M @ U)
        S_new = gam[:, None] * S + khat.T @ U
    if C_end is None:
        return O, S_new, U
    p = int(C_end)
    if p == 0:
        return O, S_new, U, S.copy()
    mask = (np.arange(c) < p)[:, None]
    khat_p = np.where(mask, k * np.exp(G[p - 1] - G), 0)
    if emulate:
        S_p = np.exp(G[p - 1])[:, None] * S + _state_update(khat_p, U, rc, dt)
    else:
        S_p = np.exp(G[p - 1])[:, None] * S + khat_p.T @ U
    return O, S_new, U, S_p


def prefill(q, k, v, g, beta, *, scale, cu_seqlens, initial_state=None, ckpt_offsets=None,
            chunk=64, emulate=False, recipe=None, ckpt_mode="split"):
    """Chunked prefill over a packed batch.  Inputs as for the oracle, but q/k/v
    already widened to float.  Returns dict(out, final, ckpt).

    ckpt_mode "split" ends a segment at the checkpoint offset (what the HIP
    kernel does: the chunk containing the offset is processed as two
    segments); "masked" keeps the chunk whole and forms the checkpoint from a
    masked partial state update."""
    T, H, K = q.shape
    V = v.shape[2]
    N = len(cu_seqlens) - 1
    dt = np.float32 if emulate else np.float64
    out = np.zeros((T, H, V), dt)
    final = np.zeros((N, H, K, V), dt)
    ck = None if ckpt_offsets is None else np.full((N, H, K, V), np.nan, dt)
    for n in range(N):
        bos, eos = int(cu_seqlens[n]), int(cu_seqlens[n + 1])
        L = eos - bos
        p = None if ckpt_offsets is None else int(ckpt_offsets[n])
        # segment boundaries: multiples of `chunk` from the sequence start, plus p
        cuts = list(range(0, L, chunk)) + [L]
        if ckpt_mode == "split" and p is not None and 0 < p < L and p not in cuts:
            cuts = sorted(cuts + [p])
        for h in range(H):
            S = np.zeros((K, V), dt) if initial_state is None else initial_state[n, h].astype(dt)
            if p == 0:
                ck[n, h] = S
            for c0, c1 in zip(cuts[:-1], cuts[1:]):
                sl = slice(bos + c0, bos + c1)
                want = ckpt_mode == "masked" and p is not None and c0 < p < c1
                res = chunk_step(S, q[sl, h], k[sl, h], v[sl, h], g[sl, h], beta[sl, h], scale,
                                 C_end=(p - c0) if want else None, emulate=emulate, recipe=recipe)
                out[sl, h] = res[0]
                if want:
                    ck[n, h] = res[3]
                S = res[1]
                if p is not None and p == c1:
                    ck[n, h] = S
            final[n, h] = S
    return {"out": out, "final": final, "ckpt": ck}


def prefill_problem(p, **kw):
    """Run on a synth.Problem."""
    return prefill(f32_from_bf16_bits(p.q), f32_from_bf16_bits(p.k), f32_from_bf16_bits(p.v), p.g,
                   p.beta, scale=p.scale, cu_seqlens=p.cu_seqlens, initial_state=p.initial_state,
                   ckpt_offsets=p.ckpt_offsets, **kw)
