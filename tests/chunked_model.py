"""Chunk-parallel form of the KDA recurrence, in numpy, for checking the maths.

This is not the oracle and not the GPU code.  It restates the chunked algebra
the HIP kernels implement, so a CPU test can show that (a) in fp64 the chunked
form reproduces the token recurrence to rounding (any chunk size, any tail),
and (b) with the rounding the kernels apply where they feed the matrix cores
(fp16 or bf16 operands, some as hi + lo pairs; see KERNEL_RECIPE), the result
still meets the parity tolerances.

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
factor is at most exp(5 * 16) when g >= -5, which fp32 and bf16 hold (fp16,
whose largest value is about exp(11), does not: those blocks use bf16).
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


def f16(x):
    """Round to fp16 (nearest even, with subnormals) and return as float32."""
    return np.asarray(x, np.float32).astype(np.float16).astype(np.float32)


def _parts(x, mode, dt):
    """x as the list of matrix-core operands a mode feeds: one rounded copy,
    or a hi + lo pair (lo = the rounding remainder, rounded again)."""
    x = np.asarray(x, dt)
    if mode == "exact":
        return [x]
    if mode in ("bf16", "fp16"):
        return [(bf16 if mode == "bf16" else f16)(x)]
    if mode in ("bf16hl", "fp16hl"):
        rnd = bf16 if mode == "bf16hl" else f16
        hi = rnd(x)
        return [hi, rnd(x.astype(np.float32) - hi)]
    raise ValueError(mode)


def _mm(a, b, modes, dt):
    """a @ b with each operand rounded as its mode says; of the hi/lo cross
    terms only lo x lo is dropped (as on the matrix cores)."""
    pa, pb = _parts(a, modes[0], dt), _parts(b, modes[1], dt)
    out = pa[0] @ pb[0]
    if len(pb) > 1:
        out = out + pa[0] @ pb[1]
    if len(pa) > 1:
        out = out + pa[1] @ pb[0]
    return out


# Where rounding is injected in "emulate" mode: the operand rounding of each
# matrix product, as (left, right) modes.
#   a_off / m_off    gated K K^T / Q K^T, blocks left of the diagonal block
#                    (both factors <= 1)
#   a_diag / m_diag  their diagonal 16-row blocks (right factor up to e^80)
#   x    K~ S            o1   Q~ S             ny   N Y
#   o2   M U             su   K^^T U (the state update)
# scale_cols: the state, V and everything derived from them are fed to the
# matrix cores multiplied by a power of two 2^s shared by groups of this many
# columns (one wave's columns); s is kept across segments and reset when the
# scaled magnitude leaves [2^2, 2^6] (0: no scaling).
KERNEL_RECIPE = {
    "a_off": ("fp16", "fp16"), "a_diag": ("bf16hl", "bf16hl"),
    "m_off": ("fp16", "fp16"), "m_diag": ("bf16hl", "bf16hl"),
    "x": ("fp16", "fp16"), "o1": ("fp16", "fp16"), "ny": ("fp16", "fp16"),
    "o2": ("fp16", "fp16"), "su": ("fp16", "fp16hl"),
    "scale_cols": 16, "fold_scale": False, "solve": "exact",
}
# The one-launch schedule: the same operands; its triangular solve merges the
# diagonal 16 x 16 inverses with fp16 matrix products.
FUSED_RECIPE = dict(KERNEL_RECIPE, solve="merge_fp16")
# The recipe the kernels used before: bf16 operands throughout, U hi + lo into
# M U and the state update, the last 16 rows of K^ hi + lo, the diagonal
# blocks of M hi + lo, the read-out scale folded into Q~ and M (the two-launch
# schedule's exact solve; the one-launch schedule merged with bf16 products).
BF16_RECIPE = {
    "a_off": ("bf16", "bf16"), "a_diag": ("bf16", "bf16"),
    "m_off": ("bf16", "bf16"), "m_diag": ("bf16hl", "bf16hl"),
    "x": ("bf16", "bf16"), "o1": ("bf16", "bf16"), "ny": ("bf16", "bf16"),
    "o2": ("bf16", "bf16hl"), "su": ("bf16hl_last16", "bf16hl"),
    "scale_cols": 0, "fold_scale": True, "solve": "exact",
}
SCALE_LO, SCALE_HI, SCALE_MID = 2.0, 6.0, 4


def _state_update(khat, U, mode, dt):
    """khat^T U; "bf16hl_last16" rounds khat to bf16 and adds the lo part of
    its last 16 rows only."""
    if mode[0] == "bf16hl_last16":
        hi = bf16(khat)
        lo = bf16(np.asarray(khat, np.float32) - hi)
        lo[:max(khat.shape[0] - 16, 0)] = 0
        return _mm(hi.T, U, ("exact", mode[1]), dt) + _mm(lo.T, U, ("exact", "bf16"), dt)
    return _mm(khat.T, U, mode, dt)


def _solve_merge(Lm, rnd):
    """(I + L)^-1 the way the one-launch schedule forms it: the four 16 x 16
    diagonal blocks inverted in fp32, then block merges on the matrix cores
    with rounded operands (rnd) and fp32 accumulation:
      T10 = -T11 (L10 T00),  T32 = -T33 (L32 T22),
      T[32:64, 0:32] = -T[32:64, 32:64] (L[32:64, 0:32] T[0:32, 0:32])."""
    f = np.float32
    T = np.zeros((64, 64), f)
    for i in range(4):
        b = slice(16 * i, 16 * i + 16)
        T[b, b] = np.linalg.inv(np.eye(16) + Lm[b, b].astype(np.float64)).astype(f)
    for i, j in ((1, 0), (3, 2)):
        bi, bj = slice(16 * i, 16 * i + 16), slice(16 * j, 16 * j + 16)
        P = rnd(Lm[bi, bj]) @ rnd(T[bj, bj])
        T[bi, bj] = -(rnd(T[bi, bi]) @ rnd(P))
    Q = rnd(Lm[32:64, 0:32]) @ rnd(T[0:32, 0:32])
    T[32:64, 0:32] = -(rnd(T[32:64, 32:64]) @ rnd(Q))
    return T


def _update_scale(s, S, v, cols):
    """Per group of `cols` columns: keep the exponent s while the scaled
    magnitude max(|S|, |V|) 2^s stays in [2^2, 2^6] (or is zero), else reset
    it so that the magnitude lands in [2^4, 2^5)."""
    s = s.copy()
    for c0 in range(0, S.shape[1], cols):
        sl = slice(c0, c0 + cols)
        m = max(float(np.max(np.abs(S[:, sl]), initial=0.0)), float(np.max(np.abs(v[:, sl]), initial=0.0)))
        ms = m * 2.0 ** s[c0]
        if m > 0 and (ms > 2.0 ** SCALE_HI or ms < 2.0 ** SCALE_LO):
            s[sl] = SCALE_MID - np.floor(np.log2(m))
    return s


def chunk_step(S, q, k, v, g, beta, scale, C_end=None, *, emulate=False, recipe=None, sexp=None):
    """One chunk from state S.  q,k [c,K] v [c,V] g [c,K] beta [c].

    Returns (O [c,V], S_new, U).  With C_end = p < c also returns the state
    after the first p rows as a fourth value (the masked partial update).
    In emulate mode with a scaling recipe, `sexp` holds the per-column scale
    exponents carried between chunks (updated in place).
    """
    rc = recipe or KERNEL_RECIPE
    dt = np.float32 if emulate else np.float64
    c, K = k.shape
    S = S.astype(dt)
    q = q.astype(dt); k = k.astype(dt); v = v.astype(dt)
    g = g.astype(dt); beta = beta.astype(dt)
    G = np.cumsum(g, axis=0, dtype=dt)
    nb = (c + SUB - 1) // SUB
    refs = [np.zeros(K, dt)] + [G[SUB * i - 1] for i in range(1, nb)]
    fold = emulate and rc["fold_scale"]
    qs = q * scale if fold else q
    A = np.zeros((c, c), dt)
    M = np.zeros((c, c), dt)
    for i in range(nb):
        r0, r1 = SUB * i, min(SUB * (i + 1), c)
        lf = np.exp(G[r0:r1] - refs[i])
        rf = np.exp(refs[i] - G[:r1])
        kl, ql, kr = k[r0:r1] * lf, qs[r0:r1] * lf, k[:r1] * rf
        if emulate:
            if r0 > 0:
                A[r0:r1, :r0] = _mm(kl, kr[:r0].T, rc["a_off"], dt)
                M[r0:r1, :r0] = _mm(ql, kr[:r0].T, rc["m_off"], dt)
            A[r0:r1, r0:r1] = _mm(kl, kr[r0:r1].T, rc["a_diag"], dt)
            M[r0:r1, r0:r1] = _mm(ql, kr[r0:r1].T, rc["m_diag"], dt)
        else:
            A[r0:r1, :r1] = kl @ kr.T
            M[r0:r1, :r1] = ql @ kr.T
    A = np.tril(A, -1)
    M = np.tril(M, 0)
    Lm = beta[:, None] * A
    if not emulate:
        T = np.linalg.inv(np.eye(c, dtype=dt) + Lm)
    elif rc.get("solve", "exact") != "exact" and c == 64:
        T = _solve_merge(Lm, f16 if rc["solve"] == "merge_fp16" else bf16)
    else:
        T = np.linalg.inv((np.eye(c) + Lm.astype(np.float64))).astype(dt)
    Nm = np.tril(T, -1)
    eG = np.exp(G)
    kt, qt = k * eG, qs * eG
    khat = k * np.exp(G[c - 1] - G)
    gam = np.exp(G[c - 1])
    if emulate:
        # the state, V and what derives from them go to the matrix cores
        # multiplied by 2^s per column (exact: a power of two)
        sig = np.ones(S.shape[1], dt)
        if rc["scale_cols"]:
            sexp[:] = _update_scale(sexp, S, v, rc["scale_cols"])
            sig = (2.0 ** sexp).astype(dt)
        Ss, vs = S * sig, v * sig
        X = _mm(kt, Ss, rc["x"], dt)
        Y = beta[:, None] * (vs - X)
        U = Y + _mm(Nm, Y, rc["ny"], dt)
        O = _mm(qt, Ss, rc["o1"], dt) + _mm(M, U, rc["o2"], dt)
        O = O / sig if fold else O * (scale / sig)
        S_new = gam[:, None] * S + _state_update(khat, U, rc["su"], dt) / sig
        U = U / sig
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
        S_p = np.exp(G[p - 1])[:, None] * S + _state_update(khat_p, U * sig, rc["su"], dt) / sig
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
            sexp = np.zeros(V)   # per-column operand scale exponents (emulate mode)
            if p == 0:
                ck[n, h] = S
            for c0, c1 in zip(cuts[:-1], cuts[1:]):
                sl = slice(bos + c0, bos + c1)
                want = ckpt_mode == "masked" and p is not None and c0 < p < c1
                res = chunk_step(S, q[sl, h], k[sl, h], v[sl, h], g[sl, h], beta[sl, h], scale,
                                 C_end=(p - c0) if want else None, emulate=emulate, recipe=recipe,
                                 sexp=sexp)
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


def _scan_bf16x3(T, S):
    """T S from bf16 hi + lo parts of both, the lo x lo product dropped
    (products exact, sums in fp32)."""
    Th = bf16(T); Tl = bf16(np.asarray(T, np.float32) - Th)
    Sh = bf16(S); Sl = bf16(np.asarray(S, np.float32) - Sh)
    f = lambda a, b: (np.asarray(a, np.float64) @ np.asarray(b, np.float64)).astype(np.float32)
    return f(Th, Sh) + f(Th, Sl) + f(Tl, Sh)


def prefill_chain(p, pieces, *, emulate=False, recipe=None, chunk=64, scan="fp32"):
    """The chain split of the two-launch schedule on a synth.Problem without
    checkpoints.  Each (sequence, head)'s chunks are cut into `pieces`
    ranges [floor(i n / P), floor((i + 1) n / P)); piece 0 runs from the
    initial state; pieces 1..P-2 run from a zero state (V as given: the
    affine part B_i) and from the identity with V = 0 (the transition T_i,
    a K x K matrix, as a K x V state with V = K columns); the incoming states
    follow from S_{i+1} = T_i S_i + B_i in the state's precision (scan
    "bf16x3": T_i S_i from bf16 hi + lo parts, the lo x lo term dropped); pieces
    1..P-1 run again from them with outputs.  Every run starts with fresh
    operand scale exponents, as each workgroup does.  Returns dict(out,
    final)."""
    assert p.ckpt_offsets is None
    dt = np.float32 if emulate else np.float64
    q, k, v = f32_from_bf16_bits(p.q), f32_from_bf16_bits(p.k), f32_from_bf16_bits(p.v)
    T, H, K = q.shape
    V = v.shape[2]
    cu = p.cu_seqlens
    out = np.zeros((T, H, V), dt)
    final = np.zeros((p.N, H, K, V), dt)

    def run(S, h, cuts, zero_v=False):
        sexp = np.zeros(S.shape[1])
        outs = []
        for c0, c1 in zip(cuts[:-1], cuts[1:]):
            vv = np.zeros((c1 - c0, S.shape[1]), np.float32) if zero_v else v[c0:c1, h]
            O, S, _ = chunk_step(S, q[c0:c1, h], k[c0:c1, h], vv, p.g[c0:c1, h], p.beta[c0:c1, h],
                                 p.scale, emulate=emulate, recipe=recipe, sexp=sexp)
            outs.append((c0, c1, O))
        return S.astype(dt), outs

    for n in range(p.N):
        bos, eos = int(cu[n]), int(cu[n + 1])
        bounds = list(range(bos, eos, chunk)) + [eos] if eos > bos else [bos]
        nseg = len(bounds) - 1
        piece_cuts = [bounds[(i * nseg) // pieces:((i + 1) * nseg) // pieces + 1] for i in range(pieces)]
        for h in range(H):
            S0 = np.zeros((K, V), dt) if p.initial_state is None else p.initial_state[n, h].astype(dt)
            S_in, _ = run(S0, h, piece_cuts[0])
            for i in range(1, pieces - 1):
                Ti, _ = run(np.eye(K, dtype=dt), h, piece_cuts[i], zero_v=True)
                Bi, _ = run(np.zeros((K, V), dt), h, piece_cuts[i])
                start = S_in
                TS = _scan_bf16x3(Ti, start) if scan == "bf16x3" else Ti @ start
                S_in = (TS + Bi).astype(dt)
                # outputs of piece i come from the run from its true state
                _, outs = run(start, h, piece_cuts[i])
                for c0, c1, O in outs:
                    out[c0:c1, h] = O
            if pieces == 1:
                _, outs = run(S0, h, piece_cuts[0])
                S_fin = S_in
            else:
                S_fin, outs = run(S_in, h, piece_cuts[-1])
                _, first = run(S0, h, piece_cuts[0])
                outs = outs + first
            for c0, c1, O in outs:
                out[c0:c1, h] = O
            final[n, h] = S_fin
    return {"out": out, "final": final}
