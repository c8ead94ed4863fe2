"""Checks that pin the fp64 oracle to facts other than itself.

Each ``pin_*`` takes ``run`` -- a callable with the signature of
``oracle.prefill`` -- and raises AssertionError when the implementation behind
it disagrees with the fact the pin states.  The same pins run against the real
oracle (tests/test_oracle.py) and against copies of the oracle with planted
mistakes, which every pin set must reject.

What the facts are:

* a hand-worked three-token example at K = V = 2 (tests/golden/hand_k2v2.json);
* the dense per-step matrix form S_t = (I - b_t k_t k_t^T) Diag(e^{g_t}) S_{t-1}
  + b_t k_t v_t^T, built as explicit K x K matrices, and its unrolled
  closed form S_T = (A_T..A_1) S_0 + sum_t (A_T..A_{t+1}) b_t k_t v_t^T;
* invariants: with g = 0 and b = 0 nothing changes; with b = 0 the state only
  decays, row d by exp(sum_t g_{t,d}); with b = 1, g = 0 and standard-basis
  keys a write overwrites exactly that row with v; a repeated key with
  constant b and g = 0 turns its row into an exponential moving average; for
  unit keys and b in [0, 1] the state's Frobenius norm grows by at most b|v|
  per token;
* bookkeeping: packed sequences are independent of each other, fixed layout
  equals packed equal lengths, a zero-length sequence keeps its state, a
  checkpoint at offset p equals the final state of the length-p prefix run on
  its own, offsets outside [0, L] export nothing, and resuming from a
  checkpoint reproduces the rest of the run.
"""
from __future__ import annotations

import json
import os

import numpy as np

from kda_gated_delta_chunked_amd.synth import bf16_bits_from_f32, f32_from_bf16_bits

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rand_inputs(rng, T, H, K, V, *, unit=True, gmin=-5.0):
    q = rng.standard_normal((T, H, K)).astype(np.float32)
    k = rng.standard_normal((T, H, K)).astype(np.float32)
    if unit:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, V)).astype(np.float32)
    g = (gmin * rng.random((T, H, K))).astype(np.float32)
    beta = rng.random((T, H)).astype(np.float32)
    return bf16_bits_from_f32(q), bf16_bits_from_f32(k), bf16_bits_from_f32(v), g, beta


def _f64(bits):
    return f32_from_bf16_bits(bits).astype(np.float64)


def _dense_reference(q, k, v, g, beta, scale, s0):
    """Per-step dense matrices for one (sequence, head): returns outs, states."""
    K = q.shape[1]
    S = s0.astype(np.float64).copy()
    outs, states = [], []
    for t in range(q.shape[0]):
        kk = _f64(k[t])
        A = (np.eye(K) - float(beta[t]) * np.outer(kk, kk)) @ np.diag(np.exp(g[t].astype(np.float64)))
        S = A @ S + float(beta[t]) * np.outer(kk, _f64(v[t]))
        outs.append(scale * (S.T @ _f64(q[t])))
        states.append(S.copy())
    return np.array(outs), states


def _assert_close(a, b, rtol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    ref = max(np.max(np.abs(b)) if b.size else 0.0, 1e-300)
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    assert err <= rtol * ref, f"{what}: max err {err:.3e} vs scale {ref:.3e}"


def pin_hand_example(run):
    with open(os.path.join(GOLDEN, "hand_k2v2.json")) as f:
        gd = json.load(f)
    q = bf16_bits_from_f32(np.array(gd["q"], np.float32)[:, None, :])
    k = bf16_bits_from_f32(np.array(gd["k"], np.float32)[:, None, :])
    v = bf16_bits_from_f32(np.array(gd["v"], np.float32)[:, None, :])
    g = np.array(gd["g"], np.float32)[:, None, :]
    beta = np.array(gd["beta"], np.float32)[:, None]
    r = run(q, k, v, g, beta, scale=gd["scale"], num_seqs=1)
    np.testing.assert_allclose(r["out"][:, 0, :], gd["expected_out"], rtol=0, atol=1e-7)
    np.testing.assert_allclose(r["final"][0, 0], gd["expected_final"], rtol=0, atol=1e-7)
    for t, st in gd["expected_state_after"].items():
        r = run(q, k, v, g, beta, scale=gd["scale"], num_seqs=1,
                ckpt_offsets=np.array([int(t)], np.int32))
        np.testing.assert_allclose(r["ckpt"][0, 0], st, rtol=0, atol=1e-7)


def pin_dense_form(run):
    rng = np.random.default_rng(11)
    for (T, H, K, V) in [(7, 2, 4, 4), (5, 1, 128, 128), (9, 1, 3, 5)]:
        q, k, v, g, beta = _rand_inputs(rng, T, H, K, V)
        s0 = (0.5 * rng.standard_normal((1, H, K, V))).astype(np.float32)
        scale = 0.3
        r = run(q, k, v, g, beta, scale=scale, num_seqs=1, initial_state=s0)
        for h in range(H):
            outs, states = _dense_reference(q[:, h], k[:, h], v[:, h], g[:, h], beta[:, h], scale,
                                            s0[0, h])
            _assert_close(r["out"][:, h, :], outs, 1e-12, f"dense outputs T{T} K{K} V{V}")
            _assert_close(r["final"][0, h], states[-1], 1e-12, f"dense final T{T} K{K} V{V}")


def pin_closed_form(run):
    rng = np.random.default_rng(12)
    T, K, V = 8, 6, 4
    q, k, v, g, beta = _rand_inputs(rng, T, 1, K, V)
    s0 = rng.standard_normal((1, 1, K, V)).astype(np.float32)
    r = run(q, k, v, g, beta, scale=1.0, num_seqs=1, initial_state=s0)
    A = []
    for t in range(T):
        kk = _f64(k[t, 0])
        A.append((np.eye(K) - float(beta[t, 0]) * np.outer(kk, kk))
                 @ np.diag(np.exp(g[t, 0].astype(np.float64))))

    def prod(lo, hi):  # A_{hi-1} ... A_{lo}
        P = np.eye(K)
        for t in range(lo, hi):
            P = A[t] @ P
        return P

    expect = prod(0, T) @ s0[0, 0].astype(np.float64)
    for t in range(T):
        expect += prod(t + 1, T) @ (float(beta[t, 0]) * np.outer(_f64(k[t, 0]), _f64(v[t, 0])))
    _assert_close(r["final"][0, 0], expect, 1e-12, "closed-form final state")
    # scalar K = V = 1: s_t = (1 - b k^2) e^g s_{t-1} + b k v, o_t = scale s_t q
    qs, ks, vs, gs, bs = _rand_inputs(rng, 12, 1, 1, 1, unit=False)
    s0s = np.array([[[[0.7]]]], np.float32)
    r = run(qs, ks, vs, gs, bs, scale=2.0, num_seqs=1, initial_state=s0s)
    s = float(np.float32(0.7))
    for t in range(12):
        kk = float(_f64(ks[t, 0])[0])
        s = (1.0 - float(bs[t, 0]) * kk * kk) * np.exp(float(gs[t, 0, 0])) * s \
            + float(bs[t, 0]) * kk * float(_f64(vs[t, 0])[0])
        assert abs(r["out"][t, 0, 0] - 2.0 * s * float(_f64(qs[t, 0])[0])) <= 1e-12 * (1 + abs(s))
    assert abs(r["final"][0, 0, 0, 0] - s) <= 1e-12 * (1 + abs(s))


def pin_identity_and_decay(run):
    rng = np.random.default_rng(13)
    T, H, K, V = 10, 2, 8, 5
    q, k, v, _, _ = _rand_inputs(rng, T, H, K, V)
    s0 = rng.standard_normal((1, H, K, V)).astype(np.float32)
    zg = np.zeros((T, H, K), np.float32)
    zb = np.zeros((T, H), np.float32)
    r = run(q, k, v, zg, zb, scale=0.5, num_seqs=1, initial_state=s0)
    assert np.array_equal(r["final"][0], s0[0].astype(np.float64)), "g=0,b=0 must keep the state"
    for h in range(H):
        expect = 0.5 * _f64(q[:, h]) @ s0[0, h].astype(np.float64)
        _assert_close(r["out"][:, h, :], expect, 1e-14, "g=0,b=0 read-out")
    g = (-3.0 * rng.random((T, H, K))).astype(np.float32)
    r = run(q, k, v, g, zb, scale=0.5, num_seqs=1, initial_state=s0)
    G = np.cumsum(g.astype(np.float64), axis=0)
    for h in range(H):
        for t in range(T):
            St = np.exp(G[t, h])[:, None] * s0[0, h].astype(np.float64)
            _assert_close(r["out"][t, h], 0.5 * St.T @ _f64(q[t, h]), 1e-12, "pure-decay read-out")
        _assert_close(r["final"][0, h], np.exp(G[-1, h])[:, None] * s0[0, h], 1e-12,
                      "pure decay, row d scaled by exp(sum g_d)")


def pin_overwrite(run):
    rng = np.random.default_rng(14)
    K = V = 16
    order = rng.permutation(K)[:10]
    T = len(order)
    k = np.zeros((T, 1, K), np.float32)
    k[np.arange(T), 0, order] = 1.0
    q = k.copy()
    v = rng.standard_normal((T, 1, V)).astype(np.float32)
    kb, qb, vb = bf16_bits_from_f32(k), bf16_bits_from_f32(q), bf16_bits_from_f32(v)
    s0 = rng.standard_normal((1, 1, K, V)).astype(np.float32)
    r = run(qb, kb, vb, np.zeros((T, 1, K), np.float32), np.ones((T, 1), np.float32),
            scale=1.0, num_seqs=1, initial_state=s0)
    vv = f32_from_bf16_bits(vb).astype(np.float64)
    expect = s0[0, 0].astype(np.float64).copy()
    for t, i in enumerate(order):
        expect[i] = vv[t, 0]
        assert np.array_equal(r["out"][t, 0], vv[t, 0]), "reading a just-written key returns its value"
    assert np.array_equal(r["final"][0, 0], expect), "b=1 with orthonormal keys overwrites rows exactly"


def pin_ema(run):
    rng = np.random.default_rng(15)
    T, K, V, b = 9, 4, 3, 0.25
    k = np.zeros((T, 1, K), np.float32)
    k[:, 0, 2] = 1.0
    v = rng.standard_normal((T, 1, V)).astype(np.float32)
    q = bf16_bits_from_f32(k)
    s0 = rng.standard_normal((1, 1, K, V)).astype(np.float32)
    r = run(q, bf16_bits_from_f32(k), bf16_bits_from_f32(v), np.zeros((T, 1, K), np.float32),
            np.full((T, 1), b, np.float32), scale=1.0, num_seqs=1, initial_state=s0)
    vv = f32_from_bf16_bits(bf16_bits_from_f32(v)).astype(np.float64)[:, 0]
    row = (1 - b) ** T * s0[0, 0, 2].astype(np.float64)
    for t in range(T):
        row = row + b * (1 - b) ** (T - 1 - t) * vv[t]
    _assert_close(r["final"][0, 0, 2], row, 1e-13, "repeated key: exponential moving average")
    others = [0, 1, 3]
    assert np.array_equal(r["final"][0, 0, others], s0[0, 0, others].astype(np.float64))


def pin_norm_growth(run):
    rng = np.random.default_rng(16)
    T, K, V = 12, 32, 32
    q, k, v, g, beta = _rand_inputs(rng, T, 1, K, V, gmin=-0.5)
    s0 = rng.standard_normal((1, 1, K, V)).astype(np.float32)
    prev = np.linalg.norm(s0[0, 0].astype(np.float64))
    vv = f32_from_bf16_bits(v).astype(np.float64)
    for t in range(1, T + 1):
        r = run(q, k, v, g, beta, scale=1.0, num_seqs=1, initial_state=s0,
                ckpt_offsets=np.array([t], np.int32))
        cur = np.linalg.norm(r["ckpt"][0, 0])
        bound = prev + float(beta[t - 1, 0]) * np.linalg.norm(vv[t - 1, 0])
        assert cur <= bound * (1 + 1e-2), f"norm grew past the bound at t={t}"
        prev = cur


def pin_bookkeeping(run):
    rng = np.random.default_rng(17)
    H, K, V = 2, 8, 8
    lens = [5, 0, 9, 1, 0, 7]
    T = sum(lens)
    q, k, v, g, beta = _rand_inputs(rng, T, H, K, V)
    N = len(lens)
    cu = np.zeros(N + 1, np.int32)
    cu[1:] = np.cumsum(lens)
    s0 = rng.standard_normal((N, H, K, V)).astype(np.float32)
    r = run(q, k, v, g, beta, scale=0.7, num_seqs=N, cu_seqlens=cu, initial_state=s0)
    for n, L in enumerate(lens):
        a, b = cu[n], cu[n + 1]
        if L == 0:
            assert np.array_equal(r["final"][n], s0[n].astype(np.float64)), "empty sequence keeps S0"
            continue
        one = run(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b], scale=0.7, num_seqs=1,
                  initial_state=s0[n:n + 1])
        assert np.array_equal(one["out"], r["out"][a:b]), "packed sequences must be independent"
        assert np.array_equal(one["final"][0], r["final"][n])
    # fixed layout == packed equal lengths
    T2 = 12
    q, k, v, g, beta = _rand_inputs(rng, 3 * T2, H, K, V)
    s0 = rng.standard_normal((3, H, K, V)).astype(np.float32)
    rf = run(q, k, v, g, beta, scale=0.7, num_seqs=3, initial_state=s0)
    rp = run(q, k, v, g, beta, scale=0.7, num_seqs=3, initial_state=s0,
             cu_seqlens=np.array([0, T2, 2 * T2, 3 * T2], np.int32))
    assert np.array_equal(rf["out"], rp["out"]) and np.array_equal(rf["final"], rp["final"])
    # a fixed batch is not one long sequence
    r1 = run(q, k, v, g, beta, scale=0.7, num_seqs=1, initial_state=s0[:1])
    assert not np.allclose(r1["out"][T2:], rf["out"][T2:])


def pin_checkpoints(run):
    rng = np.random.default_rng(18)
    H, K, V = 2, 8, 6
    lens = [11, 4, 9]
    N = len(lens)
    T = sum(lens)
    q, k, v, g, beta = _rand_inputs(rng, T, H, K, V)
    cu = np.zeros(N + 1, np.int32)
    cu[1:] = np.cumsum(lens)
    s0 = rng.standard_normal((N, H, K, V)).astype(np.float32)
    for offs in ([0, 4, 9], [5, 0, 1], [11, 3, 8], [10, 2, 0]):
        offs = np.array(offs, np.int32)
        r = run(q, k, v, g, beta, scale=0.4, num_seqs=N, cu_seqlens=cu, initial_state=s0,
                ckpt_offsets=offs)
        for n in range(N):
            p = int(offs[n])
            a = int(cu[n])
            if p == 0:
                assert np.array_equal(r["ckpt"][n], s0[n].astype(np.float64)), "offset 0 exports S0"
                continue
            pre = run(q[a:a + p], k[a:a + p], v[a:a + p], g[a:a + p], beta[a:a + p], scale=0.4,
                      num_seqs=1, initial_state=s0[n:n + 1])
            assert np.array_equal(pre["final"][0], r["ckpt"][n]), \
                f"checkpoint at offset {p} must be the state after {p} tokens"
            if p == lens[n]:
                assert np.array_equal(r["ckpt"][n], r["final"][n])
    # out-of-range offsets export nothing
    r = run(q, k, v, g, beta, scale=0.4, num_seqs=N, cu_seqlens=cu, initial_state=s0,
            ckpt_offsets=np.array([-1, 5, 3], np.int32))
    assert np.all(np.isnan(r["ckpt"][0])) and np.all(np.isnan(r["ckpt"][1]))
    assert not np.any(np.isnan(r["ckpt"][2]))
    # resume from a checkpoint reproduces the suffix
    p = 6
    full = run(q[:11], k[:11], v[:11], g[:11], beta[:11], scale=0.4, num_seqs=1,
               initial_state=s0[:1], ckpt_offsets=np.array([p], np.int32))
    rest = run(q[p:11], k[p:11], v[p:11], g[p:11], beta[p:11], scale=0.4, num_seqs=1,
               initial_state=full["ckpt"].astype(np.float32))
    _assert_close(rest["out"], full["out"][p:11], 1e-6, "resume outputs")
    _assert_close(rest["final"], full["final"], 1e-6, "resume final state")


ALL_PINS = [pin_hand_example, pin_dense_form, pin_closed_form, pin_identity_and_decay,
            pin_overwrite, pin_ema, pin_norm_growth, pin_bookkeeping, pin_checkpoints]
