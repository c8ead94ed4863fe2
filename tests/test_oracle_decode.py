"""Pins of the oracle's state-pool decode (``oracle.decode``).

The closed form of one token step, S' = (I - beta k k^T) Diag(exp(g)) S +
beta k v^T with o = scale S'^T q, is an algebraic identity of the token
recurrence (decay, delta-rule correction, read-out of the updated state); it
is written here with numpy in fp64, independently of the oracle's C loop, and
composed over the tokens of each request.  The pins also fix the pool
bookkeeping: which entry each request reads and writes, that unnamed entries
and empty request slots are left alone, and that empty slots give zeros."""
import numpy as np

import oracle
from kda_gated_delta_chunked_amd import synth


def _inputs(N, T, H, seed):
    p = synth.make_problem([T] * N, H, seed=seed, fixed=True)
    return p


def _closed_form(p, N, T, pool, idx, scale):
    pool = pool.astype(np.float64).copy()
    q = synth.f32_from_bf16_bits(p.q).astype(np.float64)
    k = synth.f32_from_bf16_bits(p.k).astype(np.float64)
    v = synth.f32_from_bf16_bits(p.v).astype(np.float64)
    g = p.g.astype(np.float64)
    beta = p.beta.astype(np.float64)
    H = p.H
    out = np.zeros(q.shape, np.float64)
    eye = np.eye(q.shape[2])
    for n in range(N):
        i = idx[n]
        if not (0 <= i < pool.shape[0]):
            continue
        for h in range(H):
            S = pool[i, h]
            for t in range(T):
                r = n * T + t
                kt, vt, qt, bt = k[r, h], v[r, h], q[r, h], beta[r, h]
                S = (eye - bt * np.outer(kt, kt)) @ (np.exp(g[r, h])[:, None] * S) + bt * np.outer(kt, vt)
                out[r, h] = scale * (S.T @ qt)
            pool[i, h] = S
    return out, pool


def test_decode_one_token_closed_form():
    N, T, H, P = 3, 1, 2, 5
    p = _inputs(N, T, H, seed=71)
    rng = np.random.default_rng(72)
    pool = rng.normal(0, 0.05, (P, H, 128, 128)).astype(np.float32)
    idx = np.array([3, -1, 0], np.int32)
    res = oracle.decode(p.q, p.k, p.v, p.g, p.beta, scale=p.scale, num_seqs=N, tokens_per_seq=T,
                        state_pool=pool, state_indices=idx)
    out, pool_ref = _closed_form(p, N, T, pool, idx, p.scale)
    assert np.allclose(res["out"], out, rtol=1e-12, atol=1e-13)
    assert np.allclose(res["pool"], pool_ref, rtol=1e-12, atol=1e-13)
    # entries no request names, and the empty slot's outputs
    for i in (1, 2, 4):
        assert np.array_equal(res["pool"][i], pool[i].astype(np.float64))
    assert not np.any(res["out"][1])


def test_decode_several_tokens_closed_form():
    N, T, H, P = 2, 4, 1, 3
    p = _inputs(N, T, H, seed=73)
    pool = np.random.default_rng(74).normal(0, 0.05, (P, H, 128, 128)).astype(np.float32)
    idx = np.array([2, 0], np.int32)
    res = oracle.decode(p.q, p.k, p.v, p.g, p.beta, scale=p.scale, num_seqs=N, tokens_per_seq=T,
                        state_pool=pool, state_indices=idx)
    out, pool_ref = _closed_form(p, N, T, pool, idx, p.scale)
    assert np.allclose(res["out"], out, rtol=1e-11, atol=1e-13)
    assert np.allclose(res["pool"], pool_ref, rtol=1e-11, atol=1e-13)
    assert np.array_equal(res["pool"][1], pool[1].astype(np.float64))


def test_decode_index_out_of_pool_is_an_empty_slot():
    N, T, H, P = 2, 1, 1, 2
    p = _inputs(N, T, H, seed=75)
    pool = np.random.default_rng(76).normal(0, 0.05, (P, H, 128, 128)).astype(np.float32)
    res = oracle.decode(p.q, p.k, p.v, p.g, p.beta, scale=p.scale, num_seqs=N, tokens_per_seq=T,
                        state_pool=pool, state_indices=np.array([2, -7], np.int32))
    assert not np.any(res["out"])
    assert np.array_equal(res["pool"], pool.astype(np.float64))
