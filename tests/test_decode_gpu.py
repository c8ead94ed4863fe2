"""State-pool decode on the GPU (kda_decode through the C ABI) against the
fp64 oracle's decode.

Tolerances: the decode runs token by token in fp32, so the state is held to
a relative L2 error of 1e-5 (a few fp32 roundings per token over 128-term
sums) and the outputs to the bf16 rounding of the store (half an ulp is
2^-9 relative: rel-L2 <= 5e-3, max-abs <= 2e-2 as for the prefill).  Pool
entries no request names stay bit for bit, empty request slots give zeros."""
import numpy as np
import pytest

import oracle
from gpu_helpers import rel_l2
from kda_gated_delta_chunked_amd import synth

pytestmark = pytest.mark.gpu

OUT_MAX_ABS = 2e-2
OUT_REL_L2 = 5e-3
POOL_REL_L2 = 1e-5


def _case(N, T, H, P, seed, empty=0, g_fill=None, beta_fill=None):
    p = synth.make_problem([T] * N, H, seed=seed, fixed=True)
    if g_fill is not None:
        p.g[...] = g_fill
    if beta_fill is not None:
        p.beta[...] = beta_fill
    rng = np.random.default_rng(seed + 1)
    pool = rng.normal(0, 0.05, (P, H, 128, 128)).astype(np.float32)
    idx = rng.permutation(P)[:N].astype(np.int32)
    if empty:
        idx[rng.choice(N, empty, replace=False)] = -1
    return p, pool, idx


def _run(p, pool, idx, T, out_alias_v=False, qk_l2norm=False, beta_logit=False):
    import torch
    import kda_gated_delta_chunked_amd as K
    dev = torch.device("cuda", 0)
    N, H = len(idx), p.H

    def bf16(bits):
        return torch.from_numpy(bits.view(np.int16).copy()).to(dev).view(torch.bfloat16)

    shp = (N, T, H, 128)
    q, k, v = bf16(p.q).view(shp), bf16(p.k).view(shp), bf16(p.v).view(shp)
    g = torch.from_numpy(p.g).to(dev).view(shp)
    beta = torch.from_numpy(p.beta).to(dev).view(N, T, H)
    dpool = torch.from_numpy(pool).to(dev)
    didx = torch.from_numpy(idx).to(dev)
    out = v if out_alias_v else torch.full(shp, float("nan"), dtype=torch.bfloat16, device=dev)
    K.decode(q, k, v, g, beta, dpool, didx, scale=p.scale, out=out, qk_l2norm=qk_l2norm,
             beta_logit=beta_logit)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().reshape(N * T, H, 128), dpool.cpu().numpy()


def _check(p, pool, idx, T, gout, gpool, what, **prologue):
    ref = oracle.decode(p.q, p.k, p.v, p.g, p.beta, scale=p.scale, num_seqs=len(idx),
                        tokens_per_seq=T, state_pool=pool, state_indices=idx, **prologue)
    assert np.all(np.isfinite(gout)), what
    err = float(np.max(np.abs(gout - ref["out"]))) if gout.size else 0.0
    assert err <= OUT_MAX_ABS, (what, err)
    if np.any(ref["out"]):
        assert rel_l2(gout, ref["out"]) <= OUT_REL_L2, what
    named = sorted(set(int(i) for i in idx if 0 <= i < pool.shape[0]))
    if named:
        assert rel_l2(gpool[named], ref["pool"][named]) <= POOL_REL_L2, what
    others = [i for i in range(pool.shape[0]) if i not in named]
    assert np.array_equal(gpool[others], pool[others]), what
    for n, i in enumerate(idx):
        if not (0 <= i < pool.shape[0]):
            assert not np.any(gout[n * T:(n + 1) * T]), what
    return ref


@pytest.mark.parametrize("N,T,H,P,empty", [(1, 1, 1, 1, 0), (37, 1, 3, 50, 5), (8, 4, 12, 9, 1),
                                           (5, 7, 2, 5, 0), (256, 1, 12, 300, 16)])
def test_decode_matches_oracle(N, T, H, P, empty):
    p, pool, idx = _case(N, T, H, P, seed=100 + N + T, empty=empty)
    gout, gpool = _run(p, pool, idx, T)
    _check(p, pool, idx, T, gout, gpool, f"N{N} T{T} H{H} P{P}")


def test_decode_gate_extremes_beta_zero_and_alias():
    for g_fill, beta_fill in ((-5.0, None), (0.0, None), (None, 0.0)):
        p, pool, idx = _case(6, 2, 2, 8, seed=131, g_fill=g_fill, beta_fill=beta_fill)
        gout, gpool = _run(p, pool, idx, 2, out_alias_v=True)
        _check(p, pool, idx, 2, gout, gpool, f"g={g_fill} beta={beta_fill}")


def test_decode_steps_in_a_row():
    # three serving steps on the same pool, the requests moving between entries
    rng = np.random.default_rng(140)
    P, H = 10, 2
    pool = rng.normal(0, 0.05, (P, H, 128, 128)).astype(np.float32)
    gpu_pool = pool.copy()
    for step in range(3):
        p = synth.make_problem([1] * 6, H, seed=141 + step, fixed=True)
        idx = rng.permutation(P)[:6].astype(np.int32)
        gout, gpool = _run(p, gpu_pool, idx, 1)
        ref = _check(p, gpu_pool, idx, 1, gout, gpool, f"step {step}")
        gpu_pool = gpool
        pool = ref["pool"].astype(np.float32)


def test_decode_equals_prefill_of_the_same_tokens():
    # a request advanced by T tokens from pool[i] matches the prefill of those
    # T tokens from the same initial state (different schedules, same function)
    from gpu_helpers import run_gpu
    N, T, H = 4, 64, 2
    p, pool, idx = _case(N, T, H, 6, seed=150)
    gout, gpool = _run(p, pool, idx, T)
    p.initial_state = pool[idx].copy()
    pre = run_gpu(p, variant="decomp")
    assert rel_l2(gout, pre["out"]) <= 2 * OUT_REL_L2
    assert rel_l2(gpool[idx], pre["final"]) <= 1e-3


def test_decode_input_prologue():
    from kda_gated_delta_chunked_amd.synth import bf16_bits_from_f32
    p, pool, idx = _case(9, 3, 4, 12, seed=160, empty=2)
    rng = np.random.default_rng(161)
    p.q = bf16_bits_from_f32(rng.normal(0, 2.0, p.q.shape).astype(np.float32))
    p.k = bf16_bits_from_f32(rng.normal(0, 2.0, p.k.shape).astype(np.float32))
    p.beta = rng.normal(0, 1.5, p.beta.shape).astype(np.float32)
    gout, gpool = _run(p, pool, idx, 3, qk_l2norm=True, beta_logit=True)
    _check(p, pool, idx, 3, gout, gpool, "decode prologue", qk_l2norm=True, beta_logit=True)
