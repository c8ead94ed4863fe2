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


# the last shape is the size the decode bench line is measured at (1024
# requests x 12 heads, one token, a pool of 1100 entries)
@pytest.mark.parametrize("N,T,H,P,empty", [(1, 1, 1, 1, 0), (37, 1, 3, 50, 5), (8, 4, 12, 9, 1),
                                           (5, 7, 2, 5, 0), (256, 1, 12, 300, 16),
                                           (1024, 1, 12, 1100, 32)])
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


def _prefix(bits, N, T, t):
    """The first t tokens of each of N requests of T tokens (token-major rows)."""
    return np.ascontiguousarray(bits.reshape(N, T, *bits.shape[1:])[:, :t]).reshape(N * t, *bits.shape[1:])


# speculative verify: T draft tokens per request, pool only read, the state
# after every token in the trace; then a commit of each request's accepted
# prefix.  The last shape is the verify bench size (1024 requests x 4 drafts,
# a 3.2 GB trace).
@pytest.mark.parametrize("N,T,H,P,empty", [(1, 1, 1, 1, 0), (6, 4, 3, 9, 1), (37, 3, 2, 40, 4),
                                           (256, 4, 12, 300, 8), (1024, 4, 12, 1100, 16)])
def test_decode_verify_trace_and_commit(N, T, H, P, empty):
    import torch
    import kda_gated_delta_chunked_amd as K
    dev = torch.device("cuda", 0)
    p, pool, idx = _case(N, T, H, P, seed=170 + N + T, empty=empty)

    def bf16(bits):
        return torch.from_numpy(bits.view(np.int16).copy()).to(dev).view(torch.bfloat16)

    shp = (N, T, H, 128)
    q, k, v = bf16(p.q).view(shp), bf16(p.k).view(shp), bf16(p.v).view(shp)
    g = torch.from_numpy(p.g).to(dev).view(shp)
    beta = torch.from_numpy(p.beta).to(dev).view(N, T, H)
    didx = torch.from_numpy(idx).to(dev)
    vpool = torch.from_numpy(pool).to(dev)
    trace = torch.full((N, T, H, 128, 128), 7.0, dtype=torch.float32, device=dev)
    vout, _ = K.decode_verify(q, k, v, g, beta, vpool, didx, scale=p.scale, state_trace=trace)
    # the same tokens through kda_decode on a copy of the pool
    dpool = torch.from_numpy(pool).to(dev)
    dout = K.decode(q, k, v, g, beta, dpool, didx, scale=p.scale)
    torch.cuda.synchronize()
    what = f"N{N} T{T} H{H} P{P}"
    gtrace = trace.cpu().numpy()
    # the pool is only read; outputs and the last traced state are kda_decode's, bit for bit
    assert np.array_equal(vpool.cpu().numpy(), pool), what
    assert torch.equal(vout.view(torch.int16), dout.view(torch.int16)), what
    gdpool = dpool.cpu().numpy()
    named = [n for n in range(N) if 0 <= idx[n] < P]
    for n in range(N):
        if n in named:
            assert np.array_equal(gtrace[n, T - 1], gdpool[idx[n]]), (what, n)
        else:
            assert np.all(gtrace[n] == 7.0), (what, n)   # no state: trace rows untouched
    # outputs against the oracle (as kda_decode's), each traced state against
    # the oracle's decode of the first t + 1 tokens
    gout = vout.float().cpu().numpy().reshape(N * T, H, 128)
    _check(p, pool, idx, T, gout, gdpool, what)
    for t in range(T):
        ref = oracle.decode(_prefix(p.q, N, T, t + 1), _prefix(p.k, N, T, t + 1),
                            _prefix(p.v, N, T, t + 1), _prefix(p.g, N, T, t + 1),
                            _prefix(p.beta, N, T, t + 1), scale=p.scale, num_seqs=N,
                            tokens_per_seq=t + 1, state_pool=pool, state_indices=idx)
        if named:
            assert rel_l2(gtrace[named, t], ref["pool"][idx[named]]) <= POOL_REL_L2, (what, t)

    # commit: every accepted length from 0 (all drafts rejected) to T, and
    # values outside [0, T] that change nothing
    rng = np.random.default_rng(180 + N)
    acc = rng.integers(0, T + 1, N).astype(np.int32)
    acc[: min(N, 2)] = T
    if N > 3:
        acc[2], acc[3] = -1, T + 1
    vpool.copy_(torch.from_numpy(pool))
    K.decode_commit(vpool, didx, trace, torch.from_numpy(acc).to(dev))
    torch.cuda.synchronize()
    want = pool.copy()
    for n in named:
        if 1 <= acc[n] <= T:
            want[idx[n]] = gtrace[n, acc[n] - 1]
    assert np.array_equal(vpool.cpu().numpy(), want), what
    # accepting every draft leaves the pool as kda_decode does
    vpool.copy_(torch.from_numpy(pool))
    K.decode_commit(vpool, didx, trace, torch.full((N,), T, dtype=torch.int32, device=dev))
    torch.cuda.synchronize()
    assert np.array_equal(vpool.cpu().numpy(), gdpool), what
    # the recompute path: a verify with no trace gives the same outputs and
    # leaves the pool alone; an advance by the accepted counts then leaves the
    # pool as the commit of the traced states did, bit for bit
    npool = torch.from_numpy(pool).to(dev)
    nout, ntrace = K.decode_verify(q, k, v, g, beta, npool, didx, scale=p.scale, state_trace=False)
    torch.cuda.synchronize()
    assert ntrace is None
    assert torch.equal(nout.view(torch.int16), dout.view(torch.int16)), what
    assert np.array_equal(npool.cpu().numpy(), pool), what
    K.decode_advance(q, k, v, g, beta, npool, didx, torch.from_numpy(acc).to(dev), scale=p.scale)
    torch.cuda.synchronize()
    assert np.array_equal(npool.cpu().numpy(), want), what


def test_decode_verify_input_prologue():
    # raw q / k and beta logits through the verify: outputs and the last traced
    # state are kda_decode's with the same flags, bit for bit, and every traced
    # state meets the oracle's decode of that prefix with the prologue
    import torch
    import kda_gated_delta_chunked_amd as K
    from kda_gated_delta_chunked_amd.synth import bf16_bits_from_f32
    dev = torch.device("cuda", 0)
    N, T, H, P = 9, 3, 4, 12
    p, pool, idx = _case(N, T, H, P, seed=190, empty=2)
    rng = np.random.default_rng(191)
    p.q = bf16_bits_from_f32(rng.normal(0, 2.0, p.q.shape).astype(np.float32))
    p.k = bf16_bits_from_f32(rng.normal(0, 2.0, p.k.shape).astype(np.float32))
    p.beta = rng.normal(0, 1.5, p.beta.shape).astype(np.float32)

    def bf16(bits):
        return torch.from_numpy(bits.view(np.int16).copy()).to(dev).view(torch.bfloat16)

    shp = (N, T, H, 128)
    q, k, v = bf16(p.q).view(shp), bf16(p.k).view(shp), bf16(p.v).view(shp)
    g = torch.from_numpy(p.g).to(dev).view(shp)
    beta = torch.from_numpy(p.beta).to(dev).view(N, T, H)
    didx = torch.from_numpy(idx).to(dev)
    flags = dict(qk_l2norm=True, beta_logit=True)
    vpool = torch.from_numpy(pool).to(dev)
    vout, trace = K.decode_verify(q, k, v, g, beta, vpool, didx, scale=p.scale, **flags)
    dpool = torch.from_numpy(pool).to(dev)
    dout = K.decode(q, k, v, g, beta, dpool, didx, scale=p.scale, **flags)
    torch.cuda.synchronize()
    assert torch.equal(vout.view(torch.int16), dout.view(torch.int16))
    gtrace, gdpool = trace.cpu().numpy(), dpool.cpu().numpy()
    named = [n for n in range(N) if 0 <= idx[n] < P]
    for n in named:
        assert np.array_equal(gtrace[n, T - 1], gdpool[idx[n]]), n
    for t in range(T):
        ref = oracle.decode(_prefix(p.q, N, T, t + 1), _prefix(p.k, N, T, t + 1), _prefix(p.v, N, T, t + 1),
                            _prefix(p.g, N, T, t + 1), _prefix(p.beta, N, T, t + 1), scale=p.scale,
                            num_seqs=N, tokens_per_seq=t + 1, state_pool=pool, state_indices=idx, **flags)
        assert rel_l2(gtrace[named, t], ref["pool"][idx[named]]) <= POOL_REL_L2, t


@pytest.mark.parametrize("mode", ["trace", "recompute"])
def test_decode_verify_commit_graph_steps(mode):
    # one speculative step (verify, then commit of the traced states or advance
    # by recompute, of the accepted prefixes) captured in a HIP graph and replayed for three steps in a row on one pool,
    # with new drafts and new accepted lengths written into the captured
    # buffers each time and eager work between replays: every replay equals the
    # same two calls made eagerly, bit for bit, and the pool follows the oracle
    import torch
    import kda_gated_delta_chunked_amd as K
    dev = torch.device("cuda", 0)
    N, T, H, P = 16, 4, 3, 20
    rng = np.random.default_rng(200)
    pool0 = rng.normal(0, 0.05, (P, H, 128, 128)).astype(np.float32)
    idx = rng.permutation(P)[:N].astype(np.int32)
    idx[[3, 11]] = -1
    shp = (N, T, H, 128)

    def bf16(bits):
        return torch.from_numpy(bits.view(np.int16).copy()).to(dev).view(torch.bfloat16)

    steps = []
    for s in range(3):
        p = synth.make_problem([T] * N, H, seed=210 + s, fixed=True)
        acc = rng.integers(0, T + 1, N).astype(np.int32)
        acc[s] = T
        steps.append((p, acc))
    p0 = steps[0][0]
    q, k, v = bf16(p0.q).view(shp), bf16(p0.k).view(shp), bf16(p0.v).view(shp)
    g = torch.from_numpy(p0.g).to(dev).view(shp)
    beta = torch.from_numpy(p0.beta).to(dev).view(N, T, H)
    pool = torch.from_numpy(pool0).to(dev)
    didx = torch.from_numpy(idx).to(dev)
    acc_d = torch.from_numpy(steps[0][1]).to(dev)
    out = torch.empty(shp, dtype=torch.bfloat16, device=dev)
    trace = torch.empty((N, T, H, 128, 128), device=dev)

    def spec_step(stream):
        if mode == "trace":
            K.decode_verify(q, k, v, g, beta, pool, didx, scale=p0.scale, out=out, state_trace=trace,
                            stream=stream)
            K.decode_commit(pool, didx, trace, acc_d, stream=stream)
        else:
            K.decode_verify(q, k, v, g, beta, pool, didx, scale=p0.scale, out=out, state_trace=False,
                            stream=stream)
            K.decode_advance(q, k, v, g, beta, pool, didx, acc_d, scale=p0.scale, stream=stream)

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(dev)
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            spec_step(side)
    torch.cuda.synchronize()

    # the eager twin on its own buffers
    epool = torch.from_numpy(pool0).to(dev)
    cpu_pool = pool0.copy()
    for s, (p, acc) in enumerate(steps):
        q.copy_(bf16(p.q).view(shp)); k.copy_(bf16(p.k).view(shp)); v.copy_(bf16(p.v).view(shp))
        g.copy_(torch.from_numpy(p.g).view(shp)); beta.copy_(torch.from_numpy(p.beta).view(N, T, H))
        acc_d.copy_(torch.from_numpy(acc))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        if mode == "trace":
            eout, etrace = K.decode_verify(q, k, v, g, beta, epool, didx, scale=p.scale)
            K.decode_commit(epool, didx, etrace, acc_d)
        else:
            eout, _ = K.decode_verify(q, k, v, g, beta, epool, didx, scale=p.scale, state_trace=False)
            K.decode_advance(q, k, v, g, beta, epool, didx, acc_d, scale=p.scale)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eout.view(torch.int16)), s
        gpool = pool.cpu().numpy()
        assert np.array_equal(gpool, epool.cpu().numpy()), s
        # the oracle: each accepted prefix from the previous pool
        for n in range(N):
            if not (0 <= idx[n] < P) or acc[n] == 0:
                continue
            a = int(acc[n])
            sl = slice(n * T, n * T + a)
            ref = oracle.decode(p.q[sl], p.k[sl], p.v[sl], p.g[sl], p.beta[sl], scale=p.scale, num_seqs=1,
                                tokens_per_seq=a, state_pool=cpu_pool, state_indices=idx[n:n + 1])
            cpu_pool_n = ref["pool"][idx[n]]
            assert rel_l2(gpool[idx[n]], cpu_pool_n) <= POOL_REL_L2, (s, n)
        untouched = [i for i in range(P) if i not in {int(idx[n]) for n in range(N) if 0 <= idx[n] < P and acc[n] > 0}]
        assert np.array_equal(gpool[untouched], cpu_pool[untouched]), s
        cpu_pool = gpool.copy()
        _ = (q.float() * 2).sum().item()   # eager work between replays


# a bf16 pool: the stored state is rounded to bf16 once per call (7 fraction
# bits, nearest even: a relative RMS error of at most 2^-7 / sqrt(12) = 2.3e-3)
# on top of the fp32 token loop, so the pool is held to 3.5e-3, the bound the
# prefill's bf16 states use
BF16_POOL_REL_L2 = 3.5e-3


def _bf16_tensor(x, dev):
    import torch
    from kda_gated_delta_chunked_amd.synth import bf16_bits_from_f32
    return torch.from_numpy(bf16_bits_from_f32(np.ascontiguousarray(x, np.float32)).view(np.int16)).to(dev) \
        .view(torch.bfloat16)


@pytest.mark.parametrize("N,T,H,P,empty", [(37, 1, 3, 50, 5), (8, 4, 12, 9, 1), (1024, 1, 12, 1100, 32)])
def test_decode_bf16_pool(N, T, H, P, empty):
    import torch
    import kda_gated_delta_chunked_amd as K
    from kda_gated_delta_chunked_amd.synth import bf16_bits_from_f32, f32_from_bf16_bits
    dev = torch.device("cuda", 0)
    p, pool, idx = _case(N, T, H, P, seed=220 + N + T, empty=empty)
    pool_b = f32_from_bf16_bits(bf16_bits_from_f32(pool))     # the values a bf16 pool holds

    def bf16(bits):
        return torch.from_numpy(bits.view(np.int16).copy()).to(dev).view(torch.bfloat16)

    shp = (N, T, H, 128)
    q, k, v = bf16(p.q).view(shp), bf16(p.k).view(shp), bf16(p.v).view(shp)
    g = torch.from_numpy(p.g).to(dev).view(shp)
    beta = torch.from_numpy(p.beta).to(dev).view(N, T, H)
    dpool = _bf16_tensor(pool_b, dev)
    didx = torch.from_numpy(idx).to(dev)
    out = K.decode(q, k, v, g, beta, dpool, didx, scale=p.scale)
    torch.cuda.synchronize()
    gout = out.float().cpu().numpy().reshape(N * T, H, 128)
    gpool = dpool.float().cpu().numpy()
    ref = oracle.decode(p.q, p.k, p.v, p.g, p.beta, scale=p.scale, num_seqs=N, tokens_per_seq=T,
                        state_pool=pool_b, state_indices=idx)
    what = f"bf16 pool N{N} T{T} H{H} P{P}"
    assert np.all(np.isfinite(gout)), what
    assert float(np.max(np.abs(gout - ref["out"]))) <= OUT_MAX_ABS, what
    assert rel_l2(gout, ref["out"]) <= OUT_REL_L2, what
    named = sorted(set(int(i) for i in idx if 0 <= i < P))
    assert rel_l2(gpool[named], ref["pool"][named]) <= BF16_POOL_REL_L2, what
    others = [i for i in range(P) if i not in named]
    assert np.array_equal(gpool[others], pool_b[others]), what
    for n, i in enumerate(idx):
        if not (0 <= i < P):
            assert not np.any(gout[n * T:(n + 1) * T]), what


# the second shape is the bf16 verify bench size (1024 requests x 4 drafts)
@pytest.mark.parametrize("N,T,H,P,empty", [(37, 3, 2, 40, 4), (1024, 4, 12, 1100, 16)])
def test_decode_bf16_pool_speculative(N, T, H, P, empty):
    # the speculative paths on a bf16 pool (a bf16 trace): outputs and the
    # last traced state are kda_decode's bit for bit, a commit of every draft
    # leaves the pool as kda_decode does, and the advance equals the commit
    import torch
    import kda_gated_delta_chunked_amd as K
    from kda_gated_delta_chunked_amd.synth import bf16_bits_from_f32, f32_from_bf16_bits
    dev = torch.device("cuda", 0)
    p, pool, idx = _case(N, T, H, P, seed=230, empty=empty)
    pool_b = f32_from_bf16_bits(bf16_bits_from_f32(pool))

    def bf16(bits):
        return torch.from_numpy(bits.view(np.int16).copy()).to(dev).view(torch.bfloat16)

    shp = (N, T, H, 128)
    q, k, v = bf16(p.q).view(shp), bf16(p.k).view(shp), bf16(p.v).view(shp)
    g = torch.from_numpy(p.g).to(dev).view(shp)
    beta = torch.from_numpy(p.beta).to(dev).view(N, T, H)
    didx = torch.from_numpy(idx).to(dev)
    acc_h = np.random.default_rng(231).integers(0, T + 1, N).astype(np.int32)
    acc_h[0] = T
    acc = torch.from_numpy(acc_h).to(dev)
    vpool = _bf16_tensor(pool_b, dev)
    vout, trace = K.decode_verify(q, k, v, g, beta, vpool, didx, scale=p.scale)
    assert trace.dtype == torch.bfloat16
    dpool = _bf16_tensor(pool_b, dev)
    dout = K.decode(q, k, v, g, beta, dpool, didx, scale=p.scale)
    torch.cuda.synchronize()
    assert torch.equal(vout.view(torch.int16), dout.view(torch.int16))
    assert torch.equal(vpool.view(torch.int16), _bf16_tensor(pool_b, dev).view(torch.int16))
    named = [n for n in range(N) if 0 <= idx[n] < P]
    for n in named:
        assert torch.equal(trace[n, T - 1].view(torch.int16), dpool[int(idx[n])].view(torch.int16)), n
    # commit of every draft == kda_decode; commit of the accepted counts == advance
    cpool = _bf16_tensor(pool_b, dev)
    K.decode_commit(cpool, didx, trace, torch.full((N,), T, dtype=torch.int32, device=dev))
    apool, bpool = _bf16_tensor(pool_b, dev), _bf16_tensor(pool_b, dev)
    K.decode_commit(apool, didx, trace, acc)
    _, none = K.decode_verify(q, k, v, g, beta, bpool, didx, scale=p.scale, state_trace=False)
    K.decode_advance(q, k, v, g, beta, bpool, didx, acc, scale=p.scale)
    torch.cuda.synchronize()
    assert none is None
    assert torch.equal(cpool.view(torch.int16), dpool.view(torch.int16))
    assert torch.equal(apool.view(torch.int16), bpool.view(torch.int16))
    # and the advanced pool against the oracle's decode of each accepted prefix
    # (every 16th request at the large size)
    gpool = bpool.float().cpu().numpy()
    for n in (named if N <= 64 else named[::16]):
        a = int(acc_h[n])
        if a == 0:
            assert np.array_equal(gpool[idx[n]], pool_b[idx[n]]), n
            continue
        sl = slice(n * T, n * T + a)
        # a one-entry pool holding this request's state
        ref = oracle.decode(p.q[sl], p.k[sl], p.v[sl], p.g[sl], p.beta[sl], scale=p.scale, num_seqs=1,
                            tokens_per_seq=a, state_pool=pool_b[idx[n]:idx[n] + 1],
                            state_indices=np.zeros(1, np.int32))
        assert rel_l2(gpool[idx[n]], ref["pool"][0]) <= BF16_POOL_REL_L2, n
