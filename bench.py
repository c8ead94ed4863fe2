#!/usr/bin/env python3
"""Benchmark: KDA multi-token recurrent prefill on one MI355X.

One step is one ``kda_prefill`` call -- the whole hot path (gate cumsum,
gated K K^T / Q K^T, triangular solve, chunk recurrence, outputs, final
state) -- over the B8 T8192 H12 K=V=128 bf16 workload with an fp32 initial
state, inputs resident in HBM before timing starts.  Prints one JSON line.
With the two-launch schedule, each launch is also timed on its own (the
library's split-stage calls) for the roofline of the dominant kernel.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

The default warm-up is 100 steps (about 60 ms of work at B8 T8192): after an
idle spell the GPU runs the first 30 ms or so about 4.5% slower (measured in
blocks of 50 calls: 0.578-0.582 ms per call in the block after a 50 ms pause,
0.553 ms in the blocks that follow it), so a shorter warm-up times part of
that ramp.  The per-call timing blocks each start with 20 untimed calls for
the same reason.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefill tokens/sec and ms/call, H=12 K=V=128 bf16 at B8 T8192; MFMA util %"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, vendor figure
MFMA_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 / fp16 matrix, vendor figure
# Context only (another vendor's part, no initial state): FlashInfer PR #4633,
# Performance, gives 0.881 ms for this shape on a 110-SM SM120 device.  The
# stated baseline of this bench is the fp64 oracle (cpu_baseline).
PAGES_CONTEXT = {"source": "FlashInfer PR #4633, Performance (110-SM SM120, BF16, no initial state)",
                 "ms": 0.881}
CSRC = os.path.join(ROOT, "kda_gated_delta_chunked_amd", "csrc")
KERNEL_SOURCES = {"fused": os.path.join(CSRC, "kda_fused.hip"), "decomp": os.path.join(CSRC, "kda_decomp.hip"),
                  "decode": os.path.join(CSRC, "kda_decode.hip")}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
MFMA_FLOPS = 16 * 16 * 32 * 2    # one v_mfma_f32_16x16x32_f16 or _bf16
MFMA_F32_FLOPS = 16 * 16 * 4 * 2  # one v_mfma_f32_16x16x4_f32


def stage_bytes(p):
    """Algorithmic HBM bytes of each launch of the two-launch schedule: the
    prepare reads q, k (bf16), g (fp32) and beta; the recurrence reads v and
    the initial state and writes out, the final state and checkpoints."""
    th = p.T_total * p.H
    state = 128 * 128 * 4 * p.N * p.H
    n_states = (1 if p.initial_state is not None else 0) + 1 + (1 if p.ckpt_offsets is not None else 0)
    return {"prepare": th * (128 * 2 * 2 + 128 * 4 + 4),
            "recurrence": th * (128 * 2 * 2) + state * n_states}


def algorithmic_bytes(p) -> int:
    """HBM bytes the method must move: q, k, v (bf16), g (fp32), beta (fp32)
    in, out (bf16) written, the fp32 state read and written per (sequence,
    head), and checkpoint states written."""
    return sum(stage_bytes(p).values())


def algorithmic_flops(p) -> float:
    """Matrix flops of the chunked form per token-head (C = 64): state read
    for X and O and the state update (3 K V), the in-chunk K K^T / Q K^T and
    M U / N Y products (C (3K + 2V) / 2), and the C^2/6 solve."""
    C, K, V = 64, 128, 128
    per = 2 * (3 * K * V + C * (3 * K + 2 * V) / 2 + C * C / 6)
    return float(per) * p.T_total * p.H


def segments(p) -> int:
    """Segments the kernels process: the 64-token chunks of every sequence,
    plus one for each distinct honoured checkpoint offset strictly inside a
    chunk (offsets are taken in order; one is honoured when it lies in
    [0, L] and is not below the previous honoured one)."""
    segs = 0
    offs = None if p.ckpt_offsets is None else np.asarray(p.ckpt_offsets).reshape(p.N, -1)
    for n in range(p.N):
        L = int(p.cu_seqlens[n + 1] - p.cu_seqlens[n])
        cuts, last = set(), 0
        for x in ([] if offs is None else [int(v) for v in offs[n]]):
            if x < last or x > L:
                continue
            last = x
            if 0 < x < L and x % 64 != 0:
                cuts.add(x)
        segs += (L + 63) // 64 + len(cuts)
    return segs


def modelled_mfma_flops(p, variant: str, vsplit: int) -> float:
    """Flops of the MFMA instructions the kernels issue (hi/lo passes
    included), counted from their schedules (a model: the committed rocprofv3
    SQ counters give the measured figure).  Per segment and head:
    * FUSED, per workgroup: 156 for the gate products (4 diagonal blocks x 4
      key blocks x 6, 6 blocks left of them x 4 x 2) and the solve merges
      (12), plus 76 per 16-column tile of the recurrence;
    * DECOMP: the prepare's 176 (4 diagonal blocks x 4 x 6, 6 off-diagonal
      x 4 x 2, 32 transposes of K^) and the recurrence's 76 per 16 columns,
      8 column tiles per (sequence, head).  The recurrence's 76: K~ S 16,
      Q~ S 16, N Y 6, M U 6, K^^T U with U hi + lo 32.  The prepare also
      issues 76 fp32 16x16x4 products (2,048 flops each) for the block
      inverse of T: 16 for its 32 x 32 halves, 60 for the lower-left quarter."""
    segs = segments(p)
    if variant == "fused":
        return float((156 + 76 * (128 // vsplit // 16)) * MFMA_FLOPS) * segs * p.H * vsplit
    return (float((176 + 8 * 76) * MFMA_FLOPS) + 76.0 * MFMA_F32_FLOPS) * segs * p.H


# headers every kernel source includes: a change there changes the kernel too
KERNEL_HEADERS = [os.path.join(CSRC, "kda_kernels.h"), os.path.join(CSRC, "kda_ckpt.h")]


def kernel_sha(variant: str) -> str:
    """SHA-256 of the kernel source followed by the shared headers."""
    h = hashlib.sha256()
    for path in [KERNEL_SOURCES[variant]] + KERNEL_HEADERS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_counters(workload: str, variant: str, kernel: str) -> dict:
    """Per-launch figures of `kernel` from the committed rocprofv3 --pmc
    summary (HBM bytes, MFMA busy fraction, MFMA flops), if they were taken on
    the current kernel source; else {}."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return {}
    e = t.get(workload, {}).get(kernel)
    if not e or e.get("source_sha256") != kernel_sha(variant):
        return {}
    return e


def measured_traffic(workload: str, variant: str, kernel: str):
    """HBM bytes per launch of `kernel` from the committed counters, or None."""
    return measured_counters(workload, variant, kernel).get("hbm_bytes_per_launch")


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(p, sample_tokens: int):
    """Time the fp64 oracle (as it stands) on the first `sample_tokens` tokens
    of every sequence of the workload, all heads, on all host cores."""
    import oracle
    oracle.build()
    idx = np.concatenate([np.arange(p.cu_seqlens[n], p.cu_seqlens[n] + min(sample_tokens,
                          p.cu_seqlens[n + 1] - p.cu_seqlens[n])) for n in range(p.N)])
    lens = [min(sample_tokens, int(p.cu_seqlens[n + 1] - p.cu_seqlens[n])) for n in range(p.N)]
    cu = np.zeros(p.N + 1, np.int32)
    cu[1:] = np.cumsum(lens)
    threads = oracle.default_threads()
    t0 = time.perf_counter()
    oracle.prefill(p.q[idx], p.k[idx], p.v[idx], p.g[idx], p.beta[idx], scale=p.scale,
                   num_seqs=p.N, cu_seqlens=cu, initial_state=p.initial_state, threads=threads)
    dt = time.perf_counter() - t0
    # one core: the first sequence of the sample, one head
    L0 = lens[0]
    sl = slice(0, L0)
    t1 = time.perf_counter()
    oracle.prefill(p.q[idx][sl, :1], p.k[idx][sl, :1], p.v[idx][sl, :1], p.g[idx][sl, :1],
                   p.beta[idx][sl, :1], scale=p.scale, num_seqs=1,
                   cu_seqlens=np.array([0, L0], np.int32),
                   initial_state=None if p.initial_state is None else p.initial_state[:1, :1],
                   threads=1)
    dt1 = time.perf_counter() - t1
    return {"value": float(cu[-1]) / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {sample_tokens} tokens of each of the {p.N} sequences, all {p.H} "
                      f"heads ({int(cu[-1]) * p.H} token-heads), fp64 token recurrence, "
                      f"{dt:.2f} s wall",
            "one_core_token_heads_per_s": round(L0 / dt1, 1), "cpu_model": _cpu_model()}


def bench_decode(args, torch, K, synth) -> int:
    """State-pool decode: N requests x T tokens, H = 12, one pool entry per
    request (a permutation), inputs resident.  HBM-bound: each (request, head)
    reads and writes its 64 KiB fp32 state once per call, plus 1,540 B per
    token-head of q, k, v, g, beta and out."""
    N, T = (int(x) for x in args.decode.split(","))
    H = 12
    dev = torch.device("cuda", 0)
    p = synth.make_problem([T] * N, H, seed=2000 + N + T, fixed=True)
    shp = (N, T, H, 128)

    def bf16(bits):
        return torch.from_numpy(bits.view(np.int16).copy()).to(dev).view(torch.bfloat16).view(shp)

    q, k, v = bf16(p.q), bf16(p.k), bf16(p.v)
    g = torch.from_numpy(p.g).to(dev).view(shp)
    beta = torch.from_numpy(p.beta).to(dev).view(N, T, H)
    rng = np.random.default_rng(2001)
    sdt = args.decode_state
    pool = torch.from_numpy(rng.normal(0, 0.02, (N, H, 128, 128)).astype(np.float32)).to(dev)
    if sdt == "bf16":
        pool = pool.to(torch.bfloat16)
    idx = torch.from_numpy(rng.permutation(N).astype(np.int32)).to(dev)
    out = torch.empty_like(v)
    stream = torch.cuda.current_stream(dev)
    prob = K.make_decode_problem(N, T, H, N, scale=p.scale, state_dtype=sdt)

    def step():
        st = K.decode_raw(prob, q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(),
                          beta.data_ptr(), pool.data_ptr(), idx.data_ptr(), out.data_ptr(),
                          stream.cuda_stream)
        if st != 0:
            raise K.KDAError(st, "kda_decode")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    ms = [a.elapsed_time(b) for a, b in zip(starts, ends)]
    ms_kernel = float(np.median(ms))
    es = 2 if sdt == "bf16" else 4
    alg = N * H * (2 * 128 * 128 * es) + N * T * H * (128 * 2 * 4 + 128 * 4 + 4)
    achieved = alg / (ms_kernel * 1e-3) / 1e9
    workload = f"decode_n{N}_t{T}" + ("_bf16" if sdt == "bf16" else "")
    res = {"metric": f"state-pool decode tokens/s (H=12, K=V=128, {sdt} state)",
           "value": round(N * T / (ms_step * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp32",
           "data": "synthetic",
           "config": {"workload": workload, "requests": N, "tokens_per_request": T,
                      "H": H, "pool_size": N, "state_dtype": sdt},
           "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                        "traffic": measured_traffic(workload, "decode", "kda_decode_kernel"),
                        "kernel": "kda_decode_kernel", "kernel_ms": round(ms_kernel, 4),
                        "algorithmic_bytes": alg}}
    print(json.dumps(res), flush=True)
    return 0


def bench_verify(args, torch, K, synth) -> int:
    """One speculative step for N requests x T draft tokens, H = 12: the verify
    (outputs for every draft, the pool only read), then the pool keeps each
    request's accepted prefix (seeded accepted counts in [0, T]), two ways:
    the verify stores every intermediate state and a commit copies the
    accepted one (trace), or the verify stores none and an advance recomputes
    the accepted prefix (recompute).  Inputs resident; `value` is the
    recompute path's draft tokens per second."""
    N, T = (int(x) for x in args.verify.split(","))
    H = 12
    dev = torch.device("cuda", 0)
    p = synth.make_problem([T] * N, H, seed=3000 + N + T, fixed=True)
    shp = (N, T, H, 128)

    def bf16(bits):
        return torch.from_numpy(bits.view(np.int16).copy()).to(dev).view(torch.bfloat16).view(shp)

    q, k, v = bf16(p.q), bf16(p.k), bf16(p.v)
    g = torch.from_numpy(p.g).to(dev).view(shp)
    beta = torch.from_numpy(p.beta).to(dev).view(N, T, H)
    rng = np.random.default_rng(3001)
    sdt = args.decode_state
    pool = torch.from_numpy(rng.normal(0, 0.02, (N, H, 128, 128)).astype(np.float32)).to(dev)
    if sdt == "bf16":
        pool = pool.to(torch.bfloat16)
    idx = torch.from_numpy(rng.permutation(N).astype(np.int32)).to(dev)
    acc_h = rng.integers(0, T + 1, N).astype(np.int32)
    acc = torch.from_numpy(acc_h).to(dev)
    out = torch.empty_like(v)
    trace = torch.empty((N, T, H, 128, 128), dtype=pool.dtype, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step_trace():
        K.decode_verify(q, k, v, g, beta, pool, idx, scale=p.scale, out=out, state_trace=trace, stream=stream)
        K.decode_commit(pool, idx, trace, acc, stream=stream)

    def step_recompute():
        K.decode_verify(q, k, v, g, beta, pool, idx, scale=p.scale, out=out, state_trace=False, stream=stream)
        K.decode_advance(q, k, v, g, beta, pool, idx, acc, scale=p.scale, stream=stream)

    def timed(step):
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / args.steps

    ms_trace = timed(step_trace)
    ms_re = timed(step_recompute)
    state = 128 * 128 * (2 if sdt == "bf16" else 4)
    taken = int(acc_h.sum())
    tok_in = 128 * 2 * 3 + 128 * 4 + 4          # q, k, v, g, beta per token-head
    # recompute: the verify reads every state, the inputs and writes the
    # outputs; the advance reads and writes the states of requests that took a
    # draft, with the inputs of the drafts taken
    alg = N * H * state + N * T * H * (tok_in + 256) + int((acc_h > 0).sum()) * H * 2 * state + taken * H * tok_in
    res = {"metric": f"speculative verify step draft tokens/s (H=12, K=V=128, {sdt} state)",
           "value": round(N * T / (ms_re * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_re, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp32",
           "data": "synthetic",
           "config": {"workload": f"verify_n{N}_t{T}" + ("_bf16" if sdt == "bf16" else ""), "requests": N,
                      "drafts_per_request": T, "H": H, "pool_size": N, "state_dtype": sdt,
                      "accepted_mean": round(float(acc_h.mean()), 3)},
           "paths": {"recompute_ms_per_step": round(ms_re, 4), "trace_ms_per_step": round(ms_trace, 4),
                     "trace_bytes": N * T * H * state},
           "roofline": {"bound": "hbm", "achieved": round(alg / (ms_re * 1e-3) / 1e9, 1),
                        "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(alg / (ms_re * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "traffic": None,
                        "kernel": "kda_decode_kernel (verify + advance)", "algorithmic_bytes": alg}}
    print(json.dumps(res), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="b8_t8192")
    ap.add_argument("--value-split", type=int, default=0, help="0 = library's choice")
    ap.add_argument("--chain-parts", type=int, default=0,
                    help="pieces of each (sequence, head)'s recurrence; 0 = library's choice")
    ap.add_argument("--variant", default="auto", choices=["auto", "decomp", "fused"])
    ap.add_argument("--cpu-sample-tokens", type=int, default=8192)
    ap.add_argument("--timing-calls", type=int, default=50,
                    help="calls per block for the median, cold-cache and graph-replay timings")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode", default="", metavar="N,T",
                    help="instead of the prefill, time the state-pool decode of N requests "
                         "advancing T tokens each (H = 12, pool of N states)")
    ap.add_argument("--verify", default="", metavar="N,T",
                    help="instead of the prefill, time a speculative step of N requests with T draft "
                         "tokens each (verify, then commit of the traced states or advance by "
                         "recompute; H = 12, pool of N states)")
    ap.add_argument("--decode-state", default="fp32", choices=("fp32", "bf16"),
                    help="state pool element type of --decode and --verify")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES, --steps times "
                         "(reference for the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this path runs per (sequence, head) on a single "
              f"MI355X and has no multi-GPU mode (asked for --gpus {args.gpus}).", file=sys.stderr)
        return 2

    import torch
    import kda_gated_delta_chunked_amd as K
    from kda_gated_delta_chunked_amd import synth

    if args.copy_calibration:
        n = args.copy_calibration // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n * 4, "steps": args.steps}), flush=True)
        return 0

    if args.decode:
        return bench_decode(args, torch, K, synth)
    if args.verify:
        return bench_verify(args, torch, K, synth)

    p = synth.workload(args.workload)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    def bf16(bits):
        return torch.from_numpy(bits.view(np.int16).copy()).to(dev).view(torch.bfloat16)

    q, k, v = bf16(p.q), bf16(p.k), bf16(p.v)
    g = torch.from_numpy(p.g).to(dev)
    beta = torch.from_numpy(p.beta).to(dev)
    cu = None if p.fixed else torch.from_numpy(p.cu_seqlens).to(dev)
    s0 = None if p.initial_state is None else torch.from_numpy(p.initial_state).to(dev)
    offs = None if p.ckpt_offsets is None else torch.from_numpy(p.ckpt_offsets).to(dev)
    out = torch.empty_like(v)
    fin = torch.empty((p.N, p.H, 128, 128), dtype=torch.float32, device=dev)
    ck = None if offs is None else torch.empty_like(fin)
    prob = K.make_problem(p.N, p.T_total, p.H, scale=p.scale, variant=args.variant,
                          value_split=args.value_split, chain_parts=args.chain_parts)
    variant, vsplit, pieces = K.plan(prob)
    ws_bytes = K.workspace_size(prob)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    stream = torch.cuda.current_stream(dev)

    def ptr(t):
        return 0 if t is None else t.data_ptr()

    def step():
        st = K.prefill_raw(prob, ptr(q), ptr(k), ptr(v), ptr(g), ptr(beta), ptr(cu), ptr(s0),
                           ptr(out), ptr(fin), ptr(offs), ptr(ck), ptr(ws), ws_bytes, stream.cuda_stream)
        if st != 0:
            raise K.KDAError(st, "kda_prefill")

    def timed(fn, steps):
        """Per-launch milliseconds from events on the call's stream, and wall ms per step."""
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            starts[i].record(stream)
            fn()
            ends[i].record(stream)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3 / steps
        return float(np.mean([a.elapsed_time(b) for a, b in zip(starts, ends)])), wall

    def per_call(fn, calls, before=None, lead=20):
        """Event-timed milliseconds of each of `calls` calls of fn (optionally
        preceded, outside the events, by `before`), after `lead` untimed
        calls."""
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(calls)]
        for _ in range(lead):
            fn()
        for a, b in ev:
            if before is not None:
                before()
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in ev]

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the timed region: exactly `steps` calls, bracketed by synchronisations,
    # with nothing else enqueued between them
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    # per-call time from events on the call's stream, in a separate pass
    ms_launch = timed(step, args.steps)[0]
    tokens = p.T_total
    value = tokens / (ms_step * 1e-3)

    # medians of two independent blocks of calls (warm), the same with 1 GiB
    # written between calls (the 256 MiB Infinity Cache then holds none of the
    # inputs), and a captured HIP graph of one call replayed
    timing = {"warm_median_ms": [round(float(np.median(per_call(step, args.timing_calls))), 4)
                                 for _ in range(2)]}
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    timing["cold_median_ms"] = round(float(np.median(
        per_call(step, max(10, args.timing_calls // 5), before=lambda: flush.fill_(1.0)))), 4)
    del flush
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(dev)
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            rc = K.prefill_raw(prob, ptr(q), ptr(k), ptr(v), ptr(g), ptr(beta), ptr(cu), ptr(s0),
                               ptr(out), ptr(fin), ptr(offs), ptr(ck), ptr(ws), ws_bytes,
                               torch.cuda.current_stream(dev).cuda_stream)
    torch.cuda.synchronize()
    if rc != 0:
        raise K.KDAError(rc, "kda_prefill (capture)")
    graph.replay()
    torch.cuda.synchronize()
    timing["graph_replay_median_ms"] = round(float(np.median(per_call(graph.replay, args.timing_calls))), 4)
    del graph

    # per-kernel times: the two launches of DECOMP enqueued by separate calls
    kernels = {}
    if variant == "decomp":
        for st, kname in (("prepare", "kda_prepare_kernel"), ("recurrence", "kda_recurrence_kernel")):
            # the call's own value split when none is given: with a chain
            # split the library may run its first launch with fewer
            # workgroups per pair than the plan reports
            sprob = K.make_problem(p.N, p.T_total, p.H, scale=p.scale, variant="decomp",
                                   value_split=args.value_split, stages=st, chain_parts=pieces)

            def one(sprob=sprob):
                rc = K.prefill_raw(sprob, ptr(q), ptr(k), ptr(v), ptr(g), ptr(beta), ptr(cu), ptr(s0),
                                   ptr(out), ptr(fin), ptr(offs), ptr(ck), ptr(ws), ws_bytes,
                                   stream.cuda_stream)
                if rc != 0:
                    raise K.KDAError(rc, "kda_prefill")
            one()
            kernels[kname] = {"stage": st, "ms": timed(one, max(5, args.steps // 2))[0]}
        step()  # leave a complete result behind
        torch.cuda.synchronize()
        sb = stage_bytes(p)
        for kname, e in kernels.items():
            e["algorithmic_bytes"] = sb[e["stage"]]
    else:
        kernels["kda_fused_kernel"] = {"stage": "both", "ms": ms_launch,
                                       "algorithmic_bytes": algorithmic_bytes(p)}
    dom = max(kernels, key=lambda kk: kernels[kk]["ms"])
    dk = kernels[dom]
    achieved = dk["algorithmic_bytes"] / (dk["ms"] * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(args.workload, variant, dom),
            "kernel": dom, "kernel_ms": round(dk["ms"], 4), "algorithmic_bytes": dk["algorithmic_bytes"]}
    alg_b = algorithmic_bytes(p)
    path = {"ms_per_call": round(ms_launch, 4), "algorithmic_bytes": alg_b,
            "achieved_GBps": round(alg_b / (ms_launch * 1e-3) / 1e9, 1),
            "frac_hbm": round(alg_b / (ms_launch * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "kernels_ms": {kk: round(e["ms"], 4) for kk, e in kernels.items()},
            # every launch's algorithmic rate against the HBM peak, not only
            # the dominant one's (at B8 T8192 the two launches take about the
            # same time, so which one is dominant can change with a change to
            # either)
            "kernels_frac_hbm": {kk: round(e["algorithmic_bytes"] / (e["ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
                                 for kk, e in kernels.items()}}
    ex_fl = modelled_mfma_flops(p, variant, vsplit)
    alg_fl = algorithmic_flops(p)
    mfma = {"modelled_executed_tflops": round(ex_fl / (ms_launch * 1e-3) / 1e12, 1),
            "modelled_executed_util": round(ex_fl / (ms_launch * 1e-3) / (MFMA_PEAK_TFLOPS * 1e12), 4),
            "algorithmic_tflops": round(alg_fl / (ms_launch * 1e-3) / 1e12, 1),
            "algorithmic_util": round(alg_fl / (ms_launch * 1e-3) / (MFMA_PEAK_TFLOPS * 1e12), 4),
            "peak_tflops": MFMA_PEAK_TFLOPS,
            # measured by rocprofv3 on the current kernel source (committed
            # profiles), per kernel: MFMA busy fraction of the SIMD cycles
            "measured_busy": {kk: measured_counters(args.workload, variant, kk).get("mfma_busy")
                              for kk in kernels}}
    res = {"metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
           "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None,
           "dtype": "bf16", "data": "synthetic",
           "config": {"workload": args.workload, "B": p.N if p.fixed else None,
                      "T": int(p.seq_lens[0]) if p.fixed else None, "num_seqs": p.N,
                      "total_tokens": p.T_total, "H": p.H, "K": 128, "V": 128,
                      "initial_state": p.initial_state is not None,
                      "checkpoints": p.ckpt_offsets is not None,
                      "variant": variant, "value_split": vsplit, "chain_parts": pieces},
           "roofline": roof, "path": path, "mfma": mfma, "timing": timing}
    if args.workload == "b8_t8192":
        res["context"] = dict(PAGES_CONTEXT, ratio_ms=round(PAGES_CONTEXT["ms"] / ms_step, 3))
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(p, args.cpu_sample_tokens)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
