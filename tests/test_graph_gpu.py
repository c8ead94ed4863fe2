"""HIP graph capture: one kda_prefill call (DECOMP with a caller workspace,
and FUSED) captured cold, then replayed after the inputs change -- q, k, v,
g, beta, the sequence lengths and the checkpoint offsets (same N and
T_total) -- with eager work and synchronisations between replays.  Every
replay is checked against the fp64 oracle."""
import numpy as np
import pytest

import oracle
from gpu_helpers import assert_parity
from kda_gated_delta_chunked_amd import synth

pytestmark = pytest.mark.gpu


def _problems():
    # 16 sequences of 512..2048 tokens (H = 2) with one checkpoint each, a
    # smaller instance of the checkpoint workload; the second input keeps N and
    # T_total but moves the lengths and the offsets
    a = synth.make_problem(synth.uniform_lengths(2004, 16, 512, 2048), 2, seed=41, init_state=True,
                           ckpt="inside", name="graph_a")
    lens = np.array(a.seq_lens, np.int64)
    lens_b = lens.copy()
    lens_b[0] += 300
    lens_b[1] -= 300
    b = synth.make_problem(list(lens_b), 2, seed=42, init_state=True, ckpt="inside", name="graph_b")
    assert a.T_total == b.T_total and a.N == b.N
    return a, b


def _full_size_problems():
    # the checkpoint workload at full size (16 sequences of 512..8192 tokens,
    # H = 12, one offset each), and a second input with the same N and T_total
    # but moved lengths and offsets
    a = synth.workload("ckpt_16_rand")
    lens_b = np.array(a.seq_lens, np.int64)
    lens_b[0] += 257
    lens_b[1] -= 257
    b = synth.make_problem(list(lens_b), a.H, seed=a.seed + 1, init_state=True, ckpt="inside",
                           name="ckpt_16_moved")
    assert a.T_total == b.T_total and a.N == b.N
    return a, b


def _few_pair_problems():
    # two long sequences (H = 2) with one checkpoint each, for the chain split
    # (its two recurrence launches and the scan between them in one graph)
    a = synth.make_problem([3000, 1100], 2, seed=43, init_state=True, ckpt="inside", name="graph_few_a")
    b = synth.make_problem([1700, 2400], 2, seed=44, init_state=True, ckpt="inside", name="graph_few_b")
    assert a.T_total == b.T_total and a.N == b.N
    return a, b


@pytest.mark.parametrize("variant,size", [("decomp", "small"), ("fused", "small"), ("decomp", "full"),
                                          ("fused", "full"), ("decomp", "split")])
def test_graph_capture_and_replay_with_new_inputs(variant, size):
    import torch
    import kda_gated_delta_chunked_amd as K
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = torch.device("cuda", 0)
    pa, pb = {"small": _problems, "full": _full_size_problems, "split": _few_pair_problems}[size]()
    N, H, T = pa.N, pa.H, pa.T_total

    def dev_bf16(bits):
        return torch.from_numpy(bits.view(np.int16).copy()).to(dev).view(torch.bfloat16)

    q, k, v = dev_bf16(pa.q), dev_bf16(pa.k), dev_bf16(pa.v)
    g = torch.from_numpy(pa.g).to(dev)
    beta = torch.from_numpy(pa.beta).to(dev)
    cu = torch.from_numpy(pa.cu_seqlens).to(dev)
    s0 = torch.from_numpy(pa.initial_state).to(dev)
    offs = torch.from_numpy(pa.ckpt_offsets).to(dev)
    out = torch.empty((T, H, 128), dtype=torch.bfloat16, device=dev)
    fin = torch.empty((N, H, 128, 128), device=dev)
    ck = torch.empty((N, H, 128, 128), device=dev)
    prob = K.make_problem(N, T, H, scale=pa.scale, variant=variant,
                          chain_parts=5 if size == "split" else 0)
    need = K.workspace_size(prob)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)

    def call(stream):
        rc = K.prefill_raw(prob, q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(), beta.data_ptr(),
                           cu.data_ptr(), s0.data_ptr(), out.data_ptr(), fin.data_ptr(), offs.data_ptr(),
                           ck.data_ptr(), ws.data_ptr(), need, stream)
        assert rc == 0

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(dev)
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            call(torch.cuda.current_stream(dev).cuda_stream)
    torch.cuda.synchronize()

    def load(p):
        q.copy_(dev_bf16(p.q)); k.copy_(dev_bf16(p.k)); v.copy_(dev_bf16(p.v))
        g.copy_(torch.from_numpy(p.g)); beta.copy_(torch.from_numpy(p.beta))
        cu.copy_(torch.from_numpy(p.cu_seqlens)); s0.copy_(torch.from_numpy(p.initial_state))
        offs.copy_(torch.from_numpy(p.ckpt_offsets))
        out.fill_(float("nan")); fin.fill_(float("nan")); ck.fill_(float("nan"))
        torch.cuda.synchronize()

    refs = {}
    for rep, p in enumerate([pa, pb, pa, pb]):
        load(p)
        graph.replay()
        torch.cuda.synchronize()
        gpu = {"out": out.float().cpu().numpy(), "final": fin.cpu().numpy(), "ckpt": ck.cpu().numpy()}
        if p.name not in refs:
            refs[p.name] = oracle.prefill_problem(p)
        m = assert_parity(gpu, refs[p.name], f"{variant} replay {rep}", p.cu_seqlens)
        print(f"[graph] {variant} replay {rep} ({p.name}): "
              + " ".join(f"{a}={b:.3e}" if isinstance(b, float) else f"{a}={b}" for a, b in m.items()),
              flush=True)
        # eager work between replays
        torch.cuda.synchronize()
        _ = (q.float() * 2).sum().item()
