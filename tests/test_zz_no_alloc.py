"""The allocation-free prefill entry point (kda_prefill_noalloc), whose DECOMP
workspace is the library's static device scratch, against kda_prefill with a
caller workspace: two calls in a row, the second on a smaller input (the
scratch then holds the first call's leftovers), each bit for bit equal to the
existing entry point's result and within the parity gates of the fp64
oracle.  Sizes past the scratch are refused on the host."""
import numpy as np
import pytest

import oracle
from gpu_helpers import assert_parity, run_gpu, to_device
from kda_gated_delta_chunked_amd import synth

pytestmark = pytest.mark.gpu


def _noalloc(p, variant, chain_parts=0):
    import torch
    import kda_gated_delta_chunked_amd as K
    d = to_device(p)
    dev = d["q"].device
    N, H, T = p.N, p.H, p.T_total
    out = torch.full((T, H, 128), float("nan"), dtype=torch.bfloat16, device=dev)
    fin = torch.full((N, H, 128, 128), float("nan"), device=dev)
    ck = None if d["offs"] is None else torch.full((N, H, 128, 128), float("nan"), device=dev)
    prob = K.make_problem(N, T, H, scale=p.scale, variant=variant, chain_parts=chain_parts)
    st = K.prefill_noalloc_raw(prob, d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(),
                               d["g"].data_ptr(), d["beta"].data_ptr(),
                               0 if d["cu"] is None else d["cu"].data_ptr(),
                               0 if d["s0"] is None else d["s0"].data_ptr(), out.data_ptr(),
                               fin.data_ptr(), 0 if d["offs"] is None else d["offs"].data_ptr(),
                               0 if ck is None else ck.data_ptr(),
                               torch.cuda.current_stream(dev).cuda_stream)
    assert st == 0, f"kda_prefill_noalloc returned {st}"
    torch.cuda.synchronize()
    return {"out": out.float().cpu().numpy(), "final": fin.cpu().numpy(),
            "ckpt": None if ck is None else ck.cpu().numpy()}


@pytest.mark.parametrize("variant", ["decomp", "auto"])
def test_noalloc_equals_prefill_two_calls_second_smaller(variant):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kda_gated_delta_chunked_amd as K
    K.load_library()
    first = synth.make_problem([3000, 0, 1111, 2049, 64], 6, seed=61, init_state=True,
                               ckpt=[1500, 0, 1111, 2000, 1])
    second = synth.make_problem([700, 130], 3, seed=62, init_state=True, ckpt=[5, 128])
    for p in (first, second):
        need = K.workspace_size(K.make_problem(p.N, p.T_total, p.H, scale=p.scale, variant="decomp"))
        assert 0 < need <= K.ops.NOALLOC_SCRATCH_BYTES
        ref = oracle.prefill_problem(p)
        want = run_gpu(p, variant=variant)
        got = _noalloc(p, variant)
        m = assert_parity(got, ref, f"noalloc {p.name}", p.cu_seqlens)
        print(f"[noalloc] {variant} {p.name}: out rel-L2 {m['out_rel_l2']:.3e} "
              f"final {m['final_rel_l2']:.3e} ckpt {m['ckpt_rel_l2']:.3e}", flush=True)
        for key in ("out", "final", "ckpt"):
            assert np.array_equal(got[key], want[key], equal_nan=True), (p.name, key)


def test_noalloc_refuses_problems_past_the_scratch():
    import kda_gated_delta_chunked_amd as K
    K.load_library()
    # B8 T8192 H12 needs about 754 MB of workspace: refused on the host, nothing enqueued
    prob = K.make_problem(8, 8 * 8192, 12, scale=0.088, variant="decomp")
    assert K.workspace_size(prob) > K.ops.NOALLOC_SCRATCH_BYTES
    st = K.prefill_noalloc_raw(prob, *([16] * 11), 0)
    assert st == -8


def test_noalloc_chain_split_two_calls_second_smaller():
    # the chain split inside the static scratch: AUTO's split of a long
    # sequence with few heads (its chain area fits the scratch), then a
    # smaller call with three pieces given; each bit for bit equal to
    # kda_prefill's with a caller workspace of kda_prefill_workspace_size
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kda_gated_delta_chunked_amd as K
    K.load_library()
    first = synth.make_problem([8192], 4, seed=63, fixed=True, init_state=True)
    second = synth.make_problem([2048, 0, 700], 2, seed=64, init_state=True)
    for p, parts in ((first, 0), (second, 3)):
        prob = K.make_problem(p.N, p.T_total, p.H, scale=p.scale, variant="auto", chain_parts=parts)
        assert 0 < K.workspace_size(prob) <= K.ops.NOALLOC_SCRATCH_BYTES
        plan = K.plan(prob)
        if torch.cuda.get_device_properties(0).multi_processor_count == 256:
            assert plan[0] == "decomp" and plan[2] >= 3, plan
        ref = oracle.prefill_problem(p)
        want = run_gpu(p, variant="auto", chain_parts=parts)
        got = _noalloc(p, "auto", chain_parts=parts)
        m = assert_parity(got, ref, f"noalloc split {p.name}", p.cu_seqlens)
        print(f"[noalloc] split {plan} {p.name}: out rel-L2 {m['out_rel_l2']:.3e} "
              f"final {m['final_rel_l2']:.3e}", flush=True)
        for key in ("out", "final"):
            assert np.array_equal(got[key], want[key]), (p.name, key)
