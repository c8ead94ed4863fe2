"""The Python binding on a side stream.  Buffers the binding allocates itself
belong to the current stream in torch's caching allocator; above all the
workspace, dropped when the call returns, must not go to a new allocation on
the current stream while the call's kernels on the side stream still use it.
A fill of a fresh buffer of the workspace's size on the current stream, issued
right after the call, must leave the results intact."""
import numpy as np
import pytest

import oracle
from gpu_helpers import assert_parity, to_device
from kda_gated_delta_chunked_amd import synth

pytestmark = pytest.mark.gpu


def test_side_stream_call_keeps_its_workspace():
    import torch
    import kda_gated_delta_chunked_amd as K
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    K.load_library()
    dev = torch.device("cuda", 0)
    p = synth.make_problem([4000, 3000, 1500], 4, seed=51, init_state=True)
    ref = oracle.prefill_problem(p)
    d = to_device(p)
    prob = K.make_problem(p.N, p.T_total, p.H, scale=p.scale, variant="decomp")
    need = K.workspace_size(prob)
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    for rep in range(3):
        out, fin = K.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu"],
                             initial_state=d["s0"], scale=p.scale, variant="decomp", stream=side)
        # right away, on the current stream: a buffer the size of the dropped
        # workspace, filled with NaN bytes
        junk = torch.empty(need, dtype=torch.uint8, device=dev)
        junk.fill_(0xFF)
        torch.cuda.synchronize()
        gpu = {"out": out.float().cpu().numpy(), "final": fin.cpu().numpy()}
        m = assert_parity(gpu, ref, f"side stream {rep}", p.cu_seqlens)
        print(f"[streams] rep {rep}: out rel-L2 {m['out_rel_l2']:.3e} final {m['final_rel_l2']:.3e}",
              flush=True)
        del junk, out, fin
