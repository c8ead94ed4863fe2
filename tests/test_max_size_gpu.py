"""Parity at the largest problem the INT32 flat-output bound admits:
T_total * H * 128 <= 2^31 - 1 with H = 1024 and T = 16383 (FlashInfer PR
#4633, Description: the bound is checked on the host; 16383 tokens pass at
H = 1024, 16384 do not).  Inputs follow the synthetic recipe but are drawn
on the GPU from a seeded torch generator (36 GiB of inputs and workspace);
the fp64 oracle checks sampled heads, and every output element must be
written (NaN sentinel)."""
import numpy as np
import pytest

import oracle
from gpu_helpers import OUT_MAX_ABS, OUT_REL_L2, STATE_REL_L2, rel_l2

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

T, H, D = 16383, 1024, 128
SAMPLED_HEADS = (0, 511, 1023)


@pytest.mark.parametrize("variant", ["decomp", "fused"])
def test_int32_bound_max_size(variant):
    import torch
    import kda_gated_delta_chunked_amd as K
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = torch.device("cuda", 0)
    gen = torch.Generator(device=dev)
    gen.manual_seed(4242)
    assert T * H * D <= 2**31 - 1 < (T + 1) * H * D

    def unit_bf16():
        x = torch.empty((T, H, D), dtype=torch.bfloat16, device=dev)
        for h0 in range(0, H, 128):     # in head blocks, to bound fp32 temporaries
            y = torch.randn((T, 128, D), generator=gen, device=dev)
            x[:, h0:h0 + 128] = (y / y.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
        return x

    q, k = unit_bf16(), unit_bf16()
    v = torch.empty((T, H, D), dtype=torch.bfloat16, device=dev)
    g = torch.empty((T, H, D), dtype=torch.float32, device=dev)
    for h0 in range(0, H, 128):
        v[:, h0:h0 + 128] = torch.randn((T, 128, D), generator=gen, device=dev).to(torch.bfloat16)
        g[:, h0:h0 + 128] = -5.0 * torch.sigmoid(torch.randn((T, 128, D), generator=gen, device=dev))
    beta = torch.sigmoid(torch.randn((T, H), generator=gen, device=dev))
    s0 = 0.02 * torch.randn((1, H, D, D), generator=gen, device=dev)
    scale = D ** -0.5

    out = torch.full((T, H, D), float("nan"), dtype=torch.bfloat16, device=dev)
    fin = torch.full((1, H, D, D), float("nan"), device=dev)
    prob = K.make_problem(1, T, H, scale=scale, variant=variant)
    need = K.workspace_size(prob)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    rc = K.prefill_raw(prob, q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(), beta.data_ptr(), 0,
                       s0.data_ptr(), out.data_ptr(), fin.data_ptr(), 0, 0, ws.data_ptr(), need,
                       torch.cuda.current_stream(dev).cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()) and bool(torch.isfinite(fin).all())
    # one token more does not fit
    assert K.validate_raw(K.make_problem(1, T + 1, H, scale=scale, variant=variant),
                          0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0) == -6   # KDA_ERR_TOO_LARGE

    def bits(t):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    for h in SAMPLED_HEADS:
        ref = oracle.prefill(bits(q[:, h:h + 1]), bits(k[:, h:h + 1]), bits(v[:, h:h + 1]),
                             g[:, h:h + 1].contiguous().cpu().numpy(), beta[:, h:h + 1].contiguous().cpu().numpy(),
                             scale=scale, num_seqs=1, initial_state=s0[:, h:h + 1].contiguous().cpu().numpy())
        o = out[:, h:h + 1].float().cpu().numpy()
        f = fin[:, h:h + 1].cpu().numpy()
        m = {"out_max_abs": float(np.max(np.abs(o - ref["out"]))), "out_rel_l2": rel_l2(o, ref["out"]),
             "final_rel_l2": rel_l2(f, ref["final"])}
        print(f"[max-size] {variant} head {h}: " + " ".join(f"{a}={b:.3e}" for a, b in m.items()), flush=True)
        assert m["out_max_abs"] <= OUT_MAX_ABS and m["out_rel_l2"] <= OUT_REL_L2, m
        assert m["final_rel_l2"] <= STATE_REL_L2, m
