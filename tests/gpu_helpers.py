"""Helpers shared by the GPU tests: move a synth.Problem to the device, run
libkda through its C ABI, and compare with the fp64 oracle."""
from __future__ import annotations

import numpy as np

from kda_gated_delta_chunked_amd import synth

# Parity gates (fp32-state KDA prefill vs the fp64 oracle).
OUT_MAX_ABS = 2e-2
OUT_REL_L2 = 5e-3
STATE_REL_L2 = 1e-3


def to_device(p: synth.Problem):
    import torch
    dev = torch.device("cuda", 0)

    def bf16(bits):
        return torch.from_numpy(bits.view(np.int16).copy()).to(dev).view(torch.bfloat16)

    d = {
        "q": bf16(p.q), "k": bf16(p.k), "v": bf16(p.v),
        "g": torch.from_numpy(p.g).to(dev), "beta": torch.from_numpy(p.beta).to(dev),
        "cu": None if p.fixed else torch.from_numpy(p.cu_seqlens).to(dev),
        "s0": None if p.initial_state is None else torch.from_numpy(p.initial_state).to(dev),
        "offs": None if p.ckpt_offsets is None else torch.from_numpy(p.ckpt_offsets).to(dev),
    }
    return d


def run_gpu(p: synth.Problem, *, variant: str = "auto", value_split: int = 0, d=None,
            sentinel: bool = True, out_alias_v: bool = False, state_in_place: bool = False,
            keep_workspace: bool = False, state_bf16: bool = False, qk_l2norm: bool = False,
            beta_logit: bool = False, cu64: bool = False, seq_order=None, chain_parts: int = 0):
    """Run kda_prefill through the C ABI on a fresh set of device buffers.

    Outputs are pre-filled with NaN so that any element the kernel fails to
    write shows up; the workspace (sized by kda_prefill_workspace_size) is
    filled with 0xFF bytes (NaN as fp32) so nothing depends on its contents.
    Returns numpy dict(out fp32, final, ckpt), and the workspace bytes under
    "workspace" when keep_workspace is set.  With state_bf16 the states are
    bf16 tensors (the initial state must hold bf16 values) and come back as
    fp32 arrays of their bf16 values.  cu64 passes the sequence offsets as
    int64; seq_order (int32 numpy [N]) is the caller's recurrence order;
    chain_parts the pieces of the two-launch schedule's chain split (0 = the
    library's choice)."""
    import torch
    import kda_gated_delta_chunked_amd as K
    d = d or to_device(p)
    dev = d["q"].device
    N, H, T = p.N, p.H, p.T_total
    out = d["v"].clone() if out_alias_v else torch.full((T, H, 128), float("nan"), dtype=torch.bfloat16,
                                                        device=dev)
    sdt = torch.bfloat16 if state_bf16 else torch.float32
    if state_in_place:
        s0 = d["s0"].clone() if d["s0"] is not None else torch.zeros((N, H, 128, 128), device=dev)
        s0 = s0.to(sdt)
        fin = s0
    else:
        s0 = None if d["s0"] is None else d["s0"].to(sdt)
        fin = torch.full((N, H, 128, 128), float("nan") if sentinel else 0.0, dtype=sdt,
                         device=dev)
    ck = None
    C = 0
    if d["offs"] is not None:
        C = 1 if d["offs"].dim() == 1 else int(d["offs"].shape[1])
        shape = (N, H, 128, 128) if d["offs"].dim() == 1 else (N, C, H, 128, 128)
        ck = torch.full(shape, float("nan"), dtype=sdt, device=dev)
    cu = d["cu"]
    if cu is not None and cu64:
        cu = cu.to(torch.int64)
    order = None if seq_order is None else torch.from_numpy(np.asarray(seq_order, np.int32)).to(dev)
    prob = K.make_problem(N, T, H, scale=p.scale, variant=variant, value_split=value_split,
                          ckpt_per_seq=C, state_dtype="bf16" if state_bf16 else "fp32",
                          qk_l2norm=qk_l2norm, beta_logit=beta_logit, cu_seqlens_int64=cu64,
                          seq_order=0 if order is None else order.data_ptr(),
                          chain_parts=chain_parts)
    need = K.workspace_size(prob)
    ws = torch.full((max(need, 1),), 255, dtype=torch.uint8, device=dev) if need else None
    stream = torch.cuda.current_stream(dev)
    v_ptr = out.data_ptr() if out_alias_v else d["v"].data_ptr()
    st = K.prefill_raw(prob, d["q"].data_ptr(), d["k"].data_ptr(), v_ptr, d["g"].data_ptr(),
                       d["beta"].data_ptr(), 0 if cu is None else cu.data_ptr(),
                       0 if s0 is None else s0.data_ptr(), out.data_ptr(), fin.data_ptr(),
                       0 if d["offs"] is None else d["offs"].data_ptr(),
                       0 if ck is None else ck.data_ptr(), 0 if ws is None else ws.data_ptr(), need,
                       stream.cuda_stream)
    assert st == 0, f"kda_prefill returned {st}"
    torch.cuda.synchronize()
    res = {"out": out.float().cpu().numpy(), "final": fin.float().cpu().numpy(),
           "ckpt": None if ck is None else ck.float().cpu().numpy()}
    if keep_workspace:
        res["workspace"] = None if ws is None else ws.cpu().numpy()
    return res


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.linalg.norm(b.ravel())
    return float(np.linalg.norm((a - b).ravel()) / den) if den > 0 else float(np.linalg.norm(a.ravel()))


def metrics(gpu, ref):
    m = {"out_max_abs": float(np.max(np.abs(gpu["out"] - ref["out"]))) if gpu["out"].size else 0.0,
         "out_rel_l2": rel_l2(gpu["out"], ref["out"]) if gpu["out"].size else 0.0,
         "final_rel_l2": rel_l2(gpu["final"], ref["final"])}
    if ref.get("ckpt") is not None:
        m["ckpt_rel_l2"] = rel_l2(gpu["ckpt"], ref["ckpt"])
    return m


def _worst_state_pair(g, r):
    """Largest relative L2 over the (sequence[, checkpoint], head) blocks of
    states shaped [..., 128, 128]; reference blocks holding NaN (nothing
    exported there) are skipped.  Returns (error, index)."""
    g = np.asarray(g, np.float64).reshape(-1, 128 * 128)
    r = np.asarray(r, np.float64).reshape(-1, 128 * 128)
    worst, where = 0.0, None
    for i in range(r.shape[0]):
        if np.isnan(r[i]).any():
            continue
        e = rel_l2(g[i], r[i])
        if not e <= worst:      # NaN counts as the worst
            worst, where = e, i
    return worst, where


def pair_metrics(gpu, ref, cu_seqlens=None):
    """Worst figures over the (sequence, head) pairs: the state's relative L2
    (final, and each exported checkpoint), and, when cu_seqlens is given, the
    output's relative L2 of each sequence and head.  One pair off by 5e-3
    among B8 H12's 96 would show as about 5e-4 over the whole tensor; here it
    shows as itself."""
    H = gpu["final"].shape[1]
    m = {}
    e, i = _worst_state_pair(gpu["final"], ref["final"])
    m["worst_final_rel_l2"] = e
    m["worst_final_pair"] = None if i is None else divmod(i, H)
    if ref.get("ckpt") is not None and gpu.get("ckpt") is not None:
        e, i = _worst_state_pair(gpu["ckpt"], ref["ckpt"])
        m["worst_ckpt_rel_l2"] = e
        m["worst_ckpt_pair"] = None if i is None else divmod(i, H)
    if cu_seqlens is not None:
        worst, where = 0.0, None
        for n in range(len(cu_seqlens) - 1):
            b, e_ = int(cu_seqlens[n]), int(cu_seqlens[n + 1])
            if e_ <= b:
                continue
            for h in range(H):
                err = rel_l2(gpu["out"][b:e_, h], ref["out"][b:e_, h])
                if not err <= worst:
                    worst, where = err, (n, h)
        m["worst_out_rel_l2"] = worst
        m["worst_out_pair"] = where
    return m


def assert_parity(gpu, ref, what="", cu_seqlens=None):
    """Gates over the whole tensors and per (sequence, head) pair: output
    max-abs <= 2e-2 and relative L2 <= 5e-3 (per pair when cu_seqlens is
    given), final and checkpoint state relative L2 <= 1e-3 for every pair."""
    assert np.all(np.isfinite(gpu["out"])), f"{what}: non-finite or unwritten outputs"
    assert np.all(np.isfinite(gpu["final"])), f"{what}: non-finite or unwritten final state"
    m = metrics(gpu, ref)
    m.update(pair_metrics(gpu, ref, cu_seqlens))
    assert m["out_max_abs"] <= OUT_MAX_ABS, f"{what}: {m}"
    assert m["out_rel_l2"] <= OUT_REL_L2, f"{what}: {m}"
    assert m["final_rel_l2"] <= STATE_REL_L2, f"{what}: {m}"
    assert m["worst_final_rel_l2"] <= STATE_REL_L2, f"{what}: {m}"
    if cu_seqlens is not None:
        assert m["worst_out_rel_l2"] <= OUT_REL_L2, f"{what}: {m}"
    if "ckpt_rel_l2" in m:
        assert np.all(np.isfinite(gpu["ckpt"][np.isfinite(ref["ckpt"])])), f"{what}: unwritten checkpoint"
        assert m["ckpt_rel_l2"] <= STATE_REL_L2, f"{what}: {m}"
        assert m["worst_ckpt_rel_l2"] <= STATE_REL_L2, f"{what}: {m}"
    return m
