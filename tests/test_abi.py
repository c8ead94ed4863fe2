"""Host-side checks of libkda's C ABI: the library loads without a GPU, exports
every entry point include/kda.h declares, and kda_validate / kda_prefill reject
bad arguments on the host before anything reaches the device."""
import ctypes
import math
import os
import re

import pytest

import kda_gated_delta_chunked_amd as K
from kda_gated_delta_chunked_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

OK, INVALID, UNSUPPORTED, ALIGN, OVERLAP, WS, TOO_LARGE = 0, -1, -2, -3, -4, -5, -6


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = K.load_library()
    names = declared_functions()
    assert {"kda_prefill", "kda_prefill_workspace_size", "kda_validate", "kda_status_string",
            "kda_plan"} <= set(names)
    for name in names:
        assert hasattr(lib, name), f"libkda.so does not export {name}"


def test_status_strings():
    lib = K.load_library()
    for code in range(-8, 1):
        s = lib.kda_status_string(code)
        assert s and s != b"unknown status"
    assert lib.kda_status_string(-99) == b"unknown status"


class Bufs:
    """Fake, 16-byte aligned, non-overlapping host addresses (never dereferenced)."""

    def __init__(self, N=2, T=256, H=4):
        self.N, self.T, self.H = N, T, H
        base = 1 << 40
        sizes = {"q": T * H * 256, "k": T * H * 256, "v": T * H * 256, "g": T * H * 512,
                 "beta": T * H * 4, "cu": (N + 1) * 4, "s0": N * H * 65536, "out": T * H * 256,
                 "fin": N * H * 65536, "offs": N * 4, "ck": N * H * 65536}
        self.addr = {}
        for k_, sz in sizes.items():
            self.addr[k_] = base
            base += (sz + 4095) // 4096 * 4096 + 4096

    def args(self, **over):
        a = dict(self.addr)
        a.update(over)
        return [a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu"], a["s0"], a["out"], a["fin"],
                a["offs"], a["ck"], 0, 0]


def validate(prob, b, **over):
    return K.validate_raw(prob, *b.args(**over))


def prob_for(b, **kw):
    return K.make_problem(b.N, b.T, b.H, scale=kw.pop("scale", 0.088), **kw)


def test_validate_accepts_a_well_formed_call():
    b = Bufs()
    assert validate(prob_for(b), b) == OK
    assert validate(prob_for(b), b, cu=0) == OK           # fixed layout, T divisible by N
    assert validate(prob_for(b), b, s0=0, fin=0) == OK     # no states
    assert validate(prob_for(b), b, offs=0, ck=0) == OK    # no checkpoints


@pytest.mark.parametrize("bound,want", [(-5.0, OK), (0.0, OK), (-2.5, OK), (-5.01, INVALID),
                                        (0.01, INVALID), (float("nan"), INVALID),
                                        (float("-inf"), INVALID)])
def test_gate_lower_bound_range_is_inclusive(bound, want):
    b = Bufs()
    assert validate(prob_for(b, gate_lower_bound=bound), b) == want


def test_shapes_and_scalars():
    b = Bufs()
    assert validate(prob_for(b, head_dim_k=64), b) == UNSUPPORTED
    assert validate(prob_for(b, head_dim_v=256), b) == UNSUPPORTED
    assert validate(prob_for(b, scale=float("inf")), b) == INVALID
    assert validate(prob_for(b, value_split=3), b) == UNSUPPORTED
    assert validate(prob_for(b, variant=7), b) == UNSUPPORTED
    assert validate(K.make_problem(0, 256, 4, scale=0.1), b) == INVALID
    assert validate(K.make_problem(2, 256, 0, scale=0.1), b) == INVALID
    assert validate(K.make_problem(3, 256, 4, scale=0.1), Bufs(N=3), cu=0) == INVALID  # 256 % 3
    assert validate(prob_for(b), b, q=0) == INVALID


def test_empty_batch_needs_no_token_buffers():
    b = Bufs(T=0)
    p = K.make_problem(2, 0, 4, scale=0.1)
    assert K.validate_raw(p, 0, 0, 0, 0, 0, b.addr["cu"], b.addr["s0"], 0, b.addr["fin"], 0, 0,
                          0, 0) == OK


def test_alignment():
    b = Bufs()
    for name in ("q", "k", "v", "g", "beta", "cu", "s0", "out", "fin", "offs", "ck"):
        assert validate(prob_for(b), b, **{name: b.addr[name] + 8}) == ALIGN, name


def test_overlap_rules():
    b = Bufs()
    p = prob_for(b)
    assert validate(p, b, out=b.addr["v"]) == OK                     # exact alias out == v
    assert validate(p, b, out=b.addr["v"] + 256) == OVERLAP          # partial
    assert validate(p, b, out=b.addr["q"]) == OVERLAP
    assert validate(p, b, fin=b.addr["s0"]) == OK                    # in-place state update
    assert validate(p, b, fin=b.addr["s0"] + 1024) == OVERLAP
    assert validate(p, b, ck=b.addr["s0"]) == OVERLAP                # checkpoints never alias
    assert validate(p, b, ck=b.addr["fin"]) == OVERLAP               # nor the final state
    assert validate(p, b, fin=b.addr["ck"]) == OVERLAP
    assert validate(p, b, out=b.addr["g"] + 512) == OVERLAP


def test_checkpoint_arguments_are_paired():
    b = Bufs()
    assert validate(prob_for(b), b, ck=0) == INVALID
    assert validate(prob_for(b), b, offs=0) == INVALID


def test_int32_flat_output_bound():
    # T_total * H * 128 must fit in int32: at H = 1024, 16383 tokens pass and 16384 do not
    for T, want in ((16383, OK), (16384, TOO_LARGE)):
        b = Bufs(N=1, T=T, H=1024)
        assert validate(K.make_problem(1, T, 1024, scale=0.1), b) == want


def test_prefill_rejects_on_the_host_without_a_device():
    b = Bufs()
    st = K.prefill_raw(prob_for(b, head_dim_k=64), *b.args()[:-2], 0, 0, 0)
    assert st == UNSUPPORTED
    st = K.prefill_raw(prob_for(b), *b.args(out=b.addr["q"])[:-2], 0, 0, 0)
    assert st == OVERLAP


def chain_cap(N, T, H):
    """The documented most chain pieces AUTO may pick: min(16, 1 + 128 // (N H),
    ceil((T // N) / 64) // 8), or 1 below 3."""
    cap = min(16, 1 + 128 // (N * H), -(-(T // N) // 64) // 8)
    return cap if cap >= 3 else 1


def decomp_bytes(N, T, H, C=1, pieces=None):
    """The documented workspace formula: 2 N + 1 int32 rounded up to 256
    bytes, then 60,416 bytes per (segment slot, head) for floor(T / 64) + N +
    N C slots (C checkpoint offsets per sequence, at least 1), then 3 x 64 KiB
    per (sequence, head, chain piece) when there are 2 or more pieces."""
    P = chain_cap(N, T, H) if pieces is None else pieces
    chain = N * H * P * 3 * 65536 if P >= 2 else 0
    return ((2 * N + 1) * 4 + 255) // 256 * 256 + (T // 64 + N + N * max(C, 1)) * H * 60416 + chain


def test_workspace_grows_with_checkpoints_per_sequence():
    for C in (0, 1, 2, 7, 64):
        p = K.make_problem(3, 1000, 2, scale=0.088, variant="decomp", ckpt_per_seq=C)
        assert K.workspace_size(p) == decomp_bytes(3, 1000, 2, C)
    with pytest.raises(K.KDAError):
        K.workspace_size(K.make_problem(3, 1000, 2, scale=0.088, ckpt_per_seq=65))
    with pytest.raises(K.KDAError):
        K.workspace_size(K.make_problem(3, 1000, 2, scale=0.088, ckpt_per_seq=-1))


def test_checkpoint_buffers_scale_with_offsets_per_sequence():
    # with C offsets per sequence the checkpoint buffer spans N C states: a
    # final state placed right after a one-state-per-sequence buffer overlaps it
    b = Bufs()
    C = 3
    prob = K.make_problem(b.N, b.T, b.H, scale=0.088, variant="fused", ckpt_per_seq=C)
    ck = b.addr["ck"]
    state = b.N * b.H * 65536
    assert ops.validate_raw(prob, *b.args(fin=0)[:-2], 0, 0) == OK
    assert ops.validate_raw(prob, *b.args(fin=ck + state)[:-2], 0, 0) == OVERLAP
    assert ops.validate_raw(prob, *b.args(fin=ck + C * state)[:-2], 0, 0) == OK


def test_periodic_offsets():
    offs = K.periodic_offsets([0, 5, 64, 200], 64)
    assert offs.dtype.name == "int32" and offs.shape == (4, 3)
    assert offs.tolist() == [[-1, -1, -1], [-1, -1, -1], [64, -1, -1], [64, 128, 192]]
    assert K.periodic_offsets([10], 64).tolist() == [[-1]]


def test_workspace_size_and_plan_arguments():
    assert K.workspace_size(K.make_problem(8, 65536, 12, scale=0.088, variant="fused")) == 0
    for var in ("auto", "decomp"):
        p = K.make_problem(8, 65536, 12, scale=0.088, variant=var)
        assert K.workspace_size(p) == decomp_bytes(8, 65536, 12)
    assert K.workspace_size(K.make_problem(3, 100, 2, scale=0.1)) == decomp_bytes(3, 100, 2)
    with pytest.raises(K.KDAError):
        K.workspace_size(K.make_problem(8, 65536, 12, scale=0.088, head_dim_k=64))


def test_workspace_rules():
    b = Bufs()
    need = decomp_bytes(b.N, b.T, b.H)
    ws = 1 << 44
    args = b.args()[:-2]

    def val(p, wsp, wsb, **over):
        return K.validate_raw(p, *b.args(**over)[:-2], wsp, wsb)

    dec = prob_for(b, variant="decomp")
    assert val(dec, 0, 0) == WS                        # DECOMP needs its workspace
    assert val(dec, ws, need - 1) == WS
    assert val(dec, ws, need) == OK
    assert val(prob_for(b), 0, 0) == OK                # AUTO falls back to FUSED
    assert val(prob_for(b), ws, need) == OK
    assert val(prob_for(b, value_split=8), 0, 0) == WS  # split 8 exists only in DECOMP
    assert val(prob_for(b, variant="fused", value_split=8), 0, 0) == UNSUPPORTED
    assert val(prob_for(b, variant="fused", value_split=1), ws, need) == UNSUPPORTED
    for vs in (1, 2, 4, 8):
        assert val(prob_for(b, variant="decomp", value_split=vs), ws, need) == OK
    assert val(dec, ws + 8, need) == ALIGN
    # the workspace overlaps nothing the call reads or writes
    assert val(dec, b.addr["out"], need) == OVERLAP
    assert val(dec, b.addr["fin"] - 4096, need) == OVERLAP
    assert val(dec, b.addr["ck"], need) == OVERLAP
    assert val(dec, b.addr["q"], need) == OVERLAP


def test_split_stages_rules():
    b = Bufs()
    need = decomp_bytes(b.N, b.T, b.H)
    ws = 1 << 44

    def val(p, wsp=ws, wsb=need):
        return K.validate_raw(p, *b.args()[:-2], wsp, wsb)

    for st in ("prepare", "recurrence"):
        assert val(prob_for(b, variant="decomp", stages=st)) == OK
        assert val(prob_for(b, variant="decomp", stages=st), 0, 0) == WS
        assert val(prob_for(b, variant="fused", stages=st)) == UNSUPPORTED
        assert val(prob_for(b, stages=st)) == UNSUPPORTED       # AUTO: the stages need DECOMP
    assert val(prob_for(b, variant="decomp", stages=3)) == INVALID
    assert val(prob_for(b, variant="decomp", stages=-1)) == INVALID


def test_plan_picks_a_schedule_without_a_device():
    # no GPU here: the CU count reads as 0, and the choice is still valid
    var, vs, parts = K.plan(K.make_problem(8, 65536, 12, scale=0.088, variant="fused"))
    assert var == "fused" and vs in (2, 4) and parts == 1
    plan = K.plan(K.make_problem(8, 65536, 12, scale=0.088, variant="decomp", value_split=4))
    assert plan == ("decomp", 4, 1)
    # with no device known, AUTO splits no chain; a given chain_parts is kept
    assert K.plan(K.make_problem(1, 8192, 12, scale=0.088))[2] == 1
    assert K.plan(K.make_problem(1, 8192, 12, scale=0.088, chain_parts=5))[2] == 5


def test_chain_split_workspace_and_rules():
    # the chain area: 3 x 64 KiB per (sequence, head, piece), for the pieces
    # given, or the most AUTO may pick; none when that is below 3
    assert chain_cap(1, 8192, 12) == 11 and chain_cap(1, 512, 12) == 1
    assert chain_cap(1, 8192, 2) == 16 and chain_cap(8, 8 * 8192, 12) == 1
    assert chain_cap(4, 4 * 2048, 4) == 4
    for N, T, H in [(1, 8192, 12), (1, 8192, 2), (1, 512, 12), (4, 4 * 2048, 4), (8, 65536, 12),
                    (2, 40, 1)]:
        for var in ("auto", "decomp"):
            assert K.workspace_size(K.make_problem(N, T, H, scale=0.088, variant=var)) == \
                decomp_bytes(N, T, H), (N, T, H, var)
        for P in (1, 2, 3, 16):
            p = K.make_problem(N, T, H, scale=0.088, variant="decomp", chain_parts=P)
            assert K.workspace_size(p) == decomp_bytes(N, T, H, pieces=P)
    with pytest.raises(K.KDAError):
        K.workspace_size(K.make_problem(1, 8192, 12, scale=0.088, chain_parts=17))
    with pytest.raises(K.KDAError):
        K.workspace_size(K.make_problem(1, 8192, 12, scale=0.088, chain_parts=-1))
    b = Bufs()
    ws = 1 << 44

    def val(p, wsp, wsb):
        return K.validate_raw(p, *b.args()[:-2], wsp, wsb)

    # FUSED runs no chain split
    assert val(prob_for(b, variant="fused", chain_parts=1), 0, 0) == OK
    assert val(prob_for(b, variant="fused", chain_parts=2), 0, 0) == UNSUPPORTED
    # a given split needs its chain area
    for P in (2, 5):
        need = decomp_bytes(b.N, b.T, b.H, pieces=P)
        for var in ("auto", "decomp"):
            p = prob_for(b, variant=var, chain_parts=P)
            assert val(p, ws, need) == OK
            assert val(p, ws, need - 1) == WS
    # AUTO runs unsplit in a workspace that holds only the slots
    assert val(prob_for(b), ws, decomp_bytes(b.N, b.T, b.H, pieces=1)) == OK
    # a given split pins AUTO to DECOMP: with no workspace it is refused, not
    # run as FUSED, and the plan says DECOMP
    assert val(prob_for(b, chain_parts=3), 0, 0) == WS
    assert K.plan(prob_for(b, chain_parts=3))[::2] == ("decomp", 3)


def test_python_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    q = torch.zeros(4, 2, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        K.prefill(q, q, q, torch.zeros(4, 2, 128), torch.zeros(4, 2))


class DecodeBufs:
    """Fake, 16-byte aligned, non-overlapping host addresses for kda_decode."""

    def __init__(self, N=4, T=2, H=3, P=6):
        self.N, self.T, self.H, self.P = N, T, H, P
        rows = N * T * H
        base = 1 << 41
        sizes = {"q": rows * 256, "k": rows * 256, "v": rows * 256, "g": rows * 512,
                 "beta": rows * 4, "pool": P * H * 65536, "idx": N * 4, "out": rows * 256,
                 "trace": rows * 65536, "acc": N * 4}
        self.addr = {}
        for k_, sz in sizes.items():
            self.addr[k_] = base
            base += (sz + 4095) // 4096 * 4096 + 4096

    def args(self, **over):
        a = dict(self.addr)
        a.update(over)
        return [a["q"], a["k"], a["v"], a["g"], a["beta"], a["pool"], a["idx"], a["out"]]


def _dprob(b, **kw):
    d = dict(scale=0.0884)
    d.update({k_: v_ for k_, v_ in kw.items() if k_ in ("scale", "gate_lower_bound", "head_dim_k",
                                                        "head_dim_v")})
    return ops.make_decode_problem(kw.get("N", b.N), kw.get("T", b.T), kw.get("H", b.H),
                                   kw.get("P", b.P), **d)


def test_decode_validation_rules():
    b = DecodeBufs()
    dv = ops.decode_validate_raw
    assert dv(_dprob(b), *b.args()) == OK
    # empty batch: nothing to check but the scalars
    assert dv(_dprob(b, N=0), *[0] * 8) == OK
    assert dv(_dprob(b, T=0), *b.args()) == INVALID
    assert dv(_dprob(b, P=0), *b.args()) == INVALID
    assert dv(_dprob(b, H=0), *b.args()) == INVALID
    assert dv(_dprob(b, head_dim_k=64), *b.args()) == UNSUPPORTED
    assert dv(_dprob(b, gate_lower_bound=-6.0), *b.args()) == INVALID
    assert dv(_dprob(b, gate_lower_bound=0.5), *b.args()) == INVALID
    assert dv(_dprob(b, scale=float("nan")), *b.args()) == INVALID
    assert dv(_dprob(b), *b.args(idx=0)) == INVALID
    assert dv(_dprob(b), *b.args(pool=b.addr["pool"] + 4)) == ALIGN
    # out may be exactly v, nothing else
    assert dv(_dprob(b), *b.args(out=b.addr["v"])) == OK
    assert dv(_dprob(b), *b.args(out=b.addr["v"] + 256)) == OVERLAP
    assert dv(_dprob(b), *b.args(out=b.addr["pool"])) == OVERLAP
    assert dv(_dprob(b), *b.args(pool=b.addr["idx"])) == OVERLAP
    assert dv(_dprob(b), *b.args(pool=b.addr["q"])) == OVERLAP
    # flat output index bound
    assert dv(_dprob(b, N=1 << 20, T=16, H=2), *b.args()) == TOO_LARGE


def test_decode_state_dtype_rules():
    # a bf16 pool holds 2-byte elements: a buffer right after its extent does
    # not overlap it, while the same placement would overlap an fp32 pool
    b = DecodeBufs()
    dv = ops.decode_validate_raw
    bad = _dprob(b)
    bad.state_dtype = 2
    assert dv(bad, *b.args()) == INVALID
    far = 1 << 47
    half = b.P * b.H * 128 * 128 * 2
    for dt, want in (("bf16", OK), ("fp32", OVERLAP)):
        prob = ops.make_decode_problem(b.N, b.T, b.H, b.P, scale=0.088, state_dtype=dt)
        assert dv(prob, *b.args(pool=far, idx=far + half)) == want, dt
    # the commit checks it too
    bad_c = _dprob(b)
    bad_c.state_dtype = 3
    assert ops.decode_commit_raw(bad_c, b.addr["pool"], b.addr["idx"], b.addr["trace"], b.addr["acc"], 0) \
        == INVALID


def test_decode_rejects_on_the_host():
    # argument errors come back before anything touches a device
    b = DecodeBufs()
    lib = K.load_library()
    prob = _dprob(b, T=0)
    P = b.args()
    assert lib.kda_decode(ctypes.byref(prob), *P, None) == INVALID
    prob = _dprob(b)
    assert lib.kda_decode(ctypes.byref(prob), *b.args(out=b.addr["pool"]), None) == OVERLAP


def test_decode_verify_and_commit_rules():
    # argument errors of the speculative pair come back on the host, before
    # anything is enqueued (the fake addresses are never dereferenced)
    b = DecodeBufs()
    a = b.addr

    def verify(prob=None, trace=a["trace"], **over):
        return ops.decode_verify_raw(prob or _dprob(b), *b.args(**over), trace, 0)

    def commit(prob=None, **over):
        d = dict(pool=a["pool"], idx=a["idx"], trace=a["trace"], acc=a["acc"])
        d.update(over)
        return ops.decode_commit_raw(prob or _dprob(b), d["pool"], d["idx"], d["trace"], d["acc"], 0)

    # the decode rules hold for a verify as well
    assert verify(_dprob(b, T=0)) == INVALID
    assert verify(_dprob(b, head_dim_k=64)) == UNSUPPORTED
    assert verify(out=a["pool"]) == OVERLAP
    assert verify(pool=a["pool"] + 4) == ALIGN
    # and the trace (optional): aligned, overlapping nothing (not even out = v)
    assert verify(trace=a["trace"] + 8) == ALIGN
    for name in ("q", "k", "v", "g", "beta", "pool", "idx", "out"):
        assert verify(trace=a[name]) == OVERLAP, name
    # the trace's extent is N T H 128 128 fp32: one that ends 16 bytes into
    # the pool overlaps it (a call that passes every check would launch, so no
    # accepted case is made here with these fake addresses)
    extent = b.N * b.T * b.H * 65536
    far = 1 << 48
    assert verify(trace=far + 16, pool=far + extent) == OVERLAP
    # an empty batch needs no buffers at all
    assert ops.decode_verify_raw(_dprob(b, N=0), *[0] * 9, 0) == OK

    assert commit(_dprob(b, T=0)) == INVALID
    assert commit(_dprob(b, P=0)) == INVALID
    assert commit(_dprob(b, head_dim_v=64)) == UNSUPPORTED
    for name in ("pool", "idx", "trace", "acc"):
        assert commit(**{name: 0}) == INVALID, name
        assert commit(**{name: a[name] + 4}) == ALIGN, name
    for name in ("idx", "trace", "acc"):
        assert commit(pool=a[name]) == OVERLAP, name
    assert ops.decode_commit_raw(_dprob(b, N=0), 0, 0, 0, 0, 0) == OK
    assert commit(_dprob(b, N=1 << 20, T=16, H=2)) == TOO_LARGE

    # the advance: the decode's inputs and pool, accepted instead of out
    def advance(prob=None, **over):
        d = dict(a)
        d.update(over)
        return ops.decode_advance_raw(prob or _dprob(b), d["q"], d["k"], d["v"], d["g"], d["beta"],
                                      d["pool"], d["idx"], d["acc"], 0)

    assert advance(_dprob(b, T=0)) == INVALID
    assert advance(_dprob(b, head_dim_k=64)) == UNSUPPORTED
    assert advance(acc=0) == INVALID
    assert advance(acc=a["acc"] + 4) == ALIGN
    for name in ("q", "k", "v", "g", "beta", "idx", "acc"):
        assert advance(pool=a[name]) == OVERLAP, name
    assert ops.decode_advance_raw(_dprob(b, N=0), *[0] * 8, 0) == OK


def test_state_dtype_rules():
    b = Bufs()
    bad = K.make_problem(2, 256, 4, scale=0.088, variant="fused")
    bad.state_dtype = 2
    with pytest.raises(K.KDAError):
        K.workspace_size(bad)
    # bf16 states take half the bytes: a final state right after a bf16
    # initial state does not overlap it, while with fp32 states it would
    half = b.N * b.H * 128 * 128 * 2
    for dt, want in (("bf16", OK), ("fp32", OVERLAP)):
        prob = K.make_problem(b.N, b.T, b.H, scale=0.088, variant="fused", state_dtype=dt)
        assert ops.validate_raw(prob, *b.args(fin=b.addr["s0"] + half)[:-2], 0, 0) == want


def test_prologue_rules():
    b = Bufs()
    lib = K.load_library()
    # unknown flag bits
    bad = K.make_problem(b.N, b.T, b.H, scale=0.088)
    bad.prologue = 4
    with pytest.raises(K.KDAError):
        K.workspace_size(bad)
    # both schedules take the prologue; AUTO with no workspace takes the
    # one-launch schedule as without it
    p = K.make_problem(b.N, b.T, b.H, scale=0.088, variant="fused", qk_l2norm=True)
    assert ops.validate_raw(p, *b.args()[:-2], 0, 0) == OK
    p = K.make_problem(b.N, b.T, b.H, scale=0.088, beta_logit=True)
    assert ops.validate_raw(p, *b.args()[:-2], 0, 0) == OK
    p = K.make_problem(b.N, b.T, b.H, scale=0.088, variant="decomp", beta_logit=True)
    assert ops.validate_raw(p, *b.args()[:-2], 0, 0) == WS
    d = DecodeBufs()
    dp = ops.make_decode_problem(d.N, d.T, d.H, d.P, scale=0.088, qk_l2norm=True, beta_logit=True)
    assert ops.decode_validate_raw(dp, *d.args()) == OK
    dp.prologue = 8
    assert ops.decode_validate_raw(dp, *d.args()) == INVALID


def test_int64_offsets_and_sequence_order_rules():
    b = Bufs()
    # int64 offsets take (N + 1) * 8 bytes: a buffer starting right after
    # the int32 extent overlaps them
    p64 = prob_for(b, cu_seqlens_int64=True)
    assert validate(p64, b) == OK
    far = 1 << 48          # cu alone at the top, out right after its int32 extent
    assert validate(prob_for(b), b, cu=far, out=far + 16) == OK
    assert validate(p64, b, cu=far, out=far + 16) == OVERLAP
    bad = prob_for(b)
    bad.cu_seqlens_int64 = 2
    assert validate(bad, b) == INVALID
    # seq_order: packed layout only, 16-byte aligned, read-only (no overlap with
    # what the call writes)
    order = 1 << 50
    assert validate(prob_for(b, seq_order=order), b) == OK
    assert validate(prob_for(b, seq_order=order), b, cu=0) == INVALID
    assert validate(prob_for(b, seq_order=order + 4), b) == ALIGN
    assert validate(prob_for(b, seq_order=b.addr["out"]), b) == OVERLAP
    assert validate(prob_for(b, seq_order=b.addr["fin"] + 64), b) == OVERLAP
    assert validate(prob_for(b, seq_order=b.addr["q"]), b) == OK   # both only read
