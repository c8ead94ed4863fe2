"""The chunked algebra the kernels implement, checked on the CPU.

(a) In fp64 the chunked form (16-row gate blocks, unit-lower-triangular solve,
chunk recurrence, checkpoint splits) reproduces the fp64 token oracle to
rounding for several chunk sizes and ragged tails.
(b) With the operand rounding the kernels apply where they feed the matrix
cores (the kernels' precision recipe, chunked_model.KERNEL_RECIPE for the
two-launch schedule and FUSED_RECIPE for the one-launch schedule), the result
meets the parity gates with margin -- also at slow decay (g near 0, inside
the gate bound [-5, 0] of lmdeploy PR #5050, Modification, which includes 0),
where rounding is not forgotten between chunks.
"""
import numpy as np
import pytest

import chunked_model as cm
import oracle
from kda_gated_delta_chunked_amd import synth


def _rel(a, b):
    return float(np.linalg.norm((a - b).ravel()) / np.linalg.norm(b.ravel()))


@pytest.mark.parametrize("chunk,mode", [(1, "split"), (16, "split"), (64, "split"),
                                        (64, "masked")])
def test_chunked_fp64_equals_token_recurrence(chunk, mode):
    lens = [1, 2, 15, 16, 17, 33, 63, 64, 65, 129]
    offs = [1, 0, 7, 16, 9, 32, 62, 64, 1, 100]
    p = synth.make_problem(lens, 2, seed=21, init_state=True, ckpt=offs)
    ref = oracle.prefill_problem(p)
    with np.errstate(over="ignore"):
        got = cm.prefill_problem(p, chunk=chunk, ckpt_mode=mode)
    assert _rel(got["out"], ref["out"]) < 1e-12
    assert _rel(got["final"], ref["final"]) < 1e-12
    assert _rel(got["ckpt"], ref["ckpt"]) < 1e-12


KERNEL_RECIPE = cm.KERNEL_RECIPE


@pytest.mark.parametrize("recipe", ["decomp", "fused"])
def test_kernel_precision_recipe_meets_gates_with_margin(recipe):
    rc = cm.KERNEL_RECIPE if recipe == "decomp" else cm.FUSED_RECIPE
    p = synth.make_problem([700, 1300, 64, 5], 2, seed=22, init_state=True, ckpt="inside")
    ref = oracle.prefill_problem(p)
    with np.errstate(over="ignore"):
        got = cm.prefill_problem(p, emulate=True, recipe=rc)
    out = synth.f32_from_bf16_bits(synth.bf16_bits_from_f32(got["out"]))
    assert np.max(np.abs(out - ref["out"])) < 2e-2 / 10
    assert _rel(out, ref["out"]) < 5e-3 / 2
    assert _rel(got["final"], ref["final"]) < 1e-3 / 10
    assert _rel(got["ckpt"], ref["ckpt"]) < 1e-3 / 10


def slow_decay_problem(kind, T, seed=11):
    """One sequence (H = 1, initial state) with a slowly decaying gate:
    "zero"  g = 0 (nothing decays);
    "weak"  g uniform in (-0.02, 0] per token and channel;
    "skew"  a per-channel decay rate log-uniform in [1e-4, 5] (times a
            per-token factor in [0.5, 1]), so that channels range from
            nearly frozen to forgetting at once, as per-channel gates allow."""
    p = synth.make_problem([T], 1, seed=seed, init_state=True,
                           gate="zero" if kind == "zero" else "random")
    rng = np.random.default_rng(seed + 7)
    if kind == "weak":
        p.g = (-0.02 * rng.random(p.g.shape)).astype(np.float32)
    elif kind == "skew":
        rate = -np.exp(rng.uniform(np.log(1e-4), np.log(5.0), size=(1, 1, p.g.shape[2])))
        p.g = np.clip(rate * rng.uniform(0.5, 1.0, size=p.g.shape), -5.0, 0.0).astype(np.float32)
    return p


@pytest.mark.parametrize("recipe", ["decomp", "fused"])
@pytest.mark.parametrize("kind", ["zero", "weak", "skew"])
def test_slow_decay_meets_state_gate_with_margin(kind, recipe):
    # at slow decay every rounding that reaches the state is carried to the
    # end of the sequence: the recipe must hold the state within half the
    # 1e-3 gate there, over 8192 tokens
    rc = cm.KERNEL_RECIPE if recipe == "decomp" else cm.FUSED_RECIPE
    p = slow_decay_problem(kind, 8192)
    ref = oracle.prefill_problem(p)
    with np.errstate(over="ignore"):
        got = cm.prefill_problem(p, emulate=True, recipe=rc)
    assert _rel(got["final"], ref["final"]) < 5e-4
    assert _rel(got["out"], ref["out"]) < 5e-3 / 4


def test_bf16_operands_fail_the_state_gate_at_slow_decay():
    # why the operands are fp16: with bf16 operands (U hi + lo into the
    # state update, the last K^ rows hi + lo) the state drifts past 1e-3 when
    # nothing decays, because K~ S, N Y and K^^T U carry their rounding along
    p = slow_decay_problem("zero", 2048)
    ref = oracle.prefill_problem(p)
    with np.errstate(over="ignore"):
        got = cm.prefill_problem(p, emulate=True, recipe=cm.BF16_RECIPE)
    assert _rel(got["final"], ref["final"]) > 1e-3


def test_plain_bf16_state_update_would_fail_the_state_gate():
    # why U goes hi + lo into the state update: a single bf16 rounding of U
    # there costs about 1.6e-3 relative, above the 1e-3 gate, even at the
    # configs' fast decay
    p = synth.make_problem([1500], 2, seed=23, init_state=True)
    ref = oracle.prefill_problem(p)
    rc = dict(cm.BF16_RECIPE, su=("bf16hl_last16", "bf16"))
    with np.errstate(over="ignore"):
        got = cm.prefill_problem(p, emulate=True, recipe=rc)
    assert _rel(got["final"], ref["final"]) > 1e-3


def test_operand_scale_follows_the_magnitude():
    # the per-wave power of two keeps max(|2^s S|, |2^s V|) in [4, 64], and
    # resets to [16, 32) when it leaves that range; zero keeps s
    S = np.zeros((128, 32))
    v = np.zeros((64, 32))
    s = np.zeros(32)
    assert np.array_equal(cm._update_scale(s, S, v, 16), s)
    v[3, 0] = 1000.0          # first group: s = -5, 1000 / 32 = 31.25
    v[5, 20] = 1e-3
    s2 = cm._update_scale(s, S, v, 16)
    assert np.all(s2[:16] == s2[0]) and np.all(s2[16:] == s2[16])
    assert 16 <= 1000.0 * 2.0 ** s2[0] < 32
    assert 16 <= 1e-3 * 2.0 ** s2[16] < 32
    # inside [4, 64] nothing changes
    S[0, 0] = 40.0 * 2.0 ** -s2[0]
    assert np.array_equal(cm._update_scale(s2, S, v, 16), s2)


@pytest.mark.parametrize("pieces", [2, 3, 7])
def test_chain_split_is_the_recurrence_in_fp64(pieces):
    # the state update is affine in the incoming state: a piece maps S to
    # T S + B, with T its end state from the identity with V = 0 and B its
    # end state from zero; composing the pieces that way reproduces the
    # token recurrence to rounding, also with empty pieces (a 1-chunk
    # sequence cut in 7) and an empty sequence
    p = synth.make_problem([0, 1, 64, 65, 700, 1300], 2, seed=31, init_state=True)
    ref = oracle.prefill_problem(p)
    got = cm.prefill_chain(p, pieces)
    assert _rel(got["out"], ref["out"]) < 1e-12
    assert _rel(got["final"], ref["final"]) < 1e-12
    assert np.array_equal(got["final"][0], p.initial_state[0])


@pytest.mark.parametrize("kind", ["zero", "weak", "random"])
def test_chain_split_with_kernel_rounding_meets_the_gates(kind):
    # with the operand rounding of the two-launch schedule in every run and
    # an fp32 scan, the split still holds the state within half the 1e-3 gate
    # (8192 tokens cut in 11 pieces), also at slow decay
    if kind == "random":
        p = synth.make_problem([8192], 1, seed=12, init_state=True)
    else:
        p = slow_decay_problem(kind, 8192, seed=12)
    ref = oracle.prefill_problem(p)
    with np.errstate(over="ignore"):
        got = cm.prefill_chain(p, 11, emulate=True, recipe=cm.KERNEL_RECIPE)
    out = synth.f32_from_bf16_bits(synth.bf16_bits_from_f32(got["out"]))
    assert _rel(got["final"], ref["final"]) < 5e-4
    assert _rel(out, ref["out"]) < 5e-3 / 2
    assert np.max(np.abs(out - ref["out"])) < 2e-2 / 2
