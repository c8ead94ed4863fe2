"""Pins of the oracle's input prologue: q and k divided by their L2 norms per
token and head, beta given as a logit (the in-kernel options FlashInfer PR
#4262 lists in its dispatch contract).

Hand-worked case, K = V = 2, scale 1, zero initial state:
  token 1: q = (3, 4), k = (0, 2), v = (1, 2), g = (0, 0), beta logit ln 3.
           q^ = (0.6, 0.8), k^ = (0, 1), beta = 1 / (1 + 1/3) = 0.75.
           p = 0, S = 0.75 k^ v^T = [[0, 0], [0.75, 1.5]],
           o = S^T q^ = (0.75 * 0.8, 1.5 * 0.8) = (0.6, 1.2).
  token 2: q = (0, 5), k = (1, 0), v = (2, 0), g = (0, 0), beta logit 0.
           q^ = (0, 1), k^ = (1, 0), beta = 0.5.
           p = S^T k^ = (0, 0) (row 0 of S is zero),
           S = S + 0.5 k^ v^T = [[1, 0], [0.75, 1.5]],
           o = S^T q^ = row 1 = (0.75, 1.5).
"""
import math
import os
import subprocess

import numpy as np
import pytest

import oracle
from kda_gated_delta_chunked_amd.synth import bf16_bits_from_f32


def _hand_inputs():
    q = np.array([[[3.0, 4.0]], [[0.0, 5.0]]], np.float32)
    k = np.array([[[0.0, 2.0]], [[1.0, 0.0]]], np.float32)
    v = np.array([[[1.0, 2.0]], [[2.0, 0.0]]], np.float32)
    g = np.zeros((2, 1, 2), np.float32)
    beta = np.array([[math.log(3.0)], [0.0]], np.float32)
    return (bf16_bits_from_f32(q), bf16_bits_from_f32(k), bf16_bits_from_f32(v), g, beta)


def test_hand_worked_two_tokens():
    q, k, v, g, beta = _hand_inputs()
    r = oracle.prefill(q, k, v, g, beta, scale=1.0, num_seqs=1, qk_l2norm=True, beta_logit=True,
                       threads=1)
    # the fp32 logit ln 3 gives beta = 0.75 to within 1e-7
    assert np.allclose(r["out"][0, 0], [0.6, 1.2], rtol=0, atol=1e-7)
    assert np.allclose(r["out"][1, 0], [0.75, 1.5], rtol=0, atol=1e-7)
    assert np.allclose(r["final"][0, 0], [[1.0, 0.0], [0.75, 1.5]], rtol=0, atol=1e-7)


def test_flags_off_leave_inputs_as_given():
    # without the prologue the inputs are used as they are: token 1 then has
    # beta = b = ln 3, S = b k v^T = [[0, 0], [2b, 4b]] and o = S^T q = (8b, 16b)
    q, k, v, g, beta = _hand_inputs()
    r = oracle.prefill(q, k, v, g, beta, scale=1.0, num_seqs=1, threads=1)
    b = float(np.float32(math.log(3.0)))
    assert np.allclose(r["out"][0, 0], [b * 2 * 4 * 1, b * 2 * 4 * 2], rtol=1e-12)


def test_normalisation_removes_power_of_two_scales():
    # scaling q and k by powers of two is exact in bf16 and fp64, so with the
    # prologue the results are bit for bit those of the unscaled inputs
    from kda_gated_delta_chunked_amd import synth
    p = synth.make_problem([40, 25], 2, seed=90, init_state=True)
    base = oracle.prefill_problem(p, qk_l2norm=True, beta_logit=True, threads=1)
    q = synth.f32_from_bf16_bits(p.q) * np.float32(8.0)
    k = synth.f32_from_bf16_bits(p.k) * np.float32(0.25)
    scaled = oracle.prefill(bf16_bits_from_f32(q), bf16_bits_from_f32(k), p.v, p.g, p.beta,
                            scale=p.scale, num_seqs=p.N, cu_seqlens=p.cu_seqlens,
                            initial_state=p.initial_state, qk_l2norm=True, beta_logit=True,
                            threads=1)
    assert np.array_equal(base["out"], scaled["out"])
    assert np.array_equal(base["final"], scaled["final"])


def test_zero_vectors_stay_zero():
    q, k, v, g, beta = _hand_inputs()
    k[0] = 0
    q[0] = 0
    r = oracle.prefill(q, k, v, g, beta, scale=1.0, num_seqs=1, qk_l2norm=True, threads=1)
    assert np.all(np.isfinite(r["out"])) and not np.any(r["out"][0])


def _prologue_pins(run):
    """The pins above, against a given build of the oracle."""
    q, k, v, g, beta = _hand_inputs()
    r = run(q, k, v, g, beta, scale=1.0, num_seqs=1, qk_l2norm=True, beta_logit=True, threads=1)
    assert np.allclose(r["out"][0, 0], [0.6, 1.2], rtol=0, atol=1e-7)
    assert np.allclose(r["out"][1, 0], [0.75, 1.5], rtol=0, atol=1e-7)
    k0 = k.copy()
    k0[0] = 0
    r = run(q, k0, v, g, beta, scale=1.0, num_seqs=1, qk_l2norm=True, threads=1)
    assert np.all(np.isfinite(r["out"]))


ORACLE_SRC = os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.c")
PROLOGUE_MUTANTS = {
    "q_by_key_norm": lambda s: s.replace("if (nq > 0.0) qt[d] /= nq;", "if (nk > 0.0) qt[d] /= nk;"),
    "norm_not_square_rooted": lambda s: s.replace("nk = sqrt(nk);", "nk = nk;"),
    "sigmoid_sign": lambda s: s.replace("bt = 1.0 / (1.0 + exp(-bt));", "bt = 1.0 / (1.0 + exp(bt));"),
    "logit_ignored": lambda s: s.replace("if (J->flags & 2) bt", "if (J->flags & 8) bt"),
    "zero_vector_divided": lambda s: s.replace("if (nk > 0.0) kt[d] /= nk;", "kt[d] /= nk;"),
}


@pytest.mark.parametrize("name", sorted(PROLOGUE_MUTANTS))
def test_prologue_pins_reject_planted_mistake(name, tmp_path):
    src = open(ORACLE_SRC).read()
    bad = PROLOGUE_MUTANTS[name](src)
    assert bad != src, f"mutation {name} did not apply"
    c = tmp_path / "mutant.c"
    c.write_text(bad)
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O1", "-std=c99", "-fPIC", "-shared", "-pthread", str(c), "-o",
                           str(so), "-lm"])
    run = oracle.prefill_with_library(str(so))
    with pytest.raises(AssertionError):
        with np.errstate(all="ignore"):
            _prologue_pins(run)
