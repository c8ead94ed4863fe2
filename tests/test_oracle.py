"""The fp64 oracle against its pins, and the pins against planted mistakes.

The second half copies kda_oracle.c, plants one plausible mistake per copy
(a dropped term, a wrong sign, a wrong index, a transposed operand, a wrong
order of steps, an off-by-one in the bookkeeping), builds it with gcc and
checks that at least one pin rejects it.  Mistakes are planted in the oracle's
source on the CPU only.
"""
import os
import subprocess

import numpy as np
import pytest

import oracle
from oracle_pins import ALL_PINS

ORACLE_SRC = os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.c")


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle.prefill)


def _swap_blocks(src, first, second, end):
    """Swap the source between markers first..second and second..end."""
    i, j, k = src.index(first), src.index(second), src.index(end)
    return src[:i] + src[j:k] + src[i:j] + src[k:]


MUTANTS = {
    "prediction_uses_query": lambda s: s.replace("p[j] += S[d * V + j] * kt[d];",
                                                 "p[j] += S[d * V + j] * qt[d];"),
    "correction_sign": lambda s: s.replace("S[d * V + j] += c * (vt[j] - p[j]);",
                                           "S[d * V + j] += c * (p[j] - vt[j]);"),
    "beta_dropped": lambda s: s.replace("const double c = bt * kt[d];", "const double c = kt[d];"),
    "decay_halved": lambda s: s.replace("const double a = exp((double)gt[d]);",
                                        "const double a = exp(0.5 * (double)gt[d]);"),
    "decay_wrong_axis": lambda s: s.replace(
        "const double a = exp((double)gt[d]);\n      for (int j = 0; j < V; ++j) S[d * V + j] *= a;",
        "for (int j = 0; j < V; ++j) S[d * V + j] *= exp((double)gt[j % K]);"),
    "readout_transposed": lambda s: s.replace("o[j] += S[d * V + j] * qt[d];",
                                              "o[j] += S[(j % K) * V + (d % V)] * qt[d];"),
    "scale_dropped": lambda s: s.replace("o[j] *= J->scale;", "o[j] *= 1.0;"),
    "decay_after_correction": lambda s: _swap_blocks(s, "    /* decay:", "    /* prediction",
                                                     "    /* read-out"),
    "readout_before_update": lambda s: _swap_blocks(s, "    /* prediction", "    /* read-out",
                                                    "    if (ckpt_at == t + 1)"),
    "ckpt_off_by_one": lambda s: s.replace("if (ckpt_at == t + 1)", "if (ckpt_at == t)"),
    "ckpt_zero_missing": lambda s: s.replace("if (ckpt_at == 0)", "if (ckpt_at == -2)"),
    "seq_len_short": lambda s: s.replace(
        "len = (long)J->cu_seqlens[n + 1] - (long)J->cu_seqlens[n];",
        "len = (long)J->cu_seqlens[n + 1] - (long)J->cu_seqlens[n] - (J->cu_seqlens[n + 1] > J->cu_seqlens[n]);"),
    "fixed_layout_one_sequence": lambda s: s.replace("bos = (long)n * len;", "bos = (long)n * len; if (n > 0) len = 0;"),
    "initial_state_transposed": lambda s: s.replace(
        "(double)J->initial_state[state_off + (size_t)d * V + j]",
        "(double)J->initial_state[state_off + (size_t)((d * V + j) % K) * V + (d * V + j) / K]"),
    "key_upcast_truncated": lambda s: s.replace("kt[d] = bf16_bits_to_double(J->k[row * K + d]);",
                                                "kt[d] = bf16_bits_to_double(J->k[row * K + d] & 0xFFF0);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_planted_mistake(name, tmp_path):
    src = open(ORACLE_SRC).read()
    bad = MUTANTS[name](src)
    assert bad != src, f"mutation {name} did not apply"
    c = tmp_path / "mutant.c"
    c.write_text(bad)
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O1", "-std=c99", "-fPIC", "-shared", "-pthread", str(c), "-o",
                           str(so), "-lm"])
    run = oracle.prefill_with_library(str(so))
    caught = []
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(run)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin rejects the planted mistake {name}"
