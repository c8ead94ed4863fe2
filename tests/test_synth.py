"""The seeded input generator: bf16 rounding matches torch's round-to-nearest-
even conversion, values follow the stated recipe, and seeds reproduce."""
import numpy as np
import pytest

from kda_gated_delta_chunked_amd import synth


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-8, 8, 100000),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.4e38, -3.4e38, 1e-40,
                                  np.inf, -np.inf], np.float32)]).astype(np.float32)
    ours = synth.bf16_bits_from_f32(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)
    assert np.array_equal(synth.f32_from_bf16_bits(ours),
                          torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_recipe_ranges_and_reproducibility():
    p = synth.make_problem([300, 200], 3, seed=5, init_state=True, ckpt="inside")
    q = synth.f32_from_bf16_bits(p.q).astype(np.float64)
    n = np.linalg.norm(q, axis=-1)
    assert np.all(np.abs(n - 1) < 1e-2)          # L2-normalised before the bf16 cast
    assert np.all(p.g <= 0) and np.all(p.g >= -5)
    assert np.all((p.beta > 0) & (p.beta < 1))
    assert 0.015 < p.initial_state.std() < 0.025
    assert np.all((p.ckpt_offsets >= 1) & (p.ckpt_offsets < p.seq_lens))
    p2 = synth.make_problem([300, 200], 3, seed=5, init_state=True, ckpt="inside")
    assert np.array_equal(p.q, p2.q) and np.array_equal(p.g, p2.g)
    assert list(p.cu_seqlens) == [0, 300, 500]


def test_named_workloads_shapes():
    for name, (N, T) in {"b1_t64_h1": (1, 64)}.items():
        p = synth.workload(name)
        assert p.N == N and p.T_total == T and p.H == 1
    for name, lens in {"packed_512x32": [512] * 32, "packed_128x8": [128] * 8,
                       "mixed_6": [1300, 547, 2048, 963, 271, 3063]}.items():
        p = synth.workload(name)
        assert list(p.seq_lens) == lens and not p.fixed and p.H == 12
        assert p.initial_state is not None and p.T_total == sum(lens)
    lens = synth.uniform_lengths(2003, 32, 1, 4096)
    assert len(lens) == 32 and min(lens) >= 1 and max(lens) <= 4096
