"""Host-side parts of bench.py, without a GPU: the one-GPU guard, the
algorithmic byte and flop counts the roofline uses, the segment count, and
the source key that invalidates committed traffic figures."""
import json
import os
import subprocess
import sys
import types

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def shape(N, T, H, init=True, ckpt=None, lens=None):
    lens = lens or [T] * N
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return types.SimpleNamespace(N=N, H=H, T_total=int(cu[-1]), cu_seqlens=cu,
                                 initial_state=object() if init else None,
                                 ckpt_offsets=None if ckpt is None else np.asarray(ckpt, np.int32))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


def test_algorithmic_bytes_of_the_headline_shape():
    p = shape(8, 8192, 12)
    sb = bench.stage_bytes(p)
    # 1,028 B per token-head for the prepare (q, k, g, beta); 512 B per
    # token-head (v, out) and 64 KiB per state read or written for the recurrence
    assert sb["prepare"] == 8 * 8192 * 12 * 1028 == 808_452_096
    assert sb["recurrence"] == 8 * 8192 * 12 * 512 + 2 * 96 * 65536
    assert bench.algorithmic_bytes(p) == 1_223_688_192
    # no initial state: one state fewer; checkpoints: one more
    assert bench.algorithmic_bytes(shape(8, 8192, 12, init=False)) == 1_223_688_192 - 96 * 65536
    assert bench.algorithmic_bytes(shape(8, 8192, 12, ckpt=[5] * 8)) == 1_223_688_192 + 96 * 65536


def test_algorithmic_flops_per_token_head():
    per = 2 * (3 * 128 * 128 + 64 * (3 * 128 + 2 * 128) / 2 + 64 * 64 / 6)
    assert bench.algorithmic_flops(shape(1, 64, 1)) == pytest.approx(64 * per)
    assert bench.algorithmic_flops(shape(8, 8192, 12)) == pytest.approx(1.106e11, rel=1e-3)


def brute_segments(lens, offs):
    total = 0
    for L, row in zip(lens, offs):
        bounds = set(range(64, L, 64))
        last = 0
        for x in row:
            if 0 <= x <= L and x >= last:
                last = x
                if 0 < x < L:
                    bounds.add(x)
        total += len(bounds) + (1 if L > 0 else 0)
    return total


def test_segment_count_with_several_offsets():
    rng = np.random.default_rng(3)
    for _ in range(200):
        N = int(rng.integers(1, 5))
        lens = [int(x) for x in rng.integers(0, 400, N)]
        C = int(rng.integers(1, 5))
        offs = rng.integers(-10, 420, (N, C)).astype(np.int32)
        p = shape(N, 0, 1, lens=lens, ckpt=offs)
        assert bench.segments(p) == brute_segments(lens, offs.tolist()), (lens, offs)


def test_traffic_is_dropped_when_a_source_or_header_changes(tmp_path, monkeypatch):
    src, hdr = tmp_path / "k.hip", tmp_path / "h.h"
    src.write_text("kernel v1")
    hdr.write_text("header v1")
    monkeypatch.setitem(bench.KERNEL_SOURCES, "decomp", str(src))
    monkeypatch.setattr(bench, "KERNEL_HEADERS", [str(hdr)])
    sha = bench.kernel_sha("decomp")
    tf = tmp_path / "traffic.json"
    tf.write_text(json.dumps({"w": {"kda_prepare_kernel": {"source_sha256": sha,
                                                           "hbm_bytes_per_launch": 123}}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tf))
    assert bench.measured_traffic("w", "decomp", "kda_prepare_kernel") == 123
    assert bench.measured_traffic("other", "decomp", "kda_prepare_kernel") is None
    hdr.write_text("header v2")
    assert bench.kernel_sha("decomp") != sha
    assert bench.measured_traffic("w", "decomp", "kda_prepare_kernel") is None


def test_committed_traffic_entries_name_their_profiles():
    # each figure points at the committed rocprofv3 summary it came from (a
    # figure taken on older sources is still committed; bench reports null)
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    for workload, entries in t.items():
        for kernel, e in entries.items():
            assert len(e["source_sha256"]) == 64 and e["hbm_bytes_per_launch"] > 0
            assert os.path.exists(os.path.join(ROOT, "profiles", e["profile"])), (workload, kernel)
