"""The segment boundaries both schedules derive from the checkpoint offsets
(kda_ckpt.h, built here for the host), against a brute-force reading of the
rule: offsets are taken in order and honoured when inside [0, L] and not
below the previous honoured one; the segments are the 64-token chunks from
the sequence start, each cut at every honoured offset strictly inside it."""
import ctypes
import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "kda_gated_delta_chunked_amd", "csrc")


@pytest.fixture(scope="module")
def lib(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("ckpt") / "libckpt_host.so")
    subprocess.check_call([hipcc, "-O1", "-std=c++17", "-fPIC", "-shared", "--offload-arch=gfx950",
                           "-I", CSRC, os.path.join(os.path.dirname(__file__), "ckpt_segments_host.cpp"),
                           "-o", out])
    return ctypes.CDLL(out)


def _brute(offs, L):
    honoured, last = [], 0
    for c, p in enumerate(offs):
        if 0 <= p <= L and p >= last:
            honoured.append(c)
            last = p
    cuts = {offs[c] for c in honoured if 0 < offs[c] < L and offs[c] % 64}
    points = sorted(set(range(64, L, 64)) | cuts)
    edges = [0] + points + [L] if L > 0 else [0]
    segs = [(edges[i], edges[i + 1]) for i in range(len(edges) - 1)]
    return honoured, segs


def _call(lib, offs, L):
    a = np.asarray(offs, np.int32)
    C = len(a)
    P = ctypes.c_void_p
    cap = 4096
    lo_hi = np.zeros(2 * cap, np.int32)
    n = lib.kda_test_segments(P(a.ctypes.data) if C else None, C, L, P(lo_hi.ctypes.data), cap)
    ends = np.zeros(cap, np.int32)
    m = lib.kda_test_walk(P(a.ctypes.data) if C else None, C, L, P(ends.ctypes.data), cap)
    mask = np.zeros(max(C, 1), np.int32)
    lib.kda_test_honoured(P(a.ctypes.data) if C else None, C, L, P(mask.ctypes.data))
    segs = [(int(lo_hi[2 * j]), int(lo_hi[2 * j + 1])) for j in range(n)]
    return [c for c in range(C) if mask[c]], segs, [int(e) for e in ends[:m]]


@pytest.mark.parametrize("offs,L", [([], 0), ([], 1), ([], 64), ([], 65), ([5], 200), ([64], 200),
                                    ([0, 200], 200), ([77, 5], 300), ([5, 5, 70, 64, 300], 300),
                                    ([-1, 130, -1], 130), ([201, 100], 200), ([63, 65, 127, 129], 192)])
def test_cases(lib, offs, L):
    honoured, segs = _brute(offs, L)
    h, s, ends = _call(lib, offs, L)
    assert h == honoured and s == segs and ends == [b for _, b in segs]


def test_random(lib):
    rng = np.random.default_rng(3)
    for _ in range(2000):
        L = int(rng.integers(0, 700))
        C = int(rng.integers(0, 9))
        offs = [int(x) for x in rng.integers(-3, L + 4, size=C)]
        if rng.random() < 0.5:
            offs.sort()
        honoured, segs = _brute(offs, L)
        h, s, ends = _call(lib, offs, L)
        assert h == honoured, (offs, L)
        assert s == segs, (offs, L)
        assert ends == [b for _, b in segs], (offs, L)
        assert all(0 < b - a <= 64 for a, b in segs)


def test_sequence_range_stays_inside_the_tensors(lib):
    # cu_seqlens that break the contract (negative, past T_total, decreasing)
    # give a shorter or empty range inside [0, T_total], never one outside;
    # well-formed entries pass through unchanged
    out = np.zeros(2, np.int64)
    P = ctypes.c_void_p
    f = lib.kda_test_seq_range
    f.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, P]
    rng = np.random.default_rng(4)
    for _ in range(2000):
        T = int(rng.integers(0, 1000))
        b, e = (int(x) for x in rng.integers(-50, T + 50, size=2))
        f(b, e, T, P(out.ctypes.data))
        bos, ln = int(out[0]), int(out[1])
        assert 0 <= bos <= T and 0 <= ln and bos + ln <= T, (b, e, T, bos, ln)
        if 0 <= b <= e <= T:
            assert (bos, ln) == (b, e - b)
        else:
            # the clamped range is the part of [b, e) inside [0, T] (empty when there is none)
            assert bos == min(max(b, 0), T) and ln == max(min(e, T) - bos, 0), (b, e, T)
