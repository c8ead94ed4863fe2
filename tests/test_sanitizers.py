"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The fp64 oracle (oracle/kda_oracle.c), built with gcc's sanitizers, runs
  every oracle pin, threads included.
* The segment walk of kda_ckpt.h (tests/ckpt_segments_host.cpp) and libkda's
  host side (argument checks, overlap rules, workspace size, schedule choice,
  the allocation-free entry point's refusal) are built through hipcc with the
  sanitizers on the host pass only.  They run the 2000 random boundary cases
  and the C-ABI host checks of tests/test_abi.py.
* A planted heap overflow in a scratch C file must be reported, so a silent
  setup cannot pass.

Each build runs in a child process with the sanitizer runtime preloaded (the
Python interpreter is not instrumented). Any report fails the test: UBSan
halts on its first error, and ASan's leak check is off because the
interpreter keeps memory until it exits.  The analog on the pages is the
memcheck / synccheck run with zero errors (FlashInfer PR #4262, Validation).
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")
CSRC = os.path.join(ROOT, "kda_gated_delta_chunked_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
# host-pass sanitizers for hipcc lines: each flag after -Xarch_host
HOST_SAN = ["-Xarch_host", "-fsanitize=address",
            "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined"]
GCC_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
ENV_SAN = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:exitcode=86",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1:exitcode=87"}


def _gcc_runtime():
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    return path


def _clang_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found or not os.path.exists(HIPCC):
        pytest.skip("the ROCm toolchain's AddressSanitizer runtime is not installed")
    return found[-1]


def _run_child(code, preload, extra_env=None, timeout=600):
    env = dict(os.environ, LD_PRELOAD=preload, **ENV_SAN)
    env.update(extra_env or {})
    env["PYTHONPATH"] = os.pathsep.join([ROOT, TESTS, env.get("PYTHONPATH", "")])
    res = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                         timeout=timeout, cwd=ROOT)
    report = "ERROR: AddressSanitizer" in res.stderr or "runtime error:" in res.stderr
    return res, report


def test_sanitizer_reports_a_planted_overflow(tmp_path):
    rt = _gcc_runtime()
    c = tmp_path / "overflow.c"
    c.write_text("#include <stdlib.h>\n"
                 "int overflow(int n) { int* a = malloc(4 * n); int s = a[n]; free(a); return s; }\n")
    so = tmp_path / "liboverflow.so"
    subprocess.check_call(["gcc", "-O0", "-fPIC", "-shared", *GCC_SAN, str(c), "-o", str(so)])
    res, report = _run_child(f"import ctypes; ctypes.CDLL({str(so)!r}).overflow(8)", rt)
    assert report and res.returncode != 0, res.stderr[-2000:]


def test_oracle_pins_under_sanitizers(tmp_path):
    rt = _gcc_runtime()
    so = tmp_path / "liboracle_san.so"
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c99", "-fPIC", "-shared", "-pthread", *GCC_SAN,
                           "-ffp-contract=off", os.path.join(ROOT, "oracle", "kda_oracle.c"), "-o",
                           str(so), "-lm"])
    code = ("import oracle\n"
            "from oracle_pins import ALL_PINS\n"
            f"run = oracle.prefill_with_library({str(so)!r})\n"
            "for pin in ALL_PINS:\n"
            "    pin(run)\n"
            "print('pins', len(ALL_PINS))\n")
    res, report = _run_child(code, rt)
    assert res.returncode == 0 and not report, res.stderr[-4000:]
    assert "pins" in res.stdout


def test_segment_walk_under_sanitizers(tmp_path):
    rt = _clang_runtime()
    so = tmp_path / "libckpt_san.so"
    subprocess.check_call([HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
                           "--offload-arch=gfx950", *HOST_SAN, "-I", CSRC,
                           os.path.join(TESTS, "ckpt_segments_host.cpp"), "-o", str(so)])
    code = ("import ctypes, numpy as np\n"
            "import test_ckpt_segments as t\n"
            f"lib = ctypes.CDLL({str(so)!r})\n"
            "rng = np.random.default_rng(5)\n"
            "for _ in range(2000):\n"
            "    L = int(rng.integers(0, 700)); C = int(rng.integers(0, 9))\n"
            "    offs = [int(x) for x in rng.integers(-3, L + 4, size=C)]\n"
            "    honoured, segs = t._brute(offs, L)\n"
            "    h, s, ends = t._call(lib, offs, L)\n"
            "    assert h == honoured and s == segs and ends == [b for _, b in segs], (offs, L)\n"
            "print('walks ok')\n")
    res, report = _run_child(code, rt)
    assert res.returncode == 0 and not report, res.stderr[-4000:]
    assert "walks ok" in res.stdout


def test_library_host_checks_under_sanitizers(tmp_path):
    rt = _clang_runtime()
    so = tmp_path / "libkda_san.so"
    srcs = [os.path.join(CSRC, s) for s in ("kda_api.hip", "kda_fused.hip", "kda_decomp.hip",
                                             "kda_decode.hip")]
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
                           "-shared", *HOST_SAN, "-Xclang", "-target-feature", "-Xclang",
                           "-packed-fp32-ops", "-I", INCLUDE, "-I", CSRC, *srcs, "-o", str(so)],
                          stderr=subprocess.DEVNULL)
    code = ("import sys, pytest\n"
            "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', '-m', 'not gpu', "
            f"{os.path.join(TESTS, 'test_abi.py')!r}]))\n")
    res, report = _run_child(code, rt, {"KDA_LIBRARY": str(so)})
    assert res.returncode == 0 and not report, (res.stdout[-3000:], res.stderr[-3000:])
    assert " passed" in res.stdout
