"""The C ABI from C: tests/c_consumer.c, compiled as C99 against include/kda.h
and linked to libkda.so, calls the host-only entry points (no device).  Its
struct layouts must equal the Python binding's ctypes mirrors, and its results
must equal the same calls made through the binding."""
import ctypes
import os
import shutil
import subprocess

import pytest

import kda_gated_delta_chunked_amd as K
from kda_gated_delta_chunked_amd import ops

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.fixture(scope="module")
def consumer_output(tmp_path_factory):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    K.load_library()
    libdir = os.path.dirname(ops.library_path())
    exe = str(tmp_path_factory.mktemp("c_consumer") / "c_consumer")
    cmd = [gcc, "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror",
           "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "c_consumer.c"),
           "-L", libdir, "-lkda", f"-Wl,-rpath,{libdir}", "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stderr
    out = {}
    for line in run.stdout.splitlines():
        key, _, val = line.partition(" ")
        out[key] = val
    return out


@pytest.mark.parametrize("struct, name", [(ops.Problem, "kda_problem"),
                                          (ops.DecodeProblem, "kda_decode_problem")])
def test_struct_layouts_match_the_binding(consumer_output, struct, name):
    assert int(consumer_output[f"sizeof.{name}"]) == ctypes.sizeof(struct)
    fields = [f for f, _ in struct._fields_]
    seen = [k.split(".", 1)[1] for k in consumer_output if k.startswith(name + ".")]
    assert seen == fields, "field order of the header and the binding differ"
    for f in fields:
        off, size = (int(x) for x in consumer_output[f"{name}.{f}"].split())
        desc = getattr(struct, f)
        assert (off, size) == (desc.offset, desc.size), f


def test_workspace_sizes_match_the_binding(consumer_output):
    probs = [K.make_problem(8, 8 * 8192, 12, scale=0.0884, variant="auto"),
             K.make_problem(5, 1000, 3, scale=0.0884, variant="decomp", ckpt_per_seq=3),
             K.make_problem(8, 8 * 8192, 12, scale=0.0884, variant="fused"),
             K.make_problem(1, 8192, 12, scale=0.0884, variant="auto"),
             K.make_problem(1, 8192, 12, scale=0.0884, variant="decomp", chain_parts=4)]
    for i, p in enumerate(probs):
        status, nbytes = (int(x) for x in consumer_output[f"workspace.{i}"].split())
        assert status == 0
        assert nbytes == K.workspace_size(p)
    assert int(consumer_output["workspace.2"].split()[1]) == 0


def test_validation_results_from_c(consumer_output):
    OK, INVALID, UNSUPPORTED, ALIGN, OVERLAP, WS = 0, -1, -2, -3, -4, -5
    want = {"validate.good": OK, "validate.misaligned": ALIGN, "validate.alias_out_v": OK,
            "validate.overlap_out_q": OVERLAP, "validate.head_dim": UNSUPPORTED,
            "validate.bound": INVALID, "validate.no_workspace": WS,
            "decode.good": OK, "decode.empty_pool": INVALID,
            "verify.no_out": INVALID, "verify.trace_on_pool": OVERLAP,
            "commit.no_accepted": INVALID, "commit.trace_on_pool": OVERLAP,
            "advance.no_accepted": INVALID}
    for key, status in want.items():
        assert int(consumer_output[key]) == status, key


def test_status_strings_from_c(consumer_output):
    lib = K.load_library()
    for s in range(-8, 1):
        assert consumer_output[f"status.{s}"] == lib.kda_status_string(s).decode()
