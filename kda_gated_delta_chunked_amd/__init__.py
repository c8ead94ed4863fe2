"""MI355X-native Kimi Delta Attention (KDA) multi-token recurrent prefill.

``prefill`` runs the chunked KDA recurrence in libkda's HIP kernels for gfx950
(the library's C ABI is declared in include/kda.h); ``decode`` advances
requests held in a state pool by a few tokens.  ``synth`` draws the
seeded synthetic workloads used by the tests and the benchmark.
"""
from .ops import (DecodeProblem, KDAError, Problem, decode, decode_raw, decode_validate_raw,
                  load_library, library_path, make_decode_problem, make_problem, periodic_offsets,
                  plan, prefill, prefill_noalloc_raw, prefill_raw, validate_raw,
                  workspace_size)

__all__ = ["DecodeProblem", "KDAError", "Problem", "decode", "decode_raw", "decode_validate_raw",
           "load_library", "library_path", "make_decode_problem", "make_problem",
           "periodic_offsets", "plan", "prefill", "prefill_noalloc_raw", "prefill_raw",
           "validate_raw", "workspace_size"]
