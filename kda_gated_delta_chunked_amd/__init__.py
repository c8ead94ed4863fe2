"""MI355X-native Kimi Delta Attention (KDA) multi-token recurrent prefill.

``prefill`` runs the chunked KDA recurrence in libkda's HIP kernels for gfx950
(the library's C ABI is declared in include/kda.h).  ``synth`` draws the
seeded synthetic workloads used by the tests and the benchmark.
"""
from .ops import (KDAError, Problem, load_library, library_path, make_problem, plan, prefill,
                  prefill_raw, validate_raw, workspace_size)

__all__ = ["KDAError", "Problem", "load_library", "library_path", "make_problem", "plan",
           "prefill", "prefill_raw", "validate_raw", "workspace_size"]
