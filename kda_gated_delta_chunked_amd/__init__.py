"""MI355X-native Kimi Delta Attention (KDA) multi-token recurrent prefill.

``prefill`` runs the chunked KDA recurrence in libkda's HIP kernels for gfx950
(the library's C ABI is declared in include/kda.h); ``decode`` advances
requests held in a state pool by a few tokens, and ``decode_verify`` then
``decode_commit`` or ``decode_advance`` do the same for speculative drafts,
keeping the state of the accepted prefix.  ``synth`` draws the
seeded synthetic workloads used by the tests and the benchmark.
"""
from .ops import (DecodeProblem, KDAError, Problem, decode, decode_advance, decode_advance_raw,
                  decode_commit, decode_commit_raw, decode_raw, decode_validate_raw, decode_verify,
                  decode_verify_raw,
                  load_library, library_path, make_decode_problem, make_problem, periodic_offsets,
                  plan, prefill, prefill_noalloc_raw, prefill_raw, validate_raw,
                  workspace_size)

__all__ = ["DecodeProblem", "KDAError", "Problem", "decode", "decode_advance", "decode_advance_raw",
           "decode_commit", "decode_commit_raw", "decode_raw", "decode_validate_raw", "decode_verify",
           "decode_verify_raw",
           "load_library", "library_path", "make_decode_problem", "make_problem",
           "periodic_offsets", "plan", "prefill", "prefill_noalloc_raw", "prefill_raw",
           "validate_raw", "workspace_size"]
