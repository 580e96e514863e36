"""CPU oracle for the single-stream DiT block (test infrastructure only).

A plain, slow, fp64 NumPy implementation of what the block computes, written
from the pages' descriptions of Qwen-Image-2.1 and its ports.  It exists to
judge the HIP path: only ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import it.  It shares no code with the HIP
path; the only module both sides use is ``ditsynth`` (seeded inputs).

Every function is pinned in ``tests/test_oracle_*.py`` against something other
than itself (brute force on tiny inputs, closed forms, invariants, library
routines, values fixed by the pages).  Precision: fp64, except where floating
point decides an integer (int8 quantization), which is taken in fp32 as the
pages fix fp32 scales.
"""
from .dit_oracle import *  # noqa: F401,F403
