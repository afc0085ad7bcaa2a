"""Plain, slow, fp64 CPU oracle for the KDA mixer core.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call, link or
run anything in this package; only the tests, the smoke check and the benchmark's
CPU-baseline leg do.  It shares no code with the HIP library.

Contents
  kda_ref.py   numpy fp64: the token-by-token recurrence, the sigmoid-gated RMSNorm,
               and a chunked (UT-transform) form of the same recurrence used only to
               check that algebra.
  kda_ref.c    the same token-by-token recurrence and norm in C (fp64, OpenMP over
               independent (sequence, head) units), for the full-size workloads.
  cref.py      ctypes wrapper and gcc build step for kda_ref.c.

Parity status: every function is pinned by tests/test_oracle_pins.py (closed forms,
invariants, a hand-worked example, textbook/library special cases).
"""
