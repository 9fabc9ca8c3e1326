"""Plain, slow fp64 CPU oracle of the DeepSeek-V4-Flash compressed attention layer.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import this package.
The product path (the HIP library and its Python binding) never calls it and never
falls back to it.  It shares no code with the HIP path: inputs arrive as arrays, and
the only thing both sides share is the seeded input generator.

Modules:
  csa_oracle  vectorised numpy fp64 implementation, processed per query, with
              per-row entry points for sampled checks at full size.
  brute       pure-Python scalar loops for tiny inputs (S <= 64), a second and
              independent transcription used to pin csa_oracle.
"""
from .csa_oracle import *  # noqa: F401,F403
