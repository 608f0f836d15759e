"""Oracle: a plain, slow CPU implementation of the batched forward pass and its
epilogues, written from the pages with contiguous (unpaged) KV.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package; only the tests, the smoke check and the CPU-baseline leg
of the benchmark do.  It shares no code with the HIP path: the only common
dependency is the seeded input generator ``synth``, which holds none of the
method's arithmetic.

Arithmetic is IEEE double, with rounding applied only at the storage points
that the GPU path also has (bf16 GEMM inputs, bf16 q, bf16 or e4m3 KV, fp32
residual stream, fp32 logits).  ``exact=True`` turns every intermediate
rounding off (used to compare against an independent library model).

Pins (tests/test_oracle_*.py) tie every function to something other than
itself: closed forms, brute force, library routines and invariants.  The one
function without such a pin is listed in its docstring as "parity unpinned".

Modules:
  numerics  - fp32 / bf16 / e4m3 rounding
  philox    - Philox4x32-10 counter-based generator
  model     - RMSNorm, RoPE, attention, SwiGLU, one decoder layer, the forward
  epilogue  - reduce_argmax and gumbel_max
  run       - driving whole workloads (chains and trees of chunks)
"""
from . import numerics, philox, model, epilogue, run  # noqa: F401
