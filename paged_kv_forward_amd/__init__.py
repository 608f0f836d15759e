"""Batched paged-KV forward pass of a Llama-style decoder with fused on-device
sampling epilogues, as hand-written HIP kernels for AMD gfx950 behind a C ABI
(include/pie.h).  This package holds the kernels and the host engine
(csrc/), their build (build.py), the ctypes binding of the C ABI (_native.py)
and a small owner of torch device buffers (runtime.py)."""
from ._native import PieError  # noqa: F401
