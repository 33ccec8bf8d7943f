"""ADA (Angle-Domain Attention) paged decode for MI355X (gfx950).

Keys live in a paged cache as an 8-bit radius code plus packed b-bit
hyperspherical angle codes; the decode kernels compute attention logits from
those codes, then softmax and the bf16 value sum, without a dense key in HBM.

Submodules (imported on demand so that loading the input generator does not
require the HIP library):
  ska        ctypes binding of the C ABI in include/ska.h (libska.so)
  workloads  seeded synthetic inputs
  build      compiles libska.so for gfx950
"""
__all__ = ["ska", "workloads", "build"]
