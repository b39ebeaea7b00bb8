"""DSpark confidence-scheduled speculative decoding: the per-token draft
sampling / confidence / prefix scheduling / lossless verification path as
hand-written HIP kernels for AMD Instinct MI355X (gfx950), behind the C-ABI of
libdsp.so (include/dsp.h).

Modules:
  dsp        ctypes binding with the C-ABI names (marshalling only)
  engine     Round: the four entry points issued in order for one decode round
  workloads  seeded synthetic inputs of the workloads the path is measured on
  build      in-tree hipcc build of libdsp.so
"""
