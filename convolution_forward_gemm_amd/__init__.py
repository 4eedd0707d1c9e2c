"""MI355X-native 2D convolution forward (fprop) as an implicit GEMM.

The compute path is the C-ABI library ``libconvfprop.so`` (hand-written HIP
kernels for gfx950), declared in ``include/convfprop.h``.  ``binding`` is the
thin ctypes layer over it; importing it loads the library and raises if the
library is missing.  ``workloads`` holds the seeded synthetic inputs.
"""
