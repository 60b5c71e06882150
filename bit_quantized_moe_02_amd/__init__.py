"""MI355X-native (gfx950) quantized routed-MoE layer: HIP kernels behind a
C ABI (include/qmoe.h, libqmoe.so) and a thin Python binding (qmoe.py)."""
