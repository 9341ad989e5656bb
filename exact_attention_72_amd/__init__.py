"""MI355X-native fused exact-attention forward (gfx950 HIP kernels behind a C ABI)."""
