"""MI355X-native quantized mixture-of-experts FFN layer (gfx950 HIP kernels behind a C ABI)."""
