"""MI355X-native EXL3 trellis-quantized linear (HIP kernels behind a C ABI)."""
