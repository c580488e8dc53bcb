"""MI355X-native ragged per-row top-K (gfx950 HIP kernels behind a C ABI)."""
