"""MI355X-native causal packed microscaled (E4M3 / UE8M0) flash attention.

The computation lives in libflamia.so (HIP kernels for gfx950, C ABI in
include/flamia.h); ``bit_causal_flash_amd.flamia`` is its ctypes binding."""
