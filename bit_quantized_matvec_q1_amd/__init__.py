"""Packed 1-bit and ternary weight x int8 activation products on AMD Instinct MI355X (gfx950).

The product lives in liblowbit.so (hand-written HIP kernels behind the C ABI in include/lowbit.h);
``bit_quantized_matvec_q1_amd.lowbit`` is its Python binding.
"""
