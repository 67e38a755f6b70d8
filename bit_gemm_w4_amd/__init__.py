"""MI355X-native W4A16 / W8A8 quantized linear layer (HIP kernels for gfx950).

The operations live in :mod:`bit_gemm_w4_amd.ops`, a thin ctypes binding over
``libbitgemm.so``; importing this package does not load the library, so the
seeded input generator (:mod:`bit_gemm_w4_amd.synth`) stays usable on hosts
without a GPU.
"""
__all__ = ["ops", "synth"]
