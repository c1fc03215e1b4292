"""Block-wise FP8 linear layer for AMD Instinct MI355X (gfx950).

The compute path is the HIP library ``libfp8bs.so`` (C ABI declared in
``include/fp8bs.h``); ``fp8_block_scaled_x128_amd.ops`` is its thin ctypes
binding.  ``inputs`` holds the seeded synthetic workload generators.
"""
__all__ = ["ops", "inputs"]
