"""STCA target-to-history cross-attention forward for MI355X (gfx950).

The compute path is the HIP library ``libstca.so`` behind the C ABI in
``include/stca.h``; ``recsys_ultra_long_amd.stca`` is its thin Python binding.
Importing the package loads nothing; ``stca.load()`` loads the library.
"""
__all__ = ["inputs", "stca"]
