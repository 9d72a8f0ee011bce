"""MI355X-native fused Gaussian-mixture EM iteration.

The compute runs in hand-written HIP kernels for gfx950 inside libgmm.so
(C ABI declared in include/gmm.h); `soft_clustering_amd.gmm` is the thin
ctypes binding.  Importing this package loads nothing; the library is opened
on first use and its absence is an error, never a fallback.
"""
__all__ = ["gmm", "synth"]
