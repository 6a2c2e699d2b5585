"""MI355X-native slow-fast decode attention (SFI) with verification-guided selection.

The compute path is ``libsfi.so`` (HIP kernels for gfx950 behind a C ABI,
declared in ``include/sfi.h``); :mod:`dynamic_sparse_kv_amd.sfi` is its thin
ctypes binding.  Importing the package loads nothing; the binding loads the
library on first use and raises if it has not been built.
"""
__all__ = ["workload", "sfi"]
