"""MI355X-native chunk-parallel gated delta-rule (GDN / KDA) prefill.

The compute path is the C-ABI library ``libgdn_mi355x.so`` (hand-written HIP
kernels for gfx950, declared in ``include/gdn.h``); :mod:`.gdn` is its thin
ctypes binding.  Importing this package loads nothing; the library is loaded on
first use and a missing library is an error, never a fallback.
"""
