"""Single-pass attention backward for AMD MI355X (gfx950).

The compute lives in ``libfa_bwd.so`` (HIP kernels behind a C ABI, declared in
``include/fa_bwd.h``); ``attention_backward_fa_amd.binding`` is the thin ctypes
layer over it. Importing this package loads nothing; the library is opened on
first use and the call fails loudly if it has not been built.
"""
