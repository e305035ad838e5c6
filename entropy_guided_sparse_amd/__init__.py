"""Entropy-guided, head-adaptive sparse prefill attention and decode-time KV
retention for AMD Instinct MI355X (gfx950).

The compute path is libegs.so (hand-written HIP kernels behind the C ABI in
include/egs.h); `api` marshals torch tensors onto it.  Importing `api`
requires the built library.
"""
__version__ = "0.1.0"
