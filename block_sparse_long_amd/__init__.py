"""MI355X-native exact-score-gated block-sparse causal prefill attention.

The compute lives in ``libbsfa.so`` (HIP kernels for gfx950 behind a C ABI declared in
include/bsfa.h). ``block_sparse_long_amd._lib`` is the thin ctypes binding; importing this
package does not load the library, the first call does, and it raises if the library is
missing (there is no CPU fallback).
"""
__version__ = "0.1.0"
