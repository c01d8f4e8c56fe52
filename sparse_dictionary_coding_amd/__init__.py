"""FAD-KV screening sparse coder with fixed-size dictionary adaptation, for MI355X (gfx950).

The compute path lives in ``libfadkv.so`` (hand-written HIP kernels behind a C ABI declared in
``include/fadkv.h``); ``fadkv`` is its thin ctypes binding.  Importing this package does not
load the library; the first call into :mod:`sparse_dictionary_coding_amd.fadkv` does, and it
raises if the library is missing.
"""
__all__ = ["fadkv", "synth"]
