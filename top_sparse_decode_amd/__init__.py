"""MI355X-native top-k sparse decode attention over a paged KV cache.

The compute path is the HIP library ``libsparse_decode.so`` (built from
``csrc/``) behind the C ABI declared in ``include/sparse_decode.h``; the
binding in :mod:`top_sparse_decode_amd.api` only marshals arguments into it.
:mod:`top_sparse_decode_amd.synth` draws seeded synthetic inputs.

Importing this package loads nothing: the library is opened on first use, and
a missing library is an error (there is no fallback path).
"""

__all__ = ["api", "synth"]
