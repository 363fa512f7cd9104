"""MI355X-native paged KV append + PagedAttention forward (HIP, gfx950).

The compute lives in ``libpa.so`` (built from ``csrc/``) behind a C ABI
declared in ``include/pa.h``; this package only marshals arguments to it.
"""
