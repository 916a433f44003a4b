"""Weight-only-quantized decode GEMV for MI355X (gfx950).

The compute lives in the HIP library ``libwqd.so`` behind a C ABI; the Python
binding (``weight_quantized_decode_block_amd.wqd``) only marshals arguments.
Importing this package does not load the library; the first call does, and
raises if it has not been built.
"""
