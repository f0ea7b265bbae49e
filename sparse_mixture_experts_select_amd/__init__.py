"""MI355X (gfx950) sparse mixture-of-experts feed-forward layer.

The layer runs in hand-written HIP kernels behind the C ABI of
``include/moe_ffn.h`` (``libmoe_ffn.so``); ``binding`` is a thin ctypes
wrapper with the same entry-point names.  ``inputs`` draws the seeded
synthetic workloads.  Importing this package loads nothing; importing
``binding`` loads the GPU library and raises if it has not been built.
"""
