"""MI355X-native paged, quantized KV-cache decode attention.

``kvq`` is the thin ctypes binding over the C-ABI library ``libkvq.so``
(hand-written HIP kernels for gfx950); ``workloads`` and ``block_manager``
build seeded inputs and block tables on the host.
"""
