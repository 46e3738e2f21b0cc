"""Paged KV-cache attention for AMD Instinct MI355X (gfx950).

The compute path lives in ``libpa.so`` (hand-written HIP kernels plus the host
block manager behind a C ABI, declared in ``include/pa.h``); ``binding`` is a
thin ctypes layer over it.  ``workloads`` draws seeded synthetic inputs.
"""
