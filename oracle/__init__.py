"""CPU oracle for paged KV-cache attention.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
reference used by the test suite, by ``__graft_entry__.smoke()`` and by the
benchmark's ``cpu_baseline`` leg.  The GPU library (``paged_kv_cache_442_amd``)
never imports, links or calls anything here, and nothing here imports the GPU
library: the two share no code.  The only shared module is the seeded input
generator, which holds none of the method's arithmetic.

Contents (each function cites the page passage it follows):

* ``fpbits``        -- exact decoding of fp16 / bf16 / fp32 bit patterns to float64.
* ``sizes``         -- KV bytes per token and per block, pool sizing, internal waste.
* ``attention``     -- gather through the block table, then textbook two-pass
                       softmax attention in float64 (decode rows and causal
                       chunked-prefill rows); partition statistics and the
                       log-sum-exp merge of partitions.
* ``cache_ops``     -- slot-mapped K/V writes and whole-block copies as bit copies.
* ``block_manager`` -- a pure-Python model of the block manager (free list,
                       reference counts, block tables, copy-on-write, release of
                       blocks behind a sliding window).
* ``fp8``           -- exact decoding of e4m3 codes and quantization (scale, clamp,
                       round to nearest even) for an FP8 KV cache.

Every function here is pinned by ``-m "not gpu"`` tests to facts fixed by the
pages and by mathematics (closed forms, special cases, brute force); none is
marked "parity unpinned".
"""

from . import fpbits, sizes, attention, cache_ops, block_manager, fp8  # noqa: F401
