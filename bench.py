"""Paged-attention decode benchmark on one MI355X.

A step is one decode step of one layer over the whole batch: the newest token of
every sequence is written into its slot and the decode runs over every context
(``pa_cache_and_decode``: the cache write and the work plan in one launch, then the
per-partition attention, then the log-sum-exp merge of partitions).
Inputs (pool, tables, queries) are resident in HBM before timing starts.

The JSON line reports:
  value      algorithmic K+V+Q bytes per step / step time, in GB/s, where the step time
             is the median over regions (at least five) of the timed steps, each timed by
             events at its boundaries only (p10 / p90 over the regions beside it);
  roofline   the partition kernel's algorithmic bytes / its mean duration (fence-free HIP
             events on the launch stream around each launch of an instrumented pass of
             the same steps) against 8 TB/s HBM peak;
  read_ceilings_GBps  what a read-only probe kernel gets from HBM over a pool-sized
             buffer: one stream, random 4 KiB tiles, random 32 KiB tiles;
  cpu_baseline  the float64 CPU oracle timed on a bounded sample of the same
             workload (a few sequences), as GB/s of algorithmic bytes.
"""

import argparse
import json
import math
import os
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0

WORKLOADS = {
    "llama3_70b": "Llama-3-70B-shaped GQA decode layer: 128 seqs, 64 query / 8 KV heads, d 128, "
                  "bf16, block 16, lengths log-uniform [256, 8192]",
    "llama2_7b": "Llama-2-7B-shaped MHA decode layer: 64 seqs, 32/32 heads, d 128, fp16, "
                 "block 16, lengths uniform [128, 2048]",
    "mixed_chunked": "Mixed batch, one layer: 8 prefill chunks of 256-512 causal query rows over "
                     "cached prefixes of 0-4096 tokens plus 96 decode rows of 1-4096 tokens; GQA "
                     "32/8, d 128, bf16, block 32",
    "shared_prefix": "Parallel sampling, one layer: 32 groups x 4 branches forked from a 1024-token "
                     "prompt plus 1-15 decoded tokens, tails of 1-256 tokens, GQA 32/8, d 128, bf16, "
                     "block 16; 96 copy-on-write block copies, then decode of the 128 branches",
    "swap": "Swap preemption, one Llama-3-70B-shaped layer (the llama3_70b cache): every 4th of "
            "the 128 sequences swapped out to pinned host memory and back in",
    "prefix_cache": "Prefix caching, one layer: 256 requests served in order over 8 system prompts "
                    "of 512-4096 tokens plus 16-256 own tokens, 128 live at a time, GQA 64/8, d 128, "
                    "bf16, block 16; decode of the 128 live requests over shared cached blocks",
}
MFMA_BF16_PEAK_TFLOPS = 2500.0


def algorithmic_bytes(w, window=0, kv_bytes=None):
    """K+V read once per (sequence, KV head) plus Q: sum_s L_s*H_kv*d*2*e + S*H_q*d*e_q
    (with a sliding window, L_s counts only the tokens inside the window; an FP8 cache
    has e = 1 for K/V and bf16 queries)."""
    eq = 4 if w.dtype == 0 else 2
    e = eq if kv_bytes is None else kv_bytes
    lens = np.asarray(w.context_lens, dtype=np.int64)
    if window:
        lens = np.minimum(lens, window)
    kv = int(np.sum(lens)) * w.num_kv_heads * w.head_dim * 2 * e
    q = w.num_seqs * w.num_q_heads * w.head_dim * eq
    return kv + q


def counter_traffic(root, partition_tokens):
    """HBM bytes per launch of the partition kernel from the committed rocprofv3 counters.

    The counters (FETCH_SIZE, WRITE_SIZE in KiB per dispatch, each scaled by what the
    same counter reads for a plain copy of known size) hold only for the kernel source and
    the partition size they were taken on: if either differs, the figure is stale and None
    is returned.
    """
    import hashlib
    path = os.path.join(root, "profiles", "decode_partition_kernel_llama3_70b.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("partition_tokens") != partition_tokens:
        return None
    h = hashlib.sha256()
    for name in rec["source_files"]:
        with open(os.path.join(root, name), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != rec["source_sha256"]:
        return None
    return int(round(rec["fetch_kib_per_launch"] * 1024 * rec["fetch_scale"] +
                     rec["write_kib_per_launch"] * 1024 * rec["write_scale"]))


class FenceFreeEvents:
    """HIP timing events recorded without the system-scope memory fence
    (``hipEventDisableSystemFence``): a default event record writes back and invalidates
    the caches, which costs the stream several microseconds and slows the kernel after
    it.  These events only time the stream; the results are read after a device-wide
    synchronize.  They come from the HIP runtime torch has loaded (one runtime per
    process)."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, count):
        import ctypes
        import torch
        torch.cuda.init()
        path = next(line.split()[-1] for line in open("/proc/self/maps")
                    if "libamdhip64" in line and line.split()[-1].startswith("/"))
        self.hip = ctypes.CDLL(path)
        self.c = ctypes
        self.ev = []
        for _ in range(count):
            e = ctypes.c_void_p()
            rc = self.hip.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE)
            if rc != 0:
                raise RuntimeError("hipEventCreateWithFlags failed (%d)" % rc)
            self.ev.append(e)

    def record(self, i, stream):
        rc = self.hip.hipEventRecord(self.ev[i], self.c.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError("hipEventRecord failed (%d)" % rc)

    def elapsed_ms(self, i, j):
        ms = self.c.c_float()
        rc = self.hip.hipEventElapsedTime(self.c.byref(ms), self.ev[i], self.ev[j])
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed (%d)" % rc)
        return ms.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)
        self.ev = []


def worse_err(worst, got, want):
    """The larger of ``worst`` and the largest |got - want|; NaN anywhere counts as inf
    (``max`` would drop it)."""
    d = np.abs(np.asarray(got, dtype=np.float64) - np.asarray(want, dtype=np.float64))
    if not np.all(np.isfinite(d)):
        return float("inf")
    return max(worst, float(d.max()))


def make_workload(name, num_q_heads=None, fixed_len=0):
    from paged_kv_cache_442_amd import workloads as wl
    if name == "llama3_70b" and (num_q_heads or fixed_len):
        return wl.llama3_70b(num_q_heads=num_q_heads or 64, fixed_len=fixed_len)
    return {"llama3_70b": wl.llama3_70b, "llama2_7b": wl.llama2_7b}[name]()


def cpu_baseline(w, budget_s):
    """Time the float64 oracle on whole sequences until ``budget_s`` is spent."""
    from oracle import attention, fpbits
    scale = attention.default_scale(w.head_dim)
    e = 4 if w.dtype == 0 else 2
    order = np.random.default_rng(0).permutation(w.num_seqs)
    done, nbytes, t_total = [], 0, 0.0
    for s in order:
        t0 = time.perf_counter()
        kt, vt = w.seq_tokens(int(s))
        attention.contiguous_decode(w.dtype, w.q[s], fpbits.decode(w.dtype, kt),
                                    fpbits.decode(w.dtype, vt), scale)
        t_total += time.perf_counter() - t0
        done.append(int(s))
        nbytes += int(w.context_lens[s]) * w.num_kv_heads * w.head_dim * 2 * e + \
            w.num_q_heads * w.head_dim * e
        if t_total >= budget_s:
            break
    return {
        "value": round(nbytes / t_total / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": "%d of %d sequences (%d tokens), float64 numpy oracle, single thread, %.1f s"
                  % (len(done), w.num_seqs, int(np.sum(np.asarray(w.context_lens)[done])), t_total),
    }


_POOL_WORKLOAD = None


def _oracle_sequence(s):
    from oracle import attention, fpbits
    w = _POOL_WORKLOAD
    kt, vt = w.seq_tokens(int(s))
    attention.contiguous_decode(w.dtype, w.q[s], fpbits.decode(w.dtype, kt),
                                fpbits.decode(w.dtype, vt), attention.default_scale(w.head_dim))
    return int(s)


def cpu_baseline_all_cores(w, max_workers=16):
    """The same oracle over every sequence, one sequence per task (longest first) on a pool
    of worker processes, timed by the wall clock.  The pool is forked before the GPU is
    touched; each worker's numpy runs its elementwise work on one thread."""
    import multiprocessing as mp
    global _POOL_WORKLOAD
    from oracle import attention, fpbits  # noqa: F401  (imported once, before the fork)
    cores = max(1, min(max_workers, len(os.sched_getaffinity(0))))
    _POOL_WORKLOAD = w
    e = 4 if w.dtype == 0 else 2
    seqs = sorted(range(w.num_seqs), key=lambda s: -int(w.context_lens[s]))
    with mp.get_context("fork").Pool(cores) as pool:
        t0 = time.perf_counter()
        for _ in pool.imap_unordered(_oracle_sequence, seqs):
            pass
        dt = time.perf_counter() - t0
    _POOL_WORKLOAD = None
    lens = np.asarray(w.context_lens, dtype=np.int64)
    nbytes = int(lens.sum()) * w.num_kv_heads * w.head_dim * 2 * e + \
        w.num_seqs * w.num_q_heads * w.head_dim * e
    return {
        "value": round(nbytes / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": "all %d sequences (%d tokens), float64 numpy oracle, one sequence per task on "
                  "%d worker processes, %.2f s wall clock" % (w.num_seqs, int(lens.sum()), cores, dt),
    }


def copy_ceiling_gbps(torch, nbytes=1 << 30, reps=20):
    """Read+write GB/s of a plain device-to-device copy (a measured ceiling)."""
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b
    return 2 * nbytes / (ms * 1e-3) / 1e9


def region_bounds(n, min_regions=5, min_steps=50):
    """Step indices cutting K = n timed steps into regions: at least ``min_regions``, each
    of at least ``min_steps`` steps when n allows it (else min_regions equal regions)."""
    regions = max(min_regions, n // min_steps) if n >= min_regions * min_steps else min_regions
    regions = max(1, min(regions, n))
    return [round(i * n / regions) for i in range(regions + 1)]


def read_ceilings(torch, pool_bytes, reps=10, log=None):
    """Read-only GB/s that the memory system delivers to a kernel that only reads
    (libpa_probe.so), over a buffer the size of the decode pool, for three patterns: one
    contiguous stream (64 KiB tiles in order), random 4 KiB tiles (the decode kernel's
    pattern: one tile per block and KV head) and random 32 KiB tiles (all 8 KV heads of a
    block as one run).  Two ways of reading, each swept over its depth: "wg" (a workgroup
    reads whole tiles, 1-8 tiles in flight per workgroup, 1-8 workgroups of 256 threads
    per CU) and "interleaved" (consecutive threads of the whole grid read consecutive
    16-byte chunks, 4 in flight per thread, 1-16 workgroups per CU).  Each figure is the
    mean over ``reps`` launches timed by events; the best per pattern is reported with the
    configuration that reached it, the whole sweep goes to ``log``."""
    import ctypes
    from paged_kv_cache_442_amd.build import PROBE_LIB_PATH
    if not os.path.exists(PROBE_LIB_PATH):
        raise RuntimeError("libpa_probe.so is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(PROBE_LIB_PATH)
    inter = lib.pa_probe_read_tiles
    inter.restype = ctypes.c_int
    inter.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                      ctypes.c_void_p, ctypes.c_void_p]
    wg = lib.pa_probe_read_tiles_wg
    wg.restype = ctypes.c_int
    wg.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                   ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    nbytes = max(1 << 30, (pool_bytes + (1 << 20) - 1) >> 20 << 20)
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.zeros(16 * cus, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    out = {}
    rng = np.random.default_rng(0)

    def timed(launch, nbytes_read):
        if launch() != 0:
            raise RuntimeError("read probe launch failed")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            launch()
        e1.record(stream)
        torch.cuda.synchronize()
        return nbytes_read / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9

    for name, tile, shuffle in (("stream", 1 << 16, False), ("random_4KiB", 4096, True),
                                ("random_32KiB", 32768, True)):
        n_tiles = nbytes // tile
        order = rng.permutation(n_tiles) if shuffle else np.arange(n_tiles)
        assert order.max() < n_tiles and order.min() >= 0
        ids = torch.from_numpy(order.astype(np.int32)).cuda()
        args = (buf.data_ptr(), ids.data_ptr(), n_tiles, tile)
        best, where = 0.0, None
        for per_cu in (1, 2, 4, 8):
            for u in (1, 2, 4, 8):
                g = timed(lambda: wg(*args, per_cu * cus, u, sink.data_ptr(), stream.cuda_stream),
                          n_tiles * tile)
                kib = per_cu * cus * u * tile / 1024
                if log:
                    print("[read probe] %-13s wg  %d WG/CU x %d tiles in flight (%7.0f KiB chip-wide): "
                          "%7.1f GB/s" % (name, per_cu, u, kib, g), file=log, flush=True)
                if g > best:
                    best, where = g, "wg: %d workgroups/CU, %d tiles in flight each" % (per_cu, u)
        for per_cu in (1, 2, 4, 8, 16):
            g = timed(lambda: inter(*args, per_cu * cus, sink.data_ptr(), stream.cuda_stream),
                      n_tiles * tile)
            if log:
                print("[read probe] %-13s interleaved %2d WG/CU x 64 B per thread: %7.1f GB/s"
                      % (name, per_cu, g), file=log, flush=True)
            if g > best:
                best, where = g, "interleaved: %d workgroups/CU, 4 loads in flight per thread" % per_cu
        out[name] = {"GBps": round(best, 1), "config": where}
    out["bytes_read"] = int(nbytes)
    del buf
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=250,
                    help="timed steps K (cut into at least 5 regions of at least 50 steps)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="llama3_70b")
    ap.add_argument("--partition", type=int, default=0, help="partition tokens (0 = library default)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="time budget of the CPU-oracle baseline (0 disables it)")
    ap.add_argument("--no-copy-ceiling", action="store_true")
    ap.add_argument("--no-read-ceilings", action="store_true",
                    help="skip the read-probe sweep (e.g. under a profiler)")
    ap.add_argument("--num-q-heads", type=int, default=0,
                    help="diagnostic: query heads of the llama3_70b shape (default 64)")
    ap.add_argument("--kv-fp8", action="store_true",
                    help="keep K/V in an FP8 (e4m3) cache (bf16 workloads)")
    ap.add_argument("--window", type=int, default=0,
                    help="sliding-window decode over the last W tokens (pa_decode_window)")
    ap.add_argument("--fixed-len", type=int, default=0,
                    help="diagnostic: every llama3_70b sequence this many tokens long")
    ap.add_argument("--contiguous-blocks", action="store_true",
                    help="hand out blocks in order 0, 1, 2, ... (a diagnostic: no scattering)")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    from paged_kv_cache_442_amd import binding as pa
    from paged_kv_cache_442_amd import workloads as wl
    from paged_kv_cache_442_amd.session import DecodeSession

    if torch.cuda.device_count() == 0:  # counts devices without initializing the GPU
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    pa.lib()  # fail loudly if the library is missing
    if args.workload == "mixed_chunked":
        return bench_mixed(args, torch)
    if args.workload == "prefix_cache":
        return bench_prefix_cache(args, torch)
    if args.workload == "swap":
        return bench_swap(args, torch)
    if args.workload == "shared_prefix":
        return bench_shared_prefix(args, torch)

    t0 = time.perf_counter()
    w = make_workload(args.workload, args.num_q_heads, args.fixed_len)
    if args.contiguous_blocks:
        w.free_order = np.arange(w.num_blocks, dtype=np.int32)
    print("[bench] workload %s drawn in %.1f s" % (args.workload, time.perf_counter() - t0),
          file=sys.stderr, flush=True)
    # The CPU oracle baselines run before the GPU is initialized (the all-cores one forks
    # worker processes).
    cpu = cpu_all = None
    if args.cpu_seconds > 0 and not args.window:
        cpu = cpu_baseline(w, args.cpu_seconds)
        cpu_all = cpu_baseline_all_cores(w)
        print("[bench] CPU oracle baselines: %.4f GB/s on 1 core, %.4f GB/s on %d"
              % (cpu["value"], cpu_all["value"], cpu_all["cores"]), file=sys.stderr, flush=True)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    t0 = time.perf_counter()
    sess = DecodeSession(w, partition_tokens=args.partition, cache_fp8=args.kv_fp8)
    print("[bench] cache written in %.1f s" % (time.perf_counter() - t0), file=sys.stderr, flush=True)

    B = algorithmic_bytes(w, args.window, 1 if args.kv_fp8 else None)
    stream = torch.cuda.current_stream()
    if args.window:
        return bench_window(args, torch, pa, sess, w, B, stream)
    for _ in range(args.warmup):
        sess.step()
    torch.cuda.synchronize()

    n = args.steps
    # The timed region: exactly K steps of pa_cache_and_decode, synchronized on both sides,
    # cut into regions (at least five, of at least 50 steps when K allows) by fence-free
    # events at the region boundaries only: no event inside a region.  `value` comes from
    # the median region's step time; p10 / p90 over the regions are reported beside it.
    bounds = region_bounds(n)
    rev = FenceFreeEvents(len(bounds))
    # One untimed pass over the same events first: the first records of new events cost
    # the stream several microseconds more than later ones.
    for i in range(len(bounds)):
        rev.record(i, stream)
        sess.step()
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    rev.record(0, stream)
    for r in range(1, len(bounds)):
        for _ in range(bounds[r] - bounds[r - 1]):
            sess.step()
        rev.record(r, stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t_wall) * 1e3
    region_ms = np.array([rev.elapsed_ms(r - 1, r) / (bounds[r] - bounds[r - 1])
                          for r in range(1, len(bounds))])
    rev.close()
    ms_step = float(np.median(region_ms))
    total_ms = float(np.sum(region_ms * np.diff(bounds)))

    # The instrumented pass (after the timed region, same steps, same stream): fence-free
    # events around every partition-kernel launch of K steps, for the roofline.
    ev = FenceFreeEvents(2 * n)

    def instrumented():
        for i in range(n):
            sess.cache_and_decode_plan()       # the cache write and the plan: one launch
            ev.record(2 * i, stream)
            sess.decode_partitions()
            ev.record(2 * i + 1, stream)
            sess.decode_reduce()

    instrumented()                             # untimed: first records of the events
    torch.cuda.synchronize()
    instrumented()
    torch.cuda.synchronize()
    part_ms = np.array([ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(n)])
    ev.close()

    # Outside the timed region: the other kernels' times (events around every kernel).
    nb = min(n, 20)
    bev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(nb)]
    for e in bev:
        e[0].record(stream)
        sess.write_new_tokens()
        e[1].record(stream)
        sess.decode_plan()
        e[2].record(stream)
        sess.cache_and_decode_plan()
        e[3].record(stream)
        sess.decode_partitions()
        e[4].record(stream)
        sess.decode_reduce()
        e[5].record(stream)
    torch.cuda.synchronize()
    write_ms = np.array([e[0].elapsed_time(e[1]) for e in bev])
    plan_ms = np.array([e[1].elapsed_time(e[2]) for e in bev])
    fused_ms = np.array([e[2].elapsed_time(e[3]) for e in bev])
    red_ms = np.array([e[4].elapsed_time(e[5]) for e in bev])

    def plain_ms(step):
        u0, u1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        u0.record(stream)
        for _ in range(n):
            step()
        u1.record(stream)
        torch.cuda.synchronize()
        return u0.elapsed_time(u1) / n

    ms_step_separate = plain_ms(sess.step_separate)

    part_avg_s = float(part_ms.mean()) * 1e-3
    achieved = B / part_avg_s / 1e9
    part_tokens = args.partition or pa.pa_decode_default_partition(sess.pool, w.num_q_heads)
    value = B / (ms_step * 1e-3) / 1e9

    # sampled parity against the oracle on the timed output
    from oracle import attention, fpbits
    got = sess.out.cpu().numpy().astype(np.float64)
    lens = np.asarray(w.context_lens)
    worst = 0.0
    def cache_values(bits, scale):
        x = fpbits.decode(w.dtype, bits)
        if not args.kv_fp8:
            return x
        from oracle import fp8
        codes = fp8.quantize(x.astype(np.float32), np.float32(1.0) / np.float32(scale))
        return fp8.dequantize(codes, scale)

    for s in sorted({int(np.argmin(lens)), int(np.argmax(lens))}):
        kt, vt = w.seq_tokens(s)
        want = attention.contiguous_decode(w.dtype, w.q[s], cache_values(kt, sess.k_scale),
                                           cache_values(vt, sess.v_scale),
                                           attention.default_scale(w.head_dim))
        worst = worse_err(worst, got[s], want)

    # host block manager: one appended token per sequence (A1), on a host-only pool
    hp = pa.pa_alloc_pool(pa.make_desc(1, w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim,
                                       w.dtype), None, w.free_order)
    hseqs = [pa.pa_seq_new(hp) for _ in range(w.num_seqs)]
    for s, L in zip(hseqs, lens):
        pa.pa_seq_append(hp, s, int(L) - 1)
    t0 = time.perf_counter()
    pa.pa_seq_append_batch(hp, hseqs)      # one scheduling step: one token per sequence
    host_mgr_us = (time.perf_counter() - t0) * 1e6

    blocks = sum(-(-int(L) // w.block_size) for L in lens)
    waste = 1.0 - float(lens.sum()) / (blocks * w.block_size)

    ceiling = None if args.no_copy_ceiling else copy_ceiling_gbps(torch)
    rceiling = None if args.no_read_ceilings else read_ceilings(torch, sess.storage.numel(), log=sys.stderr)

    line = {
        "metric": "paged-decode KV GB/s and % of HBM peak at 1 MI355X; tokens/sec per layer",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": n,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 kv, bf16 q" if args.kv_fp8 else
                 ("bf16" if w.dtype == wl.BF16 else ("f16" if w.dtype == wl.F16 else "f32")),
        "data": "synthetic (seeded N(0,1) K/V/Q, seeded block permutation)",
        "config": {
            "workload": args.workload,
            "description": WORKLOADS[args.workload],
            "num_seqs": w.num_seqs, "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
            "head_dim": w.head_dim, "block_size": w.block_size, "num_blocks": w.num_blocks,
            "total_context_tokens": int(lens.sum()), "max_context": int(lens.max()),
            "partition_tokens": part_tokens,
            "block_placement": "contiguous" if args.contiguous_blocks else "seeded permutation",
            "kv_cache": "fp8-e4m3" if args.kv_fp8 else "same as q",
            "algorithmic_bytes_per_step": B,
        },
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "tokens_per_s_per_layer": round(w.num_seqs / (ms_step * 1e-3), 1),
        "ms_per_step_p10_p50_p90": [round(float(x), 5) for x in np.percentile(region_ms, [10, 50, 90])],
        "timing": {"regions": len(bounds) - 1, "steps_per_region": [int(x) for x in np.diff(bounds)],
                   "statistic": "median of the regions' mean step times (fence-free events at "
                                "region boundaries only)",
                   "timed_steps_gpu_ms": round(total_ms, 4), "timed_steps_wall_ms": round(wall_ms, 3)},
        "ms_per_step_four_launches": round(ms_step_separate, 5),
        "partition_ms_p10_p50_p90": [round(float(x), 5) for x in np.percentile(part_ms, [10, 50, 90])],
        "kernel_ms": {"cache_write_and_plan": round(float(fused_ms.mean()), 5),
                      "decode_partitions": round(float(part_ms.mean()), 5),
                      "decode_reduce": round(float(red_ms.mean()), 5),
                      "reshape_and_cache_alone": round(float(write_ms.mean()), 5),
                      "decode_plan_alone": round(float(plan_ms.mean()), 5)},
        "roofline": {
            "bound": "hbm",
            "kernel": "decode_partition_kernel",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "launches_timed": "%d, by fence-free HIP events around each partition launch in an "
                              "instrumented pass of %d steps right after the timed region" % (n, n),
            # The committed counters belong to the default Llama-3-70B run.
            "traffic": counter_traffic(os.path.dirname(os.path.abspath(__file__)), part_tokens)
            if (args.workload == "llama3_70b" and not args.kv_fp8 and not args.num_q_heads
                and not args.fixed_len and not args.contiguous_blocks) else None,
        },
        "copy_ceiling_GBps": None if ceiling is None else round(ceiling, 1),
        "read_ceilings_GBps": rceiling,
        "max_abs_err_sampled": worst,
        "internal_waste_pct": round(100 * waste, 3),
        "host_manager_us_per_step": round(host_mgr_us, 1),
        "cpu_baseline": cpu,
        "cpu_baseline_all_cores": cpu_all,
    }
    print(json.dumps(line), flush=True)


def bench_window(args, torch, pa, sess, w, B, stream):
    """Sliding-window decode: a step is one pa_cache_and_decode_window call (the new
    tokens' write with the plan, partitions, merge); its time is the decode figure."""
    import math as _m
    tables = sess.tables
    def decode():
        pa.pa_cache_and_decode_window(sess.pool, 0, sess.new_k, sess.new_v, sess.new_slots, sess.q,
                                      tables, sess.ctx, sess.max_context, args.window, sess.scale,
                                      sess.out, sess.workspace, sess.partition_tokens)
    for _ in range(args.warmup):
        decode()
    torch.cuda.synchronize()
    n = args.steps
    ev = FenceFreeEvents(2 * n)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def steps():
        for i in range(n):
            ev.record(2 * i, stream)
            decode()
            ev.record(2 * i + 1, stream)

    steps()  # untimed: warms the events
    torch.cuda.synchronize()
    t0.record(stream)
    steps()
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / n
    dec_ms = float(np.mean([ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(n)]))
    ev.close()
    from oracle import attention, fpbits
    got = sess.out.cpu().numpy().astype(np.float64)
    lens = np.asarray(w.context_lens)
    worst = 0.0
    for s_ in sorted({int(np.argmin(lens)), int(np.argmax(lens))}):
        kt, vt = w.seq_tokens(s_)
        want = attention.window_decode(w.dtype, w.q[s_], fpbits.decode(w.dtype, kt),
                                       fpbits.decode(w.dtype, vt), attention.default_scale(w.head_dim),
                                       args.window)
        worst = worse_err(worst, got[s_], want)
    achieved = B / (dec_ms * 1e-3) / 1e9
    line = {
        "metric": "paged-decode KV GB/s and % of HBM peak at 1 MI355X; tokens/sec per layer",
        "value": round(B / (ms_step * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1, "steps": n,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if w.dtype == 2 else "f16",
        "data": "synthetic (seeded N(0,1) K/V/Q, seeded block permutation)",
        "config": {"workload": args.workload + "_window", "window": args.window,
                   "algorithmic_bytes_per_step": B,
                   # windowed calls take at most 2048-token partitions by default
                   "partition_tokens": args.partition or min(
                       pa.pa_decode_default_partition(sess.pool, w.num_q_heads), 2048)},
        "tokens_per_s_per_layer": round(w.num_seqs / (ms_step * 1e-3), 1),
        "kernel_ms": {"decode_window (plan + partitions + merge)": round(dec_ms, 5)},
        "roofline": {"bound": "hbm", "kernel": "pa_cache_and_decode_window (write + plan, partitions, merge)", "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": None},
        "max_abs_err_sampled": worst, "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def bench_mixed(args, torch):
    """The mixed chunked-prefill + decode batch: one step = the chunk rows' and decode rows'
    K/V writes, pa_prefill_chunked over the chunks, pa_decode over the decode rows."""
    from paged_kv_cache_442_amd import workloads as wl
    from paged_kv_cache_442_amd.session import PrefillSession

    t0 = time.perf_counter()
    w = wl.chunked_prefill()
    sess = PrefillSession(w, partition_tokens=args.partition)
    print("[bench] mixed batch ready in %.1f s" % (time.perf_counter() - t0), file=sys.stderr,
          flush=True)
    e = 2
    Hq, Hkv, d = w.num_q_heads, w.num_kv_heads, w.head_dim
    # Prefill: every visible (row, key) pair costs 2 MACs per query head and dim (QK, PV).
    visible = sum(int(w.chunk_lens[i]) * int(w.prefix_lens[i]) +
                  int(w.chunk_lens[i]) * (int(w.chunk_lens[i]) + 1) // 2 for i in range(sess.n_chunks))
    prefill_flops = 4 * Hq * d * visible
    prefill_kv_bytes = int(np.sum(w.prefix_lens + w.chunk_lens)) * Hkv * d * 2 * e
    prefill_q_bytes = int(np.sum(w.chunk_lens)) * Hq * d * e
    decode_bytes = int(np.sum(w.decode_lens)) * Hkv * d * 2 * e + sess.n_decode * Hq * d * e
    B = prefill_kv_bytes + prefill_q_bytes + decode_bytes

    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        sess.step()
    torch.cuda.synchronize()
    n = args.steps
    # The timed region: events only around the prefill and decode calls.
    ev = FenceFreeEvents(3 * n)
    t_start = torch.cuda.Event(enable_timing=True)
    t_stop = torch.cuda.Event(enable_timing=True)

    def steps():
        for i in range(n):
            sess.write_step_tokens()
            ev.record(3 * i, stream)
            sess.prefill()
            ev.record(3 * i + 1, stream)
            sess.decode()
            ev.record(3 * i + 2, stream)

    steps()  # untimed: warms the events
    torch.cuda.synchronize()
    t_start.record(stream)
    steps()
    t_stop.record(stream)
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_stop) / n
    prefill_ms = float(np.mean([ev.elapsed_ms(3 * i, 3 * i + 1) for i in range(n)]))
    decode_ms = float(np.mean([ev.elapsed_ms(3 * i + 1, 3 * i + 2) for i in range(n)]))
    ev.close()
    # outside it: the cache write's time
    wev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(min(n, 20))]
    for e in wev:
        e[0].record(stream)
        sess.write_step_tokens()
        e[1].record(stream)
        sess.prefill()
        sess.decode()
    torch.cuda.synchronize()
    write_ms = float(np.mean([x[0].elapsed_time(x[1]) for x in wev]))
    prefill_tflops = prefill_flops / (prefill_ms * 1e-3) / 1e12
    value = B / (ms_step * 1e-3) / 1e9
    # The same step with the decode rows on a second (default-priority) stream, overlapping
    # the prefill; timed with no event inside the loop.
    side = torch.cuda.Stream()
    sess.step_overlapped(side)
    torch.cuda.synchronize()
    o0, o1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    o0.record(stream)
    for _ in range(n):
        sess.step_overlapped(side)
    o1.record(stream)
    torch.cuda.synchronize()
    ms_step_overlapped = o0.elapsed_time(o1) / n

    # sampled parity against the oracle on the timed outputs: first and last rows of the
    # first and last chunks, first and last decode rows
    from oracle import attention, fpbits
    scale = attention.default_scale(d)

    def seq_kv(i):
        a_, b_ = w.token_offsets[i], w.token_offsets[i + 1]
        return fpbits.decode(w.dtype, w.k_tokens[a_:b_]), fpbits.decode(w.dtype, w.v_tokens[a_:b_])

    got_c = sess.out_c.cpu().numpy().astype(np.float64)
    got_d = sess.out_d.cpu().numpy().astype(np.float64)
    worst = 0.0
    for i in sorted({0, sess.n_chunks - 1}):
        kc, vc = seq_kv(i)
        for r in sorted({0, int(w.chunk_lens[i]) - 1}):
            pos = int(w.prefix_lens[i]) + r
            want = attention.contiguous_decode(w.dtype, w.q_chunks[int(w.chunk_offsets[i]) + r],
                                               kc[:pos + 1], vc[:pos + 1], scale)
            worst = worse_err(worst, got_c[int(w.chunk_offsets[i]) + r], want)
    for j in sorted({0, sess.n_decode - 1}):
        kc, vc = seq_kv(sess.n_chunks + j)
        want = attention.contiguous_decode(w.dtype, w.q_decode[j], kc, vc, scale)
        worst = worse_err(worst, got_d[j], want)
    rows = int(np.sum(w.chunk_lens)) + sess.n_decode
    line = {
        "metric": "paged-decode KV GB/s and % of HBM peak at 1 MI355X; tokens/sec per layer",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": n,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) K/V/Q, seeded block permutation)",
        "config": {
            "workload": "mixed_chunked",
            "description": WORKLOADS["mixed_chunked"],
            "chunk_rows": int(np.sum(w.chunk_lens)), "decode_rows": sess.n_decode,
            "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": d, "block_size": w.block_size,
            "algorithmic_bytes_per_step": B, "prefill_algorithmic_flops": prefill_flops,
        },
        "tokens_per_s_per_layer": round(rows / (ms_step * 1e-3), 1),
        "kernel_ms": {"reshape_and_cache": round(write_ms, 5), "prefill_chunked": round(prefill_ms, 5),
                      "decode": round(decode_ms, 5)},
        "roofline": {
            "bound": "mfma",
            "kernel": "prefill_kernel",
            "achieved": round(prefill_tflops, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(prefill_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": None,
        },
        "decode_rows_GBps": round(decode_bytes / (decode_ms * 1e-3) / 1e9, 2),
        "ms_per_step_overlapped": round(ms_step_overlapped, 5),
        "value_overlapped": round(B / (ms_step_overlapped * 1e-3) / 1e9, 2),
        "tokens_per_s_per_layer_overlapped": round(rows / (ms_step_overlapped * 1e-3), 1),
        "max_abs_err_sampled": worst,
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def bench_shared_prefix(args, torch):
    """Parallel sampling: decode of 128 branches whose tables share their group's context
    blocks, and the 96 copy-on-write block copies.  Logical bytes count every branch's
    tokens; unique bytes count each distinct block once."""
    from paged_kv_cache_442_amd import workloads as wl
    from paged_kv_cache_442_amd.session import SharedPrefixSession
    from oracle import attention, fpbits

    w = wl.shared_prefix()
    sess = SharedPrefixSession(w)
    torch.cuda.synchronize()
    e, Hq, Hkv, d, bs = 2, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    S = len(sess.seqs)
    B = int(np.sum(sess.lens)) * Hkv * d * 2 * e + S * Hq * d * e
    t = sess.tables_host
    B_unique = int(np.unique(t[t >= 0]).size) * bs * Hkv * d * 2 * e + S * Hq * d * e
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    for _ in range(args.warmup):
        sess.decode()
    torch.cuda.synchronize()
    n = args.steps
    dec = [(ev(), ev()) for _ in range(n)]
    for i in range(n):
        dec[i][0].record(stream)
        sess.decode()
        dec[i][1].record(stream)
    torch.cuda.synchronize()
    dec_ms = float(np.mean([a.elapsed_time(b) for a, b in dec]))
    # The copies again, from the same sources into free blocks: the real destinations now
    # hold the branches' own tokens and must not be overwritten.
    from paged_kv_cache_442_amd import binding as pa
    free = pa.pa_export_free_stack(sess.pool)[:len(sess.cow_pairs)]
    timing_pairs = torch.tensor([(s_, int(f)) for (s_, _), f in zip(sess.cow_pairs, free)],
                                dtype=torch.int32, device="cuda")
    for _ in range(args.warmup):
        pa.pa_copy_blocks(sess.pool, timing_pairs)
    cp = [(ev(), ev()) for _ in range(n)]
    for i in range(n):
        cp[i][0].record(stream)
        pa.pa_copy_blocks(sess.pool, timing_pairs)
        cp[i][1].record(stream)
    torch.cuda.synchronize()
    cp_ms = float(np.mean([a.elapsed_time(b) for a, b in cp]))
    copy_bytes = 2 * len(sess.cow_pairs) * pa_block_bytes_of(sess)
    got = sess.out.cpu().numpy().astype(np.float64)
    worst = 0.0
    for idx in (0, S - 1):
        s_ = sess.seqs[idx]
        kt, vt = sess.branch_tokens(s_)
        want = attention.contiguous_decode(w.dtype, w.q[sess.branch_of[s_]], fpbits.decode(w.dtype, kt),
                                           fpbits.decode(w.dtype, vt), attention.default_scale(d))
        worst = worse_err(worst, got[idx], want)
    value = B / (dec_ms * 1e-3) / 1e9
    line = {
        "metric": "paged-decode KV GB/s and % of HBM peak at 1 MI355X; tokens/sec per layer",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": n, "warmup": args.warmup,
        "ms_per_step": round(dec_ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) K/V/Q, seeded block permutation)",
        "config": {"workload": "shared_prefix", "description": WORKLOADS["shared_prefix"],
                   "branches": S, "cow_pairs": len(sess.cow_pairs), "num_blocks": w.num_blocks,
                   "logical_bytes_per_step": B, "unique_bytes_per_step": B_unique},
        "tokens_per_s_per_layer": round(S / (dec_ms * 1e-3), 1),
        "roofline": {"bound": "hbm", "kernel": "pa_decode (plan + partitions + merge)",
                     "achieved": round(value, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(value / HBM_PEAK_GBPS, 4), "traffic": None,
                     "note": "logical bytes; the unique set (unique_bytes_per_step) is read once "
                             "per branch, mostly from cache"},
        "unique_GBps": round(B_unique / (dec_ms * 1e-3) / 1e9, 2),
        "copy_blocks": {"pairs": len(sess.cow_pairs), "ms": round(cp_ms, 5),
                        "GBps_read_plus_write": round(copy_bytes / (cp_ms * 1e-3) / 1e9, 2)},
        "max_abs_err_sampled": worst, "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def pa_block_bytes_of(sess):
    from paged_kv_cache_442_amd import binding as pa
    return pa.pa_block_bytes(sess.desc)


def bench_swap(args, torch):
    """Swap preemption: pa_seq_swap_out / pa_seq_swap_in on the host, pa_swap_blocks
    (one launch moving whole blocks over the host link) timed each way; a torch copy of
    the same byte count between pinned host memory and the device is the measured
    ceiling of the link."""
    from paged_kv_cache_442_amd import binding as pa
    from paged_kv_cache_442_amd import workloads as wl
    from paged_kv_cache_442_amd.session import DecodeSession
    from oracle import attention, fpbits

    w = wl.llama3_70b()
    sess = DecodeSession(w)
    sess.write_new_tokens()          # every token of every sequence is in the cache
    torch.cuda.synchronize()
    pool = sess.pool
    victims = list(range(0, w.num_seqs, 4))
    vseqs = [sess.seqs[i] for i in victims]
    tables, _ = pa.pa_export_block_tables(pool, vseqs, sess.max_blocks)
    n_blocks = int((tables >= 0).sum())
    M = n_blocks
    pa.pa_pool_set_swap_space(pool, M)
    host = torch.empty(pa.pa_swap_space_bytes(sess.desc, M), dtype=torch.uint8, pin_memory=True)
    block_bytes = pa.pa_block_bytes(sess.desc)
    nbytes = n_blocks * block_bytes
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    out_ms, in_ms = [], []
    for it in range(args.warmup + max(1, args.steps // 10)):
        t0 = time.perf_counter()
        pairs = pa.pa_seq_swap_out(pool, vseqs)
        host_out_us = (time.perf_counter() - t0) * 1e6
        p_out = torch.tensor(pairs, dtype=torch.int32).reshape(-1, 2).cuda()
        e0, e1 = ev(), ev()
        e0.record(stream)
        pa.pa_swap_blocks(pool, host, p_out, True)
        e1.record(stream)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        pairs_in = pa.pa_seq_swap_in(pool, vseqs)
        host_in_us = (time.perf_counter() - t0) * 1e6
        p_in = torch.tensor(pairs_in, dtype=torch.int32).reshape(-1, 2).cuda()
        e2, e3 = ev(), ev()
        e2.record(stream)
        pa.pa_swap_blocks(pool, host, p_in, False)
        e3.record(stream)
        torch.cuda.synchronize()
        if it >= args.warmup:
            out_ms.append(e0.elapsed_time(e1))
            in_ms.append(e2.elapsed_time(e3))
    # The swapped sequences decode correctly from their new blocks.
    tables, ctx = pa.pa_export_block_tables(pool, sess.seqs, sess.max_blocks)
    sess.tables.copy_(torch.from_numpy(tables))
    sess.decode()
    torch.cuda.synchronize()
    got = sess.out.cpu().numpy().astype(np.float64)
    worst = 0.0
    for s_ in victims[:2]:
        kt, vt = w.seq_tokens(s_)
        want = attention.contiguous_decode(w.dtype, w.q[s_], fpbits.decode(w.dtype, kt),
                                           fpbits.decode(w.dtype, vt), attention.default_scale(w.head_dim))
        worst = worse_err(worst, got[s_], want)
    # Ceiling: one contiguous DMA copy of the same size each way.
    dev = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    hview = host[:nbytes]
    ceil = {}
    for name, fn in (("d2h", lambda: hview.copy_(dev, non_blocking=True)),
                     ("h2d", lambda: dev.copy_(hview, non_blocking=True))):
        fn()
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record(stream)
        for _ in range(3):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ceil[name] = nbytes / (e0.elapsed_time(e1) / 3 * 1e-3) / 1e9
    out_gbps = nbytes / (float(np.mean(out_ms)) * 1e-3) / 1e9
    in_gbps = nbytes / (float(np.mean(in_ms)) * 1e-3) / 1e9
    line = {
        "metric": "paged-decode KV GB/s and % of HBM peak at 1 MI355X; tokens/sec per layer",
        "value": round(min(out_gbps, in_gbps), 2), "unit": "GB/s", "n_gpus": 1,
        "steps": len(out_ms), "warmup": args.warmup,
        "ms_per_step": round(float(np.mean(out_ms)) + float(np.mean(in_ms)), 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) K/V/Q, seeded block permutation)",
        "config": {"workload": "swap", "description": WORKLOADS["swap"],
                   "swapped_sequences": len(victims), "blocks_moved": n_blocks,
                   "bytes_each_way": nbytes},
        "swap_out_GBps": round(out_gbps, 2), "swap_in_GBps": round(in_gbps, 2),
        "swap_out_ms": round(float(np.mean(out_ms)), 4), "swap_in_ms": round(float(np.mean(in_ms)), 4),
        "host_manager_us": {"swap_out": round(host_out_us, 1), "swap_in": round(host_in_us, 1)},
        "roofline": {"bound": "host link", "kernel": "swap_blocks_kernel",
                     "achieved": round(min(out_gbps, in_gbps), 2),
                     "peak": round(min(ceil["d2h"], ceil["h2d"]), 2), "unit": "GB/s",
                     "frac": round(min(out_gbps / ceil["d2h"], in_gbps / ceil["h2d"]), 4),
                     "traffic": None,
                     "note": "peak = measured contiguous DMA copy of the same size (torch), each way"},
        "dma_ceiling_GBps": {k: round(v, 2) for k, v in ceil.items()},
        "max_abs_err_sampled": worst, "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def bench_prefix_cache(args, torch):
    """Prefix caching: every request is admitted through the caching manager (its host
    calls timed), only its uncached tokens' K/V are written, then pa_decode over the live
    requests is timed.  Logical bytes count every token of every sequence; unique bytes
    count each distinct block once (shared system-prompt blocks are read by many
    sequences in one launch)."""
    from paged_kv_cache_442_amd import workloads as wl
    from paged_kv_cache_442_amd.session import PrefixCacheSession
    from oracle import attention, fpbits

    t0 = time.perf_counter()
    w = wl.prefix_cache(seed=7, num_requests=256, num_system=8, min_system=512, max_system=4096,
                        min_user=16, max_user=256, num_q_heads=64, num_kv_heads=8, block_size=16,
                        release_after=127, pool_fraction=0.0)
    sess = PrefixCacheSession(w)
    for i in range(w.num_requests):
        sess.admit(i)
    torch.cuda.synchronize()
    print("[bench] %d requests admitted in %.1f s" % (w.num_requests, time.perf_counter() - t0),
          file=sys.stderr, flush=True)
    live = sess.live()
    a = sess.decode_args(live)
    e, Hq, Hkv, d, bs = 2, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    lens = np.array([len(w.tokens(r)) for r in live], dtype=np.int64)
    B = int(lens.sum()) * Hkv * d * 2 * e + len(live) * Hq * d * e
    tables = a["tables_host"]
    unique_blocks = int(np.unique(tables[tables >= 0]).size)
    B_unique = unique_blocks * bs * Hkv * d * 2 * e + len(live) * Hq * d * e

    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        sess.run_decode(a)
    torch.cuda.synchronize()
    n = args.steps
    t_start, t_stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for _ in range(n):
        sess.run_decode(a)
    t_stop.record(stream)
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_stop) / n

    got = a["out"].cpu().numpy().astype(np.float64)
    worst = 0.0
    for j in sorted({int(np.argmin(lens)), int(np.argmax(lens))}):
        toks = w.tokens(live[j])
        k, v = w.kv_rows(toks, np.arange(len(toks)))
        want = attention.contiguous_decode(w.dtype, w.q[live[j]], fpbits.decode(w.dtype, k),
                                           fpbits.decode(w.dtype, v), attention.default_scale(d))
        worst = worse_err(worst, got[j], want)

    prompt_tokens = sum(len(w.prompt(i)) for i in range(w.num_requests))
    cached = int(sess.cached_tokens.sum())
    value = B / (ms_step * 1e-3) / 1e9
    line = {
        "metric": "paged-decode KV GB/s and % of HBM peak at 1 MI355X; tokens/sec per layer",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": n, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded token ids; K/V rows a seeded function of id and position)",
        "config": {"workload": "prefix_cache", "description": WORKLOADS["prefix_cache"],
                   "requests": w.num_requests, "live_decoded": len(live), "num_blocks": w.num_blocks,
                   "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": d, "block_size": bs,
                   "logical_bytes_per_step": B, "unique_bytes_per_step": B_unique},
        "tokens_per_s_per_layer": round(len(live) / (ms_step * 1e-3), 1),
        "roofline": {"bound": "hbm", "kernel": "pa_decode (plan + partitions + merge)",
                     "achieved": round(value, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(value / HBM_PEAK_GBPS, 4), "traffic": None,
                     "note": "logical bytes: shared blocks are read once per sequence, mostly "
                             "from cache; unique bytes / time is unique_GBps"},
        "unique_GBps": round(B_unique / (ms_step * 1e-3) / 1e9, 2),
        "prompt_tokens": prompt_tokens, "cached_prompt_tokens": cached,
        "cached_fraction": round(cached / prompt_tokens, 4),
        "cached_blocks_evicted": int(sess.evicted.sum()),
        "host_admission_us_mean": round(float(sess.host_seconds.mean()) * 1e6, 1),
        "host_admission_us_max": round(float(sess.host_seconds.max()) * 1e6, 1),
        "max_abs_err_sampled": worst, "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
