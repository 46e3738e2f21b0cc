"""Drive libpa end to end for one workload: pool, block manager, slot writes, decode.

A ``DecodeSession`` places a ``workloads.DecodeWorkload`` into a paged cache the way
a serving engine would: the block manager allocates blocks as each sequence grows
(blocks taken from the seeded free order, so they land scattered), the history
tokens' K/V rows go to their slots with ``pa_reshape_and_cache``, and one decode
step then writes each sequence's newest token and runs ``pa_decode``.  Everything
here is argument marshalling and call order; every computation runs in libpa.
"""

import math
import time

import numpy as np
import torch

from . import binding as pa
from . import workloads as wl

_TORCH = {wl.F32: torch.float32, wl.F16: torch.float16, wl.BF16: torch.bfloat16}
FP8 = pa.FP8_E4M3


def bits_to_device(bits, dtype, device):
    """Raw-bit numpy array -> GPU tensor of the storage dtype (a bit copy)."""
    if dtype == wl.F32:
        host = torch.from_numpy(np.ascontiguousarray(bits).view(np.float32))
    else:
        host = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(_TORCH[dtype])
    return host.to(device)


def nan_fill(storage, dtype):
    """Fill a pool's bytes with the quiet-NaN pattern of its dtype."""
    if dtype == FP8:
        storage.fill_(0x7F)
    else:
        storage.view(_TORCH[dtype]).fill_(float("nan"))


def fp8_scale(bits, dtype):
    """A per-tensor FP8 scale for bf16/fp16 rows: the largest magnitude maps to 448."""
    x = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(_TORCH[dtype]).float()
    amax = float(x.abs().max()) if x.numel() else 1.0
    return max(amax, 1e-30) / 448.0


class DecodeSession:
    def __init__(self, w, device="cuda", partition_tokens=0, num_layers=1, layer=0, poison=True,
                 max_context=None, chunk_tokens=1 << 16, cache_fp8=False):
        """``cache_fp8``: keep the (bf16) workload's K/V in an FP8 cache, with per-tensor
        scales from the data's largest magnitude."""
        self.w = w
        self.device = device
        self.layer = layer
        self.partition_tokens = partition_tokens
        self.dtype = w.dtype
        self.cache_dtype = FP8 if cache_fp8 else w.dtype
        if cache_fp8 and w.dtype != wl.BF16:
            raise ValueError("an FP8 cache takes bf16 rows")
        self.desc = pa.make_desc(num_layers, w.num_blocks, w.block_size, w.num_kv_heads,
                                 w.head_dim, self.cache_dtype)
        nbytes = pa.pa_pool_bytes(self.desc)
        self.storage = torch.empty(nbytes, dtype=torch.uint8, device=device)
        if poison:
            nan_fill(self.storage, self.cache_dtype)
        self.pool = pa.pa_alloc_pool(self.desc, self.storage, w.free_order)
        self.k_scale = self.v_scale = 1.0
        if cache_fp8:
            self.k_scale = fp8_scale(w.k_tokens, w.dtype)
            self.v_scale = fp8_scale(w.v_tokens, w.dtype)
            pa.pa_pool_set_kv_scales(self.pool, layer, self.k_scale, self.v_scale)
        S = w.num_seqs
        lens = np.asarray(w.context_lens, dtype=np.int64)
        self.seqs = [pa.pa_seq_new(self.pool) for _ in range(S)]

        # History: every token but the newest of each sequence.
        hist_slots = []
        for s in range(S):
            n = int(lens[s]) - 1 if lens[s] > 0 else 0
            hist_slots.append(pa.pa_seq_append(self.pool, self.seqs[s], n)[0])
        # The step's new token (one per non-empty sequence).
        new_slots = np.full(S, -1, dtype=np.int64)
        for s in range(S):
            if lens[s] > 0:
                new_slots[s] = pa.pa_seq_append(self.pool, self.seqs[s], 1)[0][0]
        self.history_slots = hist_slots
        self.new_slots_host = new_slots

        # Write history rows in bounded chunks (keeps device staging small).
        offs = w.token_offsets
        rows = np.concatenate([np.arange(offs[s], offs[s] + len(hist_slots[s])) for s in range(S)]) \
            if S else np.zeros(0, np.int64)
        slots = np.concatenate(hist_slots) if S else np.zeros(0, np.int64)
        for a in range(0, len(rows), chunk_tokens):
            idx = rows[a:a + chunk_tokens]
            k = bits_to_device(w.k_tokens[idx], w.dtype, device)
            v = bits_to_device(w.v_tokens[idx], w.dtype, device)
            sl = torch.from_numpy(slots[a:a + chunk_tokens]).to(device)
            pa.pa_reshape_and_cache(self.pool, layer, k, v, sl)
        torch.cuda.synchronize()

        last = np.where(lens > 0, offs[1:] - 1, 0)
        self.new_k = bits_to_device(w.k_tokens[last] if S else w.k_tokens[:0], w.dtype, device)
        self.new_v = bits_to_device(w.v_tokens[last] if S else w.v_tokens[:0], w.dtype, device)
        self.new_slots = torch.from_numpy(new_slots).to(device)

        self.max_blocks = max(1, max((-(-int(L) // w.block_size) for L in lens), default=1))
        tables, ctx = pa.pa_export_block_tables(self.pool, self.seqs, self.max_blocks)
        self.tables_host, self.ctx_host = tables, ctx
        self.tables = torch.from_numpy(tables).to(device)
        self.ctx = torch.from_numpy(ctx).to(device)
        self.max_context = int(lens.max()) if (max_context is None and S) else (max_context or 0)
        self.q = bits_to_device(w.q, w.dtype, device)
        self.out = torch.empty(S, w.num_q_heads, w.head_dim, dtype=torch.float32, device=device)
        ws = pa.pa_decode_workspace_bytes(self.pool, S, w.num_q_heads, self.max_context,
                                          partition_tokens)
        self.workspace = torch.empty(ws, dtype=torch.uint8, device=device)
        self.scale = 1.0 / math.sqrt(w.head_dim)

    # ---------------------------------------------------------------- one decode step
    def write_new_tokens(self, stream=None):
        pa.pa_reshape_and_cache(self.pool, self.layer, self.new_k, self.new_v, self.new_slots,
                                stream)

    def decode(self, stream=None):
        pa.pa_decode(self.pool, self.layer, self.q, self.tables, self.ctx, self.max_context,
                     self.scale, self.out, self.workspace, self.partition_tokens, stream)

    def decode_plan(self, stream=None):
        pa.pa_decode_plan(self.pool, self.layer, self.q, self.tables, self.ctx, self.max_context,
                          self.scale, self.out, self.workspace, self.partition_tokens, stream)

    def decode_partitions(self, stream=None):
        pa.pa_decode_partitions(self.pool, self.layer, self.q, self.tables, self.ctx,
                                self.max_context, self.scale, self.out, self.workspace,
                                self.partition_tokens, stream)

    def decode_reduce(self, stream=None):
        pa.pa_decode_reduce(self.pool, self.layer, self.q, self.tables, self.ctx,
                            self.max_context, self.scale, self.out, self.workspace,
                            self.partition_tokens, stream)

    def cache_and_decode_plan(self, stream=None):
        pa.pa_cache_and_decode_plan(self.pool, self.layer, self.new_k, self.new_v, self.new_slots,
                                    self.q, self.tables, self.ctx, self.max_context, self.scale,
                                    self.out, self.workspace, self.partition_tokens, stream)

    def step(self, stream=None):
        """One decode step: the new tokens' cache write and the decode, in three launches."""
        pa.pa_cache_and_decode(self.pool, self.layer, self.new_k, self.new_v, self.new_slots,
                               self.q, self.tables, self.ctx, self.max_context, self.scale,
                               self.out, self.workspace, self.partition_tokens, stream)

    def step_separate(self, stream=None):
        """The same step as ``pa_reshape_and_cache`` then ``pa_decode`` (four launches)."""
        self.write_new_tokens(stream)
        self.decode(stream)

    def layer_cache(self):
        """(K, V) of the session's layer as ``[N][H_kv][bs][d]`` tensors of the pool dtype
        (uint8 codes for an FP8 cache)."""
        w = self.w
        per = w.num_blocks * w.num_kv_heads * w.block_size * w.head_dim
        flat = self.storage if self.cache_dtype == FP8 else self.storage.view(_TORCH[w.dtype])
        base = 2 * self.layer * per
        shape = (w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim)
        return flat[base:base + per].view(shape), flat[base + per:base + 2 * per].view(shape)


class PrefillSession:
    """A mixed batch: prefill chunks over cached prefixes plus single-token decode rows.

    Every sequence's tokens (prefix, chunk, decode history) get blocks from the block
    manager and are written to their slots.  One step then rewrites the chunk rows and
    the decode rows' newest tokens (``pa_reshape_and_cache``), runs the chunks through
    ``pa_prefill_chunked`` and the decode rows through ``pa_decode``.
    """

    def __init__(self, w, device="cuda", partition_tokens=0, poison=True, chunk_tokens=1 << 16):
        self.w = w
        self.device = device
        self.partition_tokens = partition_tokens
        self.desc = pa.make_desc(1, w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, w.dtype)
        self.storage = torch.empty(pa.pa_pool_bytes(self.desc), dtype=torch.uint8, device=device)
        if poison:
            nan_fill(self.storage, w.dtype)
        self.pool = pa.pa_alloc_pool(self.desc, self.storage, w.free_order)
        lens = w.seq_lens()
        self.n_chunks = len(w.chunk_lens)
        self.n_decode = len(w.decode_lens)
        self.seqs = [pa.pa_seq_new(self.pool) for _ in range(len(lens))]
        slots = [pa.pa_seq_append(self.pool, s, int(L))[0] if L > 0 else np.zeros(0, np.int64)
                 for s, L in zip(self.seqs, lens)]
        offs = w.token_offsets
        all_rows = np.arange(offs[-1])
        all_slots = np.concatenate(slots) if slots else np.zeros(0, np.int64)
        for a in range(0, len(all_rows), chunk_tokens):
            idx = all_rows[a:a + chunk_tokens]
            pa.pa_reshape_and_cache(self.pool, 0, bits_to_device(w.k_tokens[idx], w.dtype, device),
                                    bits_to_device(w.v_tokens[idx], w.dtype, device),
                                    torch.from_numpy(all_slots[a:a + chunk_tokens]).to(device))
        torch.cuda.synchronize()

        # The step's writes: each chunk's rows and each decode row's newest token.
        step_rows, step_slots = [], []
        for i in range(self.n_chunks):
            c = int(w.chunk_lens[i])
            step_rows.append(np.arange(offs[i + 1] - c, offs[i + 1]))
            step_slots.append(slots[i][len(slots[i]) - c:])
        for j in range(self.n_decode):
            s = self.n_chunks + j
            if lens[s] > 0:
                step_rows.append(np.array([offs[s + 1] - 1]))
                step_slots.append(slots[s][-1:])
        rows = np.concatenate(step_rows) if step_rows else np.zeros(0, np.int64)
        self.step_k = bits_to_device(w.k_tokens[rows], w.dtype, device)
        self.step_v = bits_to_device(w.v_tokens[rows], w.dtype, device)
        self.step_slots = torch.from_numpy(np.concatenate(step_slots) if step_slots
                                           else np.zeros(0, np.int64)).to(device)

        def tables_of(seqs):
            mb = max(1, max((-(-pa.pa_seq_length(self.pool, s) // w.block_size) for s in seqs),
                            default=1))
            t, c = pa.pa_export_block_tables(self.pool, seqs, mb)
            return t, c

        chunk_seqs = self.seqs[:self.n_chunks]
        dec_seqs = self.seqs[self.n_chunks:]
        tc, cc = tables_of(chunk_seqs)
        self.tables_c_host, self.ctx_c_host = tc, cc
        self.tables_c = torch.from_numpy(tc).to(device)
        self.ctx_c = torch.from_numpy(cc).to(device)
        self.max_ctx_c = int(cc.max()) if len(cc) else 0
        qs = np.concatenate([[0], np.cumsum(np.asarray(w.chunk_lens, dtype=np.int64))]).astype(np.int32)
        self.query_start = torch.from_numpy(qs).to(device)
        self.max_query_len = int(np.max(w.chunk_lens)) if self.n_chunks else 0
        self.q_c = bits_to_device(w.q_chunks, w.dtype, device)
        self.out_c = torch.empty(int(qs[-1]), w.num_q_heads, w.head_dim, dtype=torch.float32,
                                 device=device)
        pws = pa.pa_prefill_workspace_bytes(self.pool, int(qs[-1]), w.num_q_heads, self.max_ctx_c)
        self.workspace_c = torch.empty(pws, dtype=torch.uint8, device=device) if pws else None
        td, cd = tables_of(dec_seqs) if dec_seqs else (np.zeros((0, 1), np.int32), np.zeros(0, np.int32))
        self.tables_d_host, self.ctx_d_host = td, cd
        self.tables_d = torch.from_numpy(td).to(device)
        self.ctx_d = torch.from_numpy(cd).to(device)
        self.max_ctx_d = int(cd.max()) if len(cd) else 0
        self.q_d = bits_to_device(w.q_decode, w.dtype, device)
        self.out_d = torch.empty(self.n_decode, w.num_q_heads, w.head_dim, dtype=torch.float32,
                                 device=device)
        ws = pa.pa_decode_workspace_bytes(self.pool, self.n_decode, w.num_q_heads, self.max_ctx_d,
                                          partition_tokens)
        self.workspace = torch.empty(ws, dtype=torch.uint8, device=device)
        self.scale = 1.0 / math.sqrt(w.head_dim)

    def write_step_tokens(self, stream=None):
        pa.pa_reshape_and_cache(self.pool, 0, self.step_k, self.step_v, self.step_slots, stream)

    def prefill(self, stream=None):
        pa.pa_prefill_chunked(self.pool, 0, self.q_c, self.query_start, self.tables_c, self.ctx_c,
                              self.max_ctx_c, self.max_query_len, self.scale, self.out_c,
                              self.workspace_c, stream)

    def decode(self, stream=None):
        if self.n_decode:
            pa.pa_decode(self.pool, 0, self.q_d, self.tables_d, self.ctx_d, self.max_ctx_d,
                         self.scale, self.out_d, self.workspace, self.partition_tokens, stream)

    def step(self, stream=None):
        self.write_step_tokens(stream)
        self.prefill(stream)
        self.decode(stream)

    def step_overlapped(self, side_stream):
        """The same step with the decode rows on ``side_stream`` (a default-priority
        stream): both wait for the cache write, the prefill runs on the current stream,
        and the current stream waits for the decode at the end.  The decode's persistent
        workgroups then take the compute-unit slots the prefill's shorter workgroups leave
        free (the two kernels read the pool only and write separate outputs)."""
        main = torch.cuda.current_stream()
        self.write_step_tokens()
        written = torch.cuda.Event()
        written.record(main)
        side_stream.wait_event(written)
        self.prefill()
        self.decode(side_stream.cuda_stream)
        decoded = torch.cuda.Event()
        decoded.record(side_stream)
        main.wait_event(decoded)



class PrefixCacheSession:
    """Serve a ``workloads.PrefixCacheWorkload`` on a pool with prefix caching.

    Requests are admitted one after another.  Admitting request ``i`` frees request
    ``i - release_after - 1`` (its full blocks stay cached until evicted), looks the
    prompt up (``pa_seq_new_prefix``), appends the rest of the prompt and the decode
    tokens with their ids, and writes K/V rows for those tokens only: the cached
    blocks already hold the rest.  ``decode`` then runs ``pa_decode`` over any set of
    live requests.
    """

    def __init__(self, w, device="cuda", poison=True):
        self.w = w
        self.device = device
        self.desc = pa.make_desc(1, w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, w.dtype)
        self.storage = torch.empty(pa.pa_pool_bytes(self.desc), dtype=torch.uint8, device=device)
        if poison:
            nan_fill(self.storage, w.dtype)
        self.pool = pa.pa_alloc_pool(self.desc, self.storage, w.free_order)
        pa.pa_pool_enable_prefix_caching(self.pool)
        self.scale = 1.0 / math.sqrt(w.head_dim)
        self.seq_of = {}
        R = w.num_requests
        self.cached_tokens = np.zeros(R, dtype=np.int64)
        self.evicted = np.zeros(R, dtype=np.int64)   # cached blocks evicted to admit request i
        self.host_seconds = np.zeros(R)              # manager calls of each admission

    def admit(self, i, stream=None):
        w = self.w
        gone = i - w.release_after - 1
        if gone >= 0 and gone in self.seq_of:
            pa.pa_seq_free(self.pool, self.seq_of.pop(gone))
        toks = w.tokens(i)
        prompt = w.prompt(i)
        empty = len(pa.pa_export_free_stack(self.pool))
        t0 = time.perf_counter()
        seq, hit = pa.pa_seq_new_prefix(self.pool, prompt)
        slots, cow = pa.pa_seq_append_tokens(self.pool, seq, toks[hit:])
        self.host_seconds[i] = time.perf_counter() - t0
        new_blocks = -(-len(toks) // w.block_size) - hit // w.block_size
        self.evicted[i] = max(0, new_blocks - empty)
        if cow:
            raise RuntimeError("no sequence is shared by forking here")
        self.seq_of[i] = seq
        self.cached_tokens[i] = hit
        k, v = w.kv_rows(toks[hit:], np.arange(hit, len(toks)))
        pa.pa_reshape_and_cache(self.pool, 0, bits_to_device(k, w.dtype, self.device),
                                bits_to_device(v, w.dtype, self.device),
                                torch.from_numpy(np.ascontiguousarray(slots)).to(self.device), stream)

    def live(self):
        return sorted(self.seq_of)

    def decode_args(self, requests):
        """Device-resident decode arguments for ``requests`` (tables exported now)."""
        w = self.w
        seqs = [self.seq_of[r] for r in requests]
        lens = [len(w.tokens(r)) for r in requests]
        max_blocks = max(1, max(-(-L // w.block_size) for L in lens))
        tables, ctx = pa.pa_export_block_tables(self.pool, seqs, max_blocks)
        dev = self.device
        return {
            "q": bits_to_device(w.q[list(requests)], w.dtype, dev),
            "tables": torch.from_numpy(tables).to(dev),
            "ctx": torch.from_numpy(ctx).to(dev),
            "max_context": max(lens),
            "out": torch.empty(len(requests), w.num_q_heads, w.head_dim, dtype=torch.float32,
                               device=dev),
            "ws": torch.empty(pa.pa_decode_workspace_bytes(self.pool, len(requests), w.num_q_heads,
                                                           max(lens), 0),
                              dtype=torch.uint8, device=dev),
            "tables_host": tables,
        }

    def run_decode(self, a, stream=None):
        pa.pa_decode(self.pool, 0, a["q"], a["tables"], a["ctx"], a["max_context"], self.scale,
                     a["out"], a["ws"], 0, stream)
        return a["out"]

    def decode(self, requests, stream=None):
        """Decode the newest token of each request in ``requests``; returns ``out``."""
        return self.run_decode(self.decode_args(requests), stream)


class SharedPrefixSession:
    """Parallel sampling over a ``workloads.SharedPrefixWorkload``.

    Each group's shared context is written once and forked into its branches; every
    branch's first divergent token triggers copy-on-write (the reported pairs are
    copied with ``pa_copy_blocks``), then the rest of each tail is appended and written.
    ``decode`` runs ``pa_decode`` over all branches, whose tables share the groups'
    full context blocks.
    """

    def __init__(self, w, device="cuda", poison=True):
        self.w = w
        self.device = device
        self.desc = pa.make_desc(1, w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, w.dtype)
        self.storage = torch.empty(pa.pa_pool_bytes(self.desc), dtype=torch.uint8, device=device)
        if poison:
            nan_fill(self.storage, w.dtype)
        pool = self.pool = pa.pa_alloc_pool(self.desc, self.storage, w.free_order)

        def write(k, v, slots):
            pa.pa_reshape_and_cache(pool, 0, bits_to_device(k, w.dtype, device),
                                    bits_to_device(v, w.dtype, device),
                                    torch.from_numpy(np.ascontiguousarray(slots, dtype=np.int64)).to(device))

        groups = []
        for g in range(w.groups):
            root = pa.pa_seq_new(pool)
            a, b = w.shared_offsets[g], w.shared_offsets[g + 1]
            write(w.shared_k[a:b], w.shared_v[a:b], pa.pa_seq_append(pool, root, b - a)[0])
            groups.append([root] + [pa.pa_seq_fork(pool, root) for _ in range(w.branches - 1)])
        self.seqs = sorted(s for grp in groups for s in grp)
        self.branch_of = {s: g * w.branches + b for g, grp in enumerate(groups) for b, s in enumerate(grp)}
        # First divergent token of every branch: copy-on-write pairs, then the copies.
        pairs, first_slots, first_rows = [], [], []
        for s in self.seqs:
            slots, p = pa.pa_seq_append(pool, s, 1)
            pairs += p
            first_slots.append(slots[0])
            first_rows.append(w.tail_offsets[self.branch_of[s]])
        self.cow_pairs = pairs
        self.pairs_dev = torch.tensor(pairs, dtype=torch.int32, device=device).reshape(-1, 2)
        pa.pa_copy_blocks(pool, self.pairs_dev)
        rows = np.array(first_rows)
        write(w.tail_k[rows], w.tail_v[rows], first_slots)
        for s in self.seqs:
            i = self.branch_of[s]
            a, e = w.tail_offsets[i] + 1, w.tail_offsets[i + 1]
            if e > a:
                slots, p = pa.pa_seq_append(pool, s, e - a)
                if p:
                    raise RuntimeError("a second copy-on-write in one branch")
                write(w.tail_k[a:e], w.tail_v[a:e], slots)
        self.lens = [pa.pa_seq_length(pool, s) for s in self.seqs]
        self.max_blocks = max(-(-L // w.block_size) for L in self.lens)
        tables, ctx = pa.pa_export_block_tables(pool, self.seqs, self.max_blocks)
        self.tables_host = tables
        self.tables = torch.from_numpy(tables).to(device)
        self.ctx = torch.from_numpy(ctx).to(device)
        order = [self.branch_of[s] for s in self.seqs]   # q row i belongs to branch i
        self.q = bits_to_device(w.q[order], w.dtype, device)
        self.max_context = max(self.lens)
        self.out = torch.empty(len(self.seqs), w.num_q_heads, w.head_dim, dtype=torch.float32,
                               device=device)
        self.workspace = torch.empty(pa.pa_decode_workspace_bytes(pool, len(self.seqs), w.num_q_heads,
                                                                  self.max_context, 0),
                                     dtype=torch.uint8, device=device)
        self.scale = 1.0 / math.sqrt(w.head_dim)

    def copy_blocks(self, stream=None):
        pa.pa_copy_blocks(self.pool, self.pairs_dev, stream)

    def decode(self, stream=None):
        pa.pa_decode(self.pool, 0, self.q, self.tables, self.ctx, self.max_context, self.scale,
                     self.out, self.workspace, 0, stream)

    def branch_tokens(self, s):
        """(K, V) raw bits of branch sequence ``s``, in token order."""
        w = self.w
        i = self.branch_of[s]
        g = i // w.branches
        sk = slice(w.shared_offsets[g], w.shared_offsets[g + 1])
        tk = slice(w.tail_offsets[i], w.tail_offsets[i + 1])
        return (np.concatenate([w.shared_k[sk], w.tail_k[tk]]),
                np.concatenate([w.shared_v[sk], w.tail_v[tk]]))
