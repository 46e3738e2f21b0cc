"""Drive libpa end to end for one workload: pool, block manager, slot writes, decode.

A ``DecodeSession`` places a ``workloads.DecodeWorkload`` into a paged cache the way
a serving engine would: the block manager allocates blocks as each sequence grows
(blocks taken from the seeded free order, so they land scattered), the history
tokens' K/V rows go to their slots with ``pa_reshape_and_cache``, and one decode
step then writes each sequence's newest token and runs ``pa_decode``.  Everything
here is argument marshalling and call order; every computation runs in libpa.
"""

import math

import numpy as np
import torch

from . import binding as pa
from . import workloads as wl

_TORCH = {wl.F32: torch.float32, wl.F16: torch.float16, wl.BF16: torch.bfloat16}


def bits_to_device(bits, dtype, device):
    """Raw-bit numpy array -> GPU tensor of the storage dtype (a bit copy)."""
    if dtype == wl.F32:
        host = torch.from_numpy(np.ascontiguousarray(bits).view(np.float32))
    else:
        host = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(_TORCH[dtype])
    return host.to(device)


def nan_fill(storage, dtype):
    """Fill a pool's bytes with the quiet-NaN pattern of its dtype."""
    storage.view(_TORCH[dtype]).fill_(float("nan"))


class DecodeSession:
    def __init__(self, w, device="cuda", partition_tokens=0, num_layers=1, layer=0, poison=True,
                 max_context=None, chunk_tokens=1 << 16):
        self.w = w
        self.device = device
        self.layer = layer
        self.partition_tokens = partition_tokens
        self.dtype = w.dtype
        self.desc = pa.make_desc(num_layers, w.num_blocks, w.block_size, w.num_kv_heads,
                                 w.head_dim, w.dtype)
        nbytes = pa.pa_pool_bytes(self.desc)
        self.storage = torch.empty(nbytes, dtype=torch.uint8, device=device)
        if poison:
            nan_fill(self.storage, w.dtype)
        self.pool = pa.pa_alloc_pool(self.desc, self.storage, w.free_order)
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

    def step(self, stream=None):
        self.write_new_tokens(stream)
        self.decode(stream)

    def layer_cache(self):
        """(K, V) of the session's layer as ``[N][H_kv][bs][d]`` tensors of the pool dtype."""
        w = self.w
        per = w.num_blocks * w.num_kv_heads * w.block_size * w.head_dim
        flat = self.storage.view(_TORCH[w.dtype])
        base = 2 * self.layer * per
        shape = (w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim)
        return flat[base:base + per].view(shape), flat[base + per:base + 2 * per].view(shape)
