"""Swap preemption: the manager model pinned by hand-worked cases, the C++ manager
bit-exact against it over random runs, and the block copies to and from pinned host
memory on the GPU, bit-exact, with decode after swapping back in.

"vLLM explained" (jackchen890311.github.io), in its table on when KV may be
overwritten, gives preemption under memory pressure by recomputing or by swapping the
KV to CPU memory.  The readings (host free stack, first-use order of the copy pairs,
one host block per distinct device block, references dropped as a free would) are in
``oracle/block_manager.py``.

Every random run tracks which token each physical slot holds, on the device and in the
swap space, from the slots and copy pairs the manager returns, and checks after every
operation that each live sequence's table addresses exactly its own tokens.
"""

import copy
import math
import random
import sys

import numpy as np
import pytest

from oracle.block_manager import BlockManagerModel, OutOfBlocks
from paged_kv_cache_442_amd import binding as pa


def pair_model(n, bs, m_host, order=None, caching=False):
    model = BlockManagerModel(n, bs, order)
    pool = pa.pa_alloc_pool(pa.make_desc(1, n, bs, 1, 8, pa.F16), None, order)
    if caching:
        model.enable_prefix_caching()
        pa.pa_pool_enable_prefix_caching(pool)
    model.set_swap_space(m_host)
    pa.pa_pool_set_swap_space(pool, m_host)
    return model, pool


# ------------------------------------------------------------------ hand-worked

def test_swap_out_copies_each_shared_block_once_and_frees_like_a_free():
    m = BlockManagerModel(8, 2)
    m.set_swap_space(4)
    a = m.seq_new()
    m.seq_append(a, 5)                          # blocks 0, 1, 2 (2 partial)
    b = m.seq_fork(a)
    _, cow = m.seq_append(b, 1)                 # copy-on-write of block 2 -> 3
    assert cow == [(2, 3)] and m.table(b) == [0, 1, 3]
    pairs = m.seq_swap_out([a, b])
    assert pairs == [(0, 0), (1, 1), (2, 2), (3, 3)]
    assert m.host_refcount == [2, 2, 1, 1]
    # a drops 0, 1, 2 (2 reaches zero), then b drops 0, 1, 3: pushed in that order.
    assert m.free_stack_top_first()[:4] == [3, 1, 0, 2]
    assert m.host_free_stack_top_first() == []
    pairs = m.seq_swap_in([b])
    assert pairs == [(0, 3), (1, 1), (3, 0)] and m.table(b) == [3, 1, 0]
    assert m.host_refcount == [1, 1, 1, 0] and m.host_free_stack_top_first() == [3]
    m.check_invariants()
    with pytest.raises(ValueError):
        m.seq_append(a, 1)                      # a is still swapped out
    m.seq_free(a)
    assert m.host_free_stack_top_first() == [2, 1, 0, 3]
    m.check_invariants()


def test_swap_is_all_or_nothing():
    m = BlockManagerModel(6, 2)
    m.set_swap_space(2)
    a = m.seq_new()
    m.seq_append(a, 5)                          # 3 blocks > 2 host blocks
    before = copy.deepcopy(m)
    with pytest.raises(OutOfBlocks):
        m.seq_swap_out([a])
    assert m.tables == before.tables and m.refcount == before.refcount
    m.set_swap_space(3)
    assert m.seq_swap_out([a]) == [(0, 0), (1, 1), (2, 2)]
    assert m.free_stack_top_first() == [2, 1, 0, 3, 4, 5]
    b = m.seq_new()
    m.seq_append(b, 8)                          # blocks 2, 1, 0, 3
    c = m.seq_new()
    m.seq_append(c, 3)                          # blocks 4, 5: none left
    before = copy.deepcopy(m)
    with pytest.raises(OutOfBlocks):
        m.seq_swap_in([a])
    assert m.tables == before.tables and m.host_refcount == before.host_refcount
    m.seq_free(b)                               # pushes 2, 1, 0, 3
    assert m.seq_swap_in([a]) == [(0, 3), (1, 0), (2, 1)]
    assert m.table(a) == [3, 0, 1] and m.host_free_stack_top_first() == [2, 1, 0]
    m.check_invariants()


def test_capi_rejects_operations_on_swapped_sequences():
    pool = pa.pa_alloc_pool(pa.make_desc(1, 8, 4, 1, 8, pa.F16), None, None)
    pa.pa_pool_set_swap_space(pool, 4)
    s = pa.pa_seq_new(pool)
    pa.pa_seq_append(pool, s, 6)
    assert pa.pa_seq_swap_out(pool, [s]) == [(0, 0), (1, 1)]
    assert pa.pa_seq_swapped(pool, s)
    for call in (lambda: pa.pa_seq_append(pool, s, 1), lambda: pa.pa_seq_fork(pool, s),
                 lambda: pa.pa_seq_release_before(pool, s, 4),
                 lambda: pa.pa_export_block_tables(pool, [s], 4),
                 lambda: pa.pa_seq_swap_out(pool, [s]),
                 lambda: pa.pa_pool_set_swap_space(pool, 8)):
        with pytest.raises(pa.PAError) as e:
            call()
        assert e.value.code == pa.PA_E_INVAL
    assert pa.pa_seq_swap_in(pool, [s]) == [(0, 1), (1, 0)]
    with pytest.raises(pa.PAError):
        pa.pa_seq_swap_in(pool, [s])
    assert [pa.pa_host_block_refcount(pool, h) for h in range(4)] == [0, 0, 0, 0]
    assert list(pa.pa_export_host_free_stack(pool)) == [1, 0, 2, 3]   # dropped 0 then 1
    assert pa.pa_swap_space_bytes(pa.make_desc(2, 8, 16, 8, 128, pa.BF16), 10) == \
        10 * pa.pa_block_bytes(pa.make_desc(2, 8, 16, 8, 128, pa.BF16))


# ------------------------------------------------------------------ random runs

class Slots:
    """Token ids held by device slots and host (swap space) slots."""

    def __init__(self, n, m, bs):
        self.bs = bs
        self.dev = np.full(n * bs, -1, dtype=np.int64)
        self.host = np.full(m * bs, -1, dtype=np.int64)

    def copy(self, pairs, src, dst):
        for a, b in pairs:
            dst[b * self.bs:(b + 1) * self.bs] = src[a * self.bs:(a + 1) * self.bs]

    def check(self, table, tokens, side):
        arr = self.host if side == "host" else self.dev
        for pos, t in enumerate(tokens):
            blk = table[pos // self.bs]
            if blk >= 0:
                assert arr[blk * self.bs + pos % self.bs] == t, (side, pos, blk)


def state(m, pool, live, swapped, n, m_host):
    res = [s for s in sorted(live) if s not in swapped]
    if res:
        t, c = pa.pa_export_block_tables(pool, res, 512)
        tc = [[int(x) for x in row[:-(-int(L) // pool.desc.block_size)]] for row, L in zip(t, c)]
    else:
        tc = []
    capi = (tc, [pa.pa_block_refcount(pool, b) for b in range(n)], list(pa.pa_export_free_stack(pool)),
            list(pa.pa_export_evictable(pool)), [pa.pa_host_block_refcount(pool, h) for h in range(m_host)],
            list(pa.pa_export_host_free_stack(pool)), [pa.pa_seq_swapped(pool, s) for s in sorted(live)])
    mod = ([m.table(s) for s in res], list(m.refcount), m.free_stack_top_first(), m.evictable(),
           list(m.host_refcount), m.host_free_stack_top_first(), [s in m.swapped for s in sorted(live)])
    return capi, mod


def run_random(seed, n, m_host, bs, ops, caching):
    rnd = random.Random(seed)
    order = list(range(n))
    rnd.shuffle(order)
    m, pool = pair_model(n, bs, m_host, order, caching)
    slots = Slots(n, m_host, bs)
    live = {}
    swapped = set()
    counts = {"swap_out": 0, "swap_in": 0}
    for _ in range(ops):
        r = rnd.random()
        resident = sorted(s for s in live if s not in swapped)
        if r < 0.2 or not resident:
            s = m.seq_new()
            assert pa.pa_seq_new(pool) == s
            live[s] = []
            continue
        if r < 0.5:
            s = rnd.choice(resident)
            k = rnd.randrange(0, 3 * bs)
            toks = [rnd.randrange(1000) for _ in range(k)]
            try:
                sl, cw = m.seq_append(s, k, toks)
            except OutOfBlocks:
                with pytest.raises(pa.PAError):
                    pa.pa_seq_append_tokens(pool, s, toks)
            else:
                sl_c, cw_c = pa.pa_seq_append_tokens(pool, s, toks)
                assert list(sl) == list(sl_c) and cw == cw_c
                slots.copy(cw, slots.dev, slots.dev)
                slots.dev[np.asarray(sl, np.int64)] = toks
                live[s] += toks
        elif r < 0.6:
            s = rnd.choice(resident)
            c = m.seq_fork(s)
            assert pa.pa_seq_fork(pool, s) == c
            live[c] = list(live[s])
        elif r < 0.75:
            group = rnd.sample(resident, rnd.randrange(1, min(3, len(resident)) + 1))
            try:
                pairs = m.seq_swap_out(group)
            except OutOfBlocks:
                with pytest.raises(pa.PAError) as e:
                    pa.pa_seq_swap_out(pool, group)
                assert e.value.code == pa.PA_E_NOMEM
            else:
                assert pa.pa_seq_swap_out(pool, group) == pairs
                slots.copy(pairs, slots.dev, slots.host)
                swapped |= set(group)
                counts["swap_out"] += 1
        elif r < 0.9 and swapped:
            group = rnd.sample(sorted(swapped), rnd.randrange(1, min(3, len(swapped)) + 1))
            try:
                pairs = m.seq_swap_in(group)
            except OutOfBlocks:
                with pytest.raises(pa.PAError) as e:
                    pa.pa_seq_swap_in(pool, group)
                assert e.value.code == pa.PA_E_NOMEM
            else:
                assert pa.pa_seq_swap_in(pool, group) == pairs
                slots.copy(pairs, slots.host, slots.dev)
                swapped -= set(group)
                counts["swap_in"] += 1
        else:
            s = rnd.choice(sorted(live))
            m.seq_free(s)
            pa.pa_seq_free(pool, s)
            del live[s]
            swapped.discard(s)
        capi, mod = state(m, pool, live, swapped, n, m_host)
        assert capi == mod
        m.check_invariants()
        for s, toks in live.items():
            slots.check(m.tables[s], toks, "host" if s in swapped else "dev")
    return counts


@pytest.mark.parametrize("seed,n,m_host,bs,caching", [
    (1, 24, 16, 2, False), (2, 40, 24, 4, False), (3, 16, 30, 1, False), (4, 64, 40, 16, False),
    (5, 24, 16, 2, True), (6, 40, 12, 4, True), (7, 20, 20, 3, True),
])
def test_manager_matches_the_model_with_swaps(seed, n, m_host, bs, caching):
    counts = run_random(seed, n, m_host, bs, 300, caching)
    assert counts["swap_out"] > 0 and counts["swap_in"] > 0


# ------------------------------------------------------------------ GPU

def announce(msg):
    print("\n[case] " + msg, flush=True)
    sys.stdout.flush()


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,layers", [(2, 1), (1, 2)])
def test_swap_round_trip_is_bit_exact_and_decode_after_swap_in(dtype, layers):
    import torch
    from oracle import attention, fpbits
    from paged_kv_cache_442_amd import workloads as wl
    from paged_kv_cache_442_amd.session import DecodeSession

    announce(f"swap round trip dtype={dtype} layers={layers}")
    lens = [1, 15, 16, 17, 100, 257, 600, 1000]
    w = wl.custom_decode(31 + dtype, dtype, lens, 16, 4, block_size=16, num_blocks=200)
    sess = DecodeSession(w, num_layers=layers, layer=layers - 1)
    sess.write_new_tokens()                     # each sequence's newest token too
    torch.cuda.synchronize()
    pool = sess.pool
    M = 96
    pa.pa_pool_set_swap_space(pool, M)
    host = torch.zeros(pa.pa_swap_space_bytes(sess.desc, M), dtype=torch.uint8, pin_memory=True)
    per = sess.storage.numel() // (2 * layers)           # bytes of one (layer, K|V) array
    blk = per // w.num_blocks
    hper = M * blk
    dev_before = sess.storage.cpu()

    out_seqs = [sess.seqs[i] for i in (1, 4, 5, 7)]
    pairs = pa.pa_seq_swap_out(pool, out_seqs)
    dpairs = torch.tensor(pairs, dtype=torch.int32, device="cuda").reshape(-1, 2)
    pa.pa_swap_blocks(pool, host, dpairs, True)
    torch.cuda.synchronize()
    hb = host.numpy()
    db = dev_before.numpy()
    for a in range(2 * layers):
        for d, h in pairs:
            assert np.array_equal(hb[a * hper + h * blk:a * hper + (h + 1) * blk],
                                  db[a * per + d * blk:a * per + (d + 1) * blk]), (a, d, h)
    # The freed device blocks are overwritten before the sequences come back.
    sess.storage.view(-1)[:].fill_(0x7F)
    pairs_in = pa.pa_seq_swap_in(pool, out_seqs)
    dpairs = torch.tensor(pairs_in, dtype=torch.int32, device="cuda").reshape(-1, 2)
    pa.pa_swap_blocks(pool, host, dpairs, False)
    torch.cuda.synchronize()
    after = sess.storage.cpu().numpy()
    for a in range(2 * layers):
        for h, d in pairs_in:
            assert np.array_equal(after[a * per + d * blk:a * per + (d + 1) * blk],
                                  hb[a * hper + h * blk:a * hper + (h + 1) * blk]), (a, h, d)

    tables, ctx = pa.pa_export_block_tables(pool, out_seqs, sess.max_blocks)
    idx = [1, 4, 5, 7]
    q = sess.q[idx].contiguous()
    out = torch.empty(len(idx), w.num_q_heads, w.head_dim, dtype=torch.float32, device="cuda")
    ws = torch.empty(pa.pa_decode_workspace_bytes(pool, len(idx), w.num_q_heads, max(lens), 0),
                     dtype=torch.uint8, device="cuda")
    pa.pa_decode(pool, layers - 1, q, torch.from_numpy(tables).cuda(), torch.from_numpy(ctx).cuda(),
                 max(lens), 1.0 / math.sqrt(w.head_dim), out, ws)
    got = out.cpu().numpy().astype(np.float64)
    for j, s in enumerate(idx):
        kt, vt = w.seq_tokens(s)
        want = attention.contiguous_decode(w.dtype, w.q[s], fpbits.decode(w.dtype, kt),
                                           fpbits.decode(w.dtype, vt), attention.default_scale(w.head_dim))
        assert np.max(np.abs(got[j] - want)) <= 2e-3, s


@pytest.mark.gpu
def test_swap_rejects_unpinned_host_memory():
    import torch
    announce("swap with unpinned host memory -> PA_E_INVAL before any launch")
    desc = pa.make_desc(1, 8, 16, 2, 128, pa.BF16)
    storage = torch.zeros(pa.pa_pool_bytes(desc), dtype=torch.uint8, device="cuda")
    pool = pa.pa_alloc_pool(desc, storage)
    pa.pa_pool_set_swap_space(pool, 4)
    plain = np.zeros(pa.pa_swap_space_bytes(desc, 4), dtype=np.uint8)
    pairs = torch.zeros(1, 2, dtype=torch.int32, device="cuda")
    rc = pa.lib().pa_swap_blocks(pool.handle, plain.ctypes.data, plain.nbytes,
                                 pairs.data_ptr(), 1, 1, None)
    assert rc == pa.PA_E_INVAL
