"""Automatic prefix caching: the manager model pinned to the pages' rules, the C++
manager bit-exact against it, and decode over cached blocks on the GPU.

The rules come from "vLLM explained" (jackchen890311.github.io), section on prefix
caching: the cache shares the block pool; blocks are in use, free and empty, or free
and cached; a request takes empty blocks first, then evicts free cached blocks least
recently used first; blocks in use are never evicted.  The readings where the page is
silent (identity = the whole token prefix, first block with an identity is the cached
one, at least one prompt token left to compute, tail blocks released first) are in
``oracle/block_manager.py``.

Besides hand-worked cases, every run checks the property a cache hit must keep:
each live sequence's table addresses slots that hold exactly its own tokens.  The
test tracks which token id sits in each physical slot from the slots and copy pairs
the manager returns, so a stale or wrong hit (a block reused after eviction, a block
of another prefix) shows as a slot holding another token.
"""

import copy
import math
import random
import sys

import numpy as np
import pytest

from oracle.block_manager import BlockManagerModel, OutOfBlocks
from paged_kv_cache_442_amd import binding as pa

EMPTY, IN_USE, CACHED = 0, 1, 2


def model(n, bs, order=None):
    m = BlockManagerModel(n, bs, order)
    m.enable_prefix_caching()
    return m


def admit(m, prompt):
    """New request: look up, then append the rest of the prompt with its ids."""
    seq, hit = m.seq_new_prefix(prompt)
    m.seq_append(seq, len(prompt) - hit, list(prompt[hit:]))
    return seq, hit


# ------------------------------------------------------------------ hand-worked pins

def test_a_second_request_with_the_same_prompt_reuses_the_full_blocks():
    m = model(8, 4)
    p = list(range(100, 110))                   # 10 tokens: 2 full blocks + 2 tokens
    a, hit = admit(m, p)
    assert hit == 0 and m.table(a) == [0, 1, 2]
    m.seq_free(a)
    # Block 2 is partial, so never cached: back on the free stack.  Blocks 1 and 0
    # are cached; released last to first, so block 1 is evicted first.
    assert m.evictable() == [1, 0]
    assert [m.block_state(b) for b in range(3)] == [CACHED, CACHED, EMPTY]
    b, hit = admit(m, p)
    assert hit == 8 and m.table(b)[:2] == [0, 1]
    assert m.evictable() == [] and m.block_state(0) == IN_USE
    m.check_invariants()


def test_a_fully_cached_prompt_still_leaves_one_token_to_compute():
    m = model(8, 4)
    p = list(range(8))                          # exactly two full blocks
    a, _ = admit(m, p)
    m.seq_free(a)
    _, hit = admit(m, p)
    assert hit == 4                             # (8 - 1) // 4 = 1 block
    _, hit = admit(m, p + [99])
    assert hit == 8


@pytest.mark.parametrize("common", [0, 3, 4, 5, 11, 12, 13])
def test_prompts_that_diverge_at_token_k_share_k_div_bs_blocks(common):
    bs = 4
    m = model(32, bs)
    p = list(range(16))
    q = p[:common] + [1000 + i for i in range(16 - common)]
    a, _ = admit(m, p)
    b, hit = admit(m, q)
    assert hit == min(common // bs, (16 - 1) // bs) * bs
    assert m.table(b)[:hit // bs] == m.table(a)[:hit // bs]
    assert m.refcount[m.table(a)[0]] == (2 if hit else 1)


def test_empty_blocks_are_taken_before_cached_ones_then_lru():
    m = model(7, 2)
    a, _ = admit(m, [1, 2, 3, 4, 5])            # blocks 0, 1 full (cached), 2 partial
    b, _ = admit(m, [7, 8, 9])                  # block 3 full (cached), 4 partial
    m.seq_free(a)                               # LRU: 1, 0 ; stack gets 2
    m.seq_free(b)                               # LRU: 1, 0, 3 ; stack gets 4
    assert m.evictable() == [1, 0, 3]
    assert m.free_stack_top_first() == [4, 2, 5, 6]
    c, hit = admit(m, list(range(20, 29)))      # 5 blocks: 4, 2, 5, 6, then evict 1
    assert hit == 0 and m.table(c) == [4, 2, 5, 6, 1]
    assert m.evictable() == [0, 3]
    # Block 1's identity is gone, block 0's is still there; the new block evicts 3.
    d, hit = admit(m, [1, 2, 3])
    assert hit == 2 and m.table(d) == [0, 3]
    assert m.evictable() == [] and m.num_free() == 0
    m.check_invariants()


def test_blocks_in_use_are_never_evicted():
    m = model(4, 2)
    a, _ = admit(m, [1, 2, 3, 4, 5])            # blocks 0, 1 cached and in use, 2 partial
    b, hit = admit(m, [1, 2, 3, 4, 9])          # shares 0 and 1, takes 3
    assert hit == 4
    with pytest.raises(OutOfBlocks):            # nothing free, nothing evictable
        m.seq_append(b, 2, [9, 9])
    m.seq_free(a)                               # 0 and 1 still held by b; 2 freed
    assert m.evictable() == [] and m.free_stack_top_first() == [2]
    m.check_invariants()


def test_an_append_without_ids_stops_caching_for_that_sequence():
    m = model(8, 2)
    a, _ = admit(m, [1, 2, 3])                  # block 0 cached
    m.seq_append(a, 1)                          # ids unknown from now on
    m.seq_append(a, 2, [7, 7])
    assert len(m.cache) == 1
    child = m.seq_fork(a)
    m.seq_append(child, 2, [8, 8])
    assert len(m.cache) == 1


def test_the_first_block_with_an_identity_is_the_cached_one():
    m = model(8, 2)
    a = m.seq_new()
    b = m.seq_new()
    m.seq_append(a, 2, [5, 6])
    m.seq_append(b, 2, [5, 6])                  # same content, not shared
    assert m.cache == {(5, 6): m.table(a)[0]}
    m.seq_free(b)
    assert m.block_state(m.table(a)[0]) == IN_USE
    assert m.free_stack_top_first()[0] == 1     # b's block was never cached


# ------------------------------------------------------------------ random runs

class Contents:
    """Which token id each physical slot holds, from the manager's own outputs."""

    def __init__(self, n, bs):
        self.bs = bs
        self.slot = np.full(n * bs, -1, dtype=np.int64)

    def write(self, slots, tokens):
        self.slot[np.asarray(slots, dtype=np.int64)] = tokens

    def copy(self, pairs):
        for src, dst in pairs:
            self.slot[dst * self.bs:(dst + 1) * self.bs] = self.slot[src * self.bs:(src + 1) * self.bs]

    def check(self, table, tokens, released_ok=True):
        for pos, t in enumerate(tokens):
            blk = table[pos // self.bs]
            if blk < 0 and released_ok:
                continue
            assert self.slot[blk * self.bs + pos % self.bs] == t, (pos, blk)


def snapshot_capi(pool, seqs, n):
    bs = pool.desc.block_size
    tables, ctx = pa.pa_export_block_tables(pool, seqs, 1024)
    return ([[int(b) for b in row[:-(-int(c) // bs)]] for row, c in zip(tables, ctx)],
            [int(c) for c in ctx],
            [pa.pa_block_refcount(pool, b) for b in range(n)],
            list(pa.pa_export_free_stack(pool)),
            list(pa.pa_export_evictable(pool)),
            [pa.pa_block_state(pool, b) for b in range(n)])


def snapshot_model(m, seqs, n):
    return ([m.table(s) for s in seqs], [m.length(s) for s in seqs], list(m.refcount),
            m.free_stack_top_first(), m.evictable(), [m.block_state(b) for b in range(n)])


def run_random(seed, n_blocks, bs, ops):
    rnd = random.Random(seed)
    order = list(range(n_blocks))
    rnd.shuffle(order)
    m = model(n_blocks, bs, order)
    pool = pa.pa_alloc_pool(pa.make_desc(1, n_blocks, bs, 1, 8, pa.F16), None, order)
    pa.pa_pool_enable_prefix_caching(pool)
    contents = Contents(n_blocks, bs)
    systems = [[rnd.randrange(50) for _ in range(rnd.randrange(1, 4 * bs))] for _ in range(3)]
    live = {}                                   # seq -> token list (None: ids unknown)
    hits = 0
    for _ in range(ops):
        r = rnd.random()
        if r < 0.3 or not live:
            prompt = list(rnd.choice(systems)) + [rnd.randrange(50) for _ in range(rnd.randrange(0, 2 * bs))]
            if not prompt:
                prompt = [1]
            s_m, h_m = m.seq_new_prefix(prompt)
            s_c, h_c = pa.pa_seq_new_prefix(pool, prompt)
            assert (s_m, h_m) == (s_c, h_c)
            hits += h_m
            live[s_m] = list(prompt[:h_m])
            rest = prompt[h_m:]
            try:
                sl_m, cw_m = m.seq_append(s_m, len(rest), rest)
            except OutOfBlocks:
                with pytest.raises(pa.PAError) as e:
                    pa.pa_seq_append_tokens(pool, s_c, rest)
                assert e.value.code == pa.PA_E_NOMEM
            else:
                sl_c, cw_c = pa.pa_seq_append_tokens(pool, s_c, rest)
                assert list(sl_m) == list(sl_c) and cw_m == cw_c
                contents.copy(cw_m)
                contents.write(sl_m, rest)
                live[s_m] += rest
        elif r < 0.55:
            s = rnd.choice(sorted(live))
            k = rnd.randrange(0, 3 * bs)
            ids = rnd.random() < 0.9
            toks = [rnd.randrange(50) for _ in range(k)]
            try:
                sl_m, cw_m = m.seq_append(s, k, toks if ids else None)
            except OutOfBlocks:
                with pytest.raises(pa.PAError) as e:
                    (pa.pa_seq_append_tokens(pool, s, toks) if ids else pa.pa_seq_append(pool, s, k))
                assert e.value.code == pa.PA_E_NOMEM
            else:
                sl_c, cw_c = (pa.pa_seq_append_tokens(pool, s, toks) if ids
                              else pa.pa_seq_append(pool, s, k))
                assert list(sl_m) == list(sl_c) and cw_m == cw_c
                contents.copy(cw_m)
                contents.write(sl_m, toks if ids else [-2] * k)
                live[s] = live[s] + (toks if ids else [-2] * k)
        elif r < 0.65:
            seqs = rnd.sample(sorted(live), rnd.randrange(1, len(live) + 1))
            counts = [rnd.randrange(0, 3) for _ in seqs]
            toks = [rnd.randrange(50) for _ in range(sum(counts))]
            # All-or-nothing, by its definition: consecutive appends, undone if one fails.
            saved = copy.deepcopy(m)
            try:
                out_m, at = [], 0
                for q, c in zip(seqs, counts):
                    out_m.append(m.seq_append(q, c, toks[at:at + c]))
                    at += c
            except OutOfBlocks:
                m = saved
                with pytest.raises(pa.PAError) as e:
                    pa.pa_seq_append_batch_tokens(pool, seqs, toks, counts)
                assert e.value.code == pa.PA_E_NOMEM
            else:
                sl_c, cw_c = pa.pa_seq_append_batch_tokens(pool, seqs, toks, counts)
                sl_m = [x for o in out_m for x in o[0]]
                assert sl_m == list(sl_c)
                assert [p for o in out_m for p in o[1]] == cw_c
                at = 0
                for (sl, cw), q, c in zip(out_m, seqs, counts):
                    contents.copy(cw)
                    contents.write(sl, toks[at:at + c])
                    live[q] = live[q] + toks[at:at + c]
                    at += c
        elif r < 0.75:
            s = rnd.choice(sorted(live))
            c_m = m.seq_fork(s)
            assert pa.pa_seq_fork(pool, s) == c_m
            live[c_m] = list(live[s])
        elif r < 0.82:
            s = rnd.choice(sorted(live))
            t = rnd.randrange(0, len(live[s]) + 1)
            assert m.seq_release_before(s, t) == pa.pa_seq_release_before(pool, s, t)
        else:
            s = rnd.choice(sorted(live))
            m.seq_free(s)
            pa.pa_seq_free(pool, s)
            del live[s]
        seqs = sorted(live)
        assert snapshot_model(m, seqs, n_blocks) == snapshot_capi(pool, seqs, n_blocks)
        m.check_invariants()
        for s in seqs:
            contents.check(m.table(s), live[s])
    return hits


@pytest.mark.parametrize("seed,n_blocks,bs", [(1, 24, 2), (2, 40, 4), (3, 16, 1), (4, 64, 16),
                                             (5, 12, 3), (6, 30, 2), (7, 80, 4), (8, 20, 2)])
def test_manager_matches_the_model_bit_exact_and_tables_hold_their_tokens(seed, n_blocks, bs):
    hits = run_random(seed, n_blocks, bs, 300)
    assert hits > 0


def test_contents_check_catches_a_stale_hit():
    """Plant a mistake in the model: eviction keeps the evicted block's identity."""
    class Stale(BlockManagerModel):
        def _pop(self):
            if self.stack:
                return self.stack.pop()
            return self.lru.pop(0)              # identity not forgotten

    m = Stale(3, 2)
    m.enable_prefix_caching()
    contents = Contents(3, 2)
    a, _ = m.seq_new_prefix([1, 2, 3])
    sl, _ = m.seq_append(a, 3, [1, 2, 3])
    contents.write(sl, [1, 2, 3])
    m.seq_free(a)
    b, _ = m.seq_new_prefix([5, 6, 7, 8, 9])
    sl, _ = m.seq_append(b, 5, [5, 6, 7, 8, 9])  # evicts the block holding (1, 2)
    contents.write(sl, [5, 6, 7, 8, 9])
    c, hit = m.seq_new_prefix([1, 2, 3])
    assert hit == 2
    with pytest.raises(AssertionError):
        contents.check(m.table(c), [1, 2])


# ------------------------------------------------------------------ C ABI errors

def test_enable_needs_no_live_sequences_and_lookup_needs_caching():
    pool = pa.pa_alloc_pool(pa.make_desc(1, 8, 4, 1, 8, pa.F16), None, None)
    with pytest.raises(pa.PAError) as e:
        pa.pa_seq_new_prefix(pool, [1, 2, 3])
    assert e.value.code == pa.PA_E_INVAL
    s = pa.pa_seq_new(pool)
    with pytest.raises(pa.PAError) as e:
        pa.pa_pool_enable_prefix_caching(pool)
    assert e.value.code == pa.PA_E_INVAL
    pa.pa_seq_free(pool, s)
    pa.pa_pool_enable_prefix_caching(pool)
    assert pa.pa_seq_new_prefix(pool, []) == (1, 0)


def test_ids_are_ignored_without_prefix_caching():
    a = pa.pa_alloc_pool(pa.make_desc(1, 8, 4, 1, 8, pa.F16), None, None)
    b = pa.pa_alloc_pool(pa.make_desc(1, 8, 4, 1, 8, pa.F16), None, None)
    sa, sb = pa.pa_seq_new(a), pa.pa_seq_new(b)
    assert list(pa.pa_seq_append_tokens(a, sa, list(range(9)))[0]) == list(pa.pa_seq_append(b, sb, 9)[0])
    pa.pa_seq_free(a, sa)
    pa.pa_seq_free(b, sb)
    assert list(pa.pa_export_free_stack(a)) == list(pa.pa_export_free_stack(b))
    assert len(pa.pa_export_evictable(a)) == 0


# ------------------------------------------------------------------ GPU

def announce(msg):
    print("\n[case] " + msg, flush=True)
    sys.stdout.flush()


@pytest.mark.gpu
@pytest.mark.parametrize("bs,H_q,release_after", [(16, 32, 4), (32, 8, 2), (16, 64, 6)])
def test_decode_over_cached_blocks_matches_the_oracle(bs, H_q, release_after):
    import torch
    from oracle import attention, fpbits
    from paged_kv_cache_442_amd import workloads as wl
    from paged_kv_cache_442_amd.session import PrefixCacheSession

    announce(f"prefix cache decode bs={bs} H_q={H_q} release_after={release_after}")
    w = wl.prefix_cache(seed=10 + bs + H_q, num_requests=24, block_size=bs, num_q_heads=H_q,
                        release_after=release_after, pool_fraction=0.2)
    sess = PrefixCacheSession(w)
    scale = 1.0 / math.sqrt(w.head_dim)
    worst = 0.0
    for i in range(w.num_requests):
        sess.admit(i)
        out = sess.decode([i]).cpu().numpy().astype(np.float64)[0]
        toks = w.tokens(i)
        k, v = w.kv_rows(toks, np.arange(len(toks)))
        want = attention.contiguous_decode(w.dtype, w.q[i], fpbits.decode(w.dtype, k),
                                           fpbits.decode(w.dtype, v), scale)
        assert np.isfinite(out).all(), i
        worst = max(worst, float(np.max(np.abs(out - want))))
    # The live requests again, in one batch.
    live = sess.live()
    out = sess.decode(live).cpu().numpy().astype(np.float64)
    for j, i in enumerate(live):
        toks = w.tokens(i)
        k, v = w.kv_rows(toks, np.arange(len(toks)))
        want = attention.contiguous_decode(w.dtype, w.q[i], fpbits.decode(w.dtype, k),
                                           fpbits.decode(w.dtype, v), scale)
        worst = max(worst, float(np.max(np.abs(out[j] - want))))
    torch.cuda.synchronize()
    assert worst <= 2e-3, worst
    assert sess.cached_tokens.sum() > 0, "no request hit the cache"
    assert sess.evicted.sum() > 0, "no cached block was evicted"
