"""Seeded synthetic workloads (inputs only).

This module draws the inputs that both the GPU path and the CPU oracle consume.
It holds none of the method's arithmetic: no attention, no block mapping, no slot
computation.  It only draws context lengths, a block permutation (the free list's
initial pop order) and the Q/K/V values, and rounds them to the storage format.

Shapes follow the workloads the pages talk about (models named only for their
shapes; no weights are involved):

* ``tiny``     -- one layer, 4 sequences of lengths 17, 64, 100, 255; 8 query heads
                  over 8 KV heads, head_dim 128, block size 16, fp32; 64 pool blocks.
* ``llama2_7b``-- one Llama-2-7B-shaped layer: 32 query = 32 KV heads, head_dim 128,
                  fp16, block size 16, 64 sequences, lengths uniform in [128, 2048].
* ``llama3_70b``-- one Llama-3-70B-shaped GQA layer: 64 query heads over 8 KV heads,
                  head_dim 128, bf16, block size 16, 128 sequences, lengths
                  log-uniform in [256, 8192] (``floor(256 * 32**u)``, u ~ U[0, 1)).
* ``shared_prefix`` -- parallel sampling: 32 groups x 4 branches sharing a
                  1024-token prompt plus ``s_g ~ U[1, 15]`` tokens decoded before the
                  fork, then per-branch tails of 1..256 tokens; GQA 32/8, bf16, bs 16.
* ``chunked_prefill`` -- 8 prefill chunks of 256..512 query tokens over cached
                  prefixes of 0..4096 tokens plus 96 decode rows of length 1..4096;
                  GQA 32/8, bf16, block size 32.
* ``prefix_cache`` -- requests that share system prompts (prefix caching): each
                  prompt is one of a few system prompts followed by the request's own
                  tokens; a token's K/V rows depend only on its id and position.

Values are float32 draws from N(0, 1) (numpy PCG64, ``default_rng(seed)``) rounded
to the storage format with round-to-nearest-even; arrays hold raw bits (uint16
for fp16/bf16, uint32 for fp32).  Draw order is fixed per workload (lengths, block
permutation, Q, K, V) so a seed fixes every byte.
"""

from dataclasses import dataclass, field
import math

import numpy as np

F32, F16, BF16 = 0, 1, 2
DTYPE_NAMES = {F32: "f32", F16: "f16", BF16: "bf16"}
BITS_DTYPE = {F32: np.uint32, F16: np.uint16, BF16: np.uint16}
NAN_BITS = {F32: 0x7FC00000, F16: 0x7E00, BF16: 0x7FC0}


def round_to_bits(x, dtype):
    """Round float32 values to the storage format (RNE) and return the raw bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == F32:
        return x.view(np.uint32).copy()
    if dtype == F16:
        return x.astype(np.float16).view(np.uint16)
    u = x.view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def _normal_bits(rng, shape, dtype):
    return round_to_bits(rng.standard_normal(shape, dtype=np.float32), dtype)


def _blocks(length, block_size):
    return -(-int(length) // block_size)


@dataclass
class DecodeWorkload:
    """Sequences to be written into a paged cache and then decoded (one layer).

    ``k_tokens``/``v_tokens`` hold every sequence's tokens back to back in logical
    order, ``[sum(L)][H_kv][d]``; sequence ``s`` owns rows
    ``token_offsets[s] : token_offsets[s+1]``.  ``free_order`` is the pool's
    initial pop order (a seeded permutation, so blocks land scattered).
    """
    name: str
    dtype: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    context_lens: np.ndarray
    free_order: np.ndarray
    q: np.ndarray
    k_tokens: np.ndarray
    v_tokens: np.ndarray
    token_offsets: np.ndarray = field(init=False)

    def __post_init__(self):
        self.token_offsets = np.concatenate(
            [[0], np.cumsum(np.asarray(self.context_lens, dtype=np.int64))])

    @property
    def num_seqs(self):
        return len(self.context_lens)

    def seq_tokens(self, s):
        a, b = self.token_offsets[s], self.token_offsets[s + 1]
        return self.k_tokens[a:b], self.v_tokens[a:b]


def _decode_workload(name, rng, dtype, lens, H_q, H_kv, d, bs, num_blocks):
    lens = np.asarray(lens, dtype=np.int32)
    perm = rng.permutation(num_blocks).astype(np.int32)
    q = _normal_bits(rng, (len(lens), H_q, d), dtype)
    total = int(lens.sum())
    k = _normal_bits(rng, (total, H_kv, d), dtype)
    v = _normal_bits(rng, (total, H_kv, d), dtype)
    return DecodeWorkload(name, dtype, H_q, H_kv, d, bs, num_blocks, lens, perm, q, k, v)


def tiny(seed=1):
    """Single-layer tiny decode: lengths {17, 64, 100, 255}, 8/8 heads, fp32, 64 blocks."""
    rng = np.random.default_rng(seed)
    return _decode_workload("tiny", rng, F32, [17, 64, 100, 255], 8, 8, 128, 16, 64)


def llama2_7b(seed=2, num_seqs=64, min_len=128, max_len=2048):
    """Llama-2-7B-shaped MHA layer: 32/32 heads, fp16, lengths U[min_len, max_len]."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(min_len, max_len + 1, size=num_seqs)
    N = math.ceil(1.25 * sum(_blocks(L, 16) for L in lens))
    return _decode_workload("llama2_7b", rng, F16, lens, 32, 32, 128, 16, N)


def llama3_70b(seed=3, num_seqs=128, min_len=256, max_len=8192, num_q_heads=64, fixed_len=0):
    """Llama-3-70B-shaped GQA layer: 64 query / 8 KV heads, bf16, log-uniform lengths
    (or every sequence ``fixed_len`` tokens long when that is given)."""
    rng = np.random.default_rng(seed)
    u = rng.random(num_seqs)
    lens = np.clip(np.floor(min_len * (max_len / min_len) ** u), min_len, max_len).astype(np.int64)
    if fixed_len:
        lens = np.full(num_seqs, fixed_len, dtype=np.int64)
    N = math.ceil(1.25 * sum(_blocks(L, 16) for L in lens))
    return _decode_workload("llama3_70b", rng, BF16, lens, num_q_heads, 8, 128, 16, N)


def custom_decode(seed, dtype, lens, num_q_heads, num_kv_heads, head_dim=128, block_size=16,
                  num_blocks=None, name="custom"):
    """Any decode shape; the pool defaults to 1.25x the blocks needed (at least 1)."""
    rng = np.random.default_rng(seed)
    if num_blocks is None:
        num_blocks = max(1, math.ceil(1.25 * sum(_blocks(L, block_size) for L in lens)))
    return _decode_workload(name, rng, dtype, lens, num_q_heads, num_kv_heads, head_dim,
                            block_size, num_blocks)


@dataclass
class SharedPrefixWorkload:
    """Parallel sampling: groups of branches forked from one shared context.

    Group ``g`` first holds ``prompt_len + pre_fork[g]`` tokens (``shared_k``/``shared_v``
    rows ``shared_offsets[g]:shared_offsets[g+1]``); it is then forked into
    ``branches`` sequences, and branch ``b`` of group ``g`` appends
    ``tails[g][b]`` tokens (``tail_k``/``tail_v`` rows ``tail_offsets[g*branches+b] :
    ... + 1]``).  Each branch has one decode query ``q[g*branches+b]``.
    """
    dtype: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    groups: int
    branches: int
    prompt_len: int
    pre_fork: np.ndarray
    tails: np.ndarray
    free_order: np.ndarray
    q: np.ndarray
    shared_k: np.ndarray
    shared_v: np.ndarray
    tail_k: np.ndarray
    tail_v: np.ndarray
    shared_offsets: np.ndarray = field(init=False)
    tail_offsets: np.ndarray = field(init=False)

    def __post_init__(self):
        shared = self.prompt_len + np.asarray(self.pre_fork, dtype=np.int64)
        self.shared_offsets = np.concatenate([[0], np.cumsum(shared)])
        self.tail_offsets = np.concatenate([[0], np.cumsum(np.asarray(self.tails).reshape(-1))])


def shared_prefix(seed=4, groups=32, branches=4, prompt_len=1024, max_pre_fork=15,
                  max_tail=256, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                  dtype=BF16):
    """Shared-prefix parallel sampling workload (fork, then copy-on-write on divergence)."""
    rng = np.random.default_rng(seed)
    pre_fork = rng.integers(1, max_pre_fork + 1, size=groups) if max_pre_fork > 0 \
        else np.zeros(groups, dtype=np.int64)
    tails = rng.integers(1, max_tail + 1, size=(groups, branches))
    blocks = 0
    for g in range(groups):
        shared = prompt_len + int(pre_fork[g])
        full_shared = shared // block_size
        for b in range(branches):
            blocks += _blocks(shared + int(tails[g, b]), block_size) - full_shared
        blocks += full_shared
    N = math.ceil(1.25 * blocks)
    perm = rng.permutation(N).astype(np.int32)
    q = _normal_bits(rng, (groups * branches, num_q_heads, head_dim), dtype)
    n_shared = int(groups * prompt_len + pre_fork.sum())
    n_tail = int(tails.sum())
    shared_k = _normal_bits(rng, (n_shared, num_kv_heads, head_dim), dtype)
    tail_k = _normal_bits(rng, (n_tail, num_kv_heads, head_dim), dtype)
    shared_v = _normal_bits(rng, (n_shared, num_kv_heads, head_dim), dtype)
    tail_v = _normal_bits(rng, (n_tail, num_kv_heads, head_dim), dtype)
    return SharedPrefixWorkload(dtype, num_q_heads, num_kv_heads, head_dim, block_size, N,
                                groups, branches, prompt_len, pre_fork, tails, perm, q,
                                shared_k, shared_v, tail_k, tail_v)


@dataclass
class ChunkedPrefillWorkload:
    """Prefill chunks over cached prefixes, plus single-token decode rows.

    Sequence ``i < num_chunks`` holds a cached prefix of ``prefix_lens[i]`` tokens and
    then a chunk of ``chunk_lens[i]`` new tokens whose query rows are ``q_chunks``
    rows ``chunk_offsets[i]:chunk_offsets[i+1]`` (positions ``prefix .. prefix+C-1``).
    Sequence ``num_chunks + j`` is a decode sequence of ``decode_lens[j]`` tokens
    with one query row ``q_decode[j]`` at position ``decode_lens[j] - 1``.  Every
    sequence's K/V (prefix, chunk and decode tokens) are ``k_tokens``/``v_tokens``
    rows ``token_offsets[s]:token_offsets[s+1]`` in logical order.
    """
    dtype: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    prefix_lens: np.ndarray
    chunk_lens: np.ndarray
    decode_lens: np.ndarray
    free_order: np.ndarray
    q_chunks: np.ndarray
    q_decode: np.ndarray
    k_tokens: np.ndarray
    v_tokens: np.ndarray
    chunk_offsets: np.ndarray = field(init=False)
    token_offsets: np.ndarray = field(init=False)

    def __post_init__(self):
        self.chunk_offsets = np.concatenate([[0], np.cumsum(np.asarray(self.chunk_lens, np.int64))])
        self.token_offsets = np.concatenate([[0], np.cumsum(self.seq_lens())])

    def seq_lens(self):
        return np.concatenate([np.asarray(self.prefix_lens) + np.asarray(self.chunk_lens),
                               np.asarray(self.decode_lens)]).astype(np.int64)


def chunked_prefill(seed=5, num_chunks=8, min_chunk=256, max_chunk=512, max_prefix=4096,
                    num_decode=96, max_decode_len=4096, num_q_heads=32, num_kv_heads=8,
                    head_dim=128, block_size=32, dtype=BF16):
    """Mixed batch: causal prefill chunks over paged prefixes plus decode rows."""
    rng = np.random.default_rng(seed)
    chunk_lens = rng.integers(min_chunk, max_chunk + 1, size=num_chunks)
    prefix_lens = rng.integers(0, max_prefix + 1, size=num_chunks)
    decode_lens = rng.integers(1, max_decode_len + 1, size=num_decode)
    lens = np.concatenate([prefix_lens + chunk_lens, decode_lens])
    N = math.ceil(1.25 * sum(_blocks(L, block_size) for L in lens))
    perm = rng.permutation(N).astype(np.int32)
    q_chunks = _normal_bits(rng, (int(chunk_lens.sum()), num_q_heads, head_dim), dtype)
    q_decode = _normal_bits(rng, (num_decode, num_q_heads, head_dim), dtype)
    total = int(lens.sum())
    k = _normal_bits(rng, (total, num_kv_heads, head_dim), dtype)
    v = _normal_bits(rng, (total, num_kv_heads, head_dim), dtype)
    return ChunkedPrefillWorkload(dtype, num_q_heads, num_kv_heads, head_dim, block_size, N,
                                  prefix_lens, chunk_lens, decode_lens, perm, q_chunks, q_decode,
                                  k, v)


def custom_chunked(seed, dtype, prefix_lens, chunk_lens, decode_lens, num_q_heads, num_kv_heads,
                   head_dim=128, block_size=16, num_blocks=None):
    """Any chunked-prefill shape: the given prefixes and chunks, plus decode rows."""
    rng = np.random.default_rng(seed)
    chunk_lens = np.asarray(chunk_lens, dtype=np.int64)
    prefix_lens = np.asarray(prefix_lens, dtype=np.int64)
    decode_lens = np.asarray(decode_lens, dtype=np.int64)
    lens = np.concatenate([prefix_lens + chunk_lens, decode_lens])
    if num_blocks is None:
        num_blocks = max(1, math.ceil(1.25 * sum(_blocks(L, block_size) for L in lens)))
    perm = rng.permutation(num_blocks).astype(np.int32)
    q_chunks = _normal_bits(rng, (int(chunk_lens.sum()), num_q_heads, head_dim), dtype)
    q_decode = _normal_bits(rng, (len(decode_lens), num_q_heads, head_dim), dtype)
    total = int(lens.sum())
    k = _normal_bits(rng, (total, num_kv_heads, head_dim), dtype)
    v = _normal_bits(rng, (total, num_kv_heads, head_dim), dtype)
    return ChunkedPrefillWorkload(dtype, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                                  prefix_lens, chunk_lens, decode_lens, perm, q_chunks, q_decode,
                                  k, v)



@dataclass
class PrefixCacheWorkload:
    """Requests sharing system prompts, served one after another by a prefix-caching pool.

    Request ``i`` has prompt ``system[sys_of[i]] + user[i]`` and then decodes ``steps``
    tokens ``decode_tokens[i]``.  Token ids are drawn from ``[0, vocab)``.  K and V rows of
    a token are ``(tok[id] + pos[position]) / sqrt(2)`` from two seeded tables each,
    rounded to the storage format: equal prefixes always give equal rows, which is what
    a cache hit relies on (in a model the rows depend on the whole prefix; a function
    of (id, position) is the simplest stand-in with that property).
    """
    dtype: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    vocab: int
    system: list
    sys_of: np.ndarray
    user: list
    decode_tokens: np.ndarray
    release_after: int
    free_order: np.ndarray
    q: np.ndarray
    tok_k: np.ndarray
    tok_v: np.ndarray
    pos_k: np.ndarray
    pos_v: np.ndarray

    @property
    def num_requests(self):
        return len(self.user)

    def prompt(self, i):
        return np.concatenate([self.system[int(self.sys_of[i])], self.user[i]]).astype(np.int32)

    def tokens(self, i):
        """Every token of request ``i`` after its decode steps."""
        return np.concatenate([self.prompt(i), self.decode_tokens[i]]).astype(np.int32)

    def kv_rows(self, token_ids, positions):
        """Raw bits of the K and V rows ``[n][H_kv][d]`` of tokens at positions."""
        t = np.asarray(token_ids, dtype=np.int64)
        p = np.asarray(positions, dtype=np.int64) % self.pos_k.shape[0]
        c = np.float32(1.0 / math.sqrt(2.0))
        k = (self.tok_k[t] + self.pos_k[p]) * c
        v = (self.tok_v[t] + self.pos_v[p]) * c
        return round_to_bits(k, self.dtype), round_to_bits(v, self.dtype)


def prefix_cache(seed=6, num_requests=48, num_system=4, min_system=100, max_system=700,
                 min_user=1, max_user=200, steps=1, vocab=512, num_q_heads=32, num_kv_heads=8,
                 head_dim=128, block_size=16, pool_fraction=0.5, release_after=4, dtype=BF16,
                 num_positions=4096):
    """Prefix-cache workload.  The pool holds ``pool_fraction`` of the blocks the requests
    would take without sharing (so cached blocks are evicted); a request is freed
    ``release_after`` requests after it starts."""
    rng = np.random.default_rng(seed)
    sys_lens = rng.integers(min_system, max_system + 1, size=num_system)
    system = [rng.integers(0, vocab, size=int(n)).astype(np.int32) for n in sys_lens]
    sys_of = rng.integers(0, num_system, size=num_requests)
    user_lens = rng.integers(min_user, max_user + 1, size=num_requests)
    user = [rng.integers(0, vocab, size=int(n)).astype(np.int32) for n in user_lens]
    decode_tokens = rng.integers(0, vocab, size=(num_requests, steps)).astype(np.int32)
    total = sum(_blocks(len(system[int(sys_of[i])]) + len(user[i]) + steps, block_size)
                for i in range(num_requests))
    live_peak = max(sum(_blocks(len(system[int(sys_of[j])]) + len(user[j]) + steps, block_size)
                        for j in range(i, min(i + release_after + 1, num_requests)))
                    for i in range(num_requests))
    N = max(live_peak + 2, int(math.ceil(pool_fraction * total)))
    perm = rng.permutation(N).astype(np.int32)
    q = _normal_bits(rng, (num_requests, num_q_heads, head_dim), dtype)
    tok_k = rng.standard_normal((vocab, num_kv_heads, head_dim), dtype=np.float32)
    tok_v = rng.standard_normal((vocab, num_kv_heads, head_dim), dtype=np.float32)
    pos_k = rng.standard_normal((num_positions, num_kv_heads, head_dim), dtype=np.float32)
    pos_v = rng.standard_normal((num_positions, num_kv_heads, head_dim), dtype=np.float32)
    return PrefixCacheWorkload(dtype, num_q_heads, num_kv_heads, head_dim, block_size, N, vocab,
                               system, sys_of, user, decode_tokens, release_after, perm, q,
                               tok_k, tok_v, pos_k, pos_v)
