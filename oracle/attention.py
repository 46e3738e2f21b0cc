"""Paged attention in float64: gather through the block table, then textbook softmax
attention.  TEST INFRASTRUCTURE ONLY.

What is computed (plain definitions, no blocking, fusion or reordering):

1. Decode the raw bits of q, K and V to float64 exactly (``oracle.fpbits``).
2. Gather.  The KV cache of one layer is a pool of fixed-size physical blocks laid
   out ``[num_blocks][num_kv_heads][block_size][head_dim]``.  Token ``t`` of a
   sequence lives in physical block ``table[t // block_size]`` at offset
   ``t % block_size`` -- the logical-to-physical block table of "LLM inference
   optimization: KV cache & PagedAttention" (carlstack.gravito.dev), section 三.1
   and its block-mapping figure; "vLLM explained" (jackchen890311.github.io),
   section on PagedAttention (block table as a page table).  Gathering every
   token in logical order gives contiguous ``[L][num_kv_heads][head_dim]`` arrays.
3. Attend.  ``softmax(q K^T / sqrt(d_k)) V`` -- carlstack page, section 二 (the
   attention formula), with ``d_k = head_dim``.  Query head ``h`` reads KV head
   ``h // (num_q_heads // num_kv_heads)`` (contiguous query groups; the pages
   only say GQA/MQA models have fewer KV heads: "vLLM explained", block-size
   section).  The score is ``z_t = (sum_i q_i K_ti) * scale`` with
   ``scale = 1/sqrt(head_dim)``; then ``m = max_t z_t``, ``w_t = exp(z_t - m)``,
   ``Z = sum_t w_t`` and ``out = sum_t (w_t / Z) V_t``.  This is the two-pass
   form, not an online one.
4. Paging changes only where K/V are stored and how they are read, not the
   attention math ("vLLM explained", section on the two implementation layers):
   the paged result equals the contiguous result exactly.

Decode rows attend to every cached token of their sequence, including the token
just written (each new token is combined with all history: carlstack page,
section 一.2; "vLLM explained", KV-cache prerequisites).  A chunked-prefill row at
absolute position ``pos`` attends to tokens ``0..pos`` only (causal), with the
chunk's own K/V already in the cache (carlstack page, section 六 item 2; "vLLM
explained", appendix).

Sums are taken with numpy's elementwise product followed by ``sum`` along one
axis, which gives the same result for the same values regardless of where the
arrays came from (used by the paged == contiguous pin).
"""

import math

import numpy as np

from . import fpbits


def default_scale(head_dim):
    """1/sqrt(d_k) in float64."""
    return 1.0 / math.sqrt(head_dim)


def gather_sequence(pool_bits, dtype, table_row, context_len, block_size):
    """Contiguous float64 ``[L][num_kv_heads][head_dim]`` copy of one sequence's cache.

    ``pool_bits``: raw bits ``[num_blocks][num_kv_heads][block_size][head_dim]`` of
    one layer's K (or V) pool.  ``table_row``: the sequence's physical block ids in
    logical order.  Only tokens ``0..L-1`` are read.
    """
    L = int(context_len)
    t = np.arange(L)
    table_row = np.asarray(table_row)
    phys = table_row[t // block_size]            # physical block of each token
    off = t % block_size                         # offset inside that block
    raw = pool_bits[phys, :, off, :]             # -> [L][num_kv_heads][head_dim]
    return fpbits.decode(dtype, raw)


def attend(q, keys, values, scale):
    """Two-pass softmax attention of query rows ``q [g][d]`` over ``keys, values [L][d]``.

    Returns ``[g][d]`` float64.  With ``L == 0`` the result is all zeros.
    """
    q = np.asarray(q, dtype=np.float64)
    g, d = q.shape
    L = keys.shape[0]
    if L == 0:
        return np.zeros((g, d))
    z = (q[:, None, :] * keys[None, :, :]).sum(axis=-1) * scale        # [g][L]
    m = z.max(axis=1, keepdims=True)
    w = np.exp(z - m)
    Z = w.sum(axis=1, keepdims=True)
    return ((w / Z)[:, :, None] * values[None, :, :]).sum(axis=1)      # [g][d]


def contiguous_decode(dtype, q_bits, k_contig, v_contig, scale):
    """Decode for one sequence whose K/V are already contiguous.

    ``q_bits [H_q][d]`` raw bits; ``k_contig, v_contig``: float64
    ``[L][num_kv_heads][head_dim]``.  Returns ``[H_q][d]`` float64.
    """
    q = fpbits.decode(dtype, q_bits)
    H_q, d = q.shape
    H_kv = k_contig.shape[1]
    g = H_q // H_kv
    out = np.zeros((H_q, d))
    for k in range(H_kv):
        heads = slice(k * g, (k + 1) * g)
        out[heads] = attend(q[heads], k_contig[:, k, :], v_contig[:, k, :], scale)
    return out


def paged_decode(dtype, q_bits, k_pool_bits, v_pool_bits, tables, context_lens,
                 block_size, scale, seqs=None):
    """Decode rows ``[S][H_q][d]`` over a paged cache; returns float64 ``[S][H_q][d]``.

    ``seqs`` optionally restricts the work to a subset of sequence indices (rows not
    in the subset are returned as NaN so that they cannot be mistaken for results).
    """
    S, H_q, d = q_bits.shape
    out = np.full((S, H_q, d), np.nan)
    for s in (range(S) if seqs is None else seqs):
        L = int(context_lens[s])
        kc = gather_sequence(k_pool_bits, dtype, tables[s], L, block_size)
        vc = gather_sequence(v_pool_bits, dtype, tables[s], L, block_size)
        out[s] = contiguous_decode(dtype, q_bits[s], kc, vc, scale)
    return out


def prefill_rows(dtype, q_bits, row_seq, row_pos, k_pool_bits, v_pool_bits, tables,
                 context_lens, block_size, scale):
    """Causal attention of query rows over a paged cache.

    ``q_bits [R][H_q][d]``; row ``r`` belongs to sequence ``row_seq[r]`` and sits at
    absolute position ``row_pos[r]``; it attends to tokens ``t <= row_pos[r]``.  A
    decode row is the case ``row_pos = L - 1``.  Returns float64 ``[R][H_q][d]``.
    """
    R, H_q, d = q_bits.shape
    out = np.zeros((R, H_q, d))
    H_kv = k_pool_bits.shape[1]
    g = H_q // H_kv
    q_all = fpbits.decode(dtype, q_bits)
    for s in np.unique(row_seq):
        rows = np.nonzero(row_seq == s)[0]
        L = int(context_lens[s])
        if np.any(row_pos[rows] >= L) or np.any(row_pos[rows] < 0):
            raise ValueError("a query row's position lies outside its sequence")
        kc = gather_sequence(k_pool_bits, dtype, tables[s], L, block_size)
        vc = gather_sequence(v_pool_bits, dtype, tables[s], L, block_size)
        for r in rows:
            visible = int(row_pos[r]) + 1
            for k in range(H_kv):
                heads = slice(k * g, (k + 1) * g)
                out[r, heads] = attend(q_all[r, heads], kc[:visible, k, :],
                                       vc[:visible, k, :], scale)
    return out


def causal_chunk(dtype, q_bits, k_contig, v_contig, first_pos, scale):
    """Causal attention of one chunk's consecutive query rows over their sequence.

    ``q_bits [C][H_q][d]`` raw bits of the rows at absolute positions ``first_pos ..
    first_pos + C - 1``; ``k_contig, v_contig`` float64 ``[L][num_kv_heads][d]`` with
    ``L >= first_pos + C``.  Row ``r`` attends to tokens ``0 .. first_pos + r`` (the same
    definition as ``prefill_rows``).  For each query head the scores of all rows come
    from one matrix product (a library routine); tokens after a row's position get no
    weight, and the rest is the two-pass softmax of ``attend``: ``m = max z``,
    ``w = exp(z - m)``, ``out = sum (w / sum w) v``.  Returns float64 ``[C][H_q][d]``.
    """
    q = fpbits.decode(dtype, q_bits)
    C, H_q, d = q.shape
    H_kv = k_contig.shape[1]
    g = H_q // H_kv
    n = int(first_pos) + C                       # keys any row of the chunk can see
    if k_contig.shape[0] < n:
        raise ValueError("the chunk's rows lie past the end of the sequence")
    pos = int(first_pos) + np.arange(C)
    visible = np.arange(n)[None, :] <= pos[:, None]                     # [C][n]
    out = np.zeros((C, H_q, d))
    for k in range(H_kv):
        keys, values = k_contig[:n, k, :], v_contig[:n, k, :]
        for h in range(k * g, (k + 1) * g):
            z = np.where(visible, (q[:, h, :] @ keys.T) * scale, -np.inf)
            m = z.max(axis=1, keepdims=True)
            w = np.exp(z - m)
            out[:, h, :] = (w / w.sum(axis=1, keepdims=True)) @ values
    return out


def partition_stats(q, keys, values, scale):
    """Softmax statistics of one query vector over one subset of tokens.

    Returns ``(m, l, o)``: the largest score, ``l = sum exp(z - m)`` and the
    normalized output ``o = sum exp(z - m) v / l``.  An empty subset gives
    ``(-inf, 0, 0)``.
    """
    d = keys.shape[1] if keys.ndim == 2 else len(q)
    if keys.shape[0] == 0:
        return -np.inf, 0.0, np.zeros(d)
    z = (np.asarray(q)[None, :] * keys).sum(axis=-1) * scale
    m = z.max()
    w = np.exp(z - m)
    l = w.sum()
    o = (w[:, None] * values).sum(axis=0) / l
    return m, l, o


def lse_merge(parts):
    """Merge per-subset ``(m, l, o)`` statistics into the softmax result over the union.

    With ``M = max_p m_p`` and ``W_p = l_p exp(m_p - M)``, the result is
    ``sum_p W_p o_p / sum_p W_p``.  Empty subsets (``l = 0``) carry no weight.
    This is an identity of the softmax: the union's weights are each subset's
    weights rescaled to a common maximum.
    """
    live = [(m, l, o) for (m, l, o) in parts if l > 0]
    if not live:
        return np.zeros_like(parts[0][2])
    M = max(m for m, _, _ in live)
    W = [l * math.exp(m - M) for m, l, _ in live]
    num = sum(w * o for w, (_, _, o) in zip(W, live))
    return num / sum(W)


def window_decode(dtype, q_bits, k_contig, v_contig, scale, window):
    """Decode over the last ``window`` tokens of a sequence (0 = all of them): with a
    sliding-window model only those tokens are attended ("vLLM explained", table of when
    KV may be overwritten).  ``k_contig, v_contig``: float64 ``[L][num_kv_heads][d]``."""
    L = k_contig.shape[0]
    start = max(0, L - window) if window > 0 else 0
    return contiguous_decode(dtype, q_bits, k_contig[start:], v_contig[start:], scale)

