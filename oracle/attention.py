"""Float64 CPU oracle of one ragged paged attention pass (test infrastructure).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may use
this module.  It shares no code with the HIP path and imports nothing from it.

What is computed, and where the pages say so
--------------------------------------------
* A pass is a ragged batch: each sequence s contributes n_s new query tokens
  (a prompt chunk when n_s > 1, a decode when n_s == 1) on top of c_s tokens
  already in the KV cache.  Composing passes at a fixed token budget from
  prompt chunks plus decode tokens is Dynamic SplitFuse ("DeepSpeed-FastGen:
  High-throughput Text Generation for LLMs via MII and DeepSpeed-Inference",
  research summary page, section "Summary"; InfoQ news item "Microsoft
  releases DeepSpeed-FastGen", second paragraph).
* The KV cache is paged: fixed-size physical blocks, addressed per sequence
  through a block table that the attention kernel reads itself
  ("DeepSpeed-FastGen Guide: Dynamic SplitKV Serving", section "3. Paged KV
  Memory Management with Zero Overhead"; research summary, "Key points").
* Attention is exact softmax attention; splitting the KV range and chunking a
  prompt over several passes must not change the result (FastGen Guide,
  "Key Benchmark Takeaways", numerical-equivalence item).
* Split-KV: each split yields a partial output and its local log-sum-exp, and
  the partials are combined by log-sum-exp weighting (FastGen Guide, section
  "1. Dynamic SplitKV Attention", two-phase softmax item, and "Step 3: Fused
  Dynamic SplitKV Attention Layer").

Readings taken where the pages are silent (each is listed in the design notes):
* scale defaults to 1/sqrt(head_dim) (FastGen Guide, Step 3 and Step 4 code);
* LSE is the natural log of the sum of exp(scaled score) over visible keys;
* the causal boundary is inclusive and bottom-right aligned: query row j of a
  chunk (absolute position c_s + j) sees keys 0 .. c_s + j;
* the pass's own K/V are appended to the cache before attention reads it;
* grouped-query heads map contiguously: q head h reads kv head h // G;
* the merge weights each partial by exp(lse_i - max lse), not by the partial's
  local maximum that the two-phase workflow figure prints;
* an empty or fully masked split range has lse = -inf and weight 0.

Cache layout (the contract the HIP path implements independently):
* K pool: [num_blocks, num_kv_heads, block_size, head_dim]
* V pool: [num_blocks, num_kv_heads, block_size // S, head_dim, S] with
  S = min(block_size, 32): each V block is stored transposed in sub-blocks of
  S slots, token index fastest (one sub-block when block_size <= 32).
"""
import math

import numpy as np

__all__ = [
    "bf16_to_f64",
    "kv_append",
    "gather_sequence",
    "attend",
    "partial_attend",
    "merge",
    "split_ranges",
    "attend_split",
]


def bf16_to_f64(bits):
    """Decode bf16 bit patterns exactly to float64.

    bf16 is the upper half of an IEEE binary32, so widening the 16 bits into
    the high half of a 32-bit word and reading it as float32 is exact; the
    float32 -> float64 widening is exact as well.
    """
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _cu(q_lens):
    cu = np.zeros(len(q_lens) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(np.asarray(q_lens, dtype=np.int64))
    return cu


def _v_sub(v_pool, block_size):
    """Slots per transposed V sub-block, min(block_size, 32), checked against
    the pool's shape [num_blocks, Hkv, block_size // S, D, S]."""
    sub = min(int(block_size), 32)
    if v_pool.ndim != 5 or v_pool.shape[2] * v_pool.shape[4] != block_size or v_pool.shape[4] != sub:
        raise ValueError(f"V pool shape {v_pool.shape} is not [blocks, Hkv, {block_size // sub}, D, {sub}]")
    return sub


def kv_append(k_pool, v_pool, q_lens, ctx_lens, block_tables, block_size, k_new, v_new):
    """Write each new token's K and V into its cache slot; return new pools.

    Token j of sequence s sits at absolute position p = ctx_lens[s] + j, in
    physical block block_tables[s, p // block_size] at slot p % block_size.
    k_new and v_new are [T, Hkv, D], token-major in sequence order.  The copy
    is value-preserving for any dtype (bf16 bits in, bf16 bits out).
    (FastGen Guide, section "3. Paged KV Memory Management with Zero Overhead".)
    """
    sub = _v_sub(v_pool, block_size)
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    cu = _cu(q_lens)
    for s in range(len(q_lens)):
        n = int(q_lens[s])
        pos = int(ctx_lens[s]) + np.arange(n)
        blk = np.asarray(block_tables[s])[pos // block_size]
        off = pos % block_size
        k_out[blk, :, off, :] = k_new[cu[s]:cu[s] + n]                      # [n, Hkv, D]
        v_out[blk, :, off // sub, :, off % sub] = v_new[cu[s]:cu[s] + n]    # [n, Hkv, D]
    return k_out, v_out


def gather_sequence(k_pool, v_pool, table_row, length, block_size):
    """Read positions 0..length-1 of one sequence back out of the pools.

    Walks the block table (a read path, separate from kv_append's write path)
    and returns K and V as [length, Hkv, D] in logical position order: logical
    position p lives in block table_row[p // block_size] at slot
    p % block_size (FastGen Guide, section "3. Paged KV Memory Management with
    Zero Overhead").
    """
    nblk = -(-int(length) // block_size)
    ids = np.asarray(table_row[:nblk], dtype=np.int64)
    hkv, d = k_pool.shape[1], k_pool.shape[3]
    _v_sub(v_pool, block_size)
    k = k_pool[ids].transpose(0, 2, 1, 3).reshape(nblk * block_size, hkv, d)[:length]
    # [blocks, Hkv, sub-block, D, slot] -> [blocks, sub-block, slot, Hkv, D]
    v = v_pool[ids].transpose(0, 2, 4, 1, 3).reshape(nblk * block_size, hkv, d)[:length]
    return k, v


def attend(q, k_pool, v_pool, q_lens, ctx_lens, block_tables, block_size,
           num_kv_heads, scale=None, seqs=None, heads=None):
    """Ragged paged causal attention of one pass, in float64.

    q: [T, Hq, D] bf16 bits; pools: bf16 bits in the layouts above, already
    holding this pass's K/V (append first).  Returns (O [T, Hq, D],
    LSE [T, Hq]) as float64; LSE is the natural log of the softmax
    denominator.  ``seqs`` / ``heads`` restrict the work to a sample; rows
    not computed are NaN.

    For each sequence s, q head h (kv head g = h // G) and chunk row j:
        s_t = scale * <q_j, k_t>   for t = 0 .. c_s + j
        O   = sum_t softmax(s)_t v_t,   LSE = ln sum_t exp(s_t)
    """
    t_tot, hq, d = q.shape
    group = hq // num_kv_heads
    if scale is None or scale == 0:
        scale = 1.0 / math.sqrt(d)
    out = np.full((t_tot, hq, d), np.nan)
    lse = np.full((t_tot, hq), np.nan)
    cu = _cu(q_lens)
    seq_list = range(len(q_lens)) if seqs is None else seqs
    head_list = range(hq) if heads is None else heads
    for s in seq_list:
        n, c = int(q_lens[s]), int(ctx_lens[s])
        length = c + n
        k_bits, v_bits = gather_sequence(k_pool, v_pool, block_tables[s], length, block_size)
        ks, vs = bf16_to_f64(k_bits), bf16_to_f64(v_bits)
        qs = bf16_to_f64(q[cu[s]:cu[s] + n])
        visible = np.arange(length)[None, :] <= (c + np.arange(n))[:, None]   # [n, L]
        for h in head_list:
            g = h // group
            scores = (qs[:, h, :] @ ks[:, g, :].T) * scale
            scores = np.where(visible, scores, -np.inf)
            m = scores.max(axis=1)
            e = np.exp(scores - m[:, None])
            den = e.sum(axis=1)
            out[cu[s]:cu[s] + n, h, :] = (e @ vs[:, g, :]) / den[:, None]
            lse[cu[s]:cu[s] + n, h] = m + np.log(den)
    return out, lse


def partial_attend(qh, kg, vg, limits, k0, k1, scale):
    """Attention of rows qh [n, D] over key positions [k0, k1) only.

    Row r sees position t when k0 <= t < k1 and t <= limits[r].  Returns the
    split's normalised partial output O_i [n, D] and its local log-sum-exp
    lse_i [n] (FastGen Guide, "1. Dynamic SplitKV Attention", two-phase
    softmax item).  A row that sees no key in the range gets O_i = 0 and
    lse_i = -inf, so its merge weight is exactly zero.
    """
    n, d = qh.shape
    o = np.zeros((n, d))
    l_out = np.full(n, -np.inf)
    if k1 <= k0:
        return o, l_out
    pos = np.arange(k0, k1)
    scores = (qh @ kg[k0:k1].T) * scale
    visible = pos[None, :] <= np.asarray(limits)[:, None]
    scores = np.where(visible, scores, -np.inf)
    any_vis = visible.any(axis=1)
    m = np.where(any_vis, scores.max(axis=1), 0.0)
    e = np.where(visible, np.exp(scores - m[:, None]), 0.0)
    den = e.sum(axis=1)
    safe = np.where(any_vis, den, 1.0)
    o = np.where(any_vis[:, None], (e @ vg[k0:k1]) / safe[:, None], 0.0)
    l_out = np.where(any_vis, m + np.log(safe), -np.inf)
    return o, l_out


def merge(parts):
    """Combine split partials [(O_i [n, D], lse_i [n]), ...] by log-sum-exp.

    M = max_i lse_i;  w_i = exp(lse_i - M);  O = sum_i w_i O_i / sum_i w_i;
    LSE = M + ln sum_i w_i.  Partials with lse_i = -inf carry weight 0.
    (FastGen Guide, Step 3 reduction; the workflow figure's formula is read
    with m_i := lse_i.)
    """
    lses = np.stack([p[1] for p in parts])          # [k, n]
    outs = np.stack([p[0] for p in parts])          # [k, n, D]
    mx = lses.max(axis=0)
    w = np.where(np.isfinite(lses), np.exp(lses - mx[None, :]), 0.0)
    wsum = w.sum(axis=0)
    o = (w[:, :, None] * outs).sum(axis=0) / wsum[:, None]
    return o, mx + np.log(wsum)


def split_ranges(length, num_splits):
    """Partition [0, length) into num_splits contiguous ranges of ceil size.

    Ranges past the end are empty, as in the Step 3 layer's chunking.
    """
    chunk = -(-int(length) // int(num_splits))
    return [(min(i * chunk, length), min((i + 1) * chunk, length)) for i in range(num_splits)]


def attend_split(q, k_pool, v_pool, q_lens, ctx_lens, block_tables, block_size,
                 num_kv_heads, ranges_for, scale=None):
    """The same pass computed split-KV style, for the oracle's self-checks.

    ``ranges_for(s, length)`` returns the list of [k0, k1) ranges that
    partition [0, length) for sequence s.  Each range yields a partial via
    partial_attend and the partials are merged by ``merge``: the two-phase
    split-KV computation of the FastGen Guide, section "1. Dynamic SplitKV
    Attention", and its Step 3 code.
    """
    t_tot, hq, d = q.shape
    group = hq // num_kv_heads
    if scale is None or scale == 0:
        scale = 1.0 / math.sqrt(d)
    out = np.zeros((t_tot, hq, d))
    lse = np.zeros((t_tot, hq))
    cu = _cu(q_lens)
    for s in range(len(q_lens)):
        n, c = int(q_lens[s]), int(ctx_lens[s])
        length = c + n
        k_bits, v_bits = gather_sequence(k_pool, v_pool, block_tables[s], length, block_size)
        ks, vs = bf16_to_f64(k_bits), bf16_to_f64(v_bits)
        qs = bf16_to_f64(q[cu[s]:cu[s] + n])
        limits = c + np.arange(n)
        ranges = ranges_for(s, length)
        for h in range(hq):
            g = h // group
            parts = [partial_attend(qs[:, h, :], ks[:, g, :], vs[:, g, :], limits, k0, k1, scale)
                     for (k0, k1) in ranges]
            o, l_ = merge(parts)
            out[cu[s]:cu[s] + n, h, :] = o
            lse[cu[s]:cu[s] + n, h] = l_
    return out, lse
