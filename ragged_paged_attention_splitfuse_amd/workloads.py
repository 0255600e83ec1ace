"""Seeded synthetic inputs for ragged paged attention passes.

This module only draws inputs: sequence lengths, block tables and bf16 tensors.
It holds none of the attention arithmetic and none of the cache addressing:
the K/V history of each sequence is returned in logical position order, and
each consumer writes it into its own paged pool through its own append path.
Both the HIP path and the CPU oracle are fed from here.

Shapes follow the pages' workloads:
* prompt lengths ~ N(2600, sd 780) and decode contexts ~ N(2660, sd 798)
  after a 60-token mean output ("DeepSpeed-FastGen: High-throughput Text
  Generation for LLMs via MII and DeepSpeed-Inference", research summary,
  "Key points", benchmark item; its "30% variance" is read as sd = 30% of the
  mean);
* decode contexts spread over 512 .. 16000 tokens ("DeepSpeed-FastGen Guide:
  Dynamic SplitKV Serving", section "2. The GPU Underutilization Trap in
  Variable-Length Decoding"), drawn log-uniform;
* the Llama-2-7B attention shape (32 heads, head_dim 128) and a 70B one-GPU
  head share (16 q / 2 kv heads) of a four-way head split (InfoQ news item
  "Microsoft releases DeepSpeed-FastGen", Llama-2 70B on 4 GPUs).

Random-number recipe (fixed; both sides see identical bits):
* one ``numpy.random.Generator(PCG64(seed))`` draws, in this order, the
  lengths and then the physical-block permutation;
* tensors come from keyed counter streams: the flat element range of each
  tensor is cut into chunks of ``CHUNK`` elements and chunk i of tensor tag t
  is drawn from ``PCG64(SeedSequence(seed, spawn_key=(t, i)))`` as float32
  N(0, 1), then rounded to bf16 with round-to-nearest-even.  Tags: 1 history
  K, 2 history V, 3 Q, 4 new K, 5 new V.  Chunks are independent, so they are
  drawn on a thread pool and any row range can be regenerated alone.
"""
import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

CHUNK = 1 << 22
BF16_NAN = 0x7FC0

TAG_HIST_K, TAG_HIST_V, TAG_Q, TAG_K_NEW, TAG_V_NEW = 1, 2, 3, 4, 5


def bf16_round(x):
    """Round float32 values to bf16 bit patterns, nearest-even (finite input)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).copy()
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    b += np.uint32(0x7FFF)
    b += lsb
    b >>= np.uint32(16)
    return b.astype(np.uint16)


def _chunk_bits(seed, tag, index, count):
    ss = np.random.SeedSequence(seed, spawn_key=(tag, index))
    g = np.random.Generator(np.random.PCG64(ss))
    return bf16_round(g.standard_normal(count, dtype=np.float32))


def _threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_bf16_range(seed, tag, start, stop):
    """Elements [start, stop) of the flat bf16 N(0,1) stream of a tensor tag."""
    out = np.empty(stop - start, dtype=np.uint16)
    if stop <= start:
        return out
    first, last = start // CHUNK, (stop - 1) // CHUNK

    def work(i):
        lo, hi = i * CHUNK, (i + 1) * CHUNK
        bits = _chunk_bits(seed, tag, i, CHUNK)
        a, b = max(lo, start), min(hi, stop)
        out[a - start:b - start] = bits[a - lo:b - lo]

    idx = range(first, last + 1)
    if last - first >= 2:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, idx))
    else:
        for i in idx:
            work(i)
    return out


@dataclass
class PassSpec:
    """Shape and metadata of one ragged pass (no tensors)."""
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    q_lens: np.ndarray          # int32 [S]
    ctx_lens: np.ndarray        # int32 [S]
    block_tables: np.ndarray    # int32 [S, max_blocks_per_seq], unused entries -1
    seed: int
    scale: float = 0.0          # 0 selects 1/sqrt(head_dim)
    notes: dict = field(default_factory=dict)

    @property
    def num_seqs(self):
        return int(len(self.q_lens))

    @property
    def num_tokens(self):
        return int(np.sum(self.q_lens, dtype=np.int64))

    @property
    def num_hist_tokens(self):
        return int(np.sum(self.ctx_lens, dtype=np.int64))

    @property
    def kv_lens(self):
        return (self.q_lens.astype(np.int64) + self.ctx_lens).astype(np.int32)

    @property
    def max_blocks_per_seq(self):
        return int(self.block_tables.shape[1])

    def history_pass(self):
        """The sequences' already-cached tokens as a pass of their own.

        Sequences with ctx > 0 contribute q_len = ctx at ctx 0, with the same
        block tables; appending it fills the pool with this pass's history.
        Returns (q_lens, ctx_lens, block_tables, seq_index) or None.
        """
        keep = np.nonzero(self.ctx_lens > 0)[0]
        if len(keep) == 0:
            return None
        return (self.ctx_lens[keep].astype(np.int32), np.zeros(len(keep), np.int32),
                np.ascontiguousarray(self.block_tables[keep]), keep)


@dataclass
class PassTensors:
    q: np.ndarray        # uint16 [T, Hq, D]
    k_new: np.ndarray    # uint16 [T, Hkv, D]
    v_new: np.ndarray    # uint16 [T, Hkv, D]
    hist_k: np.ndarray   # uint16 [sum(ctx), Hkv, D], sequence order
    hist_v: np.ndarray


def assign_blocks(rng, kv_lens, block_size, num_blocks=None, slack=1.25):
    """Draw a physical-block permutation and hand blocks out in its order."""
    need = [-(-int(n) // block_size) for n in kv_lens]
    total = int(sum(need))
    if num_blocks is None:
        num_blocks = max(1, math.ceil(slack * total))
    if total > num_blocks:
        raise ValueError("pool too small for the pass")
    perm = rng.permutation(num_blocks).astype(np.int32)
    width = max(1, max(need) if need else 1)
    tables = np.full((len(kv_lens), width), -1, dtype=np.int32)
    off = 0
    for s, k in enumerate(need):
        tables[s, :k] = perm[off:off + k]
        off += k
    return tables, num_blocks


def custom_spec(name, q_lens, ctx_lens, num_q_heads, num_kv_heads, head_dim, block_size,
                seed, num_blocks=None, scale=0.0, rng=None, slack=1.25):
    q_lens = np.asarray(q_lens, dtype=np.int32)
    ctx_lens = np.asarray(ctx_lens, dtype=np.int32)
    if rng is None:
        rng = np.random.Generator(np.random.PCG64(seed))
    kv = q_lens.astype(np.int64) + ctx_lens
    tables, nb = assign_blocks(rng, kv, block_size, num_blocks, slack)
    return PassSpec(name, num_q_heads, num_kv_heads, head_dim, block_size, nb,
                    q_lens, ctx_lens, tables, seed, scale)


def _decode_ctx(rng, count, mean=2660.0, sd=798.0):
    return np.maximum(1, np.rint(rng.normal(mean, sd, count))).astype(np.int32)


def _chunk_ctx(rng, count, chunk, mean=2600.0, sd=780.0):
    prompts = np.maximum(chunk, np.rint(rng.normal(mean, sd, count))).astype(np.int64)
    return (prompts - chunk).astype(np.int32)


def config_spec(cfg, seed=None):
    """PassSpec of a named workload.

    cfg:
      1 / "tiny"           3 seqs (40-token chunk at ctx 0, 1 decode at ctx 100,
                           23-token chunk at ctx 64), 4 q/kv heads, D 64, B 16, 64 blocks
      2 / "7b_pass2048"    16 decodes + one 2032-token final prompt chunk, 7B shape
      "7b_decode16"        the 16 decodes of cfg 2 alone
      "7b_chunk2032"       the chunk of cfg 2 alone
      3 / "7b_decode64"    64 decodes, ctx log-uniform 512..16000, 7B shape
      4 / "70b_share4096"  32 decodes + two 2032-token chunks, 16 q / 2 kv heads
      "70b_decode32", "70b_chunks"  its two halves
      "7b_budget<N>"       token-budget sweep point: the 16 decodes of cfg 2 plus
                           one prompt chunk of N - 16 tokens, the final chunk of
                           cfg 2's prompt P (context max(0, P - (N - 16)))
    """
    names = {1: "tiny", 2: "7b_pass2048", 3: "7b_decode64", 4: "70b_share4096"}
    name = names.get(cfg, cfg)
    if isinstance(name, str) and name.startswith("7b_budget"):
        budget = int(name[len("7b_budget"):])
        if budget < 32:
            raise ValueError("budget must be at least 32 tokens")
        rng = np.random.Generator(np.random.PCG64(2 if seed is None else seed))
        dec = _decode_ctx(rng, 16)
        prompt = int(_chunk_ctx(rng, 1, 2032)[0]) + 2032
        n = budget - 16
        return custom_spec(name, [1] * 16 + [n], list(dec) + [max(0, prompt - n)],
                           32, 32, 128, 64, 2 if seed is None else seed, rng=rng)
    base = {"tiny": 1, "7b_pass2048": 2, "7b_decode16": 2, "7b_chunk2032": 2,
            "7b_decode64": 3, "70b_share4096": 4, "70b_decode32": 4, "70b_chunks": 4}
    if name not in base:
        raise ValueError(f"unknown workload {cfg!r}")
    if seed is None:
        seed = base[name]
    rng = np.random.Generator(np.random.PCG64(seed))
    if name == "tiny":
        return custom_spec(name, [40, 1, 23], [0, 100, 64], 4, 4, 64, 16, seed,
                           num_blocks=64, rng=rng)
    if base[name] == 2:
        dec = _decode_ctx(rng, 16)
        chunk = _chunk_ctx(rng, 1, 2032)
        q = [1] * 16 + [2032]
        c = list(dec) + list(chunk)
        if name == "7b_decode16":
            q, c = q[:16], c[:16]
        elif name == "7b_chunk2032":
            q, c = q[16:], c[16:]
        return custom_spec(name, q, c, 32, 32, 128, 64, seed, rng=rng)
    if name == "7b_decode64":
        ctx = np.rint(np.exp(rng.uniform(math.log(512), math.log(16000), 64))).astype(np.int32)
        return custom_spec(name, [1] * 64, ctx, 32, 32, 128, 64, seed, rng=rng)
    dec = _decode_ctx(rng, 32)
    chunks = _chunk_ctx(rng, 2, 2032)
    q = [1] * 32 + [2032, 2032]
    c = list(dec) + list(chunks)
    if name == "70b_decode32":
        q, c = q[:32], c[:32]
    elif name == "70b_chunks":
        q, c = q[32:], c[32:]
    return custom_spec(name, q, c, 16, 2, 128, 64, seed, rng=rng)


def make_tensors(spec):
    """Draw Q, new K/V and the K/V history of a pass (bf16 bits)."""
    t, c = spec.num_tokens, spec.num_hist_tokens
    hq, hkv, d = spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    s = spec.seed
    return PassTensors(
        q=normal_bf16_range(s, TAG_Q, 0, t * hq * d).reshape(t, hq, d),
        k_new=normal_bf16_range(s, TAG_K_NEW, 0, t * hkv * d).reshape(t, hkv, d),
        v_new=normal_bf16_range(s, TAG_V_NEW, 0, t * hkv * d).reshape(t, hkv, d),
        hist_k=normal_bf16_range(s, TAG_HIST_K, 0, c * hkv * d).reshape(c, hkv, d),
        hist_v=normal_bf16_range(s, TAG_HIST_V, 0, c * hkv * d).reshape(c, hkv, d),
    )


def empty_pool_bits(spec, poison=False):
    """Fresh K and V pools filled with 0 or with bf16 NaN (poison mode).

    Both pools hold num_blocks * num_kv_heads * block_size * head_dim
    elements; the V pool's blocks are transposed sub-blocks of
    min(block_size, 32) slots, [num_blocks, Hkv, block_size / S, D, S].
    """
    fill = BF16_NAN if poison else 0
    sub = min(spec.block_size, 32)
    shape = (spec.num_blocks, spec.num_kv_heads, spec.block_size, spec.head_dim)
    tshape = (spec.num_blocks, spec.num_kv_heads, spec.block_size // sub, spec.head_dim, sub)
    return np.full(shape, fill, np.uint16), np.full(tshape, fill, np.uint16)


# ---------------------------------------------------------------- keyed hash generator
#
# For request traces the K/V/Q values of a token must not depend on which pass
# processed it, so they are a pure function of (seed, kind, request, position,
# head, dim): a counter-based generator built from the 32-bit "lowbias32"
# integer hash (Chris Wellons' hash-prospector construction:
# x ^= x >> 16; x *= 0x7feb352d; x ^= x >> 15; x *= 0x846ca68b; x ^= x >> 16).
# Two hashes give four 16-bit uniforms whose sum (Irwin-Hall, n = 4) is
# centred and scaled by 2^-15, an approximately normal value with sd ~1.155,
# then rounded to bf16 nearest-even.  Everything before the final rounding is
# exact integer arithmetic, and the integer -> float32 conversion and the
# power-of-two scaling are exact, so the numpy and torch versions below give
# identical bits on any device.

KIND_Q, KIND_K, KIND_V = 1, 2, 3
_M32 = 0xFFFFFFFF


def _lowbias32(x, xp):
    x = x ^ (x >> 16)
    x = (x * 0x7FEB352D) & _M32
    x = x ^ (x >> 15)
    x = (x * 0x846CA68B) & _M32
    x = x ^ (x >> 16)
    return x


def _token_keys(seed, kind, rid, positions, xp):
    """One 32-bit key per token; rid is a scalar or an array shaped like positions."""
    k = _lowbias32(positions * 0 + ((seed * 0x9E3779B1 + kind) & _M32), xp)
    k = _lowbias32(k ^ (rid & _M32), xp)
    return _lowbias32(k ^ positions, xp)


def hash_normal_bf16(seed, kind, rid, positions, heads, head_dim):
    """numpy: bf16 bits [len(positions), len(heads), head_dim] for one request."""
    pos = np.asarray(positions, dtype=np.int64)
    hs = np.asarray(heads, dtype=np.int64)
    key = _token_keys(seed, kind, rid, pos, np)                      # [n]
    elem = (hs[:, None] * head_dim + np.arange(head_dim, dtype=np.int64)[None, :]) * 2  # [H, D]
    x0 = _lowbias32(key[:, None, None] ^ elem[None], np)
    x1 = _lowbias32(key[:, None, None] ^ (elem[None] + 1), np)
    u = (x0 & 0xFFFF) + (x0 >> 16) + (x1 & 0xFFFF) + (x1 >> 16) - 131070
    return bf16_round(u.astype(np.float32) * np.float32(2.0 ** -15))


def hash_normal_bf16_torch(seed, kind, rid, positions, num_heads, head_dim, device):
    """torch (any device): bf16 tensor [len(positions), num_heads, head_dim], same bits.

    rid may be one request id or one per position (a whole pass at once)."""
    import torch
    pos = torch.as_tensor(positions, dtype=torch.int64, device=device)
    if not isinstance(rid, int):
        rid = torch.as_tensor(rid, dtype=torch.int64, device=device)
    key = _token_keys(seed, kind, rid, pos, torch)
    elem = (torch.arange(num_heads, dtype=torch.int64, device=device)[:, None] * head_dim
            + torch.arange(head_dim, dtype=torch.int64, device=device)[None, :]) * 2
    x0 = _lowbias32(key[:, None, None] ^ elem[None], torch)
    x1 = _lowbias32(key[:, None, None] ^ (elem[None] + 1), torch)
    u = (x0 & 0xFFFF) + (x0 >> 16) + (x1 & 0xFFFF) + (x1 >> 16) - 131070
    return (u.to(torch.float32) * (2.0 ** -15)).to(torch.bfloat16)
