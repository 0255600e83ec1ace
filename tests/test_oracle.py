"""Pins of the float64 CPU oracle against facts that do not come from itself.

Each test pins the oracle to something else: the bf16 format definition,
hand-derived closed forms, a textbook library routine on a reducible case,
pure-Python brute force, a one-hot addressing probe, worked examples printed
by the pages, and invariants the pages' problem statement fixes (block
permutation, split count, chunking, head grouping, sequence order).
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention as ora
from oracle import split_policy
from ragged_paged_attention_splitfuse_amd import workloads as wl
from tests._passes import cu_seqlens, logical_kv, oracle_pools

GOLDEN = __import__("os").path.join(__import__("os").path.dirname(__file__), "golden")


# ---------------------------------------------------------------- bf16 format

@pytest.mark.parametrize("bits,value", [
    (0x3F80, 1.0), (0xBF80, -1.0), (0x4000, 2.0), (0x4049, 3.140625),
    (0x3E80, 0.25), (0x0000, 0.0), (0x7F7F, (2 - 2 ** -7) * 2.0 ** 127),
    (0x0080, 2.0 ** -126), (0x0001, 2.0 ** -133), (0xC2F7, -123.5),
])
def test_bf16_decode_known_patterns(bits, value):
    # bf16 = sign, 8 exponent bits (bias 127), 7 fraction bits.
    got = ora.bf16_to_f64(np.array([bits], np.uint16))[0]
    assert got == value


def test_bf16_decode_specials():
    got = ora.bf16_to_f64(np.array([0x7F80, 0xFF80, 0x7FC0, 0x8000], np.uint16))
    assert got[0] == np.inf and got[1] == -np.inf and np.isnan(got[2])
    assert got[3] == 0.0 and math.copysign(1.0, got[3]) < 0


def test_generator_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 37
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(wl.bf16_round(x), ref)


# ---------------------------------------------------------------- append map

def _tiny_spec(q_lens, ctx_lens, hq=4, hkv=4, d=16, b=4, seed=11, nb=None):
    return wl.custom_spec("t", q_lens, ctx_lens, hq, hkv, d, b, seed, num_blocks=nb)


@pytest.mark.parametrize("b", [4, 64])
def test_append_places_every_element_by_its_flat_address(b):
    # V blocks are transposed sub-blocks of S = min(b, 32) slots: b = 4 is one
    # sub-block, b = 64 two, and the chunk of 70 tokens crosses both.
    spec = _tiny_spec([5, 1, 70], [3, 6, 0], hkv=2, hq=2, d=8, b=b, nb=40)
    t, hkv, d = spec.num_tokens, 2, 8
    sub = min(b, 32)
    ids = np.arange(1, t * hkv * d + 1, dtype=np.uint16).reshape(t, hkv, d)
    vids = (ids + 20000).astype(np.uint16)
    canary = 0x1234
    kp = np.full((spec.num_blocks, hkv, b, d), canary, np.uint16)
    vp = np.full((spec.num_blocks, hkv, b // sub, d, sub), canary, np.uint16)
    ko, vo = ora.kv_append(kp, vp, spec.q_lens, spec.ctx_lens, spec.block_tables, b, ids, vids)
    kf, vf = ko.reshape(-1), vo.reshape(-1)
    touched = np.zeros(kf.size, bool)
    row = 0
    for s in range(spec.num_seqs):
        for j in range(int(spec.q_lens[s])):
            p = int(spec.ctx_lens[s]) + j
            blk = int(spec.block_tables[s][p // b])
            off = p % b
            for g in range(hkv):
                for e in range(d):
                    kaddr = ((blk * hkv + g) * b + off) * d + e
                    vaddr = (blk * hkv + g) * d * b + (off // sub) * (d * sub) + e * sub + off % sub
                    assert kf[kaddr] == ids[row, g, e]
                    assert vf[vaddr] == vids[row, g, e]
                    touched[kaddr] = True
            row += 1
    assert np.all(kf[~touched] == canary)
    assert np.count_nonzero(vf != canary) == t * hkv * d


@pytest.mark.parametrize("b", [4, 16, 32, 64])
def test_gather_reads_every_element_from_its_flat_address(b):
    # Read-side mirror of the append pin: pools are filled directly, element by
    # element at the flat address the layout defines (K [blk][g][slot][e]; V
    # [blk][g][slot // S][e][slot % S], S = min(b, 32)), with a value that
    # names (sequence, position, head, dim).  gather_sequence must return them
    # in logical position order, so any index mix-up in its read path (block,
    # sub-block, slot, head or dim) shows.
    hkv, d = 2, 8
    lengths = [2 * b + 7, 1, b + 1]
    spec = _tiny_spec([1, 1, 1], [n - 1 for n in lengths], hq=hkv, hkv=hkv, d=d, b=b, nb=12)
    sub = min(b, 32)
    kf = np.full(spec.num_blocks * hkv * b * d, 0xFFFF, np.uint16)
    vf = np.full(spec.num_blocks * hkv * b * d, 0xFFFF, np.uint16)

    def ident(s, p, g, e, which):
        return ((which * 4 + s) * 256 + p) * 16 + g * d + e   # < 2**16, unique

    for s, n in enumerate(lengths):
        for p in range(n):
            blk = int(spec.block_tables[s][p // b])
            off = p % b
            for g in range(hkv):
                for e in range(d):
                    kf[((blk * hkv + g) * b + off) * d + e] = ident(s, p, g, e, 0)
                    vf[(blk * hkv + g) * d * b + (off // sub) * (d * sub) + e * sub + off % sub] = \
                        ident(s, p, g, e, 1)
    kp = kf.reshape(spec.num_blocks, hkv, b, d)
    vp = vf.reshape(spec.num_blocks, hkv, b // sub, d, sub)
    for s, n in enumerate(lengths):
        k, v = ora.gather_sequence(kp, vp, spec.block_tables[s], n, b)
        assert k.shape == (n, hkv, d) and v.shape == (n, hkv, d)
        for p in range(n):
            for g in range(hkv):
                for e in range(d):
                    assert k[p, g, e] == ident(s, p, g, e, 0), ("K", s, p, g, e)
                    assert v[p, g, e] == ident(s, p, g, e, 1), ("V", s, p, g, e)


# ---------------------------------------------------------------- reference reductions

def _run(spec, poison=False, scale=None):
    tens = wl.make_tensors(spec)
    kp, vp = oracle_pools(spec, tens, poison=poison)
    o, lse = ora.attend(tens.q, kp, vp, spec.q_lens, spec.ctx_lens, spec.block_tables,
                        spec.block_size, spec.num_kv_heads, scale=scale)
    return tens, kp, vp, o, lse


def _torch_reference(spec, tens, scale):
    """Dense causal attention via torch's SDPA in float64, explicit mask."""
    o_ref = np.zeros((spec.num_tokens, spec.num_q_heads, spec.head_dim))
    l_ref = np.zeros((spec.num_tokens, spec.num_q_heads))
    g = spec.num_q_heads // spec.num_kv_heads
    cu = cu_seqlens(spec.q_lens)
    for s, (kb, vb) in enumerate(logical_kv(spec, tens)):
        c, n = int(spec.ctx_lens[s]), int(spec.q_lens[s])
        q = torch.from_numpy(ora.bf16_to_f64(tens.q[cu[s]:cu[s] + n])).permute(1, 0, 2)
        k = torch.from_numpy(ora.bf16_to_f64(kb)).permute(1, 0, 2)
        v = torch.from_numpy(ora.bf16_to_f64(vb)).permute(1, 0, 2)
        k = k.repeat_interleave(g, dim=0)
        v = v.repeat_interleave(g, dim=0)
        mask = torch.arange(c + n)[None, :] <= (c + torch.arange(n))[:, None]
        o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale)
        sc = (q @ k.transpose(1, 2).contiguous()) * scale
        lse = torch.logsumexp(sc.masked_fill(~mask, -math.inf), dim=-1)
        o_ref[cu[s]:cu[s] + n] = o.permute(1, 0, 2).numpy()
        l_ref[cu[s]:cu[s] + n] = lse.permute(1, 0).numpy()
    return o_ref, l_ref


def test_textbook_reduction_single_contiguous_sequence():
    # One sequence, ctx 0, blocks in order, G = 1: plain dense causal attention.
    spec = _tiny_spec([37], [0], hq=3, hkv=3, d=32, b=8, nb=5)
    spec.block_tables[0, :5] = np.arange(5)
    tens, _, _, o, lse = _run(spec)
    o_ref, l_ref = _torch_reference(spec, tens, 1 / math.sqrt(32))
    assert np.max(np.abs(o - o_ref)) <= 1e-12
    assert np.max(np.abs(lse - l_ref)) <= 1e-12


DENSE_REFERENCE_SPECS = {
    "tiny": lambda: wl.config_spec(1),
    "mixed_gqa_b16": lambda: _tiny_spec([17, 1, 1, 33, 2], [0, 50, 7, 21, 63], hq=8, hkv=2, d=64,
                                        b=16, seed=5),
    # B = 32: one V sub-block per block; chunks cross block boundaries.
    "mixed_mha_b32": lambda: _tiny_spec([40, 1, 17, 3], [0, 50, 20, 61], hq=4, hkv=4, d=16, b=32,
                                        seed=42),
    # B = 64: two V sub-blocks per block.  Sequence 0 (70 tokens at ctx 0)
    # fills both sub-blocks of its first block; sequence 3 appends positions
    # 90..122, across the sub-block boundary at 96; sequence 4 crosses the
    # block boundary at 64; the decodes sit at 100 and 63 (a sub-block's last
    # slot and a block's last slot).
    "mixed_gqa_b64": lambda: _tiny_spec([70, 1, 1, 33, 5], [0, 100, 63, 90, 60], hq=4, hkv=2, d=32,
                                        b=64, seed=41),
}


@pytest.mark.parametrize("name", sorted(DENSE_REFERENCE_SPECS))
def test_dense_library_reference_ragged_paged(name):
    # Shuffled blocks, nonzero ctx, GQA: the oracle's append + gather + attend
    # against SDPA on the logical (never paged) K/V arrays.
    spec = DENSE_REFERENCE_SPECS[name]()
    tens, _, _, o, lse = _run(spec, poison=True)
    o_ref, l_ref = _torch_reference(spec, tens, 1 / math.sqrt(spec.head_dim))
    assert np.max(np.abs(o - o_ref)) <= 1e-12
    assert np.max(np.abs(lse - l_ref)) <= 1e-12


def test_brute_force_scalar_loops_tiny_config():
    # Pure-Python scalar loops, math.exp + math.fsum, on the tiny config.
    spec = wl.config_spec(1)
    tens, _, _, o, lse = _run(spec)
    scale = 1 / math.sqrt(64)
    qf = ora.bf16_to_f64(tens.q).tolist()
    cu = cu_seqlens(spec.q_lens)
    worst_o = worst_l = 0.0
    for s, (kb, vb) in enumerate(logical_kv(spec, tens)):
        kf, vf = ora.bf16_to_f64(kb).tolist(), ora.bf16_to_f64(vb).tolist()
        c, n = int(spec.ctx_lens[s]), int(spec.q_lens[s])
        for h in range(4):
            for j in range(n):
                qrow = qf[cu[s] + j][h]
                sc = [scale * math.fsum(qrow[e] * kf[t][h][e] for e in range(64)) for t in range(c + j + 1)]
                m = max(sc)
                w = [math.exp(x - m) for x in sc]
                den = math.fsum(w)
                for e in range(64):
                    val = math.fsum(w[t] * vf[t][h][e] for t in range(len(w))) / den
                    worst_o = max(worst_o, abs(val - o[cu[s] + j, h, e]))
                worst_l = max(worst_l, abs(m + math.log(den) - lse[cu[s] + j, h]))
    assert worst_o <= 1e-12 and worst_l <= 1e-12


# ---------------------------------------------------------------- closed forms

def _bits(x):
    return wl.bf16_round(np.asarray(x, np.float32))


def _closed_form_pass(q, k, v, c, b=4):
    """One sequence whose logical K/V are given; history = first c tokens."""
    n = q.shape[0]
    spec = wl.custom_spec("cf", [n], [c], q.shape[1], k.shape[1], q.shape[2], b, 3)
    tens = wl.PassTensors(q=_bits(q), k_new=_bits(k[c:]), v_new=_bits(v[c:]),
                          hist_k=_bits(k[:c]), hist_v=_bits(v[:c]))
    kp, vp = oracle_pools(spec, tens)
    return ora.attend(tens.q, kp, vp, spec.q_lens, spec.ctx_lens, spec.block_tables, b, k.shape[1])


def test_first_row_of_fresh_chunk_copies_v0():
    rng = np.random.default_rng(1)
    q, k, v = (rng.standard_normal((6, 1, 8)) for _ in range(3))
    o, lse = _closed_form_pass(q, k, v, c=0)
    v0 = ora.bf16_to_f64(_bits(v[0, 0]))
    assert np.array_equal(o[0, 0], v0)
    s0 = float(ora.bf16_to_f64(_bits(q[0, 0])) @ ora.bf16_to_f64(_bits(k[0, 0]))) / math.sqrt(8)
    assert abs(lse[0, 0] - s0) <= 1e-15


def test_zero_query_averages_visible_values():
    rng = np.random.default_rng(2)
    k, v = rng.standard_normal((13, 1, 8)), rng.standard_normal((13, 1, 8))
    q = np.zeros((5, 1, 8))
    o, lse = _closed_form_pass(q, k, v, c=8)
    vb = ora.bf16_to_f64(_bits(v))
    for j in range(5):
        p = 8 + j
        assert np.max(np.abs(o[j, 0] - vb[:p + 1, 0].mean(axis=0))) <= 1e-14
        assert abs(lse[j, 0] - math.log(p + 1)) <= 1e-14


def test_equal_keys_give_uniform_weights():
    rng = np.random.default_rng(3)
    key = rng.standard_normal(8)
    k = np.tile(key, (11, 1, 1))
    q, v = rng.standard_normal((3, 1, 8)), rng.standard_normal((11, 1, 8))
    o, lse = _closed_form_pass(q, k, v, c=8)
    vb = ora.bf16_to_f64(_bits(v))
    kq = ora.bf16_to_f64(_bits(key))
    for j in range(3):
        p = 8 + j
        sc = float(ora.bf16_to_f64(_bits(q[j, 0])) @ kq) / math.sqrt(8)
        assert np.max(np.abs(o[j, 0] - vb[:p + 1, 0].mean(axis=0))) <= 1e-14
        assert abs(lse[j, 0] - (sc + math.log(p + 1))) <= 1e-13


def test_constant_values_pass_through():
    rng = np.random.default_rng(4)
    q, k = rng.standard_normal((7, 2, 8)), rng.standard_normal((12, 2, 8))
    v = np.full((12, 2, 8), -1.5)
    o, _ = _closed_form_pass(q, k, v, c=5)
    assert np.max(np.abs(o + 1.5)) <= 1e-14


def test_two_key_weights_quarter_three_quarters():
    # scores 0 and ln 3 (times scale 1/sqrt(4) = 1/2): weights 1/4 and 3/4.
    # q = (2 ln 3, 0, 0, 0) is not a bf16 value, so put ln 3 into k instead:
    # q = (2,0,0,0), k1 = (x,0,0,0) with x = bf16(ln 3); score = x exactly.
    x = float(ora.bf16_to_f64(_bits([math.log(3.0)]))[0])
    q = np.array([[[0, 0, 0, 0]], [[2, 0, 0, 0]]], float)
    k = np.array([[[0, 0, 0, 0]], [[x, 0, 0, 0]]], float)
    v = np.array([[[4, 0, -8, 1]], [[0, 8, 4, 1]]], float)
    o, lse = _closed_form_pass(q, k, v, c=0)
    w1 = math.exp(x) / (1 + math.exp(x))
    expect = (1 - w1) * v[0, 0] + w1 * v[1, 0]
    assert np.max(np.abs(o[1, 0] - expect)) <= 1e-15
    assert abs(lse[1, 0] - math.log(1 + math.exp(x))) <= 1e-15


# ---------------------------------------------------------------- addressing probe

ONE_HOT_SPECS = {
    "tiny_b16": lambda: wl.config_spec(1),
    "mixed_b32": lambda: _tiny_spec([40, 1, 9], [0, 70, 60], hq=4, hkv=4, d=64, b=32, seed=43),
    "mixed_b64": lambda: _tiny_spec([70, 1, 40], [0, 130, 90], hq=4, hkv=4, d=64, b=64, seed=44),
}


@pytest.mark.parametrize("name", sorted(ONE_HOT_SPECS))
def test_one_hot_probe_every_block_boundary(name):
    # q = 32 e0 and a single key with k[0] = 32: score 1024 / sqrt(64) = 128
    # against 0 for every other key, so exp(-128) ~ 2.6e-56 and O is V[t*]
    # to far below 1e-40.  The probe is swept over both sides of every block
    # boundary of every sequence (and of every 32-slot V sub-block boundary
    # inside 64-slot blocks), in a shuffled pool.
    spec = ONE_HOT_SPECS[name]()
    b = spec.block_size
    sub = min(b, 32)
    base = wl.make_tensors(spec)
    cu = cu_seqlens(spec.q_lens)
    for s in range(spec.num_seqs):
        c, n = int(spec.ctx_lens[s]), int(spec.q_lens[s])
        length = c + n
        targets = sorted({t for blk in range(-(-length // sub)) for t in (blk * sub, blk * sub + sub - 1)
                          if t < length})
        for tstar in targets:
            tens = wl.PassTensors(q=np.zeros_like(base.q), k_new=np.zeros_like(base.k_new),
                                  v_new=base.v_new, hist_k=np.zeros_like(base.hist_k),
                                  hist_v=base.hist_v)
            tens.q[cu[s]:cu[s] + n, :, 0] = _bits(32.0)
            h0 = int(np.sum(spec.ctx_lens[:s]))
            if tstar < c:
                tens.hist_k[h0 + tstar, :, 0] = _bits(32.0)
            else:
                tens.k_new[cu[s] + tstar - c, :, 0] = _bits(32.0)
            kp, vp = oracle_pools(spec, tens, poison=True)
            o, lse = ora.attend(tens.q, kp, vp, spec.q_lens, spec.ctx_lens, spec.block_tables,
                                b, spec.num_kv_heads, seqs=[s])
            vlog = ora.bf16_to_f64(logical_kv(spec, tens)[s][1])
            for j in range(n):
                if c + j >= tstar:
                    assert np.max(np.abs(o[cu[s] + j] - vlog[tstar])) <= 1e-40
                    assert abs(lse[cu[s] + j, 0] - 128.0) <= 1e-12


# ---------------------------------------------------------------- invariants

def test_block_permutation_is_bit_invariant():
    spec = _tiny_spec([9, 1, 20], [30, 44, 5], hq=4, hkv=2, d=32, b=8, seed=8)
    tens, _, _, o, lse = _run(spec, poison=True)
    perm = np.random.default_rng(9).permutation(spec.num_blocks).astype(np.int32)
    spec2 = wl.PassSpec(**{**spec.__dict__})
    spec2.block_tables = np.where(spec.block_tables >= 0, perm[spec.block_tables], -1).astype(np.int32)
    kp, vp = oracle_pools(spec2, tens, poison=True)
    o2, lse2 = ora.attend(tens.q, kp, vp, spec2.q_lens, spec2.ctx_lens, spec2.block_tables,
                          spec2.block_size, spec2.num_kv_heads)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


@pytest.mark.parametrize("k", [1, 2, 3, 7, 64])
def test_split_count_invariance(k):
    spec = _tiny_spec([12, 1, 1, 40], [20, 200, 3, 90], hq=4, hkv=4, d=32, b=16, seed=12)
    tens, kp, vp, o, lse = _run(spec)
    o2, l2 = ora.attend_split(tens.q, kp, vp, spec.q_lens, spec.ctx_lens, spec.block_tables,
                              spec.block_size, spec.num_kv_heads,
                              lambda s, length: ora.split_ranges(length, k))
    assert np.max(np.abs(o - o2)) <= 1e-12 and np.max(np.abs(lse - l2)) <= 1e-12


def test_merge_with_empty_and_fully_masked_ranges():
    rng = np.random.default_rng(13)
    kg, vg = rng.standard_normal((50, 16)), rng.standard_normal((50, 16))
    qh = rng.standard_normal((4, 16))
    limits = np.array([10, 20, 30, 49])
    full = ora.partial_attend(qh, kg, vg, limits, 0, 50, 0.25)
    # [40, 50) is fully masked for rows 0..2; [25, 25) is empty.
    parts = [ora.partial_attend(qh, kg, vg, limits, a, b, 0.25)
             for a, b in [(0, 5), (5, 25), (25, 25), (25, 40), (40, 50)]]
    assert np.all(parts[2][1] == -np.inf) and np.all(parts[4][1][:3] == -np.inf)
    o, lse = ora.merge(parts)
    assert np.all(np.isfinite(o))
    assert np.max(np.abs(o - full[0])) <= 1e-13 and np.max(np.abs(lse - full[1])) <= 1e-13


def test_page_recipe_dense_vs_eight_splits():
    # Step 4 harness of the FastGen Guide: 8 heads, 4096 cached keys,
    # head_dim 128, one decode query, dense vs an 8-way split merge.
    rng = np.random.default_rng(14)
    q = ora.bf16_to_f64(_bits(rng.standard_normal((8, 128))))
    k = ora.bf16_to_f64(_bits(rng.standard_normal((8, 4096, 128))))
    v = ora.bf16_to_f64(_bits(rng.standard_normal((8, 4096, 128))))
    sc = 1 / math.sqrt(128)
    for h in range(8):
        lim = np.array([4095])
        dense = ora.partial_attend(q[h:h + 1], k[h], v[h], lim, 0, 4096, sc)
        parts = [ora.partial_attend(q[h:h + 1], k[h], v[h], lim, a, b, sc)
                 for a, b in ora.split_ranges(4096, 8)]
        o, lse = ora.merge(parts)
        assert np.max(np.abs(o - dense[0])) <= 1e-12 and abs(lse[0] - dense[1][0]) <= 1e-12


def test_chunked_prompt_equals_single_chunk():
    # A prompt processed in one pass vs three SplitFuse chunks over three passes.
    p, hq, hkv, d, b = 45, 4, 2, 32, 8
    rng = np.random.default_rng(15)
    q = _bits(rng.standard_normal((p, hq, d)))
    k = _bits(rng.standard_normal((p, hkv, d)))
    v = _bits(rng.standard_normal((p, hkv, d)))
    table = np.array([[5, 0, 3, 7, 1, 6]], np.int32)
    kp0 = np.zeros((8, hkv, b, d), np.uint16)
    vp0 = np.zeros((8, hkv, 1, d, b), np.uint16)     # b = 8: one V sub-block per block
    kp, vp = ora.kv_append(kp0, vp0, [p], [0], table, b, k, v)
    o_one, l_one = ora.attend(q, kp, vp, [p], [0], table, b, hkv)
    kp, vp = kp0, vp0
    outs, lses = [], []
    start = 0
    for n in (7, 13, 25):
        kp, vp = ora.kv_append(kp, vp, [n], [start], table, b, k[start:start + n], v[start:start + n])
        o, l_ = ora.attend(q[start:start + n], kp, vp, [n], [start], table, b, hkv)
        outs.append(o)
        lses.append(l_)
        start += n
    assert np.max(np.abs(np.concatenate(outs) - o_one)) <= 1e-12
    assert np.max(np.abs(np.concatenate(lses) - l_one)) <= 1e-12


def test_gqa_equals_mha_with_replicated_kv_heads():
    spec = _tiny_spec([6, 1, 14], [10, 33, 2], hq=8, hkv=2, d=16, b=8, seed=16)
    tens, _, _, o, lse = _run(spec)
    g = 4
    rep = wl.PassTensors(q=tens.q, k_new=np.repeat(tens.k_new, g, axis=1),
                         v_new=np.repeat(tens.v_new, g, axis=1),
                         hist_k=np.repeat(tens.hist_k, g, axis=1),
                         hist_v=np.repeat(tens.hist_v, g, axis=1))
    spec_mha = wl.PassSpec(**{**spec.__dict__})
    spec_mha.num_kv_heads = 8
    kp, vp = oracle_pools(spec_mha, rep)
    o2, l2 = ora.attend(tens.q, kp, vp, spec.q_lens, spec.ctx_lens, spec.block_tables,
                        spec.block_size, 8)
    assert np.array_equal(o, o2) and np.array_equal(lse, l2)


def test_sequence_order_permutes_rows():
    spec = _tiny_spec([3, 1, 8, 1], [4, 19, 0, 2], hq=2, hkv=2, d=16, b=4, seed=17)
    tens, _, _, o, lse = _run(spec)
    order = [2, 0, 3, 1]
    cu = cu_seqlens(spec.q_lens)
    hcu = cu_seqlens(spec.ctx_lens)
    rows = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in order])
    hrows = np.concatenate([np.arange(hcu[s], hcu[s + 1]) for s in order])
    spec2 = wl.PassSpec(**{**spec.__dict__})
    spec2.q_lens, spec2.ctx_lens = spec.q_lens[order], spec.ctx_lens[order]
    spec2.block_tables = spec.block_tables[order]
    t2 = wl.PassTensors(q=tens.q[rows], k_new=tens.k_new[rows], v_new=tens.v_new[rows],
                        hist_k=tens.hist_k[hrows], hist_v=tens.hist_v[hrows])
    kp, vp = oracle_pools(spec2, t2)
    o2, l2 = ora.attend(t2.q, kp, vp, spec2.q_lens, spec2.ctx_lens, spec2.block_tables,
                        spec2.block_size, spec2.num_kv_heads)
    assert np.array_equal(o[rows], o2) and np.array_equal(lse[rows], l2)


def test_poisoned_unused_slots_do_not_leak():
    spec = wl.config_spec(1)
    tens, _, _, o, lse = _run(spec, poison=False)
    _, _, _, o2, lse2 = _run(spec, poison=True)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    assert np.all(np.isfinite(o2))


# ---------------------------------------------------------------- split policies

def _read_golden(name):
    rows = []
    with open(f"{GOLDEN}/{name}") as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line)
    return rows


def test_figure_counts_match_printed_example():
    rows = [tuple(map(int, r.split())) for r in _read_golden("figure_split_counts.txt")]
    lengths = [r[0] for r in rows]
    assert split_policy.figure_counts(lengths) == [r[1] for r in rows]


def test_engine_counts_hand_derived_cases():
    for row in _read_golden("engine_split_cases.txt"):
        head, lens, want = (part.split() for part in row.split("|"))
        sms, chunk = int(head[0]), int(head[1])
        got = split_policy.engine_counts([int(x) for x in lens], sms, chunk)
        assert got == [int(x) for x in want]
