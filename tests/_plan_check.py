"""Independent checks of a plan's work list (coverage, slots, append runs).

A plan is correct when, for every query row (s, j, h), the KV ranges of the
items that compute it partition [0, ctx + j] (plus at most the few keys past
a row's causal limit inside its tile, which the kernels mask), split partials
land in disjoint workspace rows named by one split group (whose record and
zeroed arrival counter every split item points at), and every new token is
appended to exactly the slot its block table names.
"""
from collections import defaultdict

import numpy as np


def check_plan(plan, spec):
    meta = plan.metadata()
    seqs, items, merges, runs = meta["seqs"], meta["items"], meta["merges"], meta["runs"]
    g_ratio = spec.num_q_heads // spec.num_kv_heads
    info = plan.info
    assert len(items) == info["num_items"] == info["num_mfma_items"] + info["num_valu_items"]
    assert int((items[:, 7] > 0).sum()) == info["num_mfma_items"]

    # per-sequence records
    q_start = 0
    for s in range(spec.num_seqs):
        q, c = int(spec.q_lens[s]), int(spec.ctx_lens[s])
        rec = seqs[s]
        assert tuple(rec[:4]) == (q_start, q, c, q + c)
        nblk = -(-(q + c) // spec.block_size)
        assert rec[5] == nblk
        assert np.array_equal(meta["block_ids"][rec[4]:rec[4] + nblk], spec.block_tables[s, :nblk])
        q_start += q

    # items: path, alignment, grouping
    assert items.shape[1] == 12
    groups = defaultdict(list)
    for idx, it in enumerate(items):
        seq, kvh, row0, nrows, kv0, kv1, slot, waves, grp = map(int, it[:9])
        assert not it[9:].any()
        assert 0 <= seq < spec.num_seqs and 0 <= kvh < spec.num_kv_heads
        assert nrows >= 1 and kv1 > kv0 >= 0 and kv0 % 64 == 0
        if waves > 0:
            assert waves == -(-nrows // 32) and nrows <= 128
        else:
            assert nrows <= 4
        assert (slot < 0) == (grp < 0) and -1 <= grp < len(merges)
        groups[(seq, kvh, row0, nrows)].append((kv0, kv1, slot, grp))

    # one record per split group; the in-launch groups (at most one wavefront's
    # rows, in plans with few items per slot) come first and each has a zeroed
    # counter; split tiles follow, and so does every group of a plan with many
    # items per slot
    n_inl = info["num_inlaunch_merge_groups"]
    assert len(meta["counters"]) == n_inl and not meta["counters"].any()
    for gi, m in enumerate(merges):
        assert int(m[3]) <= 32 or gi >= n_inl
    if n_inl:
        assert n_inl == sum(1 for m in merges if int(m[3]) <= 32)
        # at most four items per resident work-group slot of the launched
        # kernel (the slot count is checked against the device on the GPU)
        slots = plan.resident_slots()[0]
        assert slots in (2, 3, 4)
        assert len(items) <= 4 * slots * info["target_cus"]
    merge_by_group = {}
    for gi, m in enumerate(merges):
        seq, kvh, row0, nrows, nsplit, slot0, pad0, pad1 = map(int, m)
        assert pad0 == 0 and pad1 == 0 and nsplit >= 2
        key = (seq, kvh, row0, nrows)
        assert key not in merge_by_group
        merge_by_group[key] = (nsplit, slot0, gi)

    used_slots = np.zeros(info["num_partial_rows"], dtype=np.int32)
    rows_seen = defaultdict(int)
    for (seq, kvh, row0, nrows), parts in groups.items():
        parts.sort()
        c = int(spec.ctx_lens[seq])
        vis_end = c + (row0 + nrows - 1) // g_ratio + 1
        assert parts[0][0] == 0 and parts[-1][1] == vis_end
        for (a0, a1, _, _), (b0, b1, _, _) in zip(parts, parts[1:]):
            assert a1 == b0
        if len(parts) == 1:
            assert parts[0][2] == -1 and (seq, kvh, row0, nrows) not in merge_by_group
        else:
            nsplit, slot0, gi = merge_by_group[(seq, kvh, row0, nrows)]
            assert nsplit == len(parts)
            for i, (_, _, slot, grp) in enumerate(parts):
                assert slot == slot0 + i * nrows and grp == gi
                used_slots[slot:slot + nrows] += 1
        for r in range(row0, row0 + nrows):
            rows_seen[(seq, kvh, r)] += 1
    assert np.all(used_slots == 1)
    assert len(merge_by_group) == info["num_merge_groups"]
    for s in range(spec.num_seqs):
        for g in range(spec.num_kv_heads):
            for r in range(int(spec.q_lens[s]) * g_ratio):
                assert rows_seen[(s, g, r)] == 1

    # append runs: each new token exactly once, in its table's slot
    b = spec.block_size
    cover = {}
    for tok0, slot0, count, block in map(lambda x: map(int, x), runs):
        assert 1 <= count and slot0 + count <= b
        for i in range(count):
            assert (tok0 + i) not in cover
            cover[tok0 + i] = (block, slot0 + i)
    tok = 0
    for s in range(spec.num_seqs):
        for j in range(int(spec.q_lens[s])):
            p = int(spec.ctx_lens[s]) + j
            assert cover[tok] == (int(spec.block_tables[s, p // b]), p % b)
            tok += 1
    assert len(cover) == spec.num_tokens
    return meta
