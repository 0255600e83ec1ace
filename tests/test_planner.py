"""Host planner (fg_plan_pass) on the CPU: validation, coverage, determinism."""
import numpy as np
import pytest

from ragged_paged_attention_splitfuse_amd import binding as fgb
from ragged_paged_attention_splitfuse_amd import workloads as wl
from tests._plan_check import check_plan

CUS = 256


def plan_of(spec, **knobs):
    knobs.setdefault("target_cus", CUS)
    return fgb.Plan.from_spec(spec, **knobs)


@pytest.mark.parametrize("name", ["tiny", "7b_pass2048", "7b_decode64", "70b_share4096",
                                  "7b_decode16", "7b_chunk2032", "70b_chunks"])
def test_plan_covers_every_row_once(name):
    spec = wl.config_spec(name)
    check_plan(plan_of(spec), spec)


@pytest.mark.parametrize("k", [1, 2, 3, 7, 64])
def test_forced_splits_cover(k):
    spec = wl.custom_spec("f", [1, 300, 2, 1, 70], [2000, 40, 900, 0, 129], 8, 2, 128, 64, seed=3)
    plan = plan_of(spec, force_splits=k)
    meta = check_plan(plan, spec)
    assert plan.info["max_splits_used"] <= k
    if k > 1:
        assert len(meta["merges"]) > 0


def test_mixed_shapes_and_block_sizes_cover():
    for d in (64, 128):
        for b in (16, 32, 64):
            for hq, hkv in ((4, 4), (8, 2), (12, 4), (6, 1)):
                spec = wl.custom_spec("m", [1, 5, 130, 1, 3], [77, 0, 260, 5000, 1], hq, hkv, d, b, seed=b + d)
                check_plan(plan_of(spec), spec)
                check_plan(plan_of(spec, force_splits=5), spec)


def test_plan_is_deterministic():
    spec = wl.config_spec(3)
    a, b = plan_of(spec), plan_of(spec)
    assert np.array_equal(a.metadata()["raw"], b.metadata()["raw"])
    assert a.info == b.info


def test_plan_depends_on_lengths_not_block_ids():
    spec = wl.config_spec(2)
    perm = np.random.default_rng(1).permutation(spec.num_blocks).astype(np.int32)
    spec2 = wl.PassSpec(**{**spec.__dict__})
    spec2.block_tables = np.where(spec.block_tables >= 0, perm[spec.block_tables], -1).astype(np.int32)
    ia, ib = plan_of(spec).metadata()["items"], plan_of(spec2).metadata()["items"]
    assert np.array_equal(ia, ib)


def test_long_decodes_are_split_short_ones_not():
    spec = wl.custom_spec("d", [1] * 64, [16000] + [512] * 63, 32, 32, 128, 64, seed=4)
    meta = plan_of(spec).metadata()
    items = meta["items"]
    per_seq = np.bincount(items[:, 0], minlength=64)
    assert per_seq[0] > per_seq[1:].max()
    assert per_seq[1:].max() == 32     # one item per head, no split


def test_tile_free_plan_fits_whole_rounds_of_slots():
    """The 70B-class decode half (64 GQA groups) splits to at most one item per
    work-group slot rather than spilling a few items into a second round, and
    still covers every row once."""
    spec = wl.config_spec("70b_decode32")
    plan = plan_of(spec)
    check_plan(plan, spec)
    slots = CUS * 2
    n = plan.info["num_items"]
    assert slots * 3 // 4 < n <= slots
    assert plan.info["max_splits_used"] > 1
    # a plan with tiles is left alone: the 70B share keeps its decode splits
    assert plan_of(wl.config_spec("70b_share4096")).info["num_items"] > slots


def test_skewed_decode_only_pass_splits_only_its_longest_decodes():
    """64 decodes with contexts spread over 512..16000: at two or more groups
    per slot the split target halves, so the longest decodes split and the
    short ones stay whole."""
    spec = wl.config_spec("7b_decode64")
    meta = check_plan(plan_of(spec), spec)
    items = meta["items"]
    per_seq = np.bincount(items[:, 0], minlength=spec.num_seqs) // spec.num_kv_heads
    kv = np.asarray(spec.ctx_lens) + np.asarray(spec.q_lens)
    assert per_seq[np.argmax(kv)] >= 2
    assert (per_seq[kv <= np.median(kv)] == 1).all()
    total = float(kv.sum()) * spec.num_kv_heads
    half_target = total / (CUS * 2.0 * 2.0)
    assert (per_seq[kv * 1.0 <= half_target] == 1).all()


@pytest.mark.parametrize("seed", range(40))
def test_random_compositions_cover_every_row_once(seed):
    from tests._random_passes import random_pass
    spec, knobs = random_pass(seed)
    check_plan(plan_of(spec, **knobs), spec)


def _item_costs(items):
    lengths = (items[:, 5] - items[:, 4]).astype(np.float64)
    mf = items[:, 7] > 0
    # matrix-core cost per token grows with the tile's wavefront count
    return np.where(mf, lengths * np.maximum(0.5, items[:, 7] * 32 / 170.0), lengths), mf


def test_items_are_longest_first_per_kind_and_interleaved():
    for name in ("7b_decode64", "7b_pass2048", "70b_share4096"):
        items = plan_of(wl.config_spec(name)).metadata()["items"]
        cost, mf = _item_costs(items)
        # the resident rounds are reordered for balance: two work-groups per
        # CU in the kernel with matrix-core items, three in the decode-only
        # kernel at D = 128
        m = min(len(items), (2 if mf.any() else 3) * CUS)
        cost, mf = cost[m:], mf[m:]
        assert np.all(np.diff(cost[mf]) <= 1e-9) and np.all(np.diff(cost[~mf]) <= 0)
        if mf.any() and (~mf).any():
            # both kinds spread over the whole order
            pos = np.nonzero(mf)[0] / len(cost)
            assert pos.min() < 0.05 and pos.max() > 0.95


@pytest.mark.parametrize("name", ["7b_chunk2032", "70b_chunks", "70b_share4096", "7b_pass2048"])
def test_resident_rounds_balance_cu_pairs(name):
    # positions p and p + CUS share a CU; their summed cost is evened out
    items = plan_of(wl.config_spec(name)).metadata()["items"]
    cost, _ = _item_costs(items)
    m = min(len(items), 2 * CUS)
    loads = cost[:CUS].copy()
    loads[:m - CUS] += cost[CUS:m]
    top = np.sort(cost[:m])[::-1]            # the same items, paired in sorted order
    naive = top[:CUS].copy()
    naive[:m - CUS] += top[CUS:m]
    assert loads.max() <= naive.max() + 1e-9
    assert loads.max() - loads.min() <= cost[:m].max() + 1e-9
    if name in ("7b_chunk2032", "70b_chunks"):
        assert loads.max() <= 1.01 * loads.mean()


@pytest.mark.parametrize("name", ["7b_decode16", "7b_decode64"])
def test_resident_rounds_balance_three_slots_in_decode_only_plans(name):
    # decode-only plans at D = 128 run three work-groups per CU: positions p,
    # p + CUS and p + 2 CUS share a CU, and their summed cost is evened out
    items = plan_of(wl.config_spec(name)).metadata()["items"]
    cost, mf = _item_costs(items)
    assert not mf.any()
    m = min(len(items), 3 * CUS)
    loads = np.zeros(CUS)
    for pos in range(m):
        loads[pos % CUS] += cost[pos]
    top = np.sort(cost[:m])[::-1]            # plain longest-first dealing
    naive = np.zeros(CUS)
    for pos in range(m):
        naive[pos % CUS] += top[pos]
    assert loads.max() <= naive.max() + 1e-9
    assert loads.max() - loads.min() <= 2 * cost[:m].max() + 1e-9
    assert loads.max() <= 1.06 * loads.mean()
    if m == 3 * CUS:
        assert loads.max() <= 1.01 * loads.mean()


def test_planned_resident_slots():
    # work-groups per CU of the attention kernel a plan launches (from its
    # register count): two with matrix-core items at D = 128 or B = 64, three at
    # D = 64 with B < 64; three (D = 128) or four (D = 64) in the decode-only
    # kernel.  No GPU here, so the device count reads -1 (the GPU test compares).
    want = {(64, 16, True): 3, (64, 32, True): 3, (64, 64, True): 2,
            (128, 16, True): 2, (128, 32, True): 2, (128, 64, True): 2,
            (64, 16, False): 4, (64, 32, False): 4, (64, 64, False): 4,
            (128, 16, False): 3, (128, 32, False): 3, (128, 64, False): 3}
    for (d, b, tiles), n in want.items():
        if tiles:
            spec = wl.custom_spec("t", [1] * 8 + [300], [3000] * 8 + [500], 8, 8, d, b, seed=1)
        else:
            spec = wl.custom_spec("d", [1] * 40, [3000] * 40, 8, 8, d, b, seed=2)
        plan = plan_of(spec)
        assert (plan.info["num_mfma_items"] > 0) == tiles
        planned, device = plan.resident_slots()
        assert planned == n and device in (-1, n), (d, b, tiles)


def test_tiny_plan_has_no_splits_and_no_workspace():
    plan = plan_of(wl.config_spec(1))
    assert plan.info["num_merge_groups"] == 0 and plan.info["workspace_bytes"] == 0


def test_empty_pass():
    plan = fgb.Plan([], [], np.zeros((0, 1), np.int32), 4, 4, 64, 16, 8, target_cus=CUS)
    assert plan.info["num_tokens"] == 0 and plan.info["num_items"] == 0


def _expect(status, **over):
    base = dict(q_lens=[3, 1], ctx_lens=[0, 20], block_tables=[[0, -1], [1, 2]],
                num_q_heads=4, num_kv_heads=2, head_dim=128, block_size=16, num_blocks=4,
                target_cus=CUS)
    base.update(over)
    with pytest.raises(fgb.FgError) as e:
        fgb.Plan(**base)
    assert e.value.status == status


def test_validation_errors():
    _expect(fgb.FG_E_RANGE, block_tables=[[0, -1], [1, 7]])          # block id out of range
    _expect(fgb.FG_E_RANGE, block_tables=[[0, -1], [-1, 2]])         # negative id in use
    _expect(fgb.FG_E_ALIAS, block_tables=[[1, -1], [1, 2]])          # block shared
    _expect(fgb.FG_E_RANGE, ctx_lens=[0, 40])                        # table too short
    _expect(fgb.FG_E_RANGE, q_lens=[0, 1])                           # empty query
    _expect(fgb.FG_E_RANGE, ctx_lens=[-1, 20])
    _expect(fgb.FG_E_INVALID, num_q_heads=6, num_kv_heads=4)         # Hq % Hkv
    _expect(fgb.FG_E_UNSUPPORTED, head_dim=96)
    _expect(fgb.FG_E_UNSUPPORTED, block_size=128)
    _expect(fgb.FG_E_INVALID, num_blocks=0)
    _expect(fgb.FG_E_INVALID, scale=float("nan"))
    _expect(fgb.FG_E_INVALID, scale=-1.0)
    _expect(fgb.FG_E_INVALID, force_splits=1000)
    _expect(fgb.FG_E_INVALID, target_cus=-3)
    _expect(fgb.FG_E_INVALID, split_policy=3)
    _expect(fgb.FG_E_INVALID, split_policy=-1)


def test_unused_table_entries_are_ignored():
    # entries past ceil(kv/B) may be anything, even out of range or repeated
    plan = fgb.Plan([3, 1], [0, 20], [[0, 99], [1, 2]], 4, 2, 128, 16, 4, target_cus=CUS)
    assert plan.info["num_tokens"] == 4
    plan = fgb.Plan([3, 1], [0, 5], [[0, 1], [1, 2]], 4, 2, 128, 16, 4, target_cus=CUS)
    assert plan.info["num_tokens"] == 4


# ---- the pages' split policies, native in the planner, against the oracle's
# restatements (which the golden files pin)
from oracle.split_policy import engine_counts, figure_counts  # noqa: E402


def _aligned(k, length):
    """Parts a range of `length` tokens gets when asked for k splits of
    64-token-aligned size (the planner's own alignment step)."""
    k = max(1, min(k, -(-length // 64)))
    chunk = -(-(-(-length // k)) // 64) * 64
    return -(-length // chunk)


def _splits_per_seq(plan, num_seqs):
    items = plan.metadata()["items"]
    items = items[items[:, 3] > 0]
    out = []
    for s in range(num_seqs):
        sel = items[items[:, 0] == s]
        # one kv head suffices: every head of a sequence gets the same count
        sel = sel[sel[:, 1] == 0]
        out.append(len(sel))
    return out


@pytest.mark.parametrize("policy", ["engine", "per1k"])
@pytest.mark.parametrize("cus", [256, 108, 8])
def test_page_policies_match_oracle(policy, cus):
    rng = np.random.default_rng(11 + cus)
    for trial in range(6):
        n = int(rng.integers(1, 40))
        ctx = np.exp(rng.uniform(np.log(20), np.log(40000), n)).astype(np.int64).tolist()
        spec = wl.custom_spec("p", [1] * n, ctx, 4, 4, 64, 64, seed=trial)
        lens = [c + 1 for c in ctx]
        if policy == "engine":
            want = engine_counts(lens, num_sms=cus, min_chunk_size=256)
            plan = plan_of(spec, target_cus=cus, split_policy=fgb.FG_SPLIT_ENGINE, max_splits=256)
        else:
            want = figure_counts(lens)
            plan = plan_of(spec, target_cus=cus, split_policy=fgb.FG_SPLIT_PER_1K, max_splits=256)
        got = _splits_per_seq(plan, n)
        assert got == [_aligned(min(k, 256), L) for k, L in zip(want, lens)], (lens, want, got)
        check_plan(plan, spec)


def test_engine_policy_golden_case():
    # the page's Step 4 harness input at 108 SMs and a 512-token minimum chunk
    lens = [256, 1024, 4096, 8192]
    spec = wl.custom_spec("g", [1] * 4, [x - 1 for x in lens], 4, 4, 64, 64, seed=1)
    plan = plan_of(spec, target_cus=108, split_policy=fgb.FG_SPLIT_ENGINE,
                   min_split_tokens=512, max_splits=256)
    assert _splits_per_seq(plan, 4) == [_aligned(k, L) for k, L in zip([4, 8, 32, 64], lens)]


@pytest.mark.parametrize("q_len,hq,hkv", [
    (65536, 65536, 1),      # q_len * G = 2^32 packed rows: past int32
    (32768, 65536, 1),      # 2^31 packed rows: one past INT32_MAX
    (16384, 16384 * 16, 16),  # 2^28 rows per kv head, 2^25 row tiles: past one launch
])
def test_rows_and_launch_sizes_past_the_limits_are_rejected(q_len, hq, hkv):
    # A plan that exists is valid: packed row indices are int32 and a launch
    # holds at most 2^24 - 1 work-groups, so larger passes return FG_E_RANGE
    # instead of wrapping around.
    b = 64
    bt = np.arange(-(-q_len // b), dtype=np.int32).reshape(1, -1)
    with pytest.raises(fgb.FgError) as e:
        fgb.Plan([q_len], [0], bt, hq, hkv, 128, b, bt.size, target_cus=64)
    assert e.value.status == fgb.FG_E_RANGE


def test_large_but_valid_gqa_chunk_is_planned():
    # 8192 rows per kv head (q_len 1024, G 8): inside every limit
    b = 64
    spec = wl.custom_spec("g", [1024, 1], [0, 700], 16, 2, 128, b, seed=9)
    plan = plan_of(spec)
    check_plan(plan, spec)
