"""GPU parity: the HIP path through the C ABI against the float64 CPU oracle.

Bars: KV append and block addressing bit-exact; attention max-abs error
<= 1e-2 on O (fp32 output; bf16 in, fp32 accumulate) and <= 1e-3 on LSE.
Inputs are the seeded generator's; pools start poisoned with bf16 NaN so that
any read of an unwritten slot shows up.
"""
import ctypes
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention as ora
from ragged_paged_attention_splitfuse_amd import binding as fgb
from ragged_paged_attention_splitfuse_amd import workloads as wl
from tests import _gpu as G
from tests._passes import oracle_pools
from tests._plan_check import check_plan

pytestmark = pytest.mark.gpu

O_TOL = 1e-2
LSE_TOL = 1e-3
# Split vs unsplit on the GPU: both round P to bf16, but against different
# reference maxima, so each carries its own (independent) rounding error.
SPLIT_O_TOL = 5e-3


def _log(msg):
    print(msg, flush=True)


def compare(o_gpu, lse_gpu, o_ref, lse_ref, what, rows=None):
    o = o_gpu.float().cpu().numpy().astype(np.float64)
    lg = lse_gpu.cpu().numpy().astype(np.float64)
    if rows is not None:
        o, lg = o[rows], lg[rows]
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    eo = float(np.max(np.abs(o - o_ref))) if o.size else 0.0
    el = float(np.max(np.abs(lg - lse_ref))) if lg.size else 0.0
    _log(f"[parity] {what}: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= O_TOL, f"{what}: O error {eo}"
    assert el <= LSE_TOL, f"{what}: LSE error {el}"
    return eo, el


SMALL_SPECS = {
    "tiny": lambda: wl.config_spec(1),
    "mha_d128_b64_mixed": lambda: wl.custom_spec(
        "a", [1, 300, 1, 2, 77, 1], [2500, 131, 0, 64, 1000, 63], 4, 4, 128, 64, seed=21),
    "gqa8_d128_b64_mixed": lambda: wl.custom_spec(
        "b", [1, 1, 130, 40, 1], [700, 2, 333, 0, 129], 16, 2, 128, 64, seed=22),
    "mha_d64_b32_mixed": lambda: wl.custom_spec(
        "c", [3, 1, 90, 4], [10, 1500, 45, 300], 6, 6, 64, 32, seed=23),
    "gqa4_d64_b16_mixed": lambda: wl.custom_spec(
        "d", [1, 50, 1, 2], [333, 17, 1, 900], 8, 2, 64, 16, seed=24),
    "gqa2_d128_b16_mixed": lambda: wl.custom_spec(
        "e", [2, 1, 65, 1], [100, 999, 300, 0], 4, 2, 128, 16, seed=25),
    "gqa3_d128_b32_mixed": lambda: wl.custom_spec(
        "f", [1, 41, 7], [450, 200, 60], 6, 2, 128, 32, seed=26),
}


@pytest.mark.parametrize("name", sorted(SMALL_SPECS))
def test_attention_matches_oracle_small(name):
    spec = SMALL_SPECS[name]()
    _log(f"[case] small {name} S={spec.num_seqs} T={spec.num_tokens}")
    tens, _, _, out, lse, plan = G.full_gpu_pass(spec)
    check_plan(plan, spec)
    o_ref, l_ref = G.oracle_pass(spec, tens)
    compare(out, lse, o_ref, l_ref, name)


# FG_RANDOM_CASES widens the sweep (for example 412 for a long one-off run).
RANDOM_CASES = int(os.environ.get("FG_RANDOM_CASES", "48"))


@pytest.mark.parametrize("seed", range(RANDOM_CASES))
def test_random_compositions_match_oracle(seed):
    # seeds cycle through the three ways of running a pass (see tests/_gpu.py)
    from tests._random_passes import random_pass
    spec, knobs = random_pass(seed)
    mode = G.MODES[seed % 3]
    _log(f"[case] random {seed} ({mode}): S={spec.num_seqs} T={spec.num_tokens} q={[int(x) for x in spec.q_lens]} "
         f"ctx={[int(x) for x in spec.ctx_lens]} Hq/Hkv/D/B={spec.num_q_heads}/{spec.num_kv_heads}/"
         f"{spec.head_dim}/{spec.block_size} {knobs}")
    tens, kp, vp, out, lse, plan = G.full_gpu_pass(spec, mode=mode, **knobs)
    check_plan(plan, spec)
    o_ref, l_ref = G.oracle_pass(spec, tens)
    compare(out, lse, o_ref, l_ref, f"random {seed} ({mode})")
    if mode == "pass":
        kref, vref = oracle_pools(spec, tens, poison=True)
        assert np.array_equal(G.to_host_bits(kp), kref) and np.array_equal(G.to_host_bits(vp), vref)


@pytest.mark.parametrize("name", sorted(SMALL_SPECS))
@pytest.mark.parametrize("mode", ["pass", "direct"])
def test_single_launch_pass_and_direct_attention(name, mode):
    # fg_pass: pools bit-exact (the append runs inside the attention launch)
    # and attention on the oracle.  fg_attention_ragged_direct: the pools hold
    # only the history, their new slots stay NaN-poisoned, so a read of one
    # would show as a non-finite output.
    spec = SMALL_SPECS[name]()
    _log(f"[case] {mode} {name}")
    tens, kp, vp, out, lse, plan = G.full_gpu_pass(spec, mode=mode)
    o_ref, l_ref = G.oracle_pass(spec, tens)
    compare(out, lse, o_ref, l_ref, f"{mode} {name}")
    kref, vref = oracle_pools(spec, tens, poison=True)
    if mode == "pass":
        assert np.array_equal(G.to_host_bits(kp), kref) and np.array_equal(G.to_host_bits(vp), vref)
    else:
        # only the history was written: the new positions still hold poison
        hk, hv = oracle_pools(spec, wl.PassTensors(q=tens.q, k_new=np.full_like(tens.k_new, wl.BF16_NAN),
                                                   v_new=np.full_like(tens.v_new, wl.BF16_NAN),
                                                   hist_k=tens.hist_k, hist_v=tens.hist_v), poison=True)
        assert np.array_equal(G.to_host_bits(kp), hk) and np.array_equal(G.to_host_bits(vp), hv)


@pytest.mark.parametrize("mode", ["pass", "direct"])
@pytest.mark.parametrize("splits", [3, 64])
def test_single_launch_pass_with_split_groups(mode, splits):
    # split decode groups (merged in the attention launch) and split tiles
    # (merge launch), with the pass's own tokens read from k_new / v_new
    spec = SMALL_SPECS["gqa8_d128_b64_mixed"]()
    _log(f"[case] {mode} force_splits={splits}")
    tens, kp, vp, out, lse, plan = G.full_gpu_pass(spec, mode=mode, force_splits=splits, target_cus=16)
    assert plan.info["num_merge_groups"] > 0
    o_ref, l_ref = G.oracle_pass(spec, tens)
    compare(out, lse, o_ref, l_ref, f"{mode} force_splits={splits}")


# FG_RANDOM_BIG_CASES widens this one too (for example 400).
RANDOM_BIG_CASES = int(os.environ.get("FG_RANDOM_BIG_CASES", "8"))


@pytest.mark.parametrize("seed", range(RANDOM_BIG_CASES))
def test_random_big_compositions_match_oracle(seed):
    from tests._random_passes import random_big_pass
    spec, knobs = random_big_pass(seed)
    _log(f"[case] random big {seed}: S={spec.num_seqs} T={spec.num_tokens} max ctx={int(max(spec.ctx_lens))} "
         f"Hq/Hkv/D/B={spec.num_q_heads}/{spec.num_kv_heads}/{spec.head_dim}/{spec.block_size} {knobs}")
    tens, _, _, out, lse, plan = G.full_gpu_pass(spec, **knobs)
    check_plan(plan, spec)
    o_ref, l_ref = G.oracle_pass(spec, tens)
    compare(out, lse, o_ref, l_ref, f"random big {seed}")


@pytest.mark.parametrize("name", ["tiny", "mha_d128_b64_mixed", "gqa8_d128_b64_mixed", "gqa4_d64_b16_mixed"])
def test_append_is_bit_exact(name):
    spec = SMALL_SPECS[name]()
    _log(f"[case] append {name}")
    tens, kp, vp, _, _, _ = G.full_gpu_pass(spec)
    kref, vref = oracle_pools(spec, tens, poison=True)
    assert np.array_equal(G.to_host_bits(kp), kref)
    assert np.array_equal(G.to_host_bits(vp), vref)


@pytest.mark.parametrize("name", ["tiny", "mha_d128_b64_mixed", "gqa8_d128_b64_mixed", "gqa4_d64_b16_mixed"])
def test_upload_append_matches_separate_steps(name):
    # one launch (fg_upload_append) against fg_plan_upload + fg_kv_append:
    # same metadata bytes, bit-identical pools, bit-identical attention
    spec = SMALL_SPECS[name]()
    _log(f"[case] fused upload+append {name}")
    tens = wl.make_tensors(spec)
    q, kn, vn = G.to_dev(tens.q), G.to_dev(tens.k_new), G.to_dev(tens.v_new)
    pools = []
    for fused in (False, True):
        kp, vp = G.gpu_pools(spec, poison=True)
        G.fill_history(spec, tens, kp, vp)
        plan = fgb.Plan.from_spec(spec, target_cus=G.PLAN_CUS)
        if fused:
            meta = fgb.upload_append(plan, None, kn, vn, kp, vp)
        else:
            meta = plan.upload()
            fgb.kv_append(plan, meta, kn, vn, kp, vp)
        out = torch.full((spec.num_tokens, spec.num_q_heads, spec.head_dim), float("nan"), device="cuda")
        lse = torch.full((spec.num_tokens, spec.num_q_heads), float("nan"), device="cuda")
        fgb.attention_ragged(plan, meta, q, kp, vp, out, lse)
        torch.cuda.synchronize()
        nbytes = plan.info["metadata_bytes"]
        pools.append((G.to_host_bits(kp), G.to_host_bits(vp), meta[:nbytes].cpu().numpy(),
                      out.cpu(), lse.cpu()))
        plan.close()
    (k0, v0, m0, o0, l0), (k1, v1, m1, o1, l1) = pools
    assert np.array_equal(m0, m1)
    assert np.array_equal(k0, k1) and np.array_equal(v0, v1)
    kref, vref = oracle_pools(spec, tens, poison=True)
    assert np.array_equal(k1, kref) and np.array_equal(v1, vref)
    assert torch.equal(o0, o1) and torch.equal(l0, l1)


def test_plan_larger_than_pinned_staging():
    # 48 decodes x 16 heads (D 64) split 64 ways: about 49 k items, a plan of
    # more than 2 MiB, past the pinned staging slots.  fg_plan_upload then
    # copies with hipMemcpyAsync and fg_upload_append falls back to the
    # separate steps; both must give the plan's bytes and bit-identical
    # results, on the oracle for sampled sequences.
    spec = wl.custom_spec("big", [1] * 48, [4095] * 48, 16, 16, 64, 64, seed=28)
    _log("[case] plan larger than the pinned staging slots")
    tens = wl.make_tensors(spec)
    q, kn, vn = G.to_dev(tens.q), G.to_dev(tens.k_new), G.to_dev(tens.v_new)
    runs = []
    for fused in (False, True):
        kp, vp = G.gpu_pools(spec, poison=True)
        G.fill_history(spec, tens, kp, vp)
        plan = fgb.Plan.from_spec(spec, force_splits=64, target_cus=G.PLAN_CUS)
        assert plan.info["metadata_bytes"] > 2 << 20
        if fused:
            meta = fgb.upload_append(plan, None, kn, vn, kp, vp)
        else:
            meta = plan.upload()
            fgb.kv_append(plan, meta, kn, vn, kp, vp)
        out = torch.full((spec.num_tokens, spec.num_q_heads, spec.head_dim), float("nan"), device="cuda")
        lse = torch.full((spec.num_tokens, spec.num_q_heads), float("nan"), device="cuda")
        fgb.attention_ragged(plan, meta, q, kp, vp, out, lse)
        torch.cuda.synchronize()
        nbytes = plan.info["metadata_bytes"]
        runs.append((meta[:nbytes].cpu().numpy(), plan.metadata()["raw"], out, lse))
        plan.close()
    (m0, r0, o0, l0), (m1, r1, o1, l1) = runs
    assert np.array_equal(m0, r0) and np.array_equal(m1, r1)
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    picks = [0, 17, 47]
    sub, st, rows = G.subset(spec, tens, picks)
    o_ref, l_ref = G.oracle_pass(sub, st)
    compare(o0, l0, o_ref, l_ref, f"plan over 2 MiB, seqs {picks}", rows=rows)


@pytest.mark.parametrize("k", [1, 2, 3, 7, 64])
def test_forced_split_counts(k):
    spec = SMALL_SPECS["mha_d128_b64_mixed"]()
    _log(f"[case] forced splits k={k}")
    tens, _, _, out, lse, plan = G.full_gpu_pass(spec, force_splits=k)
    check_plan(plan, spec)
    o_ref, l_ref = G.oracle_pass(spec, tens)
    compare(out, lse, o_ref, l_ref, f"force_splits={k}")
    _, _, _, out1, lse1, _ = G.full_gpu_pass(spec, tens=tens, force_splits=1)
    do, dl = float((out - out1).abs().max()), float((lse - lse1).abs().max())
    _log(f"[split-invariance] k={k}: max|dO|={do:.3e} max|dLSE|={dl:.3e}")
    assert do <= SPLIT_O_TOL and dl <= LSE_TOL


@pytest.mark.parametrize("policy", [fgb.FG_SPLIT_ENGINE, fgb.FG_SPLIT_PER_1K])
def test_page_split_policies(policy):
    # the pages' split policies only move work around: results stay on the oracle
    spec = SMALL_SPECS["mha_d128_b64_mixed"]()
    _log(f"[case] split policy {policy}")
    tens, _, _, out, lse, plan = G.full_gpu_pass(spec, split_policy=policy, target_cus=16)
    check_plan(plan, spec)
    o_ref, l_ref = G.oracle_pass(spec, tens)
    compare(out, lse, o_ref, l_ref, f"split_policy={policy}")


def test_forced_splits_gqa_tiles():
    spec = SMALL_SPECS["gqa8_d128_b64_mixed"]()
    tens, _, _, out, lse, plan = G.full_gpu_pass(spec, force_splits=5)
    assert plan.info["num_merge_groups"] > 0
    o_ref, l_ref = G.oracle_pass(spec, tens)
    compare(out, lse, o_ref, l_ref, "gqa tiles force_splits=5")


@pytest.mark.parametrize("name,splits", [("gqa8_d128_b64_mixed", 3), ("mha_d64_b32_mixed", 4),
                                         ("over64", 100)])
def test_split_groups_merge_in_launch_and_rearm(name, splits):
    # Split decode groups (few splits) merge inside the attention launch: the
    # last split of a group to finish merges it and re-arms the group's counter;
    # split tiles and many-way splits get a merge launch.  Three launches on
    # one upload must agree bit for bit, match the oracle, and leave every
    # counter at zero.  "over64" splits a decode 71 ways (merge launch).
    if name == "over64":
        spec = wl.custom_spec("over64", [1, 1, 20], [9000, 300, 700], 8, 2, 128, 64, seed=27)
    else:
        spec = SMALL_SPECS[name]()
    _log(f"[case] in-launch merge {name} force_splits={splits}")
    tens = wl.make_tensors(spec)
    kp, vp = G.gpu_pools(spec)
    G.fill_history(spec, tens, kp, vp)
    plan = fgb.Plan.from_spec(spec, force_splits=splits, target_cus=16)
    check_plan(plan, spec)
    assert plan.info["num_merge_groups"] > 0
    if name == "over64":
        assert plan.info["max_splits_used"] > 64
    if name == "gqa8_d128_b64_mixed":
        # both kinds: decode groups merged in the launch, split tiles after it
        assert 0 < plan.info["num_inlaunch_merge_groups"] < plan.info["num_merge_groups"]
    if name == "mha_d64_b32_mixed":
        assert plan.info["num_inlaunch_merge_groups"] > 0
    meta = plan.upload()
    q, kn, vn = G.to_dev(tens.q), G.to_dev(tens.k_new), G.to_dev(tens.v_new)
    fgb.kv_append(plan, meta, kn, vn, kp, vp)
    t, hq, d = spec.num_tokens, spec.num_q_heads, spec.head_dim
    runs = []
    for _ in range(3):
        out = torch.full((t, hq, d), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full((t, hq), float("nan"), dtype=torch.float32, device="cuda")
        fgb.attention_ragged(plan, meta, q, kp, vp, out, lse)
        torch.cuda.synchronize()
        runs.append((out, lse))
    for out, lse in runs[1:]:
        assert torch.equal(out, runs[0][0]) and torch.equal(lse, runs[0][1])
    raw = meta.cpu().numpy()[:plan.info["metadata_bytes"]].view(np.int32)
    words = plan.info["num_inlaunch_merge_groups"]
    start = plan_counter_offset(plan) // 4
    counters = raw[start:start + words]
    assert len(counters) == words and not counters.any()
    o_ref, l_ref = G.oracle_pass(spec, tens)
    compare(runs[0][0], runs[0][1], o_ref, l_ref, f"in-launch merge {name}")


@pytest.mark.parametrize("hq,hkv", [(16, 2), (8, 8)])   # one-wave GQA groups; vector-ALU rows
def test_inlaunch_merge_stress_is_bit_stable(hq, hkv):
    # Regression guard for the in-launch merge's ordering: a pass whose split
    # decode and GQA groups all merge inside the attention launch, repeated 200
    # times on one upload.  Every repetition must equal the first bit for bit
    # (the merging work-group is whichever split finishes last, so a stale
    # partial row would change the result); the run stops at the first
    # mismatch.  The first result is also checked against the oracle.
    spec = wl.custom_spec("stress", [1] * 24 + [2, 4], [int(x) for x in np.linspace(300, 6000, 24)] + [800, 2000],
                          hq, hkv, 128, 64, seed=71)
    _log(f"[case] in-launch merge stress hq={hq} hkv={hkv}, 200 launches")
    tens = wl.make_tensors(spec)
    kp, vp = G.gpu_pools(spec)
    G.fill_history(spec, tens, kp, vp)
    plan = fgb.Plan.from_spec(spec, force_splits=4, target_cus=256)
    assert plan.info["num_inlaunch_merge_groups"] == plan.info["num_merge_groups"] > 0
    meta = plan.upload()
    q, kn, vn = G.to_dev(tens.q), G.to_dev(tens.k_new), G.to_dev(tens.v_new)
    fgb.kv_append(plan, meta, kn, vn, kp, vp)
    t, hq, d = spec.num_tokens, spec.num_q_heads, spec.head_dim
    ws = torch.empty(max(16, plan.info["workspace_bytes"]), dtype=torch.uint8, device="cuda")
    first = None
    for i in range(200):
        out = torch.empty((t, hq, d), dtype=torch.float32, device="cuda")
        lse = torch.empty((t, hq), dtype=torch.float32, device="cuda")
        fgb.attention_ragged(plan, meta, q, kp, vp, out, lse, workspace=ws)
        if i % 20 == 19 or first is None:
            torch.cuda.synchronize()
        if first is None:
            first = (out, lse)
            continue
        if i % 10 == 9:
            torch.cuda.synchronize()
        assert torch.equal(out, first[0]) and torch.equal(lse, first[1]), f"repetition {i} differs"
    o_ref, l_ref = G.oracle_pass(spec, tens)
    compare(first[0], first[1], o_ref, l_ref, f"in-launch merge stress hq={hq} hkv={hkv}")


def plan_counter_offset(plan):
    lay = fgb.fg_plan_layout_t()
    fgb._check(fgb.lib().fg_plan_metadata(plan.handle, None, 0, ctypes.byref(lay)), "fg_plan_metadata")
    return int(lay.counters)


def _bits_to_f32(bits):
    """bf16 bit patterns (uint16) -> the same values as float32."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


ONE_HOT_CASES = {            # Hq, Hkv, D, B
    "mha_d128_b64": (4, 4, 128, 64),
    "gqa8_d128_b16": (16, 2, 128, 16),
    "gqa4_d64_b32": (8, 2, 64, 32),
}


@pytest.mark.parametrize("name", sorted(ONE_HOT_CASES))
@pytest.mark.parametrize("splits", [0, 3])
def test_one_hot_probe_block_boundaries(name, splits):
    # Addressing pin without the oracle: every query is 40 * e_0 and the only
    # nonzero key entry is K[t*][.][0] = 40 for a per-sequence target t* at or
    # next to a block boundary, inside the cached context so every row sees
    # it.  The target's score beats every other by >= 141, so each other weight
    # is exp(-141), zero in fp32: O must be V[t*] bit for bit (fp32 output) and
    # LSE the target score, for decodes and chunk tiles, split or not.
    hq, hkv, d, b = ONE_HOT_CASES[name]
    targets = [0, b - 1, b, 2 * b - 1, 2 * b, 3 * b + 5, 5 * b - 1, 5 * b]
    ctx = [t + 1 + 37 * (i % 3) for i, t in enumerate(targets)]
    q_lens = [1, 70, 1, 3, 40, 1, 130, 2]
    spec = wl.custom_spec("probe", q_lens, ctx, hq, hkv, d, b, seed=51)
    _log(f"[case] one-hot probe {name} splits={splits}")
    base = wl.make_tensors(spec)
    t_rows, h_rows = spec.num_tokens, int(spec.ctx_lens.sum())
    q = np.zeros((t_rows, hq, d), np.float32)
    q[:, :, 0] = 40.0
    hk = np.zeros((h_rows, hkv, d), np.float32)
    hcu = np.concatenate([[0], np.cumsum(spec.ctx_lens)])
    for s, t in enumerate(targets):
        hk[hcu[s] + t, :, 0] = 40.0
    tens = wl.PassTensors(q=wl.bf16_round(q), k_new=wl.bf16_round(np.zeros((t_rows, hkv, d), np.float32)),
                          v_new=base.v_new, hist_k=wl.bf16_round(hk), hist_v=base.hist_v)
    _, _, _, out, lse, plan = G.full_gpu_pass(spec, tens=tens, force_splits=splits)
    if splits:
        assert plan.info["num_merge_groups"] > 0
    out = out.cpu().numpy()
    lse = lse.cpu().numpy().astype(np.float64)
    g_ratio = hq // hkv
    score = 1600.0 / np.sqrt(d)
    row = 0
    for s, t in enumerate(targets):
        want = _bits_to_f32(base.hist_v[hcu[s] + t])          # [Hkv, D]
        for _ in range(int(spec.q_lens[s])):
            for h in range(hq):
                assert np.array_equal(out[row, h], want[h // g_ratio]), (name, s, row, h)
            row += 1
    assert float(np.max(np.abs(lse - score))) <= 1e-4


@pytest.mark.parametrize("name", sorted(ONE_HOT_CASES))
def test_one_hot_probe_on_new_tokens_direct(name):
    # Addressing of k_new / v_new rows, bit for bit: the single key with
    # K[.][0] = 40 is one of the pass's own tokens (position ctx + n // 2 of
    # each sequence; a decode's own token), the pools hold only the history
    # (new slots poisoned), and fg_attention_ragged_direct must give O =
    # V[t*] exactly for every row at or past the target.
    hq, hkv, d, b = ONE_HOT_CASES[name]
    q_lens = [1, 70, 1, 3, 40, 1, 130, 2]
    ctx = [b - 1, 0, 2 * b, 3 * b + 5, b, 5 * b - 1, 37, 64]
    spec = wl.custom_spec("probe-new", q_lens, ctx, hq, hkv, d, b, seed=52)
    _log(f"[case] one-hot probe on new tokens {name}")
    base = wl.make_tensors(spec)
    t_rows = spec.num_tokens
    q = np.zeros((t_rows, hq, d), np.float32)
    q[:, :, 0] = 40.0
    kn = np.zeros((t_rows, hkv, d), np.float32)
    cu = np.concatenate([[0], np.cumsum(spec.q_lens)])
    targets = []
    for s_, n in enumerate(q_lens):
        j = n // 2
        kn[cu[s_] + j, :, 0] = 40.0
        targets.append(j)
    tens = wl.PassTensors(q=wl.bf16_round(q), k_new=wl.bf16_round(kn), v_new=base.v_new,
                          hist_k=wl.bf16_round(np.zeros_like(base.hist_k, dtype=np.float32)), hist_v=base.hist_v)
    _, _, _, out, lse, plan = G.full_gpu_pass(spec, tens=tens, mode="direct")
    out = out.cpu().numpy()
    g_ratio = hq // hkv
    for s_, j_t in enumerate(targets):
        want = _bits_to_f32(base.v_new[cu[s_] + j_t])            # [Hkv, D]
        for j in range(j_t, q_lens[s_]):
            for h in range(hq):
                assert np.array_equal(out[cu[s_] + j, h], want[h // g_ratio]), (name, s_, j, h)


def test_sequence_order_permutes_rows_bit_identically():
    # Shuffling the sequences of a pass permutes its output rows and changes
    # nothing else: same split structure per sequence, same arithmetic.
    spec = SMALL_SPECS["gqa8_d128_b64_mixed"]()
    tens, _, _, out, lse, _ = G.full_gpu_pass(spec)
    perm = np.array([3, 0, 4, 2, 1])
    cu = np.concatenate([[0], np.cumsum(spec.q_lens)])
    hcu = np.concatenate([[0], np.cumsum(spec.ctx_lens)])
    rows = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in perm])
    hrows = np.concatenate([np.arange(hcu[s], hcu[s + 1]) for s in perm])
    spec2 = wl.PassSpec(**{**spec.__dict__})
    spec2.q_lens, spec2.ctx_lens = spec.q_lens[perm].copy(), spec.ctx_lens[perm].copy()
    spec2.block_tables = spec.block_tables[perm].copy()
    tens2 = wl.PassTensors(q=tens.q[rows], k_new=tens.k_new[rows], v_new=tens.v_new[rows],
                           hist_k=tens.hist_k[hrows], hist_v=tens.hist_v[hrows])
    _, _, _, out2, lse2, _ = G.full_gpu_pass(spec2, tens=tens2)
    assert torch.equal(out2, out[torch.from_numpy(rows).to(out.device)])
    assert torch.equal(lse2, lse[torch.from_numpy(rows).to(lse.device)])


def test_block_permutation_is_bit_identical():
    spec = SMALL_SPECS["gqa8_d128_b64_mixed"]()
    tens, _, _, out, lse, _ = G.full_gpu_pass(spec)
    perm = np.random.default_rng(5).permutation(spec.num_blocks).astype(np.int32)
    spec2 = wl.PassSpec(**{**spec.__dict__})
    spec2.block_tables = np.where(spec.block_tables >= 0, perm[spec.block_tables], -1).astype(np.int32)
    _, _, _, out2, lse2, _ = G.full_gpu_pass(spec2, tens=tens)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


def test_repeat_runs_are_bit_identical():
    spec = SMALL_SPECS["mha_d128_b64_mixed"]()
    tens, kp, vp, out, lse, _ = G.full_gpu_pass(spec)
    out2, lse2, _ = G.run_pass(spec, tens, kp, vp)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


def test_bf16_output_mode():
    spec = SMALL_SPECS["gqa8_d128_b64_mixed"]()
    tens, _, _, out, lse, _ = G.full_gpu_pass(spec, out_dtype=torch.bfloat16)
    o_ref, l_ref = G.oracle_pass(spec, tens)
    o = out.float().cpu().numpy().astype(np.float64)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(o_ref), 1e-30))) - 7)
    assert np.all(np.abs(o - o_ref) <= O_TOL + ulp)
    assert float(np.max(np.abs(lse.cpu().numpy() - l_ref))) <= LSE_TOL


def test_chunked_prompt_matches_single_pass():
    # One 300-token prompt in one pass vs three SplitFuse chunks (ctx grows).
    p, hq, hkv, d, b = 300, 8, 2, 128, 64
    rng = np.random.default_rng(31)
    q = wl.bf16_round(rng.standard_normal((p, hq, d)).astype(np.float32))
    k = wl.bf16_round(rng.standard_normal((p, hkv, d)).astype(np.float32))
    v = wl.bf16_round(rng.standard_normal((p, hkv, d)).astype(np.float32))
    table = np.array([[4, 0, 2, 7, 1]], np.int32)
    one = wl.PassSpec("one", hq, hkv, d, b, 8, np.array([p], np.int32), np.array([0], np.int32),
                      table, 0)
    kp, vp = G.gpu_pools(one)
    t_one = wl.PassTensors(q=q, k_new=k, v_new=v, hist_k=k[:0], hist_v=v[:0])
    out1, lse1, _ = G.run_pass(one, t_one, kp, vp)
    kp, vp = G.gpu_pools(one)
    outs, lses, start = [], [], 0
    for n in (37, 200, 63):
        spec = wl.PassSpec("chunk", hq, hkv, d, b, 8, np.array([n], np.int32),
                           np.array([start], np.int32), table, 0)
        tc = wl.PassTensors(q=q[start:start + n], k_new=k[start:start + n], v_new=v[start:start + n],
                            hist_k=k[:0], hist_v=v[:0])
        o, l_, _ = G.run_pass(spec, tc, kp, vp)
        outs.append(o)
        lses.append(l_)
        start += n
    assert float((torch.cat(outs) - out1).abs().max()) <= 1e-3
    assert float((torch.cat(lses) - lse1).abs().max()) <= 1e-3


def test_empty_pass_launches_nothing():
    plan = fgb.Plan([], [], np.zeros((0, 1), np.int32), 4, 4, 64, 16, 8, target_cus=0)
    meta = plan.upload()
    kshape, vshape = fgb.pool_shapes(8, 4, 16, 64)
    kp = torch.zeros(kshape, dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros(vshape, dtype=torch.bfloat16, device="cuda")
    e = torch.empty((0, 4, 64), dtype=torch.bfloat16, device="cuda")
    fgb.kv_append(plan, meta, e, e, kp, vp)
    fgb.attention_ragged(plan, meta, e, kp, vp, torch.empty((0, 4, 64), device="cuda"))
    torch.cuda.synchronize()


def test_workspace_too_small_is_rejected():
    spec = SMALL_SPECS["mha_d128_b64_mixed"]()
    tens = wl.make_tensors(spec)
    kp, vp = G.gpu_pools(spec)
    plan = fgb.Plan.from_spec(spec, force_splits=3)
    meta = plan.upload()
    ws = torch.empty(plan.info["workspace_bytes"] - 16, dtype=torch.uint8, device="cuda")
    out = torch.empty((spec.num_tokens, spec.num_q_heads, spec.head_dim), device="cuda")
    with pytest.raises(fgb.FgError) as e:
        fgb.attention_ragged(plan, meta, G.to_dev(tens.q), kp, vp, out, workspace=ws)
    assert e.value.status == fgb.FG_E_WORKSPACE


# ---------------------------------------------------------------- full-size workloads

@pytest.mark.parametrize("name,mode", [("7b_pass2048", "separate"), ("70b_share4096", "separate"),
                                       ("7b_pass2048", "pass"), ("70b_share4096", "pass")])
def test_full_size_mixed_pass_all_rows(name, mode):
    spec = wl.config_spec(name)
    _log(f"[case] full {name} ({mode}) S={spec.num_seqs} T={spec.num_tokens}")
    tens, kp, vp, out, lse, plan = G.full_gpu_pass(spec, mode=mode)
    _log(f"[plan] {plan.info}")
    o_ref, l_ref = G.oracle_pass(spec, tens)
    compare(out, lse, o_ref, l_ref, f"{name} ({mode})")
    if mode == "pass":
        kref, vref = oracle_pools(spec, tens, poison=True)
        assert np.array_equal(G.to_host_bits(kp), kref) and np.array_equal(G.to_host_bits(vp), vref)


def test_full_size_decode64_every_row():
    # all 64 sequences x 32 heads, the oracle run on sub-passes of 8 sequences
    # (blocks relabelled: the oracle is bit-invariant under relabelling)
    spec = wl.config_spec(3)
    _log(f"[case] full 7b_decode64 kv={int(spec.kv_lens.sum())}")
    tens, _, _, out, lse, plan = G.full_gpu_pass(spec)
    _log(f"[plan] {plan.info}")
    for first in range(0, spec.num_seqs, 8):
        picks = list(range(first, min(spec.num_seqs, first + 8)))
        sub, st, rows = G.subset(spec, tens, picks)
        o_ref, l_ref = G.oracle_pass(sub, st)
        compare(out, lse, o_ref, l_ref, f"7b_decode64 seqs {picks[0]}..{picks[-1]}", rows=rows)


# ---------------------------------------------------------------- edge shapes

def test_long_context_decode_uses_many_splits():
    # a 120k-token decode next to short ones: the planner splits it up to the
    # split cap, and the merge combines all parts
    spec = wl.custom_spec("long", [1, 1, 3], [120000, 40, 70], 4, 4, 128, 64, seed=31)
    _log(f"[case] long decode kv={int(spec.kv_lens.max())}")
    tens, _, _, out, lse, plan = G.full_gpu_pass(spec, target_cus=256)
    _log(f"[plan] {plan.info}")
    assert plan.info["max_splits_used"] >= 16
    o_ref, l_ref = G.oracle_pass(spec, tens)
    compare(out, lse, o_ref, l_ref, "long decode")


@pytest.mark.parametrize("hq,hkv", [(32, 1), (32, 2)])
def test_mqa_and_wide_gqa_groups(hq, hkv):
    # G = 32 and 16: a decode is a 32- or 16-row group (one-wave matrix-core
    # item), a chunk row expands into G packed rows
    spec = wl.custom_spec("wide", [1, 5, 1, 37], [900, 300, 0, 120], hq, hkv, 128, 64, seed=32)
    _log(f"[case] hq={hq} hkv={hkv}")
    tens, _, _, out, lse, plan = G.full_gpu_pass(spec, target_cus=64)
    assert plan.info["num_mfma_items"] > 0
    o_ref, l_ref = G.oracle_pass(spec, tens)
    compare(out, lse, o_ref, l_ref, f"hq={hq} hkv={hkv}")


def test_scale_override():
    spec = wl.custom_spec("scale", [1, 70], [500, 90], 4, 2, 128, 32, seed=33, scale=0.3)
    tens, _, _, out, lse, plan = G.full_gpu_pass(spec)
    o_ref, l_ref = G.oracle_pass(spec, tens)
    compare(out, lse, o_ref, l_ref, "scale 0.3")


def test_budget8192_pass_all_heads():
    # the largest token-budget sweep point: an 8176-token chunk at context 0
    # plus 16 decodes.  Every q head is compared on all 16 decode rows and on
    # three row bands of the chunk (its first 128 rows, 128 rows mid-chunk and
    # its last 256, which see the most keys); a band is computed by the oracle
    # as a chunk of its own at the band's context.
    spec = wl.config_spec("7b_budget8192")
    _log(f"[case] 7b_budget8192 T={spec.num_tokens}")
    tens, _, _, out, lse, plan = G.full_gpu_pass(spec)
    _log(f"[plan] {plan.info}")
    decodes = [s for s in range(spec.num_seqs) if int(spec.q_lens[s]) == 1]
    chunk = next(s for s in range(spec.num_seqs) if int(spec.q_lens[s]) > 1)
    sub, st, rows = G.subset(spec, tens, decodes)
    o_ref, l_ref = G.oracle_pass(sub, st)
    compare(out, lse, o_ref, l_ref, "budget 8192 decodes, all heads", rows=rows)
    n = int(spec.q_lens[chunk])
    for j0, j1 in ((0, 128), (n // 2 - 64, n // 2 + 64), (n - 256, n)):
        sub, st, rows = G.band_subpass(spec, tens, chunk, j0, j1)
        o_ref, l_ref = G.oracle_pass(sub, st)
        compare(out, lse, o_ref, l_ref, f"budget 8192 chunk rows {j0}..{j1 - 1}, all heads", rows=rows)
