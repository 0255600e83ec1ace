"""Host Dynamic SplitFuse scheduler: composition and allocation invariants.

The composition is not unique (any valid pass order gives the same attention
results), so it is pinned by invariants: the token budget, a full budget
whenever enough work is queued, every prompt token once and in order, O - 1
decodes per request after its prompt, closed-loop admission, and block
tables that only grow and never alias.
"""
from collections import defaultdict

import numpy as np
import pytest

from ragged_paged_attention_splitfuse_amd import binding as fgb
from ragged_paged_attention_splitfuse_amd import splitfuse as sf


def _check(requests, passes, nb, clients, budget, block_size):
    req = {r.rid: r for r in requests}
    prompt_done = defaultdict(int)
    decodes = defaultdict(int)
    finished, admitted = set(), []
    tables = {}
    live_prev = set()
    for p in passes:
        rids = [int(x) for x in p.rids]
        assert p.num_tokens <= budget
        assert len(set(rids)) == len(rids)
        # decodes first
        assert np.all(p.q_lens[:p.num_decodes] == 1)
        live = set(rids)
        for rid in rids:
            if rid not in admitted:
                admitted.append(rid)
        # closed loop: at most `clients` unfinished admitted requests
        active = [r for r in admitted if r not in finished]
        assert len(active) <= clients
        # queued work at pass start: every active request's remaining prompt + decode tokens
        queued = sum((1 if prompt_done[r] == req[r].prompt and decodes[r] < req[r].output - 1 else 0)
                     + (req[r].prompt - prompt_done[r]) for r in active)
        if queued >= budget:
            assert p.num_tokens == budget
        used = set()
        for s, rid in enumerate(rids):
            r = req[rid]
            ctx, n = int(p.ctx_lens[s]), int(p.q_lens[s])
            if s < p.num_decodes:
                assert prompt_done[rid] == r.prompt and ctx == r.prompt + decodes[rid]
                decodes[rid] += 1
                assert decodes[rid] <= r.output - 1
            else:
                assert ctx == prompt_done[rid] and n >= 1
                prompt_done[rid] += n
                assert prompt_done[rid] <= r.prompt
            row = [int(b) for b in p.block_tables[s] if b >= 0]
            assert len(row) * block_size >= ctx + n
            prev = tables.get(rid, [])
            assert row[:len(prev)] == prev           # tables only grow
            tables[rid] = row
            assert not (used & set(row)) and all(0 <= b < nb for b in row)
            used |= set(row)
        for rid in rids:
            r = req[rid]
            if prompt_done[rid] == r.prompt and decodes[rid] == r.output - 1:
                finished.add(rid)
                tables.pop(rid)
        live_prev = live
    assert finished == set(req)
    assert all(prompt_done[r] == req[r].prompt for r in req)
    assert all(decodes[r] == req[r].output - 1 for r in req)


@pytest.mark.parametrize("n,clients,budget,bs", [(40, 4, 256, 16), (64, 8, 512, 64), (96, 32, 2048, 64)])
def test_small_traces_keep_invariants(n, clients, budget, bs):
    reqs = sf.trace_requests(n, seed=n, prompt_mean=700, prompt_sd=210, out_mean=12, out_sd=4)
    passes, nb = sf.schedule(reqs, clients=clients, budget=budget, block_size=bs)
    _check(reqs, passes, nb, clients, budget, bs)


def test_full_trace_keeps_invariants_and_plans():
    reqs = sf.trace_requests()
    passes, nb = sf.schedule(reqs)
    assert 665 <= len(passes) <= 1200
    assert sum(p.num_tokens for p in passes) == sum(r.prompt + r.output - 1 for r in reqs)
    _check(reqs, passes, nb, 32, 2048, 64)
    for p in passes[::7]:
        plan = fgb.Plan(p.q_lens, p.ctx_lens, p.block_tables, 32, 32, 128, 64, nb, target_cus=256)
        assert plan.info["num_tokens"] == p.num_tokens


def test_single_token_outputs_and_prompts():
    reqs = [sf.TraceRequest(0, 1, 1), sf.TraceRequest(1, 5000, 1), sf.TraceRequest(2, 3, 4)]
    passes, nb = sf.schedule(reqs, clients=2, budget=1024, block_size=16)
    _check(reqs, passes, nb, 2, 1024, 16)


def test_hash_generator_numpy_matches_torch():
    import torch
    from ragged_paged_attention_splitfuse_amd import workloads as wl
    rids = np.array([3, 3, 9, 41, 41, 41])
    pos = np.array([0, 1, 77, 5, 6, 2999])
    a = np.stack([wl.hash_normal_bf16(7, wl.KIND_K, int(r), [int(q)], range(4), 64)[0]
                  for r, q in zip(rids, pos)])
    t = wl.hash_normal_bf16_torch(7, wl.KIND_K, rids, pos, 4, 64, "cpu")
    assert np.array_equal(a, t.view(torch.int16).numpy().view(np.uint16))


# ---- baseline compositions and user-facing metrics

def _walk(requests, comp):
    """Replay a composition; check prompts whole-or-chunked in order and
    O - 1 decodes after the prompt; return per-pass (tokens, prompt kinds)."""
    req = {r.rid: r for r in requests}
    done, dec = defaultdict(int), defaultdict(int)
    for p in comp:
        for rid, ctx, n, is_dec in p:
            r = req[rid]
            if is_dec:
                assert done[rid] == r.prompt and ctx == r.prompt + dec[rid]
                dec[rid] += 1
            else:
                assert ctx == done[rid] and n >= 1
                done[rid] += n
        assert len({rid for rid, _, _, _ in p}) == len(p)
    assert all(done[r] == req[r].prompt and dec[r] == req[r].output - 1 for r in req)


@pytest.mark.parametrize("policy", ["orca", "prefill_first"])
def test_baseline_policies_run_whole_prompts(policy):
    reqs = sf.trace_requests(80, seed=9, prompt_mean=900, prompt_sd=400, out_mean=10, out_sd=3)
    comp = sf.compose(reqs, clients=8, budget=1024, policy=policy)
    _walk(reqs, comp)
    for p in comp:
        prompts = [(ctx, n) for _, ctx, n, d in p if not d]
        decodes = [1 for *_, d in p if d]
        assert all(ctx == 0 for ctx, _ in prompts)            # never split
        tokens = sum(n for _, n in prompts) + len(decodes)
        if len(prompts) > 1:
            assert tokens <= 1024                              # packing stays in budget
        if policy == "prefill_first":
            assert not (prompts and decodes)                   # prompts pause generation


def test_splitfuse_never_exceeds_budget_but_baselines_may():
    reqs = sf.trace_requests(64, seed=3)
    sizes = {pol: max(sum(n for _, _, n, _ in p) for p in sf.compose(reqs, 32, 2048, pol))
             for pol in sf.POLICIES}
    assert sizes["splitfuse"] == 2048
    assert sizes["orca"] > 2048 and sizes["prefill_first"] > 2048


def test_serving_metrics_on_a_hand_timeline():
    # request 0: prompt 3, 3 outputs; request 1 arrives after 0 finishes (1 client)
    reqs = [sf.TraceRequest(0, 3, 3), sf.TraceRequest(1, 2, 1)]
    arr = {}
    comp = sf.compose(reqs, clients=1, budget=2, policy="splitfuse", arrivals=arr)
    # passes: [0: prompt 0..1], [0: prompt 2], [0 decode], [0 decode], [1: prompt 0..1]
    assert [[(r, c, n, d) for r, c, n, d in p] for p in comp] == [
        [(0, 0, 2, False)], [(0, 2, 1, False)], [(0, 3, 1, True)], [(0, 4, 1, True)], [(1, 0, 2, False)]]
    assert arr == {0: 0, 1: 4}
    m = sf.serving_metrics(reqs, comp, arr, [10, 20, 30, 40, 50])
    # ends: 10, 30, 60, 100, 150.  r0: first token 30, then 60, 100 -> TTFT 30, TPOT 35
    # r1: arrives at 100 (start of pass 4), first (and only) token at 150 -> TTFT 50
    assert m["ttft_us"]["max"] == 50 and m["ttft_us"]["mean"] == 40
    assert m["tpot_us"]["mean"] == 35
    assert sorted([m["token_gap_us"]["max"], m["token_gap_us"]["p50"]]) == [35, 40]
    assert m["latency_us"]["max"] == 100 and m["total_us"] == 150


def test_effective_throughput_counts_requests_within_both_deadlines():
    # the hand timeline above: r0 TTFT 30 (prompt 3 = 2 chunks of budget 2),
    # TPOT 35; r1 TTFT 50 (1 chunk), a single token (no pace to judge)
    reqs = [sf.TraceRequest(0, 3, 3), sf.TraceRequest(1, 2, 1)]
    arr = {}
    comp = sf.compose(reqs, clients=1, budget=2, policy="splitfuse", arrivals=arr)
    pass_us = [10, 20, 30, 40, 50]
    # t_ref 20: r0 needs TTFT <= f1*20*2 and TPOT <= f2*20; r1 TTFT <= f1*20
    cases = [((3.0, 1.5), 1),    # r0: 30 <= 120 but 35 > 30; r1: 50 <= 60
             ((3.0, 2.0), 2),    # r0: 35 <= 40; r1 as before
             ((2.0, 2.0), 1),    # r1: 50 > 40
             ((0.5, 5.0), 0)]    # r0: 30 > 20; r1: 50 > 10
    for (f1, f2), want in cases:
        m = sf.serving_metrics(reqs, comp, arr, pass_us, sla=sf.sla_of(20.0, 2, f1, f2))
        assert m["sla_met"] == want, (f1, f2, m["sla_met"])
        assert m["effective_requests_per_s"] == round(want / 150e-6, 2)
