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
