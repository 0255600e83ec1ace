"""Trace replay on the GPU: Dynamic SplitFuse passes from the host scheduler,
every pass through fg_plan_pass -> upload -> fg_kv_append ->
fg_attention_ragged on one pool; every row (all sequences, all heads) of the
kept passes checked against the oracle.
"""
import numpy as np
import pytest
import torch

from ragged_paged_attention_splitfuse_amd import binding as fgb
from ragged_paged_attention_splitfuse_amd import splitfuse as sf
from tests import _gpu as G
from tests.test_gpu_parity import compare, _log

pytestmark = pytest.mark.gpu


def _replay(passes, nb, hq, hkv, d, bs, seed, keep):
    kshape, vshape = fgb.pool_shapes(nb, hkv, bs, d)
    kp = torch.full(kshape, 0x7FC0, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    vp = torch.full(vshape, 0x7FC0, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    kept = {}
    for p in passes[:max(keep) + 1]:
        q, k, v = G.trace_pass_inputs(p, seed, hq, hkv, d)
        plan = fgb.Plan(p.q_lens, p.ctx_lens, p.block_tables, hq, hkv, d, bs, nb)
        meta = plan.upload()
        fgb.kv_append(plan, meta, k, v, kp, vp)
        out = torch.empty((p.num_tokens, hq, d), device="cuda")
        lse = torch.empty((p.num_tokens, hq), device="cuda")
        fgb.attention_ragged(plan, meta, q, kp, vp, out, lse)
        if p.index in keep:
            torch.cuda.synchronize()
            kept[p.index] = (out.cpu(), lse.cpu())
    torch.cuda.synchronize()
    return kept


def _check_pass(p, got, seqs, heads, seed, d, bs, g=1):
    out, lse = got
    heads = list(heads)
    o_ref, l_ref = G.trace_oracle(p, seqs, heads, seed, d, bs)
    cu = np.zeros(len(p.q_lens) + 1, np.int64)
    cu[1:] = np.cumsum(p.q_lens)
    rows = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in seqs])
    o = out[rows][:, heads]
    l_ = lse[rows][:, heads]
    compare(o, l_, o_ref, l_ref, f"trace pass {p.index}: {len(seqs)} seqs x {len(heads)} heads")


@pytest.mark.parametrize("clients", [1, 8])
def test_small_gqa_trace_all_rows(clients):
    reqs = sf.trace_requests(48, seed=11, prompt_mean=600, prompt_sd=180, out_mean=10, out_sd=3)
    passes, nb = sf.schedule(reqs, clients=clients, budget=512, block_size=16, seed=11)
    keep = [3, len(passes) // 2, len(passes) - 2]
    _log(f"[case] small trace clients={clients} passes={len(passes)} nb={nb} keep={keep}")
    got = _replay(passes, nb, 8, 2, 64, 16, 11, keep)
    for i in keep:
        p = passes[i]
        # GQA 8:2 -- the oracle sub-pass is MHA per head, so check every q
        # head against its kv head's regenerated K/V
        out, lse = got[i]
        for qh in range(8):
            o_ref, l_ref = G.trace_oracle_gqa(p, list(range(len(p.q_lens))), qh, qh // 4, 11, 64, 16)
            compare(out[:, [qh]], lse[:, [qh]], o_ref, l_ref, f"small trace pass {i} q head {qh}")


def test_full_trace_kept_passes_every_row():
    reqs = sf.trace_requests()
    passes, nb = sf.schedule(reqs)
    most = max(range(len(passes)), key=lambda i: (len(passes[i].q_lens), i))
    decode_only = next(i for i in range(len(passes)) if passes[i].num_decodes == len(passes[i].q_lens)
                       and passes[i].num_decodes > 8)
    multi_chunk = next(i for i in range(len(passes))
                       if len(passes[i].q_lens) - passes[i].num_decodes >= 2)
    keep = sorted({multi_chunk, most, decode_only, 400})
    _log(f"[case] full trace passes={len(passes)} nb={nb} keep={keep}")
    got = _replay(passes, nb, 32, 32, 128, 64, 5, keep)
    for i in keep:
        p = passes[i]
        _check_pass(p, got[i], list(range(len(p.q_lens))), range(32), 5, 128, 64)


@pytest.mark.parametrize("policy", ["orca", "prefill_first"])
def test_baseline_composition_oversized_passes(policy):
    # the baselines run whole prompts, so some passes exceed the 2048 budget;
    # those passes go through the same library calls and stay on the oracle
    reqs = sf.trace_requests(40, seed=7)
    passes, nb = sf.schedule(reqs, clients=16, budget=2048, block_size=64, seed=7, policy=policy)
    big = max(range(len(passes)), key=lambda i: (passes[i].num_tokens, -i))
    keep = sorted({big, min(len(passes) - 1, big + 3)})
    _log(f"[case] {policy} passes={len(passes)} big={big} tokens={passes[big].num_tokens} keep={keep}")
    assert passes[big].num_tokens > 2048
    got = _replay(passes, nb, 32, 32, 128, 64, 7, keep)
    for i in keep:
        p = passes[i]
        _check_pass(p, got[i], list(range(len(p.q_lens))), range(32), 7, 128, 64)
