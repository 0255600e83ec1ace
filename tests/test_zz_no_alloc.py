"""fg_attention_ragged_noalloc against fg_attention_ragged, through the C ABI.

The no-allocation entry point runs the same kernels with the library's scratch
array as the workspace, so its results must equal the workspace entry point's
bit for bit.  Two calls in a row, the second on a smaller pass, both with split
KV ranges (partial rows in the scratch, merged inside the attention launch and
by the merge launch).
"""
import numpy as np
import pytest
import torch

from ragged_paged_attention_splitfuse_amd import binding as fgb
from ragged_paged_attention_splitfuse_amd import workloads as wl
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


CASES = [
    # (spec, knobs): the first is larger; both split, so the scratch is used
    (lambda: wl.custom_spec("na1", [1, 300, 1, 2, 77, 1], [2500, 131, 0, 64, 1000, 63], 8, 2, 128, 64,
                            seed=61), {"force_splits": 3, "target_cus": 16}),
    (lambda: wl.custom_spec("na2", [1, 40, 1], [700, 90, 33], 4, 4, 64, 16, seed=62),
     {"force_splits": 2, "target_cus": 16}),
]


def test_noalloc_matches_workspace_entry_point_on_two_calls():
    scratch = fgb.fg_noalloc_scratch_bytes()
    sizes = []
    for i, (make, knobs) in enumerate(CASES):
        spec = make()
        _log(f"[case] noalloc call {i}: S={spec.num_seqs} T={spec.num_tokens} {knobs}")
        tens = wl.make_tensors(spec)
        kp, vp = G.gpu_pools(spec, poison=True)
        G.fill_history(spec, tens, kp, vp)
        plan = fgb.Plan.from_spec(spec, **knobs)
        ws_bytes = plan.info["workspace_bytes"]
        assert 0 < ws_bytes <= scratch
        assert plan.info["num_merge_groups"] > 0
        sizes.append(ws_bytes)
        q, kn, vn = G.to_dev(tens.q), G.to_dev(tens.k_new), G.to_dev(tens.v_new)
        meta = fgb.upload_append(plan, None, kn, vn, kp, vp)
        t, hq, d = spec.num_tokens, spec.num_q_heads, spec.head_dim
        out_a = torch.full((t, hq, d), float("nan"), device="cuda")
        lse_a = torch.full((t, hq), float("nan"), device="cuda")
        fgb.attention_ragged(plan, meta, q, kp, vp, out_a, lse_a)
        out_b = torch.full((t, hq, d), float("nan"), device="cuda")
        lse_b = torch.full((t, hq), float("nan"), device="cuda")
        fgb.attention_ragged_noalloc(plan, meta, q, kp, vp, out_b, lse_b)
        torch.cuda.synchronize()
        assert torch.isfinite(out_b).all()
        assert torch.equal(out_a, out_b) and torch.equal(lse_a, lse_b)
        o_ref, l_ref = G.oracle_pass(spec, tens)
        eo = float(np.max(np.abs(out_b.cpu().numpy() - o_ref)))
        el = float(np.max(np.abs(lse_b.cpu().numpy() - l_ref)))
        _log(f"[parity] noalloc call {i}: max|dO|={eo:.3e} max|dLSE|={el:.3e} ws={ws_bytes}")
        assert eo <= 1e-2 and el <= 1e-3
        plan.close()
    assert sizes[1] < sizes[0]
