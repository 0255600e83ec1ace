"""GPU-side helpers for the parity tests: device pools, history fill, one pass.

Everything here goes through the C-ABI binding; the oracle side is built in
tests/_passes.py from the same generator tensors.
"""
import numpy as np
import torch

from oracle import attention as ora
from ragged_paged_attention_splitfuse_amd import binding as fgb
from ragged_paged_attention_splitfuse_amd import workloads as wl
from tests._passes import oracle_pools

PLAN_CUS = 256


def to_dev(bits):
    """uint16 bf16 bits (numpy) -> contiguous bf16 device tensor, same bits."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(torch.bfloat16)


def to_host_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def gpu_pools(spec, poison=True):
    kshape, vshape = fgb.pool_shapes(spec.num_blocks, spec.num_kv_heads, spec.block_size, spec.head_dim)
    fill = wl.BF16_NAN if poison else 0
    kp = torch.full(kshape, fill, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    vp = torch.full(vshape, fill, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    return kp, vp


def fill_history(spec, tens, kp, vp):
    """Append each sequence's cached tokens through fg_kv_append."""
    hist = spec.history_pass()
    if hist is None:
        return
    q, c, bt, _ = hist
    plan = fgb.Plan(q, c, bt, spec.num_q_heads, spec.num_kv_heads, spec.head_dim,
                    spec.block_size, spec.num_blocks, target_cus=PLAN_CUS)
    meta = plan.upload()
    fgb.kv_append(plan, meta, to_dev(tens.hist_k), to_dev(tens.hist_v), kp, vp)
    torch.cuda.synchronize()
    plan.close()


MODES = ("separate", "pass", "direct")


def run_pass(spec, tens, kp, vp, out_dtype=torch.float32, dev_inputs=None, mode="separate", **knobs):
    """Plan and run one pass; returns (out, lse, plan).

    mode "separate": fg_plan_upload, fg_kv_append, fg_attention_ragged;
    "pass": fg_pass (upload, append and attention, the append inside the
    attention launch); "direct": fg_plan_upload and fg_attention_ragged_direct
    only -- the pools keep whatever the new positions held (poison in the
    tests), since that call reads the pass's own K/V from k_new / v_new."""
    knobs.setdefault("target_cus", 0)
    plan = fgb.Plan.from_spec(spec, **knobs)
    if dev_inputs is None:
        dev_inputs = (to_dev(tens.q), to_dev(tens.k_new), to_dev(tens.v_new))
    q, kn, vn = dev_inputs
    t, hq, d = spec.num_tokens, spec.num_q_heads, spec.head_dim
    out = torch.full((t, hq, d), float("nan"), dtype=out_dtype, device="cuda")
    lse = torch.full((t, hq), float("nan"), dtype=torch.float32, device="cuda")
    if mode == "pass":
        fgb.run_pass(plan, None, q, kn, vn, kp, vp, out, lse)
    elif mode == "direct":
        meta = plan.upload()
        fgb.attention_ragged_direct(plan, meta, q, kn, vn, kp, vp, out, lse)
    else:
        meta = plan.upload()
        fgb.kv_append(plan, meta, kn, vn, kp, vp)
        fgb.attention_ragged(plan, meta, q, kp, vp, out, lse)
    torch.cuda.synchronize()
    return out, lse, plan


def full_gpu_pass(spec, tens=None, poison=True, out_dtype=torch.float32, mode="separate", **knobs):
    if tens is None:
        tens = wl.make_tensors(spec)
    kp, vp = gpu_pools(spec, poison)
    fill_history(spec, tens, kp, vp)
    out, lse, plan = run_pass(spec, tens, kp, vp, out_dtype=out_dtype, mode=mode, **knobs)
    return tens, kp, vp, out, lse, plan


def subset(spec, tens, seqs):
    """The pass restricted to `seqs`, physical blocks relabelled 0..k-1.

    Attention of a sequence depends only on its own rows and blocks, and the
    oracle's results are bit-invariant under block relabelling, so this is the
    oracle input for sampled checks of a large pass.  Returns (sub_spec,
    sub_tensors, row_index) where row_index maps the sub-pass rows back to
    rows of the full pass.
    """
    seqs = list(seqs)
    cu = np.zeros(spec.num_seqs + 1, np.int64)
    cu[1:] = np.cumsum(spec.q_lens)
    hcu = np.zeros(spec.num_seqs + 1, np.int64)
    hcu[1:] = np.cumsum(spec.ctx_lens)
    q_lens, ctx_lens = spec.q_lens[seqs], spec.ctx_lens[seqs]
    need = [-(-int(q + c) // spec.block_size) for q, c in zip(q_lens, ctx_lens)]
    tables = np.full((len(seqs), max(need)), -1, np.int32)
    nxt = 0
    for i, k in enumerate(need):
        tables[i, :k] = np.arange(nxt, nxt + k)
        nxt += k
    sub = wl.PassSpec(spec.name + "-sub", spec.num_q_heads, spec.num_kv_heads, spec.head_dim,
                      spec.block_size, nxt, q_lens.copy(), ctx_lens.copy(), tables, spec.seed, spec.scale)
    rows = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in seqs])
    hrows = np.concatenate([np.arange(hcu[s], hcu[s + 1]) for s in seqs])
    st = wl.PassTensors(q=tens.q[rows], k_new=tens.k_new[rows], v_new=tens.v_new[rows],
                        hist_k=tens.hist_k[hrows], hist_v=tens.hist_v[hrows])
    return sub, st, rows


def band_subpass(spec, tens, s, j0, j1):
    """Rows j0..j1-1 of sequence s as a pass of their own: a chunk of j1 - j0
    tokens at context ctx_s + j0, whose history is the sequence's logical K/V
    before it.  Causal attention of a row depends only on its position and the
    keys before it, so the sub-pass's rows equal those rows of the full pass.
    Returns (sub_spec, sub_tensors, row_index into the full pass)."""
    from tests._passes import logical_kv
    c = int(spec.ctx_lens[s])
    k_all, v_all = logical_kv(spec, tens)[s]
    cu = np.zeros(spec.num_seqs + 1, np.int64)
    cu[1:] = np.cumsum(spec.q_lens)
    sub = wl.custom_spec(spec.name + "-band", [j1 - j0], [c + j0], spec.num_q_heads,
                         spec.num_kv_heads, spec.head_dim, spec.block_size, seed=1, slack=1.0)
    st = wl.PassTensors(q=tens.q[cu[s] + j0:cu[s] + j1], k_new=k_all[c + j0:c + j1],
                        v_new=v_all[c + j0:c + j1], hist_k=k_all[:c + j0], hist_v=v_all[:c + j0])
    return sub, st, np.arange(cu[s] + j0, cu[s] + j1)


def oracle_pass(spec, tens):
    kp, vp = oracle_pools(spec, tens, poison=True)
    return ora.attend(tens.q, kp, vp, spec.q_lens, spec.ctx_lens, spec.block_tables,
                      spec.block_size, spec.num_kv_heads, scale=spec.scale or None)


def trace_pass_inputs(p, seed, hq, hkv, d, device="cuda"):
    """Q, new K, new V of one scheduled pass from the keyed hash generator."""
    rid_rows = np.repeat(p.rids, p.q_lens)
    pos_rows = np.concatenate([np.arange(c, c + n) for c, n in zip(p.ctx_lens, p.q_lens)])
    q = wl.hash_normal_bf16_torch(seed, wl.KIND_Q, rid_rows, pos_rows, hq, d, device)
    k = wl.hash_normal_bf16_torch(seed, wl.KIND_K, rid_rows, pos_rows, hkv, d, device)
    v = wl.hash_normal_bf16_torch(seed, wl.KIND_V, rid_rows, pos_rows, hkv, d, device)
    return q.contiguous(), k.contiguous(), v.contiguous()


def _trace_seq_bits(p, seqs, seed, num_heads, head_dim):
    """Q (this pass's rows) and whole-history K, V bits of sequences `seqs` of
    a scheduled pass, heads 0..num_heads-1, from the keyed generator on the
    CPU (torch's vectorised version; same bits as the numpy one)."""
    ctx = p.ctx_lens[seqs].astype(np.int64)
    n = p.q_lens[seqs].astype(np.int64)
    rids = p.rids[seqs].astype(np.int64)
    q_pos = np.concatenate([np.arange(c, c + m) for c, m in zip(ctx, n)])
    kv_pos = np.concatenate([np.arange(0, c + m) for c, m in zip(ctx, n)])
    def gen(kind, rid_rows, pos):
        # 64-token slices keep the int64 temporaries cache-resident
        out = np.empty((len(pos), num_heads, head_dim), np.uint16)
        for a in range(0, len(pos), 64):
            t = wl.hash_normal_bf16_torch(seed, kind, rid_rows[a:a + 64], pos[a:a + 64], num_heads,
                                          head_dim, "cpu")
            out[a:a + 64] = t.view(torch.int16).numpy().view(np.uint16)
        return out

    q = gen(wl.KIND_Q, np.repeat(rids, n), q_pos)
    k = gen(wl.KIND_K, np.repeat(rids, ctx + n), kv_pos)
    v = gen(wl.KIND_V, np.repeat(rids, ctx + n), kv_pos)
    return q, k, v


def trace_oracle(p, seqs, heads, seed, head_dim, block_size):
    """Oracle rows for sequences `seqs` of a scheduled pass, on q/kv heads `heads`.

    Each sequence's whole history is regenerated from the keyed generator (it
    does not depend on which pass wrote it), so no GPU data enters the oracle.
    The sub-pass is MHA over the chosen heads with compact block ids.
    """
    hs = list(heads)
    seqs = list(seqs)
    q_lens = p.q_lens[seqs].astype(np.int32)
    ctx = p.ctx_lens[seqs].astype(np.int32)
    qa, ka, va = _trace_seq_bits(p, seqs, seed, max(hs) + 1, head_dim)
    qa, ka, va = qa[:, hs], ka[:, hs], va[:, hs]
    hk, kn, hv, vn = [], [], [], []
    o = 0
    for c, n in zip(ctx, q_lens):
        hk.append(ka[o:o + c]); kn.append(ka[o + c:o + c + n])
        hv.append(va[o:o + c]); vn.append(va[o + c:o + c + n])
        o += c + n
    spec = wl.custom_spec("trace-sub", q_lens, ctx, len(hs), len(hs), head_dim, block_size,
                          seed=1, slack=1.0)
    tens = wl.PassTensors(q=np.ascontiguousarray(qa), k_new=np.concatenate(kn), v_new=np.concatenate(vn),
                          hist_k=np.concatenate(hk), hist_v=np.concatenate(hv))
    return oracle_pass(spec, tens)


def trace_oracle_gqa(p, seqs, q_head, kv_head, seed, head_dim, block_size):
    """Oracle rows of one q head (which reads kv_head) for sequences `seqs`."""
    q_lens = p.q_lens[seqs].astype(np.int32)
    ctx = p.ctx_lens[seqs].astype(np.int32)
    qs, kn, vn, hk, hv = [], [], [], [], []
    for s in seqs:
        rid, c, n = int(p.rids[s]), int(p.ctx_lens[s]), int(p.q_lens[s])
        qs.append(wl.hash_normal_bf16(seed, wl.KIND_Q, rid, np.arange(c, c + n), [q_head], head_dim))
        k = wl.hash_normal_bf16(seed, wl.KIND_K, rid, np.arange(0, c + n), [kv_head], head_dim)
        v = wl.hash_normal_bf16(seed, wl.KIND_V, rid, np.arange(0, c + n), [kv_head], head_dim)
        hk.append(k[:c]); kn.append(k[c:]); hv.append(v[:c]); vn.append(v[c:])
    spec = wl.custom_spec("trace-sub", q_lens, ctx, 1, 1, head_dim, block_size, seed=1, slack=1.0)
    tens = wl.PassTensors(q=np.concatenate(qs), k_new=np.concatenate(kn), v_new=np.concatenate(vn),
                          hist_k=np.concatenate(hk), hist_v=np.concatenate(hv))
    return oracle_pass(spec, tens)
