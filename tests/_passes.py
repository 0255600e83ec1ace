"""Test helpers: build oracle-side pools and logical K/V arrays from a spec.

The oracle-side pool is filled by the oracle's own append (history first,
then the pass); the logical arrays are the generator's tensors concatenated
per sequence, untouched by any addressing code.
"""
import numpy as np

from oracle import attention as ora
from ragged_paged_attention_splitfuse_amd import workloads as wl


def oracle_pools(spec, tensors, poison=False):
    """Pools after appending the history and then the pass (oracle path)."""
    kp, vp = wl.empty_pool_bits(spec, poison=poison)
    hist = spec.history_pass()
    if hist is not None:
        hq, hc, ht, _ = hist
        kp, vp = ora.kv_append(kp, vp, hq, hc, ht, spec.block_size, tensors.hist_k, tensors.hist_v)
    kp, vp = ora.kv_append(kp, vp, spec.q_lens, spec.ctx_lens, spec.block_tables,
                           spec.block_size, tensors.k_new, tensors.v_new)
    return kp, vp


def logical_kv(spec, tensors):
    """Per-sequence K, V bits in position order: [ctx history ; new tokens]."""
    out = []
    h0 = 0
    t0 = 0
    for s in range(spec.num_seqs):
        c, n = int(spec.ctx_lens[s]), int(spec.q_lens[s])
        k = np.concatenate([tensors.hist_k[h0:h0 + c], tensors.k_new[t0:t0 + n]])
        v = np.concatenate([tensors.hist_v[h0:h0 + c], tensors.v_new[t0:t0 + n]])
        out.append((k, v))
        h0 += c
        t0 += n
    return out


def cu_seqlens(q_lens):
    cu = np.zeros(len(q_lens) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(q_lens)
    return cu
