"""Seeded random pass compositions for planner and parity tests: a mix of
decodes and prompt chunks with random contexts, head layouts, head dims, block
sizes and split settings.  Inputs only; no attention arithmetic."""
import numpy as np

from ragged_paged_attention_splitfuse_amd import workloads as wl

HEAD_LAYOUTS = ((4, 4), (8, 2), (6, 2), (8, 1), (16, 2), (12, 4))


def random_pass(seed):
    """(spec, knobs) of one random pass; the same seed gives the same pass."""
    rng = np.random.default_rng(10_000 + seed)
    s = int(rng.integers(1, 9))
    q_lens, ctx_lens = [], []
    for _ in range(s):
        decode = rng.random() < 0.5
        q_lens.append(1 if decode else int(rng.integers(2, 201)))
        ctx_lens.append(0 if rng.random() < 0.15 else int(rng.integers(1, 1501)))
    hq, hkv = HEAD_LAYOUTS[int(rng.integers(len(HEAD_LAYOUTS)))]
    d = int(rng.choice([64, 128]))
    b = int(rng.choice([16, 32, 64]))
    knobs = {"force_splits": int(rng.choice([0, 0, 2, 5]))}
    spec = wl.custom_spec(f"r{seed}", q_lens, ctx_lens, hq, hkv, d, b, seed=100 + seed)
    return spec, knobs


BIG_LAYOUTS = ((8, 8), (16, 2), (8, 1), (32, 8), (12, 4), (16, 16))


def random_big_pass(seed, work_cap=6e9):
    """(spec, knobs) of a larger random pass: up to 32 sequences, contexts up to
    12,000 tokens and chunks up to 700 rows (halved until sum q*(c+q)*Hq*D is
    under work_cap, so the float64 oracle stays within seconds)."""
    rng = np.random.default_rng(77_000 + seed)
    hq, hkv = BIG_LAYOUTS[int(rng.integers(len(BIG_LAYOUTS)))]
    d = int(rng.choice([64, 128]))
    b = int(rng.choice([16, 32, 64]))
    s = int(rng.integers(1, 33))
    q = [1 if rng.random() < 0.6 else int(rng.integers(2, 700)) for _ in range(s)]
    c = [0 if rng.random() < 0.1 else int(rng.integers(1, 12001)) for _ in range(s)]
    while sum(qi * (ci + qi) for qi, ci in zip(q, c)) * hq * d > work_cap and max(q) > 1:
        i = int(np.argmax(q))
        q[i] = max(1, q[i] // 2)
    knobs = {"force_splits": int(rng.choice([0, 0, 0, 2, 7]))}
    spec = wl.custom_spec(f"big{seed}", q, c, hq, hkv, d, b, seed=500 + seed)
    return spec, knobs
