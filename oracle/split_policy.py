"""Split-count policies that the pages describe (test infrastructure).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may use
this module.  These policies decide only how many KV splits each sequence
gets; attention results do not depend on them (any partition merges to the
same output), so they matter for speed alone.

Both are stated as per-sequence formulas over the context lengths L_s of the
S sequences of a pass, and implemented as such (whole-array arithmetic, exact
integer floors).  They come from "DeepSpeed-FastGen Guide: Dynamic SplitKV
Serving", and they disagree with each other:

* ``engine_counts``: the allocation engine of section "Step 2: Dynamic
  SplitKV Allocation Engine", with N compute units and a minimum chunk of m
  tokens.  Every sequence gets one split when S >= N.  Otherwise a base count
  b_s = min(16, max(1, floor(L_s / m))) is scaled up so that the counts come
  to about N: with B = sum_s b_s, k_s = max(1, floor(b_s * N / B)) when
  B < N, else k_s = b_s.  The scaled count can exceed the base cap of 16.
  The page's code multiplies by N / B in floating point, which can land one
  below an exact integer (11 * (15 / 11) gives 14.999...); the formula is
  read with exact arithmetic.
* ``figure_counts``: the worked example of the figure "Dynamic SplitKV
  Two-Phase Attention Kernel Workflow" (512, 4096 and 16384 tokens get 1, 4
  and 16 splits).  The figure prints only the outcome; the reading taken here
  is k_s = min(16, max(1, floor(L_s / 1024))), the plainest rule that gives
  the printed numbers, with no compute-unit scaling.
"""
import numpy as np

__all__ = ["engine_counts", "figure_counts"]


def engine_counts(seq_lengths, num_sms=108, min_chunk_size=256):
    """Split counts per sequence under the Step 2 allocation engine."""
    lengths = np.asarray(seq_lengths, dtype=np.int64)
    if lengths.size >= num_sms:
        return [1] * int(lengths.size)
    base = np.clip(lengths // min_chunk_size, 1, 16)
    total = int(base.sum())
    counts = np.maximum(1, (base * num_sms) // total) if 0 < total < num_sms else base
    return [int(k) for k in counts]


def figure_counts(seq_lengths, tokens_per_split=1024, cap=16):
    """Split counts per sequence under the workflow figure's worked example."""
    lengths = np.asarray(seq_lengths, dtype=np.int64)
    return [int(k) for k in np.clip(lengths // tokens_per_split, 1, cap)]
