"""Split-count policies that the pages describe (test infrastructure).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may use
this module.  These policies decide only how many KV splits each sequence
gets; attention results do not depend on them (any partition merges to the
same output), so they matter for speed alone.

Two policies are printed on "DeepSpeed-FastGen Guide: Dynamic SplitKV
Serving" and they disagree with each other:

* ``host_heuristic`` restates the allocation engine of section "Step 2:
  Dynamic SplitKV Allocation Engine": no split at or below a minimum chunk,
  otherwise one split per minimum chunk capped at 16, then every count is
  scaled up by (SM count / total) when the total falls short of the SM count,
  and everything collapses to one split when there are at least as many
  sequences as SMs.  Note that the scaling step can push a count past its own
  cap of 16.
* ``figure_rule`` reproduces the worked example of the figure "Dynamic
  SplitKV Two-Phase Attention Kernel Workflow" (512, 4096 and 16384 tokens get
  1, 4 and 16 splits).  The figure prints only the outcome; the reading taken
  here is one split per 1024 tokens, at least 1 and at most 16, with no SM
  scaling -- the plainest rule that gives the printed numbers.
"""

__all__ = ["host_heuristic", "figure_rule"]


def host_heuristic(seq_lengths, num_sms=108, min_chunk_size=256):
    """Split counts per sequence under the Step 2 allocation engine."""
    n = len(seq_lengths)
    if n == 0:
        return []
    if n >= num_sms:
        return [1] * n
    counts = []
    for length in seq_lengths:
        if length <= min_chunk_size:
            counts.append(1)
        else:
            counts.append(min(max(1, length // min_chunk_size), 16))
    total = sum(counts)
    if total < num_sms:
        factor = num_sms / total
        counts = [max(1, int(c * factor)) for c in counts]
    return counts


def figure_rule(seq_lengths, tokens_per_split=1024, cap=16):
    """Split counts per sequence under the workflow figure's worked example."""
    return [min(max(1, length // tokens_per_split), cap) for length in seq_lengths]
