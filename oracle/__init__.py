"""CPU oracle for one ragged paged attention pass -- TEST INFRASTRUCTURE ONLY.

This package is the slow, plain, float64 definition of what a Dynamic SplitFuse
attention pass computes.  It exists to check the HIP path, never to stand in for
it: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import, call or execute anything in here.  The product package
(``ragged_paged_attention_splitfuse_amd``) never imports it, and this package
imports nothing from the product package: the two share no code.

Inputs are bf16 bit patterns (``numpy.uint16``) exactly as the GPU receives
them; every value is decoded exactly to float64 before any arithmetic.

Modules
-------
attention
    bf16 decoding, the KV-append index map, block-table gather, per-sequence
    causal attention with log-sum-exp, the split-KV partial attention and the
    log-sum-exp merge.  Every function is pinned by ``tests/test_oracle.py``
    (closed forms, brute force, a textbook library reduction, invariants).
split_policy
    The split-count policies the pages print (a host heuristic and a figure's
    worked example).  Pinned by the worked example the figure prints and by
    hand-derived cases of the printed heuristic.
"""
