"""Host Dynamic SplitFuse scheduler and paged-KV block allocator (trace replay).

Composes forward passes from a request trace at a fixed token budget, the
pass-composition strategy of "DeepSpeed-FastGen: High-throughput Text
Generation for LLMs via MII and DeepSpeed-Inference" (research summary,
"Summary" and idea I3): every request that is generating contributes one
decode token, and prompt tokens fill the rest of the budget exactly -- long
prompts are cut into chunks spread over several passes, short ones are packed
together.  Requests come from closed-loop clients, as in the benchmark setup
of the same page ("Key points": 1-32 clients, 512 requests, prompt and output
lengths normal with means 2600 and 60).

Readings where the pages leave the policy open (any composition gives the
same attention results, so none of this is parity-checked):
* decodes first, then prompt chunks FIFO by admission, the in-progress prompt
  first, several prompts fused when room remains;
* a request with output length O needs O - 1 decode passes: its first output
  token comes from the last prompt position;
* 32 closed-loop clients: a client submits its next request in the pass after
  its previous one finished;
* KV blocks come from a seeded, shuffled free list, are allocated on demand
  and returned to the back of the list when a request finishes.

This module only composes passes (lengths, positions, block tables); the
attention itself runs through the C-ABI library.
"""
from dataclasses import dataclass

import numpy as np


@dataclass
class TraceRequest:
    rid: int
    prompt: int
    output: int


def trace_requests(n=512, seed=5, prompt_mean=2600.0, prompt_sd=780.0, out_mean=60.0, out_sd=18.0):
    """Synthetic request trace: lengths clamped >= 1."""
    rng = np.random.Generator(np.random.PCG64(seed))
    p = np.maximum(1, np.rint(rng.normal(prompt_mean, prompt_sd, n))).astype(np.int64)
    o = np.maximum(1, np.rint(rng.normal(out_mean, out_sd, n))).astype(np.int64)
    return [TraceRequest(i, int(p[i]), int(o[i])) for i in range(n)]


@dataclass
class ScheduledPass:
    index: int
    rids: np.ndarray         # int64 [S] request per sequence, decodes first
    q_lens: np.ndarray       # int32 [S]
    ctx_lens: np.ndarray     # int32 [S]
    block_tables: np.ndarray  # int32 [S, width], unused -1
    num_decodes: int

    @property
    def num_tokens(self):
        return int(self.q_lens.sum())


class _Live:
    __slots__ = ("req", "prompt_done", "decodes_done", "blocks", "admitted")

    def __init__(self, req, admitted):
        self.req = req
        self.prompt_done = 0
        self.decodes_done = 0
        self.blocks = []
        self.admitted = admitted


POLICIES = ("splitfuse", "orca", "prefill_first")


def compose(requests, clients=32, budget=2048, policy="splitfuse", arrivals=None):
    """Pass composition only: list of [(rid, ctx, q_len, is_decode), ...].

    policy:
      "splitfuse"      Dynamic SplitFuse: all decodes, then prompt chunks fill
                       the budget exactly (long prompts split over passes).
      "orca"           iteration-level batching without splitting: all decodes
                       plus whole prompts in admission order while they fit
                       the budget; a prompt that fits no pass runs whole anyway.
      "prefill_first"  prefill-prioritising batching: while any live request
                       has prompt left, a pass holds only whole prompts (at
                       least one, as many as fit); decodes wait.
    The two baselines are the compositions the pages contrast with SplitFuse
    (research summary, "Summary": prompts that pause generation, and whole
    prompts run beside generation making some passes very large).
    If `arrivals` is a dict, it receives rid -> index of the first pass the
    request could have joined (its client submitted it just before that pass).
    """
    if policy not in POLICIES:
        raise ValueError(f"unknown policy {policy!r}")
    pending = list(requests)
    live = []
    order = 0
    passes = []
    for _ in range(min(clients, len(pending))):
        req = pending.pop(0)
        live.append(_Live(req, order))
        if arrivals is not None:
            arrivals[req.rid] = 0
        order += 1
    while live:
        decodes = [(lv, lv.req.prompt + lv.decodes_done, 1, True) for lv in live
                   if lv.prompt_done == lv.req.prompt and lv.decodes_done < lv.req.output - 1]
        waiting = [lv for lv in live if lv.prompt_done < lv.req.prompt]   # admission order
        seqs = []
        if policy == "splitfuse":
            seqs = list(decodes)
            left = budget - len(seqs)
            if left < 0:
                raise ValueError("more decodes than the token budget")
            for lv in waiting:
                if left == 0:
                    break
                n = min(lv.req.prompt - lv.prompt_done, left)
                seqs.append((lv, lv.prompt_done, n, False))
                left -= n
        elif policy == "orca":
            seqs = list(decodes)
            used, any_prompt = len(seqs), False
            for lv in waiting:
                n = lv.req.prompt
                if used + n <= budget or not any_prompt:
                    seqs.append((lv, 0, n, False))
                    used += n
                    any_prompt = True
                if used >= budget:
                    break
        else:
            if waiting:
                used = 0
                for lv in waiting:
                    n = lv.req.prompt
                    if used == 0 or used + n <= budget:
                        seqs.append((lv, 0, n, False))
                        used += n
                    if used >= budget:
                        break
            else:
                seqs = list(decodes)
        if not seqs:
            raise RuntimeError("scheduler made no progress")
        passes.append([(lv.req.rid, ctx, n, dec) for lv, ctx, n, dec in seqs])
        finished = []
        for lv, ctx, n, dec in seqs:
            if dec:
                lv.decodes_done += 1
            else:
                lv.prompt_done += n
            if lv.prompt_done == lv.req.prompt and lv.decodes_done == lv.req.output - 1:
                finished.append(lv)
        for lv in finished:
            live.remove(lv)
            if pending:
                req = pending.pop(0)
                live.append(_Live(req, order))
                if arrivals is not None:
                    arrivals[req.rid] = len(passes)
                order += 1
    return passes


def sla_of(t_ref_us, budget, ttft_factor=3.0, tpot_factor=1.5):
    """Attention-level service levels, in units of one full-budget pass.

    The pages judge serving by requests that complete within deadlines on the
    time to first token and on the pace of streamed tokens (research summary,
    idea I4 "effective throughput"; FastGen Guide, the goodput table and its
    per-token deadline), with whole-model values in milliseconds.  Here only
    the attention layer runs, so the deadlines are stated in units of t_ref,
    the device time of one full-budget pass of the same shape: a request
    meets them when its TTFT <= ttft_factor * t_ref * ceil(prompt / budget)
    and its TPOT <= tpot_factor * t_ref."""
    return {"t_ref_us": float(t_ref_us), "budget": int(budget), "ttft_factor": float(ttft_factor),
            "tpot_factor": float(tpot_factor)}


def serving_metrics(requests, comp, arrivals, pass_us, sla=None):
    """User-facing metrics of a composed trace on a measured timeline.

    comp: compose() output; arrivals: its rid -> first-joinable pass index;
    pass_us: duration of each pass in microseconds (passes back to back).
    A request's first output token comes at the end of the pass holding its
    last prompt token, each later token at the end of its decode pass.
    TTFT = first-token time - arrival time; TPOT = mean gap between its output
    tokens (requests with more than one); token gaps pool every such gap for
    the tail; latency = last-token time - arrival time.  Time to first token
    and a steady token pace are the user-facing measures the research summary
    names (idea I4); the pages' absolute SLA figures belong to whole-model
    passes and are not used here.  With `sla` (see sla_of), effective
    throughput counts only the requests that meet both deadlines: requests
    meeting them per second of the whole replay.
    """
    ends = np.cumsum(np.asarray(pass_us, dtype=np.float64))
    prompt_len = {r.rid: r.prompt for r in requests}

    def start(i):
        return ends[i - 1] if i > 0 else 0.0

    first, last, gaps, ntok = {}, {}, [], {}
    for i, p in enumerate(comp):
        for rid, ctx, n, dec in p:
            if dec:
                gaps.append(ends[i] - last[rid])
                last[rid] = ends[i]
                ntok[rid] += 1
            elif rid in prompt_len and ctx + n == prompt_len[rid]:
                first[rid] = last[rid] = ends[i]
                ntok[rid] = 1
    ttft, tpot, lat = [], [], []
    met = 0
    for r in requests:
        a = start(arrivals[r.rid])
        ttft.append(first[r.rid] - a)
        lat.append(last[r.rid] - a)
        pace = None
        if ntok[r.rid] > 1:
            pace = (last[r.rid] - first[r.rid]) / (ntok[r.rid] - 1)
            tpot.append(pace)
        if sla is not None:
            chunks = -(-r.prompt // sla["budget"])
            ok = ttft[-1] <= sla["ttft_factor"] * sla["t_ref_us"] * chunks
            ok = ok and (pace is None or pace <= sla["tpot_factor"] * sla["t_ref_us"])
            met += int(ok)

    def pct(x):
        x = np.asarray(x, dtype=np.float64)
        return {"mean": round(float(x.mean()), 2), "p50": round(float(np.percentile(x, 50)), 2),
                "p90": round(float(np.percentile(x, 90)), 2), "p95": round(float(np.percentile(x, 95)), 2),
                "p99": round(float(np.percentile(x, 99)), 2), "max": round(float(x.max()), 2)}

    total = float(ends[-1]) if len(ends) else 0.0
    out_tokens = sum(r.output for r in requests)
    res = {"ttft_us": pct(ttft), "tpot_us": pct(tpot) if tpot else None, "token_gap_us": pct(gaps) if gaps else None,
           "latency_us": pct(lat), "total_us": round(total, 1),
           "requests_per_s": round(len(requests) / (total * 1e-6), 2) if total else None,
           "output_tokens_per_s": round(out_tokens / (total * 1e-6), 1) if total else None,
           "passes": len(comp)}
    if sla is not None:
        res["sla"] = dict(sla)
        res["sla_met"] = met
        res["effective_requests_per_s"] = round(met / (total * 1e-6), 2) if total else None
    return res


def schedule(requests, clients=32, budget=2048, block_size=64, seed=5, slack=1.25,
             policy="splitfuse", arrivals=None):
    """Compose passes and give every sequence its block table.

    Returns (passes, num_blocks).  The pool holds slack x the peak number of
    blocks live at once; blocks come from a shuffled free list.
    """
    comp = compose(requests, clients, budget, policy, arrivals)
    last = {}
    for i, p in enumerate(comp):
        for rid, _, _, _ in p:
            last[rid] = i
    finals = [[] for _ in comp]
    for rid, i in last.items():
        finals[i].append(rid)
    need, peak = {}, 0
    for i, p in enumerate(comp):
        for rid, ctx, n, _ in p:
            need[rid] = -(-(ctx + n) // block_size)
        peak = max(peak, sum(need.values()))
        for rid in finals[i]:
            del need[rid]
    num_blocks = int(np.ceil(slack * peak))
    rng = np.random.Generator(np.random.PCG64(seed))
    free = [int(b) for b in rng.permutation(num_blocks)]
    head = 0
    tables = {}
    out = []
    for i, p in enumerate(comp):
        rows = []
        for rid, ctx, n, _ in p:
            t = tables.setdefault(rid, [])
            while len(t) * block_size < ctx + n:
                if head >= len(free):
                    raise RuntimeError("KV pool exhausted")
                t.append(free[head])
                head += 1
            rows.append(t)
        width = max(len(r) for r in rows)
        bt = np.full((len(rows), width), -1, dtype=np.int32)
        for s, r in enumerate(rows):
            bt[s, :len(r)] = r
        out.append(ScheduledPass(
            i, np.array([x[0] for x in p], np.int64), np.array([x[2] for x in p], np.int32),
            np.array([x[1] for x in p], np.int32), bt, sum(1 for x in p if x[3])))
        for rid in finals[i]:
            free.extend(tables.pop(rid))
    return out, num_blocks


def composition_of(passes):
    """schedule() output back in compose() form: [(rid, ctx, q_len, is_decode), ...]."""
    return [[(int(p.rids[s]), int(p.ctx_lens[s]), int(p.q_lens[s]), s < p.num_decodes)
             for s in range(len(p.rids))] for p in passes]
