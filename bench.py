"""Benchmark one Dynamic SplitFuse attention pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]

A step is the whole hot path over one synthetic pass: host plan
(fg_plan_pass) -> metadata upload -> fg_kv_append -> fg_attention_ragged
(split-KV attention + log-sum-exp merge).  Inputs (Q, new K/V, the K/V
history in the paged pools) are resident in HBM before timing starts.

Default workload: the Llama-2-7B attention shape (32 q/kv heads, head_dim
128, bf16, KV block 64), one 2048-token pass of 16 decodes plus one
2032-token final prompt chunk.  Prints ONE JSON line.
"""
import argparse
import gc
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs per SplitFuse attention pass + KV GB/s & MFMA TFLOP/s as % of peak, 7B shape"
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
# Sources that decide what the attention kernel reads and writes: the kernels
# themselves and the planner that cuts the work items.
KERNEL_SOURCES = [os.path.join(ROOT, "ragged_paged_attention_splitfuse_amd", "csrc", f)
                  for f in ("fg_device.hip", "plan.cpp", "plan.h", "fg_meta.h")]


def algorithmic(spec, out_bytes=4):
    """Bytes and flops the method itself must move / compute for one pass."""
    q = spec.q_lens.astype(np.int64)
    c = spec.ctx_lens.astype(np.int64)
    kv_tokens = int(np.sum(q + c))
    hq, hkv, d, t = spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.num_tokens
    kv_bytes = kv_tokens * hkv * d * 2 * 2
    attn_bytes = kv_bytes + t * hq * d * 2 + t * hq * d * out_bytes + t * hq * 4
    append_bytes = 2 * t * hkv * d * 2 * 2
    pairs = int(np.sum(q * c + q * (q + 1) // 2))
    flops = 4 * d * hq * pairs
    return {"kv_tokens": kv_tokens, "kv_bytes": kv_bytes, "attn_bytes": attn_bytes,
            "append_bytes": append_bytes, "pairs_per_head": pairs, "flops": flops}


def source_hash():
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def achievable_peaks(torch, fgb, dev, stream, copy_mib=1024, read_mib=2048, gemm_n=8192, iters=10):
    """Achievable rates measured in the same run: a device-to-device copy (HBM
    read + write), the library's read-stream probe over 2 GiB (eight times the
    MALL; attention traffic is almost all reads), a bf16 GEMM through the vendor
    BLAS and the library's matrix-core loop (with the shader clock it ran at).
    `hbm_gbs` is the larger of the two HBM rates."""
    def timed(fn):
        for _ in range(2):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(iters):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / iters
    n = copy_mib << 20
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    t_copy = timed(lambda: dst.copy_(src))
    del src, dst
    nr = read_mib << 20
    buf = torch.ones(nr, dtype=torch.uint8, device=dev)
    sink = torch.empty(1 << 20, dtype=torch.uint8, device=dev)
    t_read = timed(lambda: fgb.fg_probe_read_stream(buf, sink, stream))
    del buf, sink
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    a = torch.randn((gemm_n, gemm_n), dtype=torch.bfloat16, device=dev, generator=g)
    b = torch.randn((gemm_n, gemm_n), dtype=torch.bfloat16, device=dev, generator=g)
    t_gemm = timed(lambda: torch.mm(a, b))
    del a, b
    # the library's matrix-core loop: two work-groups per CU, 32 bf16 MFMAs per
    # wavefront per round; its per-work-group counters give the shader clock
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    loop_iters = 1024
    lsink = torch.empty(cus * 2 * 256, dtype=torch.float32, device=dev)
    lclk = torch.zeros(cus * 2 * 2, dtype=torch.int64, device=dev)
    t_loop = timed(lambda: fgb.fg_probe_mfma_loop(loop_iters, lsink, lclk, stream))
    clk = lclk.view(-1, 2).cpu().numpy().astype(np.float64)
    loop_flops = cus * 2 * 4 * loop_iters * 32 * 32 * 32 * 16 * 2
    del lsink, lclk
    copy_gbs = round(2 * n / t_copy / 1e9, 1)
    read_gbs = round(nr / t_read / 1e9, 1)
    return {"copy_gbs": copy_gbs, "read_gbs": read_gbs, "hbm_gbs": max(copy_gbs, read_gbs),
            "copy_bytes": n, "read_bytes": nr,
            "bf16_gemm_tflops": round(2 * gemm_n ** 3 / t_gemm / 1e12, 1),
            "gemm_shape": [gemm_n, gemm_n, gemm_n],
            "bf16_mfma_loop_tflops": round(loop_flops / t_loop / 1e12, 1),
            "mfma_loop_clock_ghz": round(float(np.median(clk[:, 0] / (clk[:, 1] / 100e6))) / 1e9, 3)}


def _pmc_per_dispatch(run_dir, counter):
    """{kernel name: [value per dispatch]} from one rocprofv3 --pmc csv run."""
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    per = {}
    for path in files:
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                key = (r["Kernel_Name"], path, int(r["Dispatch_Id"]))
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])   # sum over dimensions
    out = {}
    for (name, _, _), v in per.items():
        out.setdefault(name, []).append(v)
    return out


def write_traffic(workload, fetch_dir, write_dir, probe_mib):
    """Turn two rocprofv3 --pmc runs of this script (FETCH_SIZE, then WRITE_SIZE,
    both with --copy-probe-mib) into profiles/traffic_<workload>.json.

    Each counter is read in KiB per dispatch and scaled by what it reads for the
    plain device-to-device copy of probe_mib MiB in the same run (that copy
    reads and writes exactly probe_mib MiB)."""
    probe = probe_mib << 20
    flag = "" if workload == "7b_pass2048" else f" --workload {workload}"
    rec = {"workload": workload, "kernel_source_sha256_16": source_hash(),
           "copy_probe_bytes": probe,
           "commands": [f"rocprofv3 --pmc {c} -d {d} -o pmc --output-format csv -- python bench.py "
                        f"--no-cpu --no-achievable{flag} --steps 5 --warmup 1 --cold-iters 0 "
                        f"--copy-probe-mib {probe_mib}"
                        for c, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir))] +
                       [f"python bench.py{flag} --traffic-from {fetch_dir} {write_dir} "
                        f"--copy-probe-mib {probe_mib}"]}
    total = 0.0
    for counter, run_dir in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        vals = _pmc_per_dispatch(run_dir, counter)
        copies = [v for n, vs in vals.items() if "copyBuffer" in n or "copy_kernel" in n for v in vs]
        attn = [v for n, vs in vals.items() if "attn_kernel" in n for v in vs]
        if not copies or not attn:
            raise SystemExit(f"{counter}: copy probe or attn_kernel dispatches missing in {run_dir}")
        factor = max(copies) * 1024.0 / probe
        per_launch = sum(attn) / len(attn) * 1024.0 / factor
        key = "fetch" if counter == "FETCH_SIZE" else "write"
        rec[f"{key}_counter_factor"] = round(factor, 4)
        rec[f"{key}_kib_per_launch_raw"] = round(sum(attn) / len(attn), 1)
        rec[f"attn_{key}_bytes_per_launch"] = int(per_launch)
        rec[f"{key}_dispatches"] = len(attn)
        total += per_launch
    rec["attn_hbm_bytes_per_launch"] = int(total)
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


def load_traffic(workload):
    """HBM traffic per attention launch from committed rocprofv3 counters.

    profiles/traffic_<workload>.json holds FETCH/WRITE KiB per dispatch, the
    copy-kernel calibration factor and the kernel-source hash they were taken
    at; a different hash (the kernel changed since) gives null.
    """
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256_16") != source_hash():
        return None
    return rec.get("attn_hbm_bytes_per_launch")


def cpu_baseline(spec, tens, budget_s=30.0, min_s=10.0, single_thread=False):
    """The float64 oracle as it stands, timed on this host (append + attention).
    With single_thread, BLAS is limited to one thread (and the result says so)."""
    from threadpoolctl import threadpool_info, threadpool_limits
    if single_thread:
        with threadpool_limits(limits=1, user_api="blas"):
            res = cpu_baseline(spec, tens, budget_s, min_s)
        res["cores"] = 1
        res["sample"] += "; BLAS limited to one thread"
        return res

    from oracle import attention as ora
    from ragged_paged_attention_splitfuse_amd import workloads as wl

    kp, vp = wl.empty_pool_bits(spec)
    hist = spec.history_pass()
    if hist is not None:
        kp, vp = ora.kv_append(kp, vp, hist[0], hist[1], hist[2], spec.block_size,
                               tens.hist_k, tens.hist_v)
    kp2, vp2 = ora.kv_append(kp, vp, spec.q_lens, spec.ctx_lens, spec.block_tables,
                             spec.block_size, tens.k_new, tens.v_new)
    # attention: whole pass when it fits the budget, else a head sample scaled up
    heads = list(range(spec.num_q_heads))
    t0 = time.perf_counter()
    ora.attend(tens.q, kp2, vp2, spec.q_lens, spec.ctx_lens, spec.block_tables,
               spec.block_size, spec.num_kv_heads, heads=heads[:1])
    t_one = time.perf_counter() - t0
    n_heads = max(1, min(len(heads), int(budget_s / max(t_one, 1e-6))))
    # repeat the (append + sampled attention) until about min_s of CPU work
    reps, t_app_sum, t_att_sum, t_start = 0, 0.0, 0.0, time.perf_counter()
    while True:
        t0 = time.perf_counter()
        ora.kv_append(kp, vp, spec.q_lens, spec.ctx_lens, spec.block_tables,
                      spec.block_size, tens.k_new, tens.v_new)
        t1 = time.perf_counter()
        ora.attend(tens.q, kp2, vp2, spec.q_lens, spec.ctx_lens, spec.block_tables,
                   spec.block_size, spec.num_kv_heads, heads=heads[:n_heads])
        t2 = time.perf_counter()
        t_app_sum += t1 - t0
        t_att_sum += t2 - t1
        reps += 1
        if t2 - t_start >= min_s or reps >= 100000:
            break
    t_app = t_app_sum / reps
    t_att = t_att_sum / reps * len(heads) / n_heads
    blas = [i["num_threads"] for i in threadpool_info() if i.get("user_api") == "blas"]
    sample = (f"{reps} repetitions ({t_app_sum + t_att_sum:.1f} s) of one full pass: append of all "
              f"{spec.num_tokens} new tokens + attention of "
              f"{'all' if n_heads == len(heads) else n_heads} of {len(heads)} q heads"
              + ("" if n_heads == len(heads) else " (time scaled by heads)") + "; mean per pass")
    return {"value": round((t_app + t_att) * 1e6, 1), "unit": "µs",
            "cores": int(max(blas) if blas else 1), "kind": "oracle", "sample": sample,
            "host_cpus": len(os.sched_getaffinity(0))}


def trace_cpu_baseline(passes, hq, hkv, d, bs, seed, wl, n_sample=8):
    """The float64 oracle on a seeded sample of the trace's passes (append +
    attention of each sampled pass, its sequences' histories regenerated from
    the keyed generator and appended untimed).  Returns the mean per pass."""
    from threadpoolctl import threadpool_info

    from oracle import attention as ora
    rng = np.random.Generator(np.random.PCG64(seed + 1000))
    picks = sorted(int(i) for i in rng.choice(len(passes), size=min(n_sample, len(passes)),
                                               replace=False))
    qh, kh = list(range(hq)), list(range(hkv))
    times = []
    for i in picks:
        p = passes[i]
        spec = wl.custom_spec("trace-cpu", p.q_lens, p.ctx_lens, hq, hkv, d, bs, seed=1, slack=1.0)
        qs, kn, vn, hk, hv = [], [], [], [], []
        for s in range(len(p.q_lens)):
            rid, c, n = int(p.rids[s]), int(p.ctx_lens[s]), int(p.q_lens[s])
            qs.append(wl.hash_normal_bf16(seed, wl.KIND_Q, rid, np.arange(c, c + n), qh, d))
            k = wl.hash_normal_bf16(seed, wl.KIND_K, rid, np.arange(0, c + n), kh, d)
            v = wl.hash_normal_bf16(seed, wl.KIND_V, rid, np.arange(0, c + n), kh, d)
            hk.append(k[:c]); kn.append(k[c:]); hv.append(v[:c]); vn.append(v[c:])
        kp, vp = wl.empty_pool_bits(spec)
        hist = spec.history_pass()
        if hist is not None:
            kp, vp = ora.kv_append(kp, vp, hist[0], hist[1], hist[2], bs,
                                   np.concatenate(hk), np.concatenate(hv))
        t0 = time.perf_counter()
        kp2, vp2 = ora.kv_append(kp, vp, spec.q_lens, spec.ctx_lens, spec.block_tables, bs,
                                 np.concatenate(kn), np.concatenate(vn))
        ora.attend(np.concatenate(qs), kp2, vp2, spec.q_lens, spec.ctx_lens, spec.block_tables,
                   bs, hkv)
        times.append(time.perf_counter() - t0)
    blas = [i["num_threads"] for i in threadpool_info() if i.get("user_api") == "blas"]
    mean = float(np.mean(times))
    return {"value": round(mean * 1e6, 1), "unit": "µs", "cores": int(max(blas) if blas else 1),
            "kind": "oracle",
            "sample": (f"{len(picks)} of {len(passes)} passes (seeded, {sum(times):.1f} s): append + "
                       f"attention of every row of each; mean per pass; whole trace extrapolated "
                       f"to {mean * len(passes):.0f} s"),
            "host_cpus": len(os.sched_getaffinity(0))}


def replay_trace(torch, fgb, wl, reqs, clients, policy, warmup=1, trace_passes=0, separate=False,
                 record_kernels=True, api="pass"):
    """Replay a request trace through the host scheduler at `clients` closed-loop
    clients under composition `policy`.

    Every pass runs fg_plan_pass -> upload + append -> fg_attention_ragged on
    one pool.  Inputs of all passes come from the keyed hash generator and are
    placed in HBM before timing starts.  Returns the passes, per-pass device
    µs (HIP events on the launch stream, passes back to back), wall time, host
    planning times and the library's per-kernel totals."""
    from ragged_paged_attention_splitfuse_amd import splitfuse as sf

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    hq = hkv = 32
    d, bs, seed = 128, 64, 5
    arrivals = {}
    passes, nb = sf.schedule(reqs, clients=clients, budget=2048, block_size=bs, seed=seed,
                             policy=policy, arrivals=arrivals)
    full_passes = len(passes)
    if trace_passes > 0:
        # a slice of the replay (the first N passes, e.g. for a profiled run)
        passes = passes[:trace_passes]
    t_max = max(p.num_tokens for p in passes)
    kshape, vshape = fgb.pool_shapes(nb, hkv, bs, d)
    kp = torch.zeros(kshape, dtype=torch.bfloat16, device=dev)
    vp = torch.zeros(vshape, dtype=torch.bfloat16, device=dev)
    # every pass's rows, generated in a few large slices and viewed per pass
    rid_rows = np.concatenate([np.repeat(p.rids, p.q_lens) for p in passes])
    pos_rows = np.concatenate([np.arange(c, c + n) for p in passes for c, n in zip(p.ctx_lens, p.q_lens)])
    big = {}
    for kind, h in ((wl.KIND_Q, hq), (wl.KIND_K, hkv), (wl.KIND_V, hkv)):
        buf = torch.empty((len(rid_rows), h, d), dtype=torch.bfloat16, device=dev)
        for a in range(0, len(rid_rows), 16384):
            buf[a:a + 16384] = wl.hash_normal_bf16_torch(seed, kind, rid_rows[a:a + 16384],
                                                         pos_rows[a:a + 16384], h, d, dev)
        big[kind] = buf
    inputs, r0 = [], 0
    for p in passes:
        r1 = r0 + p.num_tokens
        inputs.append(tuple(big[kind][r0:r1] for kind in (wl.KIND_Q, wl.KIND_K, wl.KIND_V)))
        r0 = r1
    max_meta = max_ws = 16
    for p in passes:
        pl = fgb.Plan(p.q_lens, p.ctx_lens, p.block_tables, hq, hkv, d, bs, nb)
        max_meta = max(max_meta, pl.info["metadata_bytes"])
        max_ws = max(max_ws, pl.info["workspace_bytes"])
        pl.close()
    meta = torch.empty(max_meta, dtype=torch.uint8, device=dev)
    ws = torch.empty(max_ws, dtype=torch.uint8, device=dev)
    out = torch.empty((t_max, hq, d), dtype=torch.float32, device=dev)
    lse = torch.empty((t_max, hq), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    # Gated replays: the per-pass events must time device work only, but at
    # few clients a pass takes less device time than its host-side planning
    # and launch, so the device would idle between passes and the idle time
    # would land inside the events.  Before each chunk of 6 passes (fewer
    # than the library's pinned upload slots, so the host never waits for one
    # while the device sleeps) a bounded spin kernel (torch.cuda._sleep) holds
    # the stream for twice the wall time six passes took in the ungated
    # replay, plus 0.3 ms, so the whole chunk is queued before the device
    # reaches it and its passes run back to back.
    gate_chunk = 6   # fewer passes than the library's 8 pinned upload slots: the host never
                     # waits for a slot while the device sleeps
    # the spin kernel's counter rate, measured once (cycles per second)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(1000)
    e0.record(stream)
    torch.cuda._sleep(2_000_000)
    e1.record(stream)
    torch.cuda.synchronize()
    gate_rate = 2_000_000 / max(1e-6, e0.elapsed_time(e1) * 1e-3)
    gate_cycles = [0]

    # per-pass events, created (and recorded once, which creates the HIP
    # event) before any timed replay: event creation inside a replay can stall
    # the host for milliseconds when the runtime grows its event pool
    pass_events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in passes]
    for e0, e1 in pass_events:
        e0.record(stream)
        e1.record(stream)
    torch.cuda.synchronize()

    def replay(record, gated=False):
        keep, evs, host = [], [], []
        for i, (p, (q, k, v)) in enumerate(zip(passes, inputs)):
            if gated and i % gate_chunk == 0:
                torch.cuda._sleep(gate_cycles[0])
            h0 = time.perf_counter()
            plan = fgb.Plan(p.q_lens, p.ctx_lens, p.block_tables, hq, hkv, d, bs, nb)
            host.append(time.perf_counter() - h0)
            t = p.num_tokens
            if record:
                e0, e1 = pass_events[i]
                e0.record(stream)
            if api == "pass":
                fgb.run_pass(plan, meta, q, k, v, kp, vp, out[:t], lse[:t], workspace=ws, stream=stream)
            else:
                if separate:
                    plan.upload(meta, stream)
                    fgb.kv_append(plan, meta, k, v, kp, vp, stream)
                else:
                    fgb.upload_append(plan, meta, k, v, kp, vp, stream)
                fgb.attention_ragged(plan, meta, q, kp, vp, out[:t], lse[:t], workspace=ws, stream=stream)
            if record:
                e1.record(stream)
                evs.append((e0, e1))
            keep.append(plan)
        return keep, evs, host

    gc.collect()
    gc.disable()   # a collection pause inside a gated chunk would land in its events
    for _ in range(max(0, warmup)):
        replay(False)
        torch.cuda.synchronize()
    fgb.fg_profile_read()
    if record_kernels:
        fgb.fg_profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    keep, evs, host = replay(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fgb.fg_profile_enable(False)
    kern = fgb.fg_profile_read()
    per_ungated = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
    keep.clear()
    # the device timeline: per-pass device times from a gated replay; each
    # gate lasts twice the ungated replay's wall time for a chunk, plus 0.3 ms
    gate_cycles[0] = int(gate_rate * min(0.2, 0.0003 + 2.0 * gate_chunk * wall / len(passes)))
    print(json.dumps({"replay": f"{policy} x{clients}", "passes": len(passes), "wall_s": round(wall, 2),
                      "gate_rate_hz": round(gate_rate)}), file=sys.stderr, flush=True)
    keep, evs, _ = replay(True, gated=True)
    torch.cuda.synchronize()
    per = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
    keep.clear()
    gc.enable()
    del inputs, big, kp, vp
    torch.cuda.empty_cache()
    return {"passes": passes, "full_passes": full_passes, "arrivals": arrivals, "pool_blocks": nb,
            "per_us": per, "per_us_ungated": per_ungated, "wall_s": wall, "host_s": host, "kern": kern,
            "t_max": t_max, "shape": (hq, hkv, d, bs, seed)}


def full_budget_ref_us(passes, per_us, budget=2048):
    """Median device time of the replay's passes that hold exactly `budget` tokens."""
    full = [u for p, u in zip(passes, per_us) if p.num_tokens == budget]
    return float(np.median(full)) if full else None


def run_trace(args, torch, fgb, wl):
    """Replay the 512-request trace through the host SplitFuse scheduler."""
    from ragged_paged_attention_splitfuse_amd import splitfuse as sf

    reqs = sf.trace_requests()
    r = replay_trace(torch, fgb, wl, reqs, args.clients, args.serve_policy, warmup=args.warmup,
                     trace_passes=args.trace_passes, separate=args.separate_append, api=args.api)
    passes, per, wall, kern = r["passes"], r["per_us"], r["wall_s"], r["kern"]
    hq, hkv, d, bs, seed = r["shape"]
    serving = None
    if len(passes) == r["full_passes"]:
        t_ref = full_budget_ref_us(passes, per)
        sla = sf.sla_of(t_ref, 2048, args.sla_ttft_factor, args.sla_tpot_factor) if t_ref else None
        serving = sf.serving_metrics(reqs, sf.composition_of(passes), r["arrivals"], per, sla=sla)
    toks = sum(p.num_tokens for p in passes)
    kv_bytes = sum(int(np.sum(p.q_lens.astype(np.int64) + p.ctx_lens)) * hkv * d * 4 for p in passes)
    flops = sum(4 * d * hq * int(np.sum(p.q_lens.astype(np.int64) * p.ctx_lens
                                        + p.q_lens.astype(np.int64) * (p.q_lens + 1) // 2))
                for p in passes)
    attn_ms, attn_n = kern["attn_kernel"]
    # Roofline of the attention launches over the whole replay: algorithmic
    # bytes (KV + Q + fp32 O + LSE of every pass) over their summed event time.
    # HBM-bound like the 7B pass; no counter runs cover the trace (traffic null).
    roof = None
    if attn_ms and attn_n == len(passes):
        attn_bytes = kv_bytes + sum(p.num_tokens * hq * (d * (2 + 4) + 4) for p in passes)
        gbs = attn_bytes / (attn_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None, "kernel": "attn_kernel",
                "algorithmic_per_launch": int(attn_bytes // attn_n), "launches": attn_n}
    res = {
        "metric": METRIC, "value": round(wall * 1e6 / len(passes), 2), "unit": "µs",
        "n_gpus": 1, "steps": len(passes), "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / len(passes), 5), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "trace512", "policy": args.serve_policy, "requests": len(reqs),
                   "clients": args.clients, "budget": 2048, "max_pass_tokens": r["t_max"],
                   "q_heads": hq, "kv_heads": hkv, "head_dim": d, "block_size": bs,
                   "passes": len(passes), "trace_passes": r["full_passes"], "pool_blocks": r["pool_blocks"]},
        "roofline": roof, "cpu_baseline": None,
        "detail": {
            "total_ms": round(wall * 1e3, 3), "tokens": toks,
            "tokens_per_s": round(toks / wall, 1),
            "pass_device_us": {q: round(float(np.percentile(per, v)), 2)
                               for q, v in (("p10", 10), ("p50", 50), ("p90", 90), ("p99", 99), ("max", 100))},
            "device_total_ms": round(float(per.sum()) / 1e3, 3),
            "device_timeline": "per-pass HIP events of a second, gated replay (each chunk of 6 passes "
                               "queued behind a bounded spin, so passes run back to back)",
            "host_plan_us_median": round(float(np.median(r["host_s"])) * 1e6, 1),
            "kernel_ms_total": {k: round(v[0], 3) for k, v in kern.items()},
            "attn_gbs_avg": round(kv_bytes / (attn_ms * 1e-3) / 1e9, 1) if attn_ms else None,
            "attn_tflops_avg": round(flops / (attn_ms * 1e-3) / 1e12, 2) if attn_ms else None,
            "kv_bytes_total": kv_bytes, "flops_total": flops,
            "serving_on_device_timeline": serving,
        },
    }
    if not args.no_cpu:
        res["cpu_baseline"] = trace_cpu_baseline(passes, hq, hkv, d, bs, seed, wl)
        res["detail"]["gpu_vs_oracle"] = round(res["cpu_baseline"]["value"] / res["value"], 1)
    print(json.dumps(res), flush=True)


SERVE_CLIENTS = (1, 2, 4, 8, 16, 32)


def run_serve_sweep(args, torch, fgb, wl):
    """The 512-request trace at 1 .. 32 closed-loop clients under each pass
    composition (the benchmark setup of the research summary, "Key points"),
    with the user-facing metrics and the effective throughput on the device
    timeline.  The SLA unit t_ref is the median full-budget SplitFuse pass of
    the 32-client replay, shared by every point of the sweep."""
    from ragged_paged_attention_splitfuse_amd import splitfuse as sf

    reqs = sf.trace_requests()
    runs = {}
    order = [(c, pol) for c in sorted(SERVE_CLIENTS, reverse=True) for pol in sf.POLICIES]
    for i, (clients, pol) in enumerate(order):
        r = replay_trace(torch, fgb, wl, reqs, clients, pol, warmup=1 if i == 0 else 0,
                         separate=args.separate_append, record_kernels=False, api=args.api)
        runs[(clients, pol)] = r
        print(json.dumps({"clients": clients, "policy": pol, "passes": len(r["passes"]),
                          "device_ms": round(float(r["per_us"].sum()) / 1e3, 2)}), file=sys.stderr, flush=True)
    top = runs[(max(SERVE_CLIENTS), "splitfuse")]
    t_ref = full_budget_ref_us(top["passes"], top["per_us"])
    sla = sf.sla_of(t_ref, 2048, args.sla_ttft_factor, args.sla_tpot_factor)
    points = []
    for (clients, pol), r in sorted(runs.items()):
        m = sf.serving_metrics(reqs, sf.composition_of(r["passes"]), r["arrivals"], r["per_us"], sla=sla)
        points.append({"clients": clients, "policy": pol, "passes": m["passes"],
                       "requests_per_s": m["requests_per_s"],
                       "effective_requests_per_s": m["effective_requests_per_s"], "sla_met": m["sla_met"],
                       "ttft_us_p50": m["ttft_us"]["p50"], "ttft_us_p99": m["ttft_us"]["p99"],
                       "tpot_us_p50": m["tpot_us"]["p50"], "tpot_us_p99": m["tpot_us"]["p99"],
                       "token_gap_us_p99": m["token_gap_us"]["p99"], "token_gap_us_max": m["token_gap_us"]["max"],
                       "host_plan_us_median": round(float(np.median(r["host_s"])) * 1e6, 1)})
    best = max(p["effective_requests_per_s"] for p in points if p["policy"] == "splitfuse")
    res = {"metric": "effective throughput of the attention layer over 1-32 clients (requests/s meeting "
                     "the attention-level SLA, device timeline), 7B shape",
           "value": best, "unit": "requests/s (SplitFuse, best client count)", "n_gpus": 1,
           "steps": sum(len(r["passes"]) for r in runs.values()), "warmup": 1,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic", "config": {"workload": "serve_sweep", "requests": len(reqs),
                                           "clients": list(SERVE_CLIENTS), "policies": list(sf.POLICIES),
                                           "budget": 2048},
           "roofline": None, "cpu_baseline": None,
           "detail": {"sla": sla, "points": points}}
    print(json.dumps(res), flush=True)


def knobs_of(args, fgb):
    policy = {"balanced": fgb.FG_SPLIT_BALANCED, "engine": fgb.FG_SPLIT_ENGINE,
              "per1k": fgb.FG_SPLIT_PER_1K}[args.split_policy]
    return {"target_cus": args.target_cus, "split_policy": policy, "force_splits": args.force_splits}


def measure_pass(torch, fgb, spec, tens, dev, stream, knobs, steps, warmup, separate=False,
                 events="timed-attention", api="pass"):
    """Set up pools and inputs of one pass, then time `steps` passes (plan,
    upload + append in one launch, attention; `separate` uses the two-launch
    upload and append) back to back after `warmup` untimed ones.
    Per-kernel times come from the library's HIP events on the launch stream."""
    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    kshape, vshape = fgb.pool_shapes(spec.num_blocks, spec.num_kv_heads, spec.block_size, spec.head_dim)
    kp = torch.zeros(kshape, dtype=torch.bfloat16, device=dev)
    vp = torch.zeros(vshape, dtype=torch.bfloat16, device=dev)
    hist = spec.history_pass()
    if hist is not None:
        hplan = fgb.Plan(hist[0], hist[1], hist[2], spec.num_q_heads, spec.num_kv_heads,
                         spec.head_dim, spec.block_size, spec.num_blocks)
        fgb.kv_append(hplan, hplan.upload(), to_dev(tens.hist_k), to_dev(tens.hist_v), kp, vp)
        torch.cuda.synchronize()
        hplan.close()
    q, kn, vn = to_dev(tens.q), to_dev(tens.k_new), to_dev(tens.v_new)
    t, hq, d = spec.num_tokens, spec.num_q_heads, spec.head_dim
    out = torch.empty((t, hq, d), dtype=torch.float32, device=dev)
    lse = torch.empty((t, hq), dtype=torch.float32, device=dev)

    probe = fgb.Plan.from_spec(spec, **knobs)
    info = probe.info
    meta = torch.empty(max(16, info["metadata_bytes"]), dtype=torch.uint8, device=dev)
    ws = torch.empty(max(16, info["workspace_bytes"]), dtype=torch.uint8, device=dev)
    probe.close()

    host_plan_s = []

    def step(keep, attention=True):
        h0 = time.perf_counter()
        plan = fgb.Plan.from_spec(spec, **knobs)
        host_plan_s.append(time.perf_counter() - h0)
        if api == "pass" and attention:
            fgb.run_pass(plan, meta, q, kn, vn, kp, vp, out, lse, workspace=ws, stream=stream)
            keep.append(plan)
            return
        if separate:
            plan.upload(meta, stream)
            fgb.kv_append(plan, meta, kn, vn, kp, vp, stream)
        else:
            fgb.upload_append(plan, meta, kn, vn, kp, vp, stream)
        if attention:
            fgb.attention_ragged(plan, meta, q, kp, vp, out, lse, workspace=ws, stream=stream)
        keep.append(plan)

    keep = []
    for _ in range(warmup):
        step(keep)
    torch.cuda.synchronize()
    keep.clear()
    host_plan_s.clear()

    # Per-kernel times come from the library's HIP events on the launch stream.
    # events="timed-attention": the timed passes bracket the attention (and
    # merge) launches, the kernels `roofline` reports, and a second loop of the
    # same passes' upload+append launches alone times that launch.  "timed": the timed passes
    # bracket every launch.  "separate": the timed passes run without events
    # and a second loop brackets every launch.
    in_loop = {"timed": None, "timed-attention": (fgb.FG_KERNEL_ATTENTION, fgb.FG_KERNEL_MERGE),
               "separate": ()}[events]
    fgb.fg_profile_read()
    if in_loop != ():
        # The same passes, untimed, with the same launches bracketed: the
        # library's event pool then holds every event the timed passes use,
        # so none is created inside the timed loop (creating one can hold the
        # host for milliseconds).
        fgb.fg_profile_enable(True, in_loop)
        for _ in range(steps):
            step(keep)
        torch.cuda.synchronize()
        fgb.fg_profile_enable(False)
        fgb.fg_profile_read()
        keep.clear()
        host_plan_s.clear()
        fgb.fg_profile_enable(True, in_loop)
    gc.collect()
    gc.disable()   # no collection pause inside the timed loop
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(keep)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    gc.enable()
    fgb.fg_profile_enable(False)
    kern = fgb.fg_profile_read()
    keep.clear()
    if events != "timed":
        plan_s_timed = list(host_plan_s)
        append_only = events == "timed-attention"
        fgb.fg_profile_enable(True, (fgb.FG_KERNEL_APPEND,) if append_only else None)
        for _ in range(steps):
            step(keep, attention=not append_only)
        torch.cuda.synchronize()
        fgb.fg_profile_enable(False)
        more = fgb.fg_profile_read()
        keep.clear()
        host_plan_s[:] = plan_s_timed
        for name, (ms, n) in more.items():
            if n and not kern[name][1]:
                kern[name] = (ms, n)
    return {"step": step, "keep": keep, "kern": kern, "info": info, "host_plan_s": host_plan_s,
            "ms_per_step": (t1 - t0) * 1e3 / steps}


def kernel_us(kern):
    out = {}
    for key, name in (("append", "append_kernel"), ("attention", "attn_kernel"), ("merge", "merge_kernel")):
        ms, n = kern[name]
        out[key] = ms * 1e3 / n if n else 0.0
    return out


SWEEP_BUDGETS = (256, 512, 1024, 2048, 4096, 8192)


def run_sweep(args, torch, fgb, wl, dev, stream, knobs):
    """Token-budget sweep of the fused pass: the cfg-2 mix (16 decodes plus one
    prompt chunk filling the budget) at budgets 256 .. 8192 tokens."""
    rows = []
    for budget in SWEEP_BUDGETS:
        spec = wl.config_spec(f"7b_budget{budget}")
        tens = wl.make_tensors(spec)
        alg = algorithmic(spec)
        m = measure_pass(torch, fgb, spec, tens, dev, stream, knobs, args.steps, args.warmup,
                         args.separate_append, args.kernel_events, args.api)
        ku = kernel_us(m["kern"])
        pass_us = m["ms_per_step"] * 1e3
        rows.append({"budget": budget, "pass_us": round(pass_us, 2),
                     "tokens_per_s": round(budget / (pass_us * 1e-6), 1),
                     "kernel_us": {k: round(v, 2) for k, v in ku.items()},
                     "attn_tflops": round(alg["flops"] / (ku["attention"] * 1e-6) / 1e12, 1),
                     "attn_gbs": round(alg["attn_bytes"] / (ku["attention"] * 1e-6) / 1e9, 1),
                     "chunk_ctx": int(spec.ctx_lens[-1]), "items": m["info"]["num_items"]})
        print(json.dumps({"budget": budget, "pass_us": rows[-1]["pass_us"]}), file=sys.stderr, flush=True)
        del m, tens
        torch.cuda.empty_cache()
    tps = np.array([r["tokens_per_s"] for r in rows])
    knee = next(r["budget"] for r, v in zip(rows, tps) if v >= 0.9 * tps.max())
    # latency against tokens: least-squares line through (budget, pass µs)
    bud = np.array([r["budget"] for r in rows], dtype=np.float64)
    lat = np.array([r["pass_us"] for r in rows])
    slope, icpt = np.polyfit(bud, lat, 1)
    gain = np.diff(tps) / np.diff(np.log2(bud))   # throughput gained per doubling
    res = {
        "metric": "token-budget sweep of the fused SplitFuse pass (7B shape, 16 decodes + chunk)",
        "value": float(tps.max()), "unit": "tokens/s (max over budgets)", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "sweep", "budgets": list(SWEEP_BUDGETS)},
        "roofline": None, "cpu_baseline": None,
        "detail": {"points": rows, "knee_budget_90pct": knee,
                   "latency_fit_us": {"per_token": round(float(slope), 5),
                                      "intercept": round(float(icpt), 2)},
                   "throughput_gain_per_doubling": [round(float(x), 1) for x in gain],
                   "throughput_concave": bool(np.all(np.diff(gain) <= 0))},
    }
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="7b_pass2048")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--target-cus", type=int, default=0,
                    help="planner balance target (0 = the device's CU count)")
    ap.add_argument("--cold-iters", type=int, default=10,
                    help="extra passes timed with a 1 GiB cache flush before each")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one device-to-device copy of this many MiB (a known-size "
                         "kernel that calibrates HBM byte counters)")
    ap.add_argument("--split-policy", choices=["balanced", "engine", "per1k"], default="balanced",
                    help="planner split-count policy (speed only; results are identical)")
    ap.add_argument("--force-splits", type=int, default=0,
                    help="static split count for every row group (FlashDecoding-style)")
    ap.add_argument("--kernel-events", choices=["timed-attention", "timed", "separate"],
                    default="timed-attention",
                    help="where the per-launch HIP events go: around the attention launches "
                         "of the timed passes (default; upload+append timed in a second loop), "
                         "around every launch of the timed passes, or only in a second loop")
    ap.add_argument("--api", choices=["pass", "append-then-attention"], default="pass",
                    help="how a step runs: fg_pass (metadata upload, then one launch doing the KV "
                         "append and the attention), or the plan upload + KV append launch "
                         "followed by fg_attention_ragged")
    ap.add_argument("--separate-append", action="store_true",
                    help="upload the plan and append K/V in two launches instead of one")
    ap.add_argument("--serve-policy", choices=["splitfuse", "orca", "prefill_first"],
                    default="splitfuse", help="pass composition of the trace512 replay")
    ap.add_argument("--clients", type=int, default=32,
                    help="trace512: closed-loop clients (the pages' benchmark uses 1-32)")
    ap.add_argument("--sla-ttft-factor", type=float, default=3.0,
                    help="SLA: TTFT <= factor x t_ref x ceil(prompt / budget)")
    ap.add_argument("--sla-tpot-factor", type=float, default=1.5,
                    help="SLA: TPOT <= factor x t_ref (t_ref: median full-budget pass)")
    ap.add_argument("--trace-passes", type=int, default=0,
                    help="trace512: replay only the first N passes (0 = all; for profiled runs)")
    ap.add_argument("--no-achievable", action="store_true",
                    help="skip the achievable-peak probes (copy, read stream and bf16 GEMM)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU run: write profiles/traffic_<workload>.json from two "
                         "rocprofv3 --pmc output folders of this script (FETCH_SIZE, "
                         "WRITE_SIZE) taken with --copy-probe-mib")
    args = ap.parse_args()
    if args.traffic_from:
        if args.copy_probe_mib <= 0:
            raise SystemExit("--traffic-from needs the --copy-probe-mib the runs used")
        write_traffic(args.workload, args.traffic_from[0], args.traffic_from[1], args.copy_probe_mib)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this path runs on one GPU only; multi-GPU runs are not "
                          "part of it (sharding by kv head is described in the design notes)",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    from ragged_paged_attention_splitfuse_amd import binding as fgb
    from ragged_paged_attention_splitfuse_amd import workloads as wl

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    if args.workload == "trace512":
        run_trace(args, torch, fgb, wl)
        return
    if args.workload == "serve_sweep":
        run_serve_sweep(args, torch, fgb, wl)
        return
    if args.workload == "sweep":
        run_sweep(args, torch, fgb, wl, dev, stream, knobs_of(args, fgb))
        return
    spec = wl.config_spec(args.workload)
    tens = wl.make_tensors(spec)
    alg = algorithmic(spec)
    t, hq, d = spec.num_tokens, spec.num_q_heads, spec.head_dim
    knobs = knobs_of(args, fgb)
    m = measure_pass(torch, fgb, spec, tens, dev, stream, knobs, args.steps, args.warmup,
                     args.separate_append, args.kernel_events, args.api)
    step, keep, kern, info = m["step"], m["keep"], m["kern"], m["info"]
    host_plan_s, ms_per_step = m["host_plan_s"], m["ms_per_step"]

    # warm passes one by one: each bracketed by HIP events on the launch stream,
    # back to back, for the per-pass distribution (median, p10, p90)
    warm = []
    evs = []
    for _ in range(args.steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step(keep)
        e1.record(stream)
        evs.append((e0, e1))
    torch.cuda.synchronize()
    warm = [a.elapsed_time(b) * 1e3 for a, b in evs]
    keep.clear()

    # cold-cache passes: 1 GiB written between passes evicts L2 and the 256 MB MALL
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cold = []
    for _ in range(args.cold_iters):
        flush.fill_(1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step(keep)
        e1.record(stream)
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1) * 1e3)
    keep.clear()
    del flush

    attn_ms, attn_n = kern["attn_kernel"]
    app_ms, app_n = kern["append_kernel"]
    mrg_ms, mrg_n = kern["merge_kernel"]
    attn_us = attn_ms * 1e3 / max(1, attn_n)
    app_us = app_ms * 1e3 / max(1, app_n)
    mrg_us = mrg_ms * 1e3 / max(1, mrg_n) if mrg_n else 0.0
    attn_gbs = alg["attn_bytes"] / (attn_us * 1e-6) / 1e9
    attn_tflops = alg["flops"] / (attn_us * 1e-6) / 1e12
    pass_us = ms_per_step * 1e3
    traffic = load_traffic(args.workload)
    hbm_floor_us = alg["attn_bytes"] / (PEAK_HBM_GBS * 1e9) * 1e6
    mfma_floor_us = alg["flops"] / (PEAK_BF16_TFLOPS * 1e12) * 1e6
    bound = "hbm" if hbm_floor_us >= mfma_floor_us else "mfma"
    if bound == "hbm":
        roof = {"bound": "hbm", "achieved": round(attn_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(attn_gbs / PEAK_HBM_GBS, 4), "traffic": traffic}
    else:
        roof = {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic}
    achievable = None if args.no_achievable else achievable_peaks(torch, fgb, dev, stream)
    if achievable:
        ach = achievable["hbm_gbs"] if bound == "hbm" else achievable["bf16_gemm_tflops"]
        roof["achievable_peak"] = ach
        roof["frac_of_achievable"] = round(roof["achieved"] / ach, 4)
    roof["kernel"] = "attn_kernel"
    roof["algorithmic_per_launch"] = alg["attn_bytes"] if bound == "hbm" else alg["flops"]

    res = {
        "metric": METRIC,
        "value": round(pass_us, 2),
        "unit": "µs",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": spec.name, "seqs": spec.num_seqs, "tokens": t, "q_heads": hq,
            "kv_heads": spec.num_kv_heads, "head_dim": d, "block_size": spec.block_size,
            "kv_tokens": alg["kv_tokens"], "decodes": int(np.sum(spec.q_lens == 1)),
            "chunk_tokens": [int(x) for x in spec.q_lens[spec.q_lens > 1]],
            "chunk_ctx": [int(x) for x in spec.ctx_lens[spec.q_lens > 1]],
            "split_policy": args.split_policy if args.force_splits == 0 else f"static{args.force_splits}",
        },
        "roofline": roof,
        "cpu_baseline": None,
        "detail": {
            "tokens_per_s": round(t / (pass_us * 1e-6), 1),
            "kernel_us": {"append": round(app_us, 2), "attention": round(attn_us, 2),
                          "merge": round(mrg_us, 2)},
            "attn_gbs": round(attn_gbs, 1), "attn_hbm_frac": round(attn_gbs / PEAK_HBM_GBS, 4),
            "attn_tflops": round(attn_tflops, 2),
            "attn_mfma_frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
            "floor_us": {"hbm": round(hbm_floor_us, 2), "mfma": round(mfma_floor_us, 2)},
            "pass_roofline_frac": round(max(hbm_floor_us, mfma_floor_us) / pass_us, 4),
            "append_gbs": round(alg["append_bytes"] / (app_us * 1e-6) / 1e9, 1) if app_us > 0 else None,
            "host_plan_us_median": round(float(np.median(host_plan_s)) * 1e6, 1) if host_plan_s else None,
            "warm_pass_device_us": {"p10": round(float(np.percentile(warm, 10)), 2),
                                    "median": round(float(np.median(warm)), 2),
                                    "p90": round(float(np.percentile(warm, 90)), 2),
                                    "passes": len(warm)} if warm else None,
            "cold_pass_us": {"p10": round(float(np.percentile(cold, 10)), 2),
                             "median": round(float(np.median(cold)), 2),
                             "p90": round(float(np.percentile(cold, 90)), 2)} if cold else None,
            "plan": {k: info[k] for k in ("num_items", "num_valu_items", "num_mfma_items",
                                          "num_merge_groups", "num_inlaunch_merge_groups", "max_splits_used",
                                          "target_cus")},
            "algorithmic": alg,
            "achievable": achievable,
            "attn_frac_of_achievable": {
                "hbm": round(attn_gbs / achievable["hbm_gbs"], 4),
                "mfma": round(attn_tflops / achievable["bf16_gemm_tflops"], 4),
                "mfma_loop": round(attn_tflops / achievable["bf16_mfma_loop_tflops"], 4)} if achievable else None,
            "kernel_source_sha256_16": source_hash(),
            "kernel_events": args.kernel_events,
        },
    }
    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        res["detail"]["copy_probe_bytes"] = {"read": n, "write": n}
        del src, dst
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(spec, tens)
        res["detail"]["gpu_vs_oracle"] = round(res["cpu_baseline"]["value"] / pass_us, 1)
        if spec.name == "tiny":
            res["detail"]["cpu_baseline_single_thread"] = cpu_baseline(spec, tens, single_thread=True)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
