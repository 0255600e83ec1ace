/*
 * fg.h -- C ABI of libfg.so: ragged paged attention for Dynamic SplitFuse
 * passes on AMD Instinct MI355X (gfx950).
 *
 * A "pass" is one forward step's worth of attention at a fixed token budget:
 * each sequence s brings q_lens[s] new query tokens (a prompt chunk when > 1,
 * a decode when == 1) on top of ctx_lens[s] tokens already in a paged KV
 * cache.  Composing such passes from prompt chunks plus decode tokens is
 * Dynamic SplitFuse ("DeepSpeed-FastGen: High-throughput Text Generation for
 * LLMs via MII and DeepSpeed-Inference", research summary page, section
 * "Summary"; InfoQ news item "Microsoft releases DeepSpeed-FastGen").
 *
 * The cache is paged: fixed-size physical blocks addressed per sequence by a
 * block table that the kernels read themselves ("DeepSpeed-FastGen Guide:
 * Dynamic SplitKV Serving", section "3. Paged KV Memory Management with Zero
 * Overhead").  Long KV ranges are split over compute units and the partial
 * results merged by log-sum-exp (same page, section "1. Dynamic SplitKV
 * Attention"); for decode rows the merge runs inside the attention launch,
 * done by whichever work-group finishes a split group last, and split prefill
 * tiles are merged by a short launch after it.
 *
 * Call order for one pass, all on one HIP stream, nothing synchronises inside
 * the library:
 *     fg_plan_pass -> fg_plan_upload -> fg_kv_append -> fg_attention_ragged
 *     ... stream sync ... -> fg_plan_destroy
 * or, with the first two device steps in one launch,
 *     fg_plan_pass -> fg_upload_append -> fg_attention_ragged -> ...
 * or the whole pass in one call,
 *     fg_plan_pass -> fg_pass -> ... stream sync ... -> fg_plan_destroy
 *
 * Conventions
 * -----------
 * - Every function returns an fg_status (0 = success, negative = error); no
 *   exception crosses the ABI and nothing aborts.
 * - All validation happens in fg_plan_pass; a plan that exists is valid, and
 *   the kernels never see an index outside the pools.
 * - The library calls no device allocator.  The caller owns every device
 *   buffer (metadata, workspace, pools, inputs, outputs) and the stream; the
 *   library's only device memory of its own is the static scratch array behind
 *   fg_attention_ragged_noalloc.
 * - Device pointers must be 16-byte aligned.  `stream` is a hipStream_t passed
 *   as void* (NULL = the null stream).
 * - Plans are immutable after fg_plan_pass; functions are reentrant.  Calls
 *   that write the same device buffers must not overlap in time.
 * - bf16 means IEEE binary32's upper 16 bits (round-to-nearest-even when the
 *   library rounds).
 *
 * Tensor layouts (row-major, innermost last)
 * ------------------------------------------
 *   q          [T, Hq, D]            bf16, tokens in sequence order
 *   k_new/v_new[T, Hkv, D]           bf16, same token order
 *   k_pool     [num_blocks, Hkv, B, D]  bf16  (slot-major within a block)
 *   v_pool     [num_blocks, Hkv, B/S, D, S]  bf16, S = min(B, 32): each
 *                                      block stored transposed in sub-blocks
 *                                      of S slots (for every dim, S slots
 *                                      contiguous); B <= 32 is one sub-block
 *   out        [T, Hq, D]            fp32 or bf16
 *   lse        [T, Hq]               fp32, natural log
 * where T = sum(q_lens), B = block_size, D = head_dim.  Token j of sequence s
 * lives at absolute position p = ctx_lens[s] + j, in physical block
 * block_tables[s*max_blocks_per_seq + p / B] at slot p % B.  Query head h
 * reads kv head h / (Hq / Hkv).
 */
#ifndef FG_H
#define FG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 3: d_meta of fg_attention_ragged is writable (split-group counters).
 * 4: V pool blocks stored in transposed sub-blocks of min(B, 32) slots. */
#define FG_ABI_VERSION 4

typedef int32_t fg_status;

enum {
  FG_OK = 0,
  FG_E_INVALID = -1,     /* null pointer, negative count, Hq % Hkv != 0, bad knob */
  FG_E_RANGE = -2,       /* block id outside [0, num_blocks); table row too short
                            for ctx + q_len; q_len < 1; size overflow */
  FG_E_ALIAS = -3,       /* a physical block used twice within one pass */
  FG_E_UNSUPPORTED = -4, /* head_dim not in {64,128}, block_size not in {16,32,64},
                            unknown output dtype */
  FG_E_WORKSPACE = -5,   /* workspace smaller than the plan needs, or misaligned */
  FG_E_HIP = -6,         /* a HIP runtime call or kernel launch failed */
  FG_E_NOMEM = -7        /* host allocation failed */
};

enum { FG_DTYPE_F32 = 0, FG_DTYPE_BF16 = 1 };

/* Description of one pass.  All pointers are host pointers; the planner
 * copies what it needs, so they may be freed when fg_plan_pass returns. */
typedef struct fg_pass_desc {
  int32_t num_seqs;           /* S >= 0 (S == 0 is an empty pass) */
  int32_t num_q_heads;        /* Hq >= 1 */
  int32_t num_kv_heads;       /* Hkv >= 1, Hq % Hkv == 0 */
  int32_t head_dim;           /* D: 64 or 128 */
  int32_t block_size;         /* B: 16, 32 or 64 tokens */
  int32_t num_blocks;         /* physical blocks in each pool, >= 1 */
  int32_t max_blocks_per_seq; /* row stride of block_tables */
  float scale;                /* softmax scale; 0 selects 1/sqrt(D) */
  const int32_t* q_lens;      /* [S], each >= 1 */
  const int32_t* ctx_lens;    /* [S], each >= 0 */
  const int32_t* block_tables;/* [S * max_blocks_per_seq]; entries past
                                 ceil((ctx+q_len)/B) are ignored, the used ones
                                 must lie in [0, num_blocks) and be distinct
                                 across the whole pass */
  /* Planner knobs (0 = default).  They change speed only, never results. */
  int32_t target_cus;         /* compute units to balance over; 0 = query the
                                 current HIP device (needs a GPU) */
  int32_t min_split_tokens;   /* smallest KV range worth its own work item */
  int32_t max_splits;         /* cap on KV splits of one row group (<= 256) */
  int32_t force_splits;       /* > 0: split every row group's KV range into this
                                 many parts regardless of cost (tests, and the
                                 static FlashDecoding-style policy) */
  int32_t split_policy;       /* FG_SPLIT_*: how KV split counts are chosen when
                                 force_splits is 0 */
} fg_pass_desc;

/* Split-count policies.  All give the same attention results; only speed
 * differs.
 *   FG_SPLIT_BALANCED  (default) per row group, from a cost model in KV tokens
 *                      balanced over target_cus compute units.
 *   FG_SPLIT_ENGINE    per sequence, the allocation engine of "DeepSpeed-FastGen
 *                      Guide: Dynamic SplitKV Serving", section "Step 2: Dynamic
 *                      SplitKV Allocation Engine", as a formula: with
 *                      N = target_cus, m = min_split_tokens (default 256),
 *                      b_s = clamp(kv_len_s / m, 1, 16) and B = sum of b_s,
 *                      k_s = 1 when there are at least N sequences, else
 *                      max(1, b_s * N / B) when B < N, else b_s (integer
 *                      floors; the scaled count may exceed 16).
 *   FG_SPLIT_PER_1K    per sequence, kv_len / 1024 clamped to [1, 16]: the
 *                      reading of the same page's figure "Dynamic SplitKV
 *                      Two-Phase Attention Kernel Workflow" (512, 4096 and 16384
 *                      tokens get 1, 4 and 16 splits).
 * A sequence's count applies to each of its row groups.  Every count is then
 * capped by max_splits and by the 64-token alignment of split ranges (a range
 * of L tokens split k ways uses parts of ceil(ceil(L / k) / 64) * 64 tokens). */
enum { FG_SPLIT_BALANCED = 0, FG_SPLIT_ENGINE = 1, FG_SPLIT_PER_1K = 2 };

typedef struct fg_plan fg_plan;

typedef struct fg_plan_info_t {
  int64_t num_tokens;      /* T */
  int64_t metadata_bytes;  /* size of the device metadata buffer */
  int64_t workspace_bytes; /* size of the attention workspace (may be 0) */
  int32_t num_items;       /* attention work items (work-groups) */
  int32_t num_valu_items;  /* of which on the vector-ALU path (few query rows) */
  int32_t num_mfma_items;  /* of which on the matrix-core path (row tiles) */
  int32_t num_merge_groups;/* row groups whose KV range was split */
  int32_t num_partial_rows;/* partial (O, lse) rows held in the workspace */
  int32_t max_splits_used;
  int32_t num_append_runs; /* (sequence, block) runs the append writes */
  int32_t target_cus;      /* CU count the plan was balanced for */
  int32_t num_inlaunch_merge_groups; /* split groups merged inside the attention
                              launch (the rest get a merge launch after it) */
} fg_plan_info_t;

/* Build the plan of one pass (host only, no device call unless
 * desc->target_cus == 0): the split-KV work list whose split counts follow
 * each request's length and the compute-unit count ("DeepSpeed-FastGen Guide:
 * Dynamic SplitKV Serving", section "1. Dynamic SplitKV Attention", and its
 * "Step 2: Dynamic SplitKV Allocation Engine").  Validates every input: null
 * pointers, bad counts or knobs -> FG_E_INVALID; block ids out of range or a
 * short table row -> FG_E_RANGE; a block used twice -> FG_E_ALIAS; head_dim or
 * block_size not supported -> FG_E_UNSUPPORTED; host allocation failure ->
 * FG_E_NOMEM; a failed device query for target_cus == 0 -> FG_E_HIP.  The
 * desc's arrays are copied, so the caller may free them on return.  On
 * success *out_plan receives a plan owned by the library; free it with
 * fg_plan_destroy.  Deterministic: the same desc gives a byte-identical plan. */
fg_status fg_plan_pass(const fg_pass_desc* desc, fg_plan** out_plan);

/* Report sizes and counts of a plan. */
fg_status fg_plan_info(const fg_plan* plan, fg_plan_info_t* out);

/* Copy the plan's metadata into d_meta (device, >= metadata_bytes,
 * caller-owned, 16-byte aligned), asynchronously and in order on `stream`.
 * FG_E_INVALID for a null plan or a null or misaligned d_meta, FG_E_HIP if a
 * copy or launch fails.  Plans up to 2 MiB
 * are staged through a library-owned ring of pinned host buffers (allocated on
 * first use, held until the process ends) and copied by a small kernel on the
 * same stream; larger ones use hipMemcpyAsync, in which case the plan must stay
 * alive until the stream has passed the copy. */
fg_status fg_plan_upload(const fg_plan* plan, void* d_meta, void* stream);

/* Scatter the pass's new K and V into their cache slots (asynchronous): token
 * j of sequence s goes to block block_tables[s][p / B], slot p % B, with
 * p = ctx_lens[s] + j ("DeepSpeed-FastGen Guide: Dynamic SplitKV Serving",
 * section "3. Paged KV Memory Management with Zero Overhead").  d_meta must
 * hold this plan's uploaded metadata (read only here).  k_new, v_new:
 * [T, Hkv, D] bf16; k_pool, v_pool: pools in the layouts above; all
 * caller-owned.  Writes exactly T*Hkv K rows and T*Hkv V columns; no other
 * byte of the pools changes.  Bit-exact copy.  FG_E_INVALID for a null or
 * misaligned pointer (a pass with nothing to append returns FG_OK at once),
 * FG_E_HIP if the launch fails. */
fg_status fg_kv_append(const fg_plan* plan, const void* d_meta,
                       const void* k_new, const void* v_new,
                       void* k_pool, void* v_pool, void* stream);

/* fg_plan_upload followed by fg_kv_append, as one kernel launch (saves a launch
 * and the gap between two kernels).  Arguments as for those two calls; on
 * return d_meta holds the plan (once the stream gets there) and the pools hold
 * the pass's new K/V, bit-exact as fg_kv_append writes them.  The append reads
 * its run records from the pinned staging slot, so it does not wait for the
 * metadata copy.  Plans over 2 MiB, or a process where pinned staging could
 * not be allocated, fall back to the two separate steps. */
fg_status fg_upload_append(const fg_plan* plan, void* d_meta, const void* k_new,
                           const void* v_new, void* k_pool, void* v_pool, void* stream);

/* Attention of every query row of the pass over its sequence's cached keys
 * 0 .. ctx + j (inclusive causal bound), read through the block tables
 * (asynchronous; one kernel launch, plus a merge launch when the plan splits
 * prefill tiles).  Split KV ranges are computed as partial softmax results and
 * merged by log-sum-exp ("DeepSpeed-FastGen Guide: Dynamic SplitKV Serving",
 * section "1. Dynamic SplitKV Attention", two-phase softmax; merge weights are
 * the partials' log-sum-exp values).  Errors: FG_E_UNSUPPORTED for an unknown
 * out_dtype, FG_E_INVALID for a null or misaligned pointer, FG_E_WORKSPACE for
 * a missing, short or misaligned workspace, FG_E_HIP if a launch fails; a plan
 * with no rows returns FG_OK without a launch.  The pools must already hold this pass's
 * K/V (append first, on the same stream).  q: [T, Hq, D] bf16.  out: [T, Hq, D]
 * of out_dtype (FG_DTYPE_F32 or FG_DTYPE_BF16).  lse: [T, Hq] fp32 or NULL.
 * d_ws: caller-owned workspace of >= workspace_bytes (may be NULL when that is
 * 0); its contents on entry do not matter.
 * d_meta is written as well as read: the split groups' arrival counters live
 * in it.  They are zero after an upload and every call leaves them zero again,
 * so one upload serves any number of calls; calls sharing one d_meta must not
 * overlap in time (stream order them). */
fg_status fg_attention_ragged(const fg_plan* plan, void* d_meta,
                              const void* q, const void* k_pool, const void* v_pool,
                              void* out, int32_t out_dtype, float* lse,
                              void* d_ws, size_t ws_bytes, void* stream);

/* fg_attention_ragged with this pass's own key positions (ctx_s .. ctx_s +
 * q_len_s - 1 of each sequence) read from k_new / v_new ([T, Hkv, D] bf16, as
 * given to fg_kv_append) instead of the pools: the pools need to hold only
 * the cached context, and the pool slots of the new positions are never read.
 * The attention step of fg_pass, for a pass whose K/V is not (yet) appended.
 * Arguments and errors as for fg_attention_ragged; FG_E_INVALID for a null or
 * misaligned k_new / v_new. */
fg_status fg_attention_ragged_direct(const fg_plan* plan, void* d_meta, const void* q,
                                     const void* k_new, const void* v_new,
                                     const void* k_pool, const void* v_pool, void* out,
                                     int32_t out_dtype, float* lse, void* d_ws, size_t ws_bytes,
                                     void* stream);

/* One whole pass: the plan's metadata upload, the KV append and the attention
 * (plus the merge launch when the plan splits prefill tiles).  For a plan
 * without prefill tiles the append is done by work-groups of the attention
 * launch, and attention reads key positions below each sequence's cached
 * context from the pools and the pass's own positions straight from k_new /
 * v_new, so it does not wait for the append.  A plan with prefill tiles runs
 * the fused upload + append launch first and then the attention launch over
 * the pools (tiles staged from the pools measured faster).  Either way the
 * pools hold the pass's K/V once the stream has passed the call, bit for bit
 * as fg_kv_append writes them ("DeepSpeed-FastGen Guide: Dynamic SplitKV
 * Serving", section "3. Paged KV Memory Management with Zero Overhead": the
 * kernel reads the block tables itself, with no separate translation pass).
 * Arguments as for fg_plan_upload, fg_kv_append and fg_attention_ragged
 * (k_pool / v_pool are written); the same errors. */
fg_status fg_pass(const fg_plan* plan, void* d_meta, const void* q, const void* k_new,
                  const void* v_new, void* k_pool, void* v_pool, void* out, int32_t out_dtype,
                  float* lse, void* d_ws, size_t ws_bytes, void* stream);

/* fg_attention_ragged for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same kernels and results, bit for bit, with no workspace
 * argument.  The split partial rows go to a library-owned scratch array that
 * sits in the library's code object on each GPU (fg_noalloc_scratch_bytes()
 * bytes, 32 MiB, held by every GPU the library runs on until the process
 * ends).  The call allocates nothing, creates no events (fg_profile_enable
 * does not bracket it) and needs no initialisation.  Arguments, layouts,
 * ownership and errors as for fg_attention_ragged, plus FG_E_WORKSPACE when
 * the plan's workspace_bytes exceed the scratch size, FG_E_HIP if the
 * scratch's device address cannot be looked up, FG_E_UNSUPPORTED past 64
 * devices.  Every call on one GPU shares that GPU's scratch (its contents on
 * entry do not matter): calls that overlap in time on one GPU, on any
 * streams, race and give undefined results. */
fg_status fg_attention_ragged_noalloc(const fg_plan* plan, void* d_meta,
                                      const void* q, const void* k_pool, const void* v_pool,
                                      void* out, int32_t out_dtype, float* lse, void* stream);

/* Size in bytes of the scratch array behind fg_attention_ragged_noalloc. */
size_t fg_noalloc_scratch_bytes(void);

/* Free a plan (NULL is allowed).  Only after the stream has passed every
 * call that used it. */
void fg_plan_destroy(fg_plan* plan);

/* Static, human-readable name of a status code. */
const char* fg_status_string(fg_status status);

/* FG_ABI_VERSION of the built library. */
int32_t fg_abi_version(void);

/* ---- introspection (tests and debugging) -----------------------------------
 * Copy the plan's packed device metadata (metadata_bytes; the same bytes
 * fg_plan_upload sends) into the host buffer host_dst of `bytes` bytes, and
 * report where each record section starts.  Records are little-endian int32:
 *   sequence  8 ints: q_start, q_len, ctx, kv_len, block_id_offset, num_blocks, 0, 0
 *   block id  1 int:  physical block of each used table entry, per sequence
 *   run       4 ints: first new-token row, first slot, token count, block
 *   item     12 ints: seq, kv_head, row0, nrows, kv0, kv1, slot (-1 = final
 *                     rows, else first partial row), waves (0 = vector-ALU
 *                     path), group (split group, -1 = unsplit), 0, 0, 0
 *   merge     8 ints: seq, kv_head, row0, nrows, nsplit, slot0, 0, 0
 *                     (one per split group; the first num_counters groups are
 *                     merged inside the attention launch, the rest by a merge
 *                     launch after it)
 *   counter   1 int:  arrival counter of each in-launch split group, 0
 * Packed row r of an item is query token r / G at q head kv_head * G + r % G;
 * split i of a split group's row r sits at partial row slot0 + i * nrows + r.
 * host_dst may be NULL to query the layout only. */
typedef struct fg_plan_layout_t {
  int64_t seqs, block_ids, runs, items, merges, counters;   /* byte offsets */
  int32_t num_seqs, num_block_ids, num_runs, num_items, num_merges, num_counters;
} fg_plan_layout_t;

fg_status fg_plan_metadata(const fg_plan* plan, void* host_dst, size_t bytes,
                           fg_plan_layout_t* layout);

/* Work-groups one CU holds at once.  *planned: the count fg_plan_pass assumed
 * when it dealt the plan's first launch rounds onto the CUs (the matrix-core
 * kernel's for plans with matrix-core items, else the decode-only kernel's);
 * it affects speed only.  *device: what the HIP occupancy calculator gives for
 * the attention kernels this plan can launch on the current device (the
 * smaller of the pool-reading and the direct instantiation), or -1 when it
 * cannot be queried (no GPU).  Introspection for tests; no launch.
 * FG_E_INVALID for a null argument, FG_E_UNSUPPORTED for an unsupported
 * head_dim / block_size. */
fg_status fg_plan_resident_slots(const fg_plan* plan, int32_t* planned, int32_t* device);

/* ---- measurement hooks ------------------------------------------------------
 * fg_profile_enable(mask): bit (1 << FG_KERNEL_x) of mask makes the library
 * bracket each launch of that kernel with HIP events recorded on the launch
 * stream; 0 turns it off, -1 brackets every kernel.  fg_profile_read waits for
 * the recorded events, writes per-kernel totals (milliseconds and launch
 * counts, indexed by the FG_KERNEL_* ids) and clears the record.  Off by
 * default; the record is process-wide and not thread-safe. */
enum {
  FG_KERNEL_APPEND = 0,
  FG_KERNEL_ATTENTION = 1,
  FG_KERNEL_MERGE = 2,
  FG_KERNEL_COUNT = 3
};

fg_status fg_profile_enable(int32_t on);
fg_status fg_profile_read(double* total_ms, int32_t* launches, int32_t n_kernels);
const char* fg_kernel_name(int32_t kernel_id);

/* Achievable HBM read rate, for measurement only (no step of the method uses
 * it): one launch on `stream` streams `bytes` (a multiple of 16) from the
 * caller-owned device buffer buf (16-byte aligned) with 16-byte non-temporal
 * loads, and writes one uint32 per thread into the caller-owned device buffer
 * sink, which must hold at least 1024 bytes per compute unit of the current
 * device (256 KiB on a 256-CU part; 1 MiB covers any).  Time it with events
 * on the same stream.  FG_E_INVALID for null or misaligned pointers or a size
 * not a multiple of 16, FG_E_WORKSPACE for a short sink, FG_E_HIP if the
 * launch fails. */
fg_status fg_probe_read_stream(const void* buf, size_t bytes, void* sink, size_t sink_bytes,
                               void* stream);

/* Achievable matrix-core rate and the shader clock under matrix-core load, for
 * measurement only: one launch on `stream` of two 256-thread work-groups per
 * compute unit, each wavefront issuing iters (1..2048) rounds of 32 bf16
 * 32x32x16 MFMAs (32,768 flops each) on register operands.  Writes one float
 * per thread into sink (>= 2 KiB per compute unit; each value is 8192 * iters)
 * and, per work-group, two int64 counts into clocks (>= 32 bytes per compute
 * unit): elapsed shader-clock cycles (s_memtime) and elapsed 100 MHz ticks
 * (s_memrealtime).  Both buffers are caller-owned device memory.  Time it with
 * events on the same stream.  FG_E_INVALID for null or misaligned pointers or
 * iters out of range, FG_E_WORKSPACE for short buffers, FG_E_HIP if the launch
 * fails. */
fg_status fg_probe_mfma_loop(int32_t iters, void* sink, size_t sink_bytes, void* clocks,
                             size_t clocks_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FG_H */
