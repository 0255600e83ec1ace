// fg_meta.h -- device metadata records written by the host planner and read
// by the kernels.  Plain int32 records, 16-byte aligned sections, no pointers,
// so one host-to-device copy moves a whole plan.
#pragma once

#include <stdint.h>

namespace fg {

// Query rows per work item on the vector-ALU path (decodes and tiny chunks).
constexpr int kValuMaxRows = 4;
// Query rows per wavefront on the matrix-core path, and wavefronts per item.
constexpr int kMfmaRowsPerWave = 32;
constexpr int kMfmaMaxWaves = 4;
constexpr int kMfmaTileRows = kMfmaRowsPerWave * kMfmaMaxWaves;
// KV tokens per LDS stage on the matrix-core path; split boundaries are
// aligned to it so every item starts on a stage boundary.
constexpr int kKvTile = 64;
// KV tokens per V^T sub-block, and per vector-ALU wavefront step in the
// decode-only kernel (the mixed kernel steps two at a time); divides kKvTile.
constexpr int kValuSubTile = 32;

// Per-sequence record.
struct SeqRec {
  int32_t q_start;   // first row of this sequence in q / out / k_new
  int32_t q_len;     // n_s
  int32_t ctx;       // c_s: tokens cached before this pass
  int32_t kv_len;    // c_s + n_s
  int32_t bt_off;    // offset of this sequence's used block-table entries
  int32_t nblk;      // ceil(kv_len / B)
  int32_t pad0, pad1;
};

// One append run: up to B consecutive new tokens of one sequence that land in
// one physical block.
struct RunRec {
  int32_t tok0;      // first row in k_new / v_new
  int32_t slot0;     // slot of the first token inside the block
  int32_t count;     // tokens in the run
  int32_t block;     // physical block id
};

// One attention work item: a group of query rows of one (sequence, kv head)
// over one KV range.  Packed row r of the group is query token r / G of the
// sequence at q head kv_head * G + r % G.
struct ItemRec {
  int32_t seq;
  int32_t kv_head;
  int32_t row0;      // first packed row
  int32_t nrows;     // rows in the item
  int32_t kv0;       // KV range [kv0, kv1); kv0 is a multiple of kKvTile
  int32_t kv1;
  int32_t slot;      // -1: write final out/lse; else first partial row
  int32_t waves;     // matrix-core path: active wavefronts (1..4); else 0
  int32_t group;     // split group (index into the group records), -1 if unsplit
  int32_t pad0, pad1, pad2;
};

// A split group: the rows of one item-row range whose KV range was cut into
// `nsplit` items.  Split i of row r writes partial row slot0 + i * nrows + r.
// Groups 0 .. n_inlaunch-1 (at most one wavefront's rows -- decode rows, GQA
// decode groups -- split at most four ways) are merged inside the attention
// launch by the work-group
// that finishes the group's last split; each owns one int32 arrival counter
// in the counter section (zero on upload, reset to zero by the merging
// work-group).  The remaining groups (split prefill tiles, whose partials are
// 64 KiB per split, and many-way splits) are merged by a merge launch after
// the attention launch.
struct MergeRec {
  int32_t seq;
  int32_t kv_head;
  int32_t row0;
  int32_t nrows;
  int32_t nsplit;
  int32_t slot0;
  int32_t pad0, pad1;
};

static_assert(sizeof(SeqRec) == 32, "SeqRec layout");
static_assert(sizeof(RunRec) == 16, "RunRec layout");
static_assert(sizeof(ItemRec) == 48, "ItemRec layout");
static_assert(sizeof(MergeRec) == 32, "MergeRec layout");

}  // namespace fg
