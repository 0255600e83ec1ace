// plan.h -- the host-side plan object behind the opaque fg_plan handle.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "fg.h"
#include "fg_meta.h"

struct fg_plan {
  // Shape of the pass.
  int32_t num_seqs = 0;
  int32_t num_tokens = 0;
  int32_t hq = 0, hkv = 0, group = 0, head_dim = 0, block_size = 0, num_blocks = 0;
  float scale = 0.f;

  // Packed device metadata: [SeqRec][block ids][RunRec][ItemRec][MergeRec]
  // [int32 split-group counters, zero], each section starting on a 16-byte
  // boundary (byte offsets below).
  std::vector<uint8_t> blob;
  size_t off_seqs = 0, off_bt = 0, off_runs = 0, off_items = 0, off_merges = 0, off_counters = 0;

  int32_t n_runs = 0;
  int32_t n_items = 0;   // n_mfma matrix-core items first, then n_valu
  int32_t n_mfma = 0;
  int32_t n_valu = 0;
  int32_t n_tiles = 0;   // matrix-core items of two or more wavefronts (prefill tiles)
  int32_t n_merge_groups = 0;   // row groups that were split (one MergeRec each)
  int32_t n_inlaunch_groups = 0;  // the first of them, merged inside the attention launch
  int32_t n_partial_rows = 0;
  int32_t max_splits_used = 0;
  int32_t target_cus = 0;
  int32_t resident_slots = 0;   // work-groups per CU the dispatch order assumed

  // Workspace: partial O rows [n_partial_rows, D] fp32 then lse [n_partial_rows].
  size_t ws_o_off = 0, ws_lse_off = 0, ws_bytes = 0;
};

// Compute units of the current HIP device, or a negative value on failure.
// Defined next to the kernels so that the planner itself needs no HIP headers.
extern "C" int fg_internal_device_cu_count(void);
