// plan.cpp -- host planner of one ragged paged attention pass.
//
// Validates the pass description, packs per-sequence records and the used
// block-table entries, cuts the new tokens into per-block append runs, and
// builds the attention work list: query rows of each (sequence, kv head) are
// grouped (few rows -> vector-ALU items, many rows -> 128-row matrix-core
// tiles), and each group's visible KV range is split over compute units when
// it is long compared with the pass's total work.  Split partials are merged
// by log-sum-exp inside the attention launch: the work-group that finishes a
// split group's last split merges it.
//
// The length-aware split follows the adaptive split-KV idea of "DeepSpeed-
// FastGen Guide: Dynamic SplitKV Serving" (section "1. Dynamic SplitKV
// Attention": split counts follow each request's length and the number of
// compute units; short requests are not split).  The policy itself is ours:
// a cost model in KV tokens, a per-item target derived from the total work
// and the CU count, splits aligned to the 64-token KV stage, and
// longest-first ordering of the work items.
#include "plan.h"

#include <math.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <numeric>

namespace {

using fg::ItemRec;
using fg::MergeRec;
using fg::RunRec;
using fg::SeqRec;

constexpr int64_t kMaxTokens = int64_t(1) << 28;
constexpr int64_t kMaxKvLen = int64_t(1) << 28;
// Every launch runs 256-thread work-groups and a dispatch's work-item count
// is a 32-bit number, so one launch holds at most 2^24 - 1 work-groups: the
// attention items, the merge groups, and the append launch's (run, kv head)
// pairs plus its metadata-copy groups.  Packed query rows of a (sequence, kv
// head), q_len * G, are int32 indices in the item records.  Passes past
// either limit are rejected with FG_E_RANGE before anything is sized by them.
constexpr int64_t kMaxGroupsPerLaunch = (int64_t(1) << 24) - 1;
constexpr int64_t kMaxPackedRows = INT32_MAX;
constexpr int kDefaultMinSplitTokens = 256;
constexpr int kDefaultMaxSplits = 64;
constexpr int kMaxSplitsLimit = 256;
// Items longer than total / (CUs * kItemsPerCu) are split.  Two per CU (one
// per resident work-group slot) is enough for longest-first dispatch to end
// with every CU busy until close to the mean; a finer target buys little
// balance and costs partial-row traffic plus the merge (measured on the 7B
// 2048-token pass: 256 us per pass at 2, 280 us at 3 and 4).
constexpr double kItemsPerCu = 2.0;
// A pass whose groups all take the matrix-core path (GQA groups of more than
// kValuMaxRows rows) is split more coarsely: its items carry several query
// rows per KV stream, and each split adds a partial write and a merge for all
// of them.  Measured on the 70B GQA passes (16/2 heads): the 32-decode half
// 31.7 -> 29.4 us of attention, the 4096-token share 104 -> 102 us; at 1.0 the
// share lost (117 us).  Passes with vector-ALU decodes stay at kItemsPerCu
// (the 7B decode half: 117 us at 2.0, 127 us at 1.5).
constexpr double kMfmaOnlyItemsPerCu = 1.5;
// Matrix-core tiles: relative cost per KV token of a tile with R padded rows
// is max(kMfmaMinCost, R / kFlopPerByte), where kFlopPerByte is the ratio of
// achievable bf16 MFMA rate to achievable HBM rate on MI355X (about
// 1000 TFLOP/s : 6 TB/s).  Splitting a prefill tile (two or more wavefronts)
// buys no attention time once there are at least as many tiles as CUs, but
// moves its partial rows through the workspace and puts the merge on the
// group's last split, so such tiles are split only when they are too few to
// occupy the CUs (then to about kMfmaSlotsPerCu items per CU, never below
// kMfmaMinSplitTokens).  Measured on MI355X: splitting tiles longer than
// 1.5x the per-slot mean slowed the 70B-class chunk pass from 99 to 113 us,
// and 1.0x slowed the 7B chunk from 107 to 168 us.  One-wave
// groups (GQA decodes) are bandwidth-bound like decodes and use the common
// target.
constexpr double kFlopPerByte = 170.0;
constexpr double kMfmaMinCost = 0.5;
constexpr int kMfmaMinSplitTokens = 1024;
constexpr int kMfmaSlotsPerCu = 2;
// Split groups merged inside the attention launch: at most one wavefront's
// rows, in plans of at most this many items per work-group slot (slots of the
// kernel the plan launches).  Every split item of such a group ends with a
// store drain and a device-scope atomic round trip before it can exit, so a
// slot pays that latency once per item it runs.  Measured: 64 decodes split
// 16 ways (55 items per slot) took 1,218 us per pass in-launch and 1,064 us
// with a merge launch; the 70B-class decode half (about one item per slot, 64
// groups split 8 ways) took 59.0 us in-launch and 64.5 us with the merge
// launch; 64 decodes at the default split (2,336 items, three slots per CU)
// took 715 us in-launch and 728 us with the merge launch.
constexpr int kInLaunchMaxItemsPerSlot = 4;
// Decode-only passes with several groups per slot (many sequences, lengths
// spread widely): the longest groups are each about one slot's share, and the
// launch ends with those few streams running alone.  Halving the split target
// there splits only the longest ones.  Measured on MI355X, 64 decodes with
// contexts log-uniform over 512..16000: attention + merge 682 -> 669 us at 1/2,
// 673 us at 1/4; the 7B pass, its decode half and the 70B decode half are
// untouched by the rule (tiles present, or about one group per slot).
constexpr double kSkewedItemsPerSlot = 2.0;
constexpr double kSkewedSplitFactor = 2.0;
// Round fitting.  Items of a tile-free plan are about equal by construction,
// so a plan a few items past a whole number of work-group rounds runs one more
// round for those few: the launch takes about one item time longer.  When the
// excess is at most kRoundFitSlack of a round, the split target grows until
// the items fit the rounds (at most kRoundFitPasses re-splits).  Plans with
// tiles are left alone: there the decode items fill in beside long tiles.
// Measured on MI355X, the 70B-class decode half (32 GQA decodes, 64 groups):
// 542 items on 512 slots took 34.5 us of attention; 492 items (8 splits) took
// 28.1 us and 438 items (7 splits) 27.8 us, against 31.5 us at 546 items.
// A round is counted as two work-groups per CU for every tile-free plan: in
// the decode-only kernel's three, 64 decodes were fitted to three rounds
// (2,304 items) and took 689 us of attention against 685 us unfitted.
constexpr double kRoundFitSlack = 0.25;
constexpr int kRoundFitPasses = 4;

size_t align16(size_t x) { return (x + 15) & ~size_t(15); }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Group {
  int32_t seq, kv_head, row0, nrows, vis_end, waves;  // waves 0: vector-ALU path
  double cost;
};

struct Pending {
  ItemRec item;
  double cost;
  int32_t order;
};

// Work-groups one CU holds at once for the attention kernel a plan launches,
// from the compiled kernels' register counts (VGPRs per wavefront, allocated in
// granules of 8 from 512 per SIMD lane; the LDS never binds first):
//   with matrix-core items, D = 128:        223-240 VGPRs -> 2
//                           D = 64, B = 64: 172-174       -> 2
//                           D = 64, B < 64: 164-166       -> 3
//   decode-only kernel,     D = 128:        153-164       -> 3
//                           D = 64:         116-127       -> 4
// Only the dispatch order depends on these; tests/test_gpu_occupancy.py checks
// them against the HIP occupancy calculator for every (D, B, kernel) pair.
int resident_slots_per_cu(bool mfma, int D, int B) {
  if (mfma) return (D == 64 && B < 64) ? 3 : kMfmaSlotsPerCu;
  return D == 64 ? 4 : 3;
}

// The first launch rounds are resident together: MI355X's dispatcher hands
// work-group p of a fresh launch to CU (p mod C) in round p / C (it deals
// them round-robin over the XCDs and, within each, one per CU before a
// second; per-work-group HW_ID readings showed positions p, p + C and p + 2C on
// one CU for every position).  Work-groups on one CU share its matrix cores,
// and a CU of the decode-only kernel streams about the same total (28-29 GB/s
// at full load) whether it holds two or three work-groups, so a CU finishes
// roughly with the sum of its items' costs.  Longest-first order would put
// the longest item of every round on the same CUs; instead the first
// C * slots items are dealt costliest-first onto the least-loaded CU with a
// free slot (greedy multiway partition) and written back at positions
// cu + round * C, CUs holding more items first.  Items after those rounds
// keep their order and fill whichever CU frees a slot first.  Only speed
// depends on this.
void place_resident_rounds(std::vector<Pending>& list, int cus, int slots) {
  const size_t c = size_t(cus), k = size_t(slots);
  const size_t m = std::min(list.size(), c * k);
  if (m <= c) return;
  std::vector<double> cost(m);
  for (size_t i = 0; i < m; ++i) cost[i] = list[i].cost;
  std::vector<uint32_t> idx(m);
  std::iota(idx.begin(), idx.end(), 0u);
  std::sort(idx.begin(), idx.end(),
            [&](uint32_t x, uint32_t y) { return cost[x] != cost[y] ? cost[x] > cost[y] : x < y; });
  // The costliest c items open one bin each; the rest go, costliest first,
  // to the least-loaded bin with a free slot (ties: lower bin).  Bin u's
  // items are bin_item[u * k .. u * k + count[u]).
  std::vector<uint32_t> bin_item(c * k);
  std::vector<uint32_t> count(c, 1);
  using Entry = std::pair<double, uint32_t>;
  std::vector<Entry> heap(c);
  for (size_t u = 0; u < c; ++u) {
    bin_item[u * k] = idx[u];
    heap[u] = {cost[idx[u]], uint32_t(u)};
  }
  auto cmp = [](const Entry& x, const Entry& y) {
    return x.first != y.first ? x.first > y.first : x.second > y.second;
  };
  std::make_heap(heap.begin(), heap.end(), cmp);
  for (size_t i = c; i < m; ++i) {
    std::pop_heap(heap.begin(), heap.end(), cmp);
    const Entry e = heap.back();
    heap.pop_back();
    const uint32_t u = e.second;
    bin_item[u * k + count[u]++] = idx[i];
    if (count[u] < k) {
      heap.push_back({e.first + cost[idx[i]], u});
      std::push_heap(heap.begin(), heap.end(), cmp);
    }
  }
  // Round r takes the r-th item of every bin holding more than r items; bins
  // are ordered by item count (then bin index), so those bins come first in
  // every round and the j-th bin of that order has its items at positions j,
  // j + c, j + 2c, ...
  std::vector<uint32_t> order;
  order.reserve(c);
  for (size_t n = k; n >= 1; --n)
    for (size_t u = 0; u < c; ++u)
      if (count[u] == n) order.push_back(uint32_t(u));
  std::vector<Pending> placed;
  placed.reserve(m);
  for (size_t r = 0; r < k; ++r)
    for (size_t j = 0; j < c && count[order[j]] > r; ++j) placed.push_back(list[bin_item[order[j] * k + r]]);
  std::copy(placed.begin(), placed.end(), list.begin());
}

fg_status validate(const fg_pass_desc* d) {
  if (d->num_seqs < 0) return FG_E_INVALID;
  if (d->num_q_heads < 1 || d->num_kv_heads < 1) return FG_E_INVALID;
  if (d->num_q_heads % d->num_kv_heads != 0) return FG_E_INVALID;
  if (d->head_dim != 64 && d->head_dim != 128) return FG_E_UNSUPPORTED;
  if (d->block_size != 16 && d->block_size != 32 && d->block_size != 64) return FG_E_UNSUPPORTED;
  if (d->num_blocks < 1 || d->max_blocks_per_seq < 0) return FG_E_INVALID;
  if (!isfinite(d->scale) || d->scale < 0.f) return FG_E_INVALID;
  if (d->target_cus < 0 || d->min_split_tokens < 0) return FG_E_INVALID;
  if (d->max_splits < 0 || d->max_splits > kMaxSplitsLimit) return FG_E_INVALID;
  if (d->force_splits < 0 || d->force_splits > kMaxSplitsLimit) return FG_E_INVALID;
  if (d->split_policy < FG_SPLIT_BALANCED || d->split_policy > FG_SPLIT_PER_1K) return FG_E_INVALID;
  if (d->num_seqs > 0 && (!d->q_lens || !d->ctx_lens || !d->block_tables)) return FG_E_INVALID;
  return FG_OK;
}

}  // namespace

extern "C" fg_status fg_plan_pass(const fg_pass_desc* d, fg_plan** out_plan) {
  if (!d || !out_plan) return FG_E_INVALID;
  *out_plan = nullptr;
  fg_status st = validate(d);
  if (st != FG_OK) return st;

  try {
    const int S = d->num_seqs;
    const int B = d->block_size;
    const int D = d->head_dim;
    const int G = d->num_q_heads / d->num_kv_heads;
    const int MB = d->max_blocks_per_seq;

    // ---- per-sequence records and block-table validation
    std::vector<SeqRec> seqs(S);
    int64_t tokens = 0, used_blocks = 0;
    for (int s = 0; s < S; ++s) {
      const int64_t q = d->q_lens[s], c = d->ctx_lens[s];
      if (q < 1 || c < 0) return FG_E_RANGE;
      const int64_t kv = q + c;
      if (kv > kMaxKvLen) return FG_E_RANGE;
      const int64_t nblk = ceil_div(kv, B);
      if (nblk > MB) return FG_E_RANGE;
      SeqRec& r = seqs[s];
      r.q_start = int32_t(tokens);
      r.q_len = int32_t(q);
      r.ctx = int32_t(c);
      r.kv_len = int32_t(kv);
      r.bt_off = int32_t(used_blocks);
      r.nblk = int32_t(nblk);
      r.pad0 = r.pad1 = 0;
      tokens += q;
      used_blocks += nblk;
      if (tokens > kMaxTokens) return FG_E_RANGE;
    }
    // Packed rows per (sequence, kv head) and the row-group count, in 64-bit
    // arithmetic, before any vector is sized by them.
    int64_t group_count = 0;
    for (int s = 0; s < S; ++s) {
      const int64_t rows = int64_t(seqs[s].q_len) * G;
      if (rows > kMaxPackedRows) return FG_E_RANGE;
      const int64_t per_head = rows <= fg::kValuMaxRows ? 1 : ceil_div(rows, fg::kMfmaTileRows);
      group_count += per_head * d->num_kv_heads;
      if (group_count > kMaxGroupsPerLaunch) return FG_E_RANGE;
    }
    std::vector<int32_t> bt(static_cast<size_t>(used_blocks));
    std::vector<uint8_t> seen(size_t(d->num_blocks), 0);
    for (int s = 0; s < S; ++s) {
      const int32_t* row = d->block_tables + int64_t(s) * MB;
      for (int b = 0; b < seqs[s].nblk; ++b) {
        const int32_t id = row[b];
        if (id < 0 || id >= d->num_blocks) return FG_E_RANGE;
        if (seen[id]) return FG_E_ALIAS;
        seen[id] = 1;
        bt[size_t(seqs[s].bt_off) + b] = id;
      }
    }

    int target_cus = d->target_cus;
    if (target_cus == 0) {
      target_cus = fg_internal_device_cu_count();
      if (target_cus < 1) return FG_E_HIP;
    }
    const int min_split = d->min_split_tokens ? d->min_split_tokens : kDefaultMinSplitTokens;
    const int max_splits = d->max_splits ? d->max_splits : kDefaultMaxSplits;

    // ---- append runs: consecutive new tokens of a sequence within one block
    std::vector<RunRec> runs;
    runs.reserve(size_t(used_blocks));
    for (int s = 0; s < S; ++s) {
      const SeqRec& r = seqs[s];
      int64_t p = r.ctx;
      while (p < r.kv_len) {
        const int64_t bi = p / B;
        const int64_t end = std::min<int64_t>(r.kv_len, (bi + 1) * B);
        RunRec run;
        run.tok0 = int32_t(r.q_start + (p - r.ctx));
        run.slot0 = int32_t(p % B);
        run.count = int32_t(end - p);
        run.block = bt[size_t(r.bt_off + bi)];
        runs.push_back(run);
        p = end;
      }
    }
    if (int64_t(runs.size()) * d->num_kv_heads > kMaxGroupsPerLaunch) return FG_E_RANGE;

    // ---- row groups and their costs (KV tokens visible to the group: a
    // decode group streams them from HBM, a full 128-row tile spends about the
    // same time on matrix-core work per token at the MI355X flop:byte ratio)
    std::vector<Group> groups;
    groups.reserve(size_t(group_count));
    double total_cost = 0.0;
    for (int s = 0; s < S; ++s) {
      const SeqRec& r = seqs[s];
      const int rows = int(int64_t(r.q_len) * G);   // <= kMaxPackedRows, checked above
      for (int g = 0; g < d->num_kv_heads; ++g) {
        if (rows <= fg::kValuMaxRows) {
          Group grp{s, g, 0, rows, r.kv_len, 0, double(r.kv_len)};
          groups.push_back(grp);
          total_cost += grp.cost;
        } else {
          for (int r0 = 0; r0 < rows; r0 += fg::kMfmaTileRows) {
            const int nr = std::min(fg::kMfmaTileRows, rows - r0);
            const int j_last = (r0 + nr - 1) / G;
            const int vis = r.ctx + j_last + 1;
            const int waves = (nr + fg::kMfmaRowsPerWave - 1) / fg::kMfmaRowsPerWave;
            const double per_tok =
                std::max(kMfmaMinCost, double(waves * fg::kMfmaRowsPerWave) / kFlopPerByte);
            Group grp{s, g, r0, nr, vis, waves, per_tok * double(vis)};
            groups.push_back(grp);
            total_cost += grp.cost;
          }
        }
      }
    }

    // ---- per-sequence split counts of the pages' policies (FG_SPLIT_ENGINE,
    // FG_SPLIT_PER_1K; see fg.h), as per-sequence formulas of the KV length:
    //   engine:  b_s = clamp(L_s / m, 1, 16), B = sum b_s over the pass;
    //            k_s = 1 if S >= N, else max(1, b_s * N / B) if B < N, else b_s
    //   per 1k:  k_s = clamp(L_s / 1024, 1, 16)
    // (N = target_cus, m = min_split_tokens or 256; integer floors throughout)
    std::vector<int64_t> seq_splits(size_t(S), 1);
    if (d->split_policy == FG_SPLIT_ENGINE) {
      const int64_t m = d->min_split_tokens > 0 ? d->min_split_tokens : kDefaultMinSplitTokens;
      int64_t base_sum = 0;
      for (int s = 0; s < S; ++s) {
        seq_splits[size_t(s)] = std::clamp<int64_t>(seqs[s].kv_len / m, 1, 16);
        base_sum += seq_splits[size_t(s)];
      }
      const int64_t n_cus = target_cus;
      for (int64_t& k : seq_splits)
        k = S >= n_cus ? 1 : base_sum < n_cus ? std::max<int64_t>(1, k * n_cus / base_sum) : k;
    } else if (d->split_policy == FG_SPLIT_PER_1K) {
      for (int s = 0; s < S; ++s) seq_splits[size_t(s)] = std::clamp<int64_t>(seqs[s].kv_len / 1024, 1, 16);
    }

    // ---- split each group's visible range [0, vis_end)
    int64_t tile_groups = 0, valu_groups = 0;
    double tile_cost = 0.0;
    for (const Group& grp : groups) {
      if (grp.waves == 0) ++valu_groups;
      if (grp.waves >= 2) {
        ++tile_groups;
        tile_cost += grp.cost;
      }
    }
    const double items_per_cu = valu_groups == 0 ? kMfmaOnlyItemsPerCu : kItemsPerCu;
    // A pass of vector-ALU groups only, with at least kSkewedItemsPerSlot of
    // them per work-group slot, halves the split target (see kSkewedSplitFactor).
    const bool many_valu_groups =
        tile_groups == 0 &&
        double(groups.size()) >= kSkewedItemsPerSlot * double(target_cus) * kMfmaSlotsPerCu;
    const double target = std::max(
        1.0, total_cost / (double(target_cus) * items_per_cu * (many_valu_groups ? kSkewedSplitFactor : 1.0)));
    const double tile_target =
        tile_groups >= target_cus
            ? 1e300
            : std::max(1.0, tile_cost / (double(target_cus) * kMfmaSlotsPerCu));
    std::vector<Pending> mfma, valu;
    std::vector<MergeRec> merges, late_merges;
    int64_t partial_rows = 0;
    int max_used = 1;
    int32_t order = 0;
    // Split count and chunk of every group first: whether split groups may
    // merge inside the attention launch depends on the plan's item count.
    std::vector<int64_t> gk(groups.size()), gchunk(groups.size());
    auto split_all = [&](double valu_target) {
      int64_t items = 0;
      for (size_t gi = 0; gi < groups.size(); ++gi) {
        const Group& grp = groups[gi];
        int64_t k;
        if (d->force_splits > 0) {
          k = d->force_splits;
        } else if (d->split_policy != FG_SPLIT_BALANCED) {
          k = std::min<int64_t>(seq_splits[size_t(grp.seq)], max_splits);
        } else {
          k = int64_t(ceil(grp.cost / (grp.waves >= 2 ? tile_target : valu_target)));
          k = std::min<int64_t>(k, max_splits);
          const int floor_tokens =
              grp.waves >= 2 ? std::max(min_split, kMfmaMinSplitTokens) : min_split;
          k = std::min<int64_t>(k, std::max<int64_t>(1, grp.vis_end / std::max(1, floor_tokens)));
        }
        k = std::max<int64_t>(1, std::min<int64_t>(k, ceil_div(grp.vis_end, fg::kKvTile)));
        const int64_t chunk = ceil_div(ceil_div(grp.vis_end, k), fg::kKvTile) * fg::kKvTile;
        gk[gi] = ceil_div(grp.vis_end, chunk);
        gchunk[gi] = chunk;
        items += gk[gi];
      }
      return items;
    };
    int64_t total_items = split_all(target);
    if (total_items > kMaxGroupsPerLaunch ||
        total_items + int64_t(runs.size()) * d->num_kv_heads > kMaxGroupsPerLaunch)
      return FG_E_RANGE;   // attention items, and attention items + fused append groups
    // Round fitting (see kRoundFitSlack): a tile-free plan just past a whole
    // number of work-group rounds gets a larger target until it fits them.
    if (d->force_splits == 0 && d->split_policy == FG_SPLIT_BALANCED && tile_groups == 0) {
      const int64_t slots = int64_t(target_cus) * kMfmaSlotsPerCu;
      double valu_target = target;
      for (int pass = 0; pass < kRoundFitPasses; ++pass) {
        const int64_t rounds = total_items / slots;
        const int64_t excess = total_items - rounds * slots;
        if (rounds < 1 || excess == 0 || double(excess) > kRoundFitSlack * double(slots)) break;
        valu_target *= double(total_items) / double(rounds * slots);
        total_items = split_all(valu_target);   // a larger target: never more items
      }
    }
    const bool inlaunch_ok =
        total_items <= int64_t(kInLaunchMaxItemsPerSlot) * target_cus *
                           resident_slots_per_cu(valu_groups < int64_t(groups.size()), D, B);
    {
      int64_t n_mfma_items = 0;
      for (size_t gi = 0; gi < groups.size(); ++gi)
        if (groups[gi].waves) n_mfma_items += gk[gi];
      mfma.reserve(size_t(n_mfma_items));
      valu.reserve(size_t(total_items - n_mfma_items));
    }
    for (size_t gi = 0; gi < groups.size(); ++gi) {
      const Group& grp = groups[gi];
      const int64_t k = gk[gi], chunk = gchunk[gi];
      max_used = std::max<int>(max_used, int(k));
      int32_t slot0 = -1;
      // Split groups of at most one wavefront's rows merge inside the
      // attention launch when the plan has few items per slot (group index
      // >= 0 here); split tiles, and every group of a plan with many items per
      // slot, are merged by a merge launch (encoded -2 - index until the two
      // lists are joined).
      int32_t group = -1;
      if (k > 1) {
        if (partial_rows + k * grp.nrows > INT32_MAX) return FG_E_RANGE;
        slot0 = int32_t(partial_rows);
        partial_rows += k * grp.nrows;
        MergeRec m;
        m.seq = grp.seq;
        m.kv_head = grp.kv_head;
        m.row0 = grp.row0;
        m.nrows = grp.nrows;
        m.nsplit = int32_t(k);
        m.slot0 = slot0;
        m.pad0 = m.pad1 = 0;
        if (grp.waves <= 1 && inlaunch_ok) {
          group = int32_t(merges.size());
          merges.push_back(m);
        } else {
          group = -2 - int32_t(late_merges.size());
          late_merges.push_back(m);
        }
      }
      for (int64_t i = 0; i < k; ++i) {
        Pending p;
        p.item.seq = grp.seq;
        p.item.kv_head = grp.kv_head;
        p.item.row0 = grp.row0;
        p.item.nrows = grp.nrows;
        p.item.kv0 = int32_t(i * chunk);
        p.item.kv1 = int32_t(std::min<int64_t>(grp.vis_end, (i + 1) * chunk));
        p.item.slot = k > 1 ? int32_t(slot0 + i * grp.nrows) : -1;
        p.item.waves = grp.waves;
        p.item.group = group;
        p.item.pad0 = p.item.pad1 = p.item.pad2 = 0;
        p.cost = double(p.item.kv1 - p.item.kv0) * (grp.cost / double(grp.vis_end));
        p.order = order++;
        (grp.waves ? mfma : valu).push_back(p);
      }
    }

    // In-launch groups first, then the merge launch's; remap the items.
    const int32_t n_inl = int32_t(merges.size());
    auto remap = [n_inl](std::vector<Pending>& v) {
      for (Pending& p : v)
        if (p.item.group <= -2) p.item.group = n_inl + (-2 - p.item.group);
    };
    remap(mfma);
    remap(valu);
    merges.insert(merges.end(), late_merges.begin(), late_merges.end());

    // Longest first within each kind (ties keep plan order: deterministic).
    auto longest_first = [](const Pending& a, const Pending& b) {
      if (a.cost != b.cost) return a.cost > b.cost;
      return a.order < b.order;
    };
    std::sort(mfma.begin(), mfma.end(), longest_first);
    std::sort(valu.begin(), valu.end(), longest_first);

    // ---- pack the metadata blob
    fg_plan* plan = new fg_plan();
    plan->num_seqs = S;
    plan->num_tokens = int32_t(tokens);
    plan->hq = d->num_q_heads;
    plan->hkv = d->num_kv_heads;
    plan->group = G;
    plan->head_dim = D;
    plan->block_size = B;
    plan->num_blocks = d->num_blocks;
    plan->scale = d->scale > 0.f ? d->scale : float(1.0 / sqrt(double(D)));
    plan->n_runs = int32_t(runs.size());
    plan->n_mfma = int32_t(mfma.size());
    plan->n_valu = int32_t(valu.size());
    plan->n_tiles = int32_t(std::count_if(mfma.begin(), mfma.end(),
                                          [](const Pending& x) { return x.item.waves >= 2; }));
    plan->n_items = plan->n_mfma + plan->n_valu;
    plan->n_merge_groups = int32_t(merges.size());
    plan->n_inlaunch_groups = n_inl;
    plan->n_partial_rows = int32_t(partial_rows);
    plan->max_splits_used = max_used;
    plan->target_cus = target_cus;

    size_t off = 0;
    plan->off_seqs = off;   off = align16(off + sizeof(SeqRec) * seqs.size());
    plan->off_bt = off;     off = align16(off + sizeof(int32_t) * bt.size());
    plan->off_runs = off;   off = align16(off + sizeof(RunRec) * runs.size());
    plan->off_items = off;  off = align16(off + sizeof(ItemRec) * size_t(plan->n_items));
    plan->off_merges = off; off = align16(off + sizeof(MergeRec) * merges.size());
    plan->off_counters = off; off = align16(off + sizeof(int32_t) * size_t(n_inl));
    // the fused upload + append launch: metadata-copy groups of 4 KiB each
    // beside the (run, kv head) groups
    if (int64_t(ceil_div(int64_t(off), 4096)) + int64_t(runs.size()) * d->num_kv_heads >
        kMaxGroupsPerLaunch) {
      delete plan;
      return FG_E_RANGE;
    }
    plan->blob.assign(std::max<size_t>(off, 16), 0);
    uint8_t* base = plan->blob.data();
    if (!seqs.empty()) memcpy(base + plan->off_seqs, seqs.data(), sizeof(SeqRec) * seqs.size());
    if (!bt.empty()) memcpy(base + plan->off_bt, bt.data(), sizeof(int32_t) * bt.size());
    if (!runs.empty()) memcpy(base + plan->off_runs, runs.data(), sizeof(RunRec) * runs.size());
    ItemRec* items = reinterpret_cast<ItemRec*>(base + plan->off_items);
    {
      // Dispatch order: the two item kinds (compute-bound tiles, bandwidth-
      // bound decode rows) are spread evenly over the order, each kind
      // longest-first, so a CU holds a mix of both rather than a round of
      // tiles followed by a round of decodes.
      std::vector<Pending> order_list;
      order_list.reserve(mfma.size() + valu.size());
      size_t a = 0, b = 0;
      const double na = double(mfma.size()), nb = double(valu.size());
      while (a < mfma.size() || b < valu.size()) {
        const bool take_a = b >= valu.size() ||
                            (a < mfma.size() && (double(a) + 0.5) / na <= (double(b) + 0.5) / nb);
        order_list.push_back(take_a ? mfma[a++] : valu[b++]);
      }
      const int slots = resident_slots_per_cu(!mfma.empty(), D, B);
      plan->resident_slots = slots;
      place_resident_rounds(order_list, target_cus, slots);
      for (size_t o = 0; o < order_list.size(); ++o) items[o] = order_list[o].item;
    }
    if (!merges.empty())
      memcpy(base + plan->off_merges, merges.data(), sizeof(MergeRec) * merges.size());

    plan->ws_o_off = 0;
    plan->ws_lse_off = (size_t(partial_rows) * D * sizeof(float) + 255) & ~size_t(255);
    plan->ws_bytes = partial_rows ? plan->ws_lse_off + size_t(partial_rows) * sizeof(float) : 0;
    *out_plan = plan;
    return FG_OK;
  } catch (const std::bad_alloc&) {
    return FG_E_NOMEM;
  } catch (...) {
    return FG_E_INVALID;
  }
}

extern "C" fg_status fg_plan_info(const fg_plan* p, fg_plan_info_t* o) {
  if (!p || !o) return FG_E_INVALID;
  memset(o, 0, sizeof(*o));
  o->num_tokens = p->num_tokens;
  o->metadata_bytes = int64_t(p->blob.size());
  o->workspace_bytes = int64_t(p->ws_bytes);
  o->num_items = p->n_items;
  o->num_valu_items = p->n_valu;
  o->num_mfma_items = p->n_mfma;
  o->num_merge_groups = p->n_merge_groups;
  o->num_inlaunch_merge_groups = p->n_inlaunch_groups;
  o->num_partial_rows = p->n_partial_rows;
  o->max_splits_used = p->max_splits_used;
  o->num_append_runs = p->n_runs;
  o->target_cus = p->target_cus;
  return FG_OK;
}

extern "C" fg_status fg_plan_metadata(const fg_plan* p, void* host_dst, size_t bytes,
                                      fg_plan_layout_t* layout) {
  if (!p) return FG_E_INVALID;
  if (host_dst) {
    if (bytes < p->blob.size()) return FG_E_INVALID;
    memcpy(host_dst, p->blob.data(), p->blob.size());
  }
  if (layout) {
    memset(layout, 0, sizeof(*layout));
    layout->seqs = int64_t(p->off_seqs);
    layout->block_ids = int64_t(p->off_bt);
    layout->runs = int64_t(p->off_runs);
    layout->items = int64_t(p->off_items);
    layout->merges = int64_t(p->off_merges);
    layout->counters = int64_t(p->off_counters);
    layout->num_seqs = p->num_seqs;
    layout->num_block_ids = int32_t((p->off_runs - p->off_bt) / sizeof(int32_t));
    layout->num_runs = p->n_runs;
    layout->num_items = p->n_items;
    layout->num_merges = p->n_merge_groups;
    layout->num_counters = p->n_inlaunch_groups;
  }
  return FG_OK;
}

extern "C" void fg_plan_destroy(fg_plan* p) { delete p; }

extern "C" const char* fg_status_string(fg_status s) {
  switch (s) {
    case FG_OK: return "ok";
    case FG_E_INVALID: return "invalid argument";
    case FG_E_RANGE: return "value out of range";
    case FG_E_ALIAS: return "physical block used twice in one pass";
    case FG_E_UNSUPPORTED: return "unsupported head_dim, block_size or dtype";
    case FG_E_WORKSPACE: return "workspace too small or misaligned";
    case FG_E_HIP: return "HIP runtime error";
    case FG_E_NOMEM: return "host allocation failed";
    default: return "unknown status";
  }
}

extern "C" int32_t fg_abi_version(void) { return FG_ABI_VERSION; }
