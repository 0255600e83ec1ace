// Host-only fuzz driver for the planner's C ABI (fg_plan_pass, fg_plan_info,
// fg_plan_metadata, fg_plan_destroy), built with AddressSanitizer and UBSan by
// tests/test_planner_fuzz.py.  Random pass descriptions, valid and invalid:
// the planner must return a status for each and never read or write out of
// bounds.  Accepted plans are checked for basic consistency.
//   planner_fuzz SEED ITERATIONS
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "fg.h"

// The library's device query, stood in for on the host: target_cus = 0 asks
// the planner to balance over this many compute units.
extern "C" int fg_internal_device_cu_count(void) { return 256; }

static int fail(const char* what, unsigned seed, int it) {
  std::fprintf(stderr, "FAIL %s (seed %u, iteration %d)\n", what, seed, it);
  return 1;
}

int main(int argc, char** argv) {
  const unsigned seed = argc > 1 ? unsigned(std::strtoul(argv[1], nullptr, 10)) : 1u;
  const int iters = argc > 2 ? std::atoi(argv[2]) : 1000;
  std::mt19937 rng(seed);
  auto uni = [&](int lo, int hi) { return int(std::uniform_int_distribution<int>(lo, hi)(rng)); };
  auto chance = [&](int pct) { return uni(0, 99) < pct; };
  static const int kLayouts[][2] = {{4, 4}, {8, 2}, {16, 2}, {32, 32}, {8, 1}, {12, 4}, {0, 1}, {6, 4}};
  int ok = 0, rejected = 0, huge_ok = 0, huge_range = 0;
  for (int it = 0; it < iters; ++it) {
    // One description in 16 is "huge": few sequences, 64 to 65536 query heads
    // per kv head (1-4 kv heads) and chunks up to 66536 tokens, so packed rows
    // (q_len * G) and work-group counts cross the planner's int32 and launch
    // limits.  Those must be rejected with FG_E_RANGE, or accepted with a
    // consistent plan; nothing may overflow on the way.
    const bool huge = chance(6);
    const bool bad = !huge && chance(50);  // allow invalid fields in this description
    auto flaw = [&](int pct) { return bad && chance(pct); };
    const int S = huge ? uni(1, 3) : (flaw(5) ? uni(-2, 0) : uni(1, 70));
    const int n = S > 0 ? S : 0;
    std::vector<int32_t> q(n), c(n);
    for (int s = 0; s < n; ++s) {
      q[s] = chance(50) ? 1 : uni(2, chance(10) ? 5000 : 300);
      c[s] = chance(15) ? 0 : uni(1, chance(10) ? 60000 : 4000);
      if (huge) q[s] = chance(30) ? 1 : (1 << uni(1, 16)) + uni(0, 1000);
      if (flaw(2)) q[s] = uni(-3, 0);
      if (flaw(2)) c[s] = -uni(1, 5);
    }
    const int li = flaw(8) ? uni(6, 7) : uni(0, 5);  // the last two are invalid
    const int huge_kv = uni(1, 4);
    // half the huge draws are meant to cross the limits: G = 65536 with a chunk
    // of at least 32768 tokens (2^31 packed rows or more)
    const bool past = huge && chance(50);
    const int huge_q = huge_kv * (1 << (past ? 16 : uni(6, 16)));   // G = 64 .. 65536
    if (past) {
      for (int s = 0; s < n; ++s) q[s] = 1;
      q[uni(0, n - 1)] = uni(32768, 65536);
    }
    const int D = flaw(4) ? 96 : (chance(50) ? 64 : 128);
    const int B = flaw(4) ? 8 : (16 << uni(0, 2));
    int maxb = 1;
    std::vector<int> nb(n);
    int64_t total = 0;
    for (int s = 0; s < n; ++s) {
      const int64_t L = int64_t(q[s] > 0 ? q[s] : 0) + (c[s] > 0 ? c[s] : 0);
      nb[s] = int((L + B - 1) / B);
      if (nb[s] > maxb) maxb = nb[s];
      total += nb[s];
    }
    maxb += uni(0, 3);
    if (total > 4000000) continue;
    if (huge) {
      // Keep huge descriptions either over a limit (packed rows past int32,
      // or more row groups than one launch holds) or cheap to plan under the
      // sanitizers (under 2^18 row groups); the band between is skipped.
      int64_t groups = 0;
      bool over = false;
      for (int s = 0; s < n; ++s) {
        const int64_t rows = int64_t(q[s]) * (huge_q / huge_kv);
        over = over || rows > INT32_MAX;
        groups += (rows <= 4 ? 1 : (rows + 127) / 128) * huge_kv;
      }
      over = over || groups >= (int64_t(1) << 24);
      if (!over && groups >= (int64_t(1) << 18)) continue;
    }
    std::vector<int32_t> bt(size_t(n) * maxb, -1);
    std::vector<int32_t> perm(static_cast<size_t>(total));
    for (int64_t i = 0; i < total; ++i) perm[size_t(i)] = int32_t(i);
    std::shuffle(perm.begin(), perm.end(), rng);
    int64_t next = 0;
    for (int s = 0; s < n; ++s)
      for (int b = 0; b < nb[s]; ++b) bt[size_t(s) * maxb + b] = perm[size_t(next++)];
    if (n > 0 && flaw(5)) bt[size_t(uni(0, n - 1)) * maxb + uni(0, maxb - 1)] = uni(-5, int(total) + 5);
    int32_t num_blocks = int32_t(total) + uni(0, 10);
    if (flaw(3)) num_blocks = uni(0, int(total));

    fg_pass_desc d{};
    d.num_seqs = S;
    d.num_q_heads = huge ? huge_q : kLayouts[li][0];
    d.num_kv_heads = huge ? huge_kv : kLayouts[li][1];
    d.head_dim = D;
    d.block_size = B;
    d.num_blocks = num_blocks;
    d.max_blocks_per_seq = flaw(3) ? 0 : maxb;
    d.scale = chance(10) ? 0.1f : 0.f;
    d.q_lens = flaw(2) ? nullptr : q.data();
    d.ctx_lens = c.data();
    d.block_tables = flaw(2) ? nullptr : bt.data();
    d.target_cus = chance(5) ? 0 : uni(flaw(10) ? -2 : 1, chance(5) ? 4096 : 304);
    d.min_split_tokens = chance(20) ? uni(flaw(20) ? -1 : 0, 2048) : 0;
    d.max_splits = chance(20) ? uni(flaw(20) ? -1 : 0, flaw(20) ? 300 : 256) : 0;
    d.force_splits = chance(15) ? uni(flaw(20) ? -1 : 0, 80) : 0;
    if (huge) d.force_splits = chance(30) ? uni(1, 16) : 0;
    d.split_policy = chance(80) ? 0 : uni(flaw(20) ? -1 : 0, flaw(20) ? 4 : 2);

    fg_plan* plan = nullptr;
    const fg_status st = fg_plan_pass(&d, &plan);
    if (st != FG_OK) {
      if (plan != nullptr) return fail("error status with a plan", seed, it);
      if (huge) {
        if (st != FG_E_RANGE) {
          std::fprintf(stderr, "status %d: %s\n", int(st), fg_status_string(st));
          return fail("huge description rejected with a status other than FG_E_RANGE", seed, it);
        }
        ++huge_range;
        continue;
      }
      if (!bad) {
        std::fprintf(stderr, "status %d: %s\n", int(st), fg_status_string(st));
        return fail("valid description rejected", seed, it);
      }
      ++rejected;
      continue;
    }
    if (plan == nullptr) return fail("FG_OK without a plan", seed, it);
    fg_plan_info_t info{};
    if (fg_plan_info(plan, &info) != FG_OK) return fail("fg_plan_info", seed, it);
    int64_t tokens = 0;
    for (int s = 0; s < n; ++s) tokens += q[s];
    if (info.num_tokens != tokens) return fail("num_tokens", seed, it);
    if (info.num_items != info.num_valu_items + info.num_mfma_items) return fail("item counts", seed, it);
    if (info.metadata_bytes < 0 || info.workspace_bytes < 0) return fail("sizes", seed, it);
    if (info.max_splits_used > 256) return fail("split cap", seed, it);
    if (info.num_items < 0 || info.num_items >= (1 << 24) || info.num_partial_rows < 0 ||
        info.num_merge_groups < 0 || info.num_merge_groups > info.num_items)
      return fail("counts outside the launch limits", seed, it);
    std::vector<unsigned char> meta(size_t(info.metadata_bytes) + 1);
    fg_plan_layout_t lay{};
    if (fg_plan_metadata(plan, meta.data(), size_t(info.metadata_bytes), &lay) != FG_OK)
      return fail("fg_plan_metadata", seed, it);
    if (lay.num_items != info.num_items || lay.num_seqs != S) return fail("layout counts", seed, it);
    {
      // every item record: rows and KV range inside the sequence's own
      const int32_t* seqw = reinterpret_cast<const int32_t*>(meta.data() + lay.seqs);
      const int32_t* itw = reinterpret_cast<const int32_t*>(meta.data() + lay.items);
      const int64_t G = d.num_q_heads / d.num_kv_heads;
      for (int i = 0; i < lay.num_items; ++i) {
        const int32_t* r = itw + 12 * i;
        if (r[0] < 0 || r[0] >= S || r[1] < 0 || r[1] >= d.num_kv_heads) return fail("item seq/head", seed, it);
        const int32_t* sq = seqw + 8 * r[0];
        if (r[2] < 0 || r[3] < 1 || int64_t(r[2]) + r[3] > int64_t(sq[1]) * G) return fail("item rows", seed, it);
        if (r[4] < 0 || r[5] <= r[4] || r[5] > sq[3]) return fail("item kv range", seed, it);
      }
    }
    if (huge) ++huge_ok;
    if (info.metadata_bytes > 0 && fg_plan_metadata(plan, meta.data(), size_t(info.metadata_bytes) - 1, &lay) == FG_OK)
      return fail("short metadata buffer accepted", seed, it);
    fg_plan_destroy(plan);
    ++ok;
  }
  std::printf("planner fuzz seed %u: %d plans accepted, %d rejected; huge: %d accepted, %d out of range\n",
              seed, ok, rejected, huge_ok, huge_range);
  // every kind must occur, or the run did not exercise what it is for
  return ok > 0 && rejected > 0 && huge_ok > 0 && huge_range > 0 ? 0 : 1;
}
