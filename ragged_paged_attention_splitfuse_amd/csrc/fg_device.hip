// fg_device.hip -- gfx950 kernels of one ragged paged attention pass and the
// C-ABI entry points that launch them.
//
// Kernels
//   append_kernel   one work-group per (append run, kv head): copies the new K
//                   rows into their block (slot-major) and writes the new V
//                   rows transposed into the block's [B/S][D][S] layout,
//                   S = min(B, 32) (8x8 tiles transposed in registers, 16-byte
//                   stores).
//   attn_kernel     one work-group per work item.  Items with many query rows
//                   (prompt-chunk tiles, GQA groups) take the matrix-core path:
//                   K/V stages of 64 tokens staged in LDS, S^T = K Q^T and
//                   O^T = V^T P^T on v_mfma_f32_32x32x16_bf16, online softmax in
//                   fp32 with one query row per lane.  Items with at most four
//                   rows (decodes) take the vector-ALU path: every wavefront
//                   streams its own 32- or 64-token steps with 16-byte loads,
//                   dot products on v_dot2_f32_bf16 with DPP row reductions, and
//                   the four wavefronts merge by log-sum-exp at the end.
//                   An item that is one split of a longer KV range writes its
//                   partial rows to the workspace and counts itself in on its
//                   split group's counter; the work-group that completes the
//                   count merges the group by log-sum-exp ("DeepSpeed-FastGen
//                   Guide: Dynamic SplitKV Serving", section "1. Dynamic
//                   SplitKV Attention", two-phase softmax item; the weights are
//                   the partials' log-sum-exp values).  This is done for
//                   groups of up to one wavefront's rows (decodes).
//   merge_kernel    the same merge for split prefill tiles, one work-group per
//                   group, after the attention launch.
//
// Exponentials run base 2 on v_exp_f32 with the softmax scale folded into
// scale * log2(e); log-sum-exp values are returned in natural-log units.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "fg.h"
#include "fg_meta.h"
#include "plan.h"

namespace fg {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
// Reference-max slack of the matrix-core path's online softmax (log2 units).
constexpr float kRescaleSlack = 8.f;

struct AttnArgs {
  const SeqRec* seqs;
  const int32_t* bt;
  const ItemRec* items;
  const MergeRec* groups;   // split groups (in-launch ones first)
  int32_t* counters;        // one arrival counter per in-launch split group
  const uint16_t* q;
  const uint16_t* kpool;
  const uint16_t* vpool;
  // When set, key positions at or past a sequence's cached context (this
  // pass's own tokens) are read from k_new / v_new instead of the pools, so
  // the attention does not depend on the append of the same pass.
  const uint16_t* k_new;
  const uint16_t* v_new;
  // Fused append (fg_pass): work-groups n_items .. n_items + n_runs * hkv - 1
  // of the attention launch append run (i / hkv) for kv head (i % hkv).
  const RunRec* runs;
  uint16_t* kpool_w;
  uint16_t* vpool_w;
  int32_t n_items;
  void* out;
  float* lse;
  float* ws_o;
  float* ws_lse;
  int32_t hq, hkv, group, n_mfma;
  int32_t n_inlaunch;       // split groups merged inside the attention launch
  float scale_log2;  // softmax scale * log2(e)
  int32_t out_bf16;
};

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
// Non-temporal 16-byte load: the line is streamed rather than kept for reuse.
__device__ __forceinline__ u32x4 ld16_nt(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st16(uint16_t* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Offset of (dim d, slot t) inside one (block, kv head) region of the V pool:
// the block is stored transposed in sub-blocks of S = min(B, 32) slots, each
// [D][S] with the slot index fastest.  Eight slots starting at a multiple of 8
// are always 16 contiguous bytes.
template <int D, int B>
__device__ __forceinline__ int vt_off(int d, int t) {
  constexpr int S = B < 32 ? B : 32;
  return (t / S) * (D * S) + d * S + t % S;
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pick_lo(uint32_t a, uint32_t b) {
  // {a.lo, b.lo} as (low half, high half)
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pick_hi(uint32_t a, uint32_t b) {
  // {a.hi, b.hi}
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of LANES (4, 8 or 16) lanes; every lane of a group
// receives the group's sum.  quad_perm [1,0,3,2], quad_perm [2,3,0,1],
// row_half_mirror, row_mirror.
template <int LANES>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp_f<0xB1>(x);
  x += dpp_f<0x4E>(x);
  if constexpr (LANES >= 8) x += dpp_f<0x141>(x);
  if constexpr (LANES >= 16) x += dpp_f<0x140>(x);
  return x;
}

// Block ids of a work item's KV range, held 64 at a time in one VGPR of each
// wavefront (lane i holds table entry base + i), so that a step or stage picks
// its block with a readlane instead of a dependent memory round trip before
// its K/V loads.  `limit` is the number of used table entries of the sequence;
// lanes past it hold 0 and are never selected.  base and the selected index
// are wavefront-uniform.
struct BlockWindow {
  const int32_t* bt;
  int limit;
  int base;
  int ids;
  __device__ __forceinline__ void load(int first) {
    base = first;
    const int i = first + int(threadIdx.x & 63);
    ids = i < limit ? bt[i] : 0;
  }
  // block id of table entry e (e >= base, uniform)
  __device__ __forceinline__ int get(int e) {
    if (e - base >= 64) load(e);
    return __builtin_amdgcn_readlane(ids, e - base);
  }
};

// Zero the bf16 elements of an 8-token chunk starting at `first` whose token
// index is >= `valid` (slots past the end of a sequence may hold anything).
__device__ __forceinline__ u32x4 zero_tail(u32x4 v, int first, int valid) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int t = first + 2 * e;
    uint32_t w = v[e];
    if (t >= valid) w = 0u;
    else if (t + 1 >= valid) w &= 0x0000ffffu;
    v[e] = w;
  }
  return v;
}

// Row of k_new / v_new holding key position p (>= ctx) of a sequence.
__device__ __forceinline__ size_t new_row(const AttnArgs& a, const SeqRec& sq, int p, int g) {
  return size_t(sq.q_start + (p - sq.ctx)) * a.hkv + g;
}

// Replace the elements of an 8-token chunk of dim d (tokens first .. first+7)
// at positions in [ctx, kv_len) by this pass's new V values.
template <int D>
__device__ __forceinline__ u32x4 patch_new_v(const AttnArgs& a, const SeqRec& sq, u32x4 v, int first,
                                             int d, int g) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int t = first + e;
    if (t >= sq.ctx && t < sq.kv_len) {
      const uint32_t x = a.v_new[new_row(a, sq, t, g) * D + d];
      const uint32_t w = v[e >> 1];
      v[e >> 1] = (e & 1) ? ((w & 0x0000ffffu) | (x << 16)) : ((w & 0xffff0000u) | x);
    }
  }
  return v;
}

// Destination of packed row r of an item: final (token, head) row or a
// partial row of the workspace.
__device__ __forceinline__ void store_result(const AttnArgs& a, const SeqRec& sq, const ItemRec& it,
                                             int D, int r, int d0, const float* vals, int n,
                                             bool write_lse, float lse_val) {
  if (it.slot < 0) {
    const int row = it.row0 + r;
    const int j = row / a.group;
    const int h = it.kv_head * a.group + row % a.group;
    const size_t idx = size_t(sq.q_start + j) * a.hq + h;
    if (a.out_bf16) {
      __bf16* o = reinterpret_cast<__bf16*>(a.out) + idx * D + d0;
      for (int e = 0; e < n; ++e) o[e] = __bf16(vals[e]);
    } else {
      float* o = reinterpret_cast<float*>(a.out) + idx * D + d0;
      for (int e = 0; e < n; ++e) o[e] = vals[e];
    }
    if (write_lse && a.lse) a.lse[idx] = lse_val;
  } else if (it.group < a.n_inlaunch) {
    // Partial rows of an in-launch group are written coherently at device
    // scope (whichever work-group merges the group reads them, on any XCD),
    // so no L2 write-back is needed to publish them.
    float* o = a.ws_o + size_t(it.slot + r) * D + d0;
    for (int e = 0; e < n; ++e) __hip_atomic_store(o + e, vals[e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (write_lse)
      __hip_atomic_store(a.ws_lse + it.slot + r, lse_val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    // merged by the merge launch, which sees them after the kernel boundary
    float* o = a.ws_o + size_t(it.slot + r) * D + d0;
    for (int e = 0; e < n; ++e) o[e] = vals[e];
    if (write_lse) a.ws_lse[it.slot + r] = lse_val;
  }
}

// Read of a partial value: device-coherent for in-launch groups (see the
// partial-row stores above), a plain load in the merge launch.
template <bool COHERENT>
__device__ __forceinline__ float load_partial(const float* p) {
  if constexpr (COHERENT) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else return *p;
}

// ----------------------------------------------------------------------------
// Vector-ALU path: up to NR query rows of one (sequence, kv head) over the
// item's KV range.  Wavefront w handles ST-token steps w, w+4, w+8, ...
// (ST = 32 or 64: one or two 32-token V^T sub-blocks) with its own
// online-softmax state; the four states merge at the end.
// LDS use: per-wave probability exchange, then the cross-wave merge buffers.
template <int D, int B, int NR, int ST, bool DIRECT>
__device__ void valu_item(const AttnArgs& a, const ItemRec& it, float* smem) {
  static_assert(ST % kValuSubTile == 0 && kKvTile % ST == 0, "whole sub-blocks per step");
  constexpr int LPT = D / 8;                // lanes holding one 16-byte-chunked K row
  constexpr int TPI = 64 / LPT;             // tokens per K load instruction
  constexpr int HV = ST / kValuSubTile;     // 32-token V^T sub-blocks per step
  constexpr int UK = ST / TPI;              // K loads per step
  constexpr int UV = D / 16;                // V^T loads per half (16 dims each)
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const SeqRec sq = a.seqs[it.seq];
  const int32_t* bt = a.bt + sq.bt_off;
  const int G = a.group, g = it.kv_head;
  const int kv_valid = sq.kv_len;
  BlockWindow win{bt, sq.nblk, 0, 0};
  if constexpr (B >= ST) win.load((it.kv0 + wave * ST) / B);
  const int ktok = lane / LPT, kdc = lane % LPT;
  const int vd = lane >> 2, vtc = lane & 3;

  u32x4 q[NR];
  int lim[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    if (r < it.nrows) {
      const int row = it.row0 + r, j = row / G, h = g * G + row % G;
      q[r] = ld16(a.q + (size_t(sq.q_start + j) * a.hq + h) * D + 8 * kdc);
      lim[r] = sq.ctx + j;
    } else {
      q[r] = u32x4{0u, 0u, 0u, 0u};
      lim[r] = -1;
    }
  }
  float m[NR], l[NR], acc[NR][UV];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    m[r] = -INFINITY;
    l[r] = 0.f;
#pragma unroll
    for (int i = 0; i < UV; ++i) acc[r][i] = 0.f;
  }
  float* pbuf = smem + wave * (NR * ST);

  // With k_new / v_new (fused pass) the pool stream stops at ctx and this
  // pass's own positions are taken one token at a time after the loop; the
  // wavefront's first such token is loaded here, before the stream, so its
  // latency overlaps the loop (K chunk kdc, and the dims vd + 16 i of V as
  // bf16 pairs).
  const int main_end = DIRECT ? min(kv_valid, sq.ctx) : kv_valid;
  const int p_tail = max(it.kv0, sq.ctx) + wave;
  u32x4 kn_pre = u32x4{0u, 0u, 0u, 0u};
  uint32_t vn_pre[UV / 2];
#pragma unroll
  for (int i = 0; i < UV / 2; ++i) vn_pre[i] = 0u;
  if (DIRECT && p_tail < it.kv1) {
    const size_t nrow = new_row(a, sq, p_tail, g) * D;
    kn_pre = ld16(a.k_new + nrow + 8 * kdc);
#pragma unroll
    for (int i = 0; i < UV / 2; ++i)
      vn_pre[i] = uint32_t(a.v_new[nrow + vd + 32 * i]) | (uint32_t(a.v_new[nrow + vd + 32 * i + 16]) << 16);
  }
  const int kv_hi = min(it.kv1, main_end);
  for (int t0 = it.kv0 + wave * ST; t0 < kv_hi; t0 += kWaves * ST) {
    u32x4 kr[UK], vr[HV][UV];
    int blk_u = 0;
    if constexpr (B >= ST) blk_u = win.get(t0 / B);
#pragma unroll
    for (int i = 0; i < UK; ++i) {
      const int tok = t0 + i * TPI + ktok;
      kr[i] = u32x4{0u, 0u, 0u, 0u};
      if (tok < main_end) {
        const int blk = (B >= ST) ? blk_u : bt[tok / B];
        // Each K and V^T load instruction reads whole 128-byte lines (TPI full
        // K rows; 16 dims of one V^T sub-block) that no other load of this
        // item touches again, so both stream with the non-temporal hint.
        kr[i] = ld16_nt(a.kpool + ((size_t(blk) * a.hkv + g) * B + tok % B) * D + 8 * kdc);
      }
    }
#pragma unroll
    for (int h = 0; h < HV; ++h) {
      const int vt = t0 + kValuSubTile * h + 8 * vtc;
#pragma unroll
      for (int i = 0; i < UV; ++i) {
        vr[h][i] = u32x4{0u, 0u, 0u, 0u};
        if (vt < main_end) {
          const int blk = (B >= ST) ? blk_u : bt[vt / B];
          vr[h][i] = ld16_nt(a.vpool + (size_t(blk) * a.hkv + g) * D * B + vt_off<D, B>(vd + 16 * i, vt % B));
        }
      }
      if (vt < main_end && vt + 8 > main_end) {
#pragma unroll
        for (int i = 0; i < UV; ++i) vr[h][i] = zero_tail(vr[h][i], vt, main_end);
      }
    }

    // scores (log2 units), masked by range and causal limit
    float s[NR][UK];
#pragma unroll
    for (int i = 0; i < UK; ++i) {
      const int tok = t0 + i * TPI + ktok;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        float p = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) p = dot2(q[r][e], kr[i][e], p);
        p = group_sum<LPT>(p);
        s[r][i] = (tok < kv_hi && tok <= lim[r]) ? p * a.scale_log2 : -INFINITY;
      }
    }

    float alpha[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      float mt = s[r][0];
#pragma unroll
      for (int i = 1; i < UK; ++i) mt = fmaxf(mt, s[r][i]);
#pragma unroll
      for (int x = LPT; x < 64; x <<= 1) mt = fmaxf(mt, __shfl_xor(mt, x));
      const float mn = fmaxf(m[r], mt);
      const float mref = (mn == -INFINITY) ? 0.f : mn;
      alpha[r] = fast_exp2(m[r] - mref);
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < UK; ++i) {
        s[r][i] = fast_exp2(s[r][i] - mref);
        ps += s[r][i];
      }
      l[r] = l[r] * alpha[r] + ps;
      m[r] = mn;
    }

    // probabilities: token-per-lane-group layout -> 8-token chunk per lane
    if (kdc == 0) {
#pragma unroll
      for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int i = 0; i < UK; ++i) pbuf[r * ST + i * TPI + ktok] = s[r][i];
    }
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    float pp[HV][NR][8];
#pragma unroll
    for (int h = 0; h < HV; ++h)
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(pbuf + r * ST + kValuSubTile * h + 8 * vtc);
        const f32x4 x1 = *reinterpret_cast<const f32x4*>(pbuf + r * ST + kValuSubTile * h + 8 * vtc + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pp[h][r][e] = x0[e];
          pp[h][r][4 + e] = x1[e];
        }
      }
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");

#pragma unroll
    for (int i = 0; i < UV; ++i) {
#pragma unroll
      for (int r = 0; r < NR; ++r) acc[r][i] *= alpha[r];
#pragma unroll
      for (int h = 0; h < HV; ++h) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[2 * e] = bf_lo(vr[h][i][e]);
          v[2 * e + 1] = bf_hi(vr[h][i][e]);
        }
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          float t = acc[r][i];
#pragma unroll
          for (int u = 0; u < 8; ++u) t = fmaf(pp[h][r][u], v[u], t);
          acc[r][i] = t;
        }
      }
    }
  }

  // This pass's own positions [max(kv0, ctx), kv1) (fused pass only; one token
  // for a decode, at most kValuMaxRows for a tiny chunk): wavefront w takes
  // tokens w, w + 4, ...  Every lane reads chunk kdc of the K row, so each
  // LPT-lane group holds the full score; the weight enters l in the first
  // group's lanes and acc in the vtc == 0 lanes only, as the reductions below
  // sum over token groups and over the four vtc lanes.
  if constexpr (DIRECT) {
    for (int p = p_tail; p < it.kv1; p += kWaves) {
      u32x4 kn = kn_pre;
      float vv[UV];
      if (p == p_tail) {
#pragma unroll
        for (int i = 0; i < UV / 2; ++i) {
          vv[2 * i] = bf_lo(vn_pre[i]);
          vv[2 * i + 1] = bf_hi(vn_pre[i]);
        }
      } else {
        const size_t nrow = new_row(a, sq, p, g) * D;
        kn = ld16(a.k_new + nrow + 8 * kdc);
#pragma unroll
        for (int i = 0; i < UV; ++i) vv[i] = __uint_as_float(uint32_t(a.v_new[nrow + vd + 16 * i]) << 16);
      }
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        float sc = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) sc = dot2(q[r][e], kn[e], sc);
        sc = group_sum<LPT>(sc);
        const float x = p <= lim[r] ? sc * a.scale_log2 : -INFINITY;
        const float mn = fmaxf(m[r], x);
        if (mn != -INFINITY) {
          const float alpha = fast_exp2(m[r] - mn);
          const float w = fast_exp2(x - mn);
          l[r] = l[r] * alpha + (ktok == 0 ? w : 0.f);
#pragma unroll
          for (int i = 0; i < UV; ++i) acc[r][i] = acc[r][i] * alpha + (vtc == 0 ? w * vv[i] : 0.f);
          m[r] = mn;
        }
      }
    }
  }

  // wavefront totals: l over token groups, acc over the 4 chunk lanes
#pragma unroll
  for (int r = 0; r < NR; ++r) {
#pragma unroll
    for (int x = LPT; x < 64; x <<= 1) l[r] += __shfl_xor(l[r], x);
#pragma unroll
    for (int i = 0; i < UV; ++i) {
      float t = acc[r][i];
      t += dpp_f<0xB1>(t);
      t += dpp_f<0x4E>(t);
      acc[r][i] = t;
    }
  }

  // cross-wavefront log-sum-exp merge
  float* ms = smem + kWaves * NR * ST;
  float* ls = ms + kWaves * NR;
  float* as = ls + kWaves * NR;
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      ms[wave * NR + r] = m[r];
      ls[wave * NR + r] = l[r];
    }
  }
  if (vtc == 0) {
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int i = 0; i < UV; ++i) as[(wave * NR + r) * D + vd + 16 * i] = acc[r][i];
  }
  __syncthreads();
  for (int idx = tid; idx < NR * D; idx += kThreads) {
    const int r = idx / D, d = idx % D;
    if (r >= it.nrows) continue;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, ms[w * NR + r]);
    float o = 0.f, lse_val = -INFINITY;
    if (mx != -INFINITY) {
      float wsum = 0.f, os = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = fast_exp2(ms[w * NR + r] - mx);
        wsum += ls[w * NR + r] * f;
        os += as[(w * NR + r) * D + d] * f;
      }
      o = os / wsum;
      lse_val = (mx + fast_log2(wsum)) * kLn2;
    }
    store_result(a, sq, it, D, r, d, &o, 1, d == 0, lse_val);
  }
}

// ----------------------------------------------------------------------------
// Matrix-core path: up to 128 packed query rows (32 per wavefront, one per lane
// pair l, l^32) of one (sequence, kv head) over the item's KV range, in
// 64-token stages double-buffered in LDS.
//
// Stage layout in LDS (bf16): K rows [64][D+8] with the 32 tokens of each half
// stored at row perm32(t) (bits 2 and 3 swapped), then V^T rows [D][64+8].
// The padding keeps the 16-byte MFMA operand reads free of bank conflicts.
//
// With A = K rows and B = Q^T, lane l of the S^T product holds query row l%32
// and the 16 tokens 16*(v>>3) + 8*(l/32) + (v&7), v = 0..15, of each 32-token
// half; those are exactly the P^T operand of O^T = V^T P^T for the two 16-token
// k-steps (elements 8*ks .. 8*ks+7), and the matching V^T operand is 8
// contiguous tokens of one dimension.
__device__ __forceinline__ int perm32(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }

template <int D>
struct MfmaLds {
  static constexpr int KS = D + 8;
  static constexpr int VS = kKvTile + 8;
  static constexpr int KT = kKvTile * KS;
  static constexpr int VT = D * VS;
  static constexpr int STAGE = KT + VT;
  static constexpr int BYTES = 2 * STAGE * 2;
};

__device__ __forceinline__ void lds_dma16(const uint16_t* src, uint16_t* lds_seg) {
  using gptr = const void __attribute__((address_space(1)))*;
  using lptr = void __attribute__((address_space(3)))*;
  __builtin_amdgcn_global_load_lds((gptr)src, (lptr)lds_seg, 16, 0, 0);
}

template <int D, int B, bool DIRECT>
__device__ void mfma_item(const AttnArgs& a, const ItemRec& it, uint16_t* lds) {
  using L = MfmaLds<D>;
  constexpr int CPR = D / 8;                          // 16-byte chunks per K row
  constexpr int KCH = kKvTile * CPR / kThreads;       // K chunks per thread per stage
  constexpr int VCH = D * (kKvTile / 8) / kThreads;   // V^T chunks per thread per stage
  static_assert(KCH * kThreads == kKvTile * CPR && VCH * kThreads == D * kKvTile / 8, "stage split");
  // The wavefront index is uniform; reading it as a scalar keeps the staging
  // segments' LDS addresses in scalar registers.
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hf = lane >> 5;
  const SeqRec sq = a.seqs[it.seq];
  const int32_t* bt = a.bt + sq.bt_off;
  const int G = a.group, g = it.kv_head, kv_valid = sq.kv_len;
  const int r = wave * kMfmaRowsPerWave + l32;
  const bool row_ok = r < it.nrows;
  const int row = it.row0 + r;
  const int j = row / G, h = g * G + row % G;
  const int lim = row_ok ? sq.ctx + j : -1;
  const bool active = wave < it.waves;

  bf16x8 qb[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (row_ok) v = ld16(a.q + (size_t(sq.q_start + j) * a.hq + h) * D + 16 * kk + 8 * hf);
    qb[kk] = __builtin_bit_cast(bf16x8, v);
  }
  f32x16 o[D / 32];
#pragma unroll
  for (int dd = 0; dd < D / 32; ++dd)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[dd][v] = 0.f;
  float m = -INFINITY, lsum = 0.f;

  const int ntiles = (it.kv1 - it.kv0 + kKvTile - 1) / kKvTile;
  const size_t kv_head_base = size_t(g);
  u32x4 kst[KCH], vst[VCH];

  // Global -> register staging of one 64-token stage, for B < 64 (a stage then
  // spans 64 / B blocks; each chunk resolves its own block).  Chunk c of this
  // thread is 16-byte chunk ch = tid + 256 c of the stage.  Only the final
  // stage of a sequence (past kv_len) needs bounds checks.
  auto load_stage = [&](int tb) {
    const bool full = tb + kKvTile <= kv_valid;
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
      const int ch = tid + kThreads * c;
      const int tok = ch / CPR, dc = ch % CPR, p = tb + tok;
      kst[c] = u32x4{0u, 0u, 0u, 0u};
      if (DIRECT && p >= sq.ctx && p < kv_valid) {
        kst[c] = ld16(a.k_new + new_row(a, sq, p, g) * D + 8 * dc);
      } else if (full || p < kv_valid) {
        const int blk = bt[p / B];
        kst[c] = ld16(a.kpool + ((size_t(blk) * a.hkv + kv_head_base) * B + p % B) * D + 8 * dc);
      }
    }
#pragma unroll
    for (int c = 0; c < VCH; ++c) {
      const int ch = tid + kThreads * c;
      const int d = ch / (kKvTile / 8), tc = ch % (kKvTile / 8), p = tb + 8 * tc;
      vst[c] = u32x4{0u, 0u, 0u, 0u};
      if (full || p < kv_valid) {
        const int blk = bt[p / B];
        vst[c] = ld16(a.vpool + (size_t(blk) * a.hkv + kv_head_base) * D * B + vt_off<D, B>(d, p % B));
        if (!full && p + 8 > kv_valid) vst[c] = zero_tail(vst[c], p, kv_valid);
        if (DIRECT && p + 8 > sq.ctx) vst[c] = patch_new_v<D>(a, sq, vst[c], p, d, g);
      }
    }
  };
  auto store_stage = [&](int buf) {
    uint16_t* kt = lds + buf * L::STAGE;
    uint16_t* vt = kt + L::KT;
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
      const int ch = tid + kThreads * c;
      const int tok = ch / CPR, dc = ch % CPR;
      const int prow = (tok & ~31) | perm32(tok & 31);
      st16(kt + prow * L::KS + 8 * dc, kst[c]);
    }
#pragma unroll
    for (int c = 0; c < VCH; ++c) {
      const int ch = tid + kThreads * c;
      const int d = ch / (kKvTile / 8), tc = ch % (kKvTile / 8);
      st16(vt + d * L::VS + 8 * tc, vst[c]);
    }
  };

  // Causal limit of the wave's first packed row: a stage ending at or below it,
  // and inside the item's range, needs no mask for any row of the wave.
  const int lim_lo = sq.ctx + (it.row0 + wave * kMfmaRowsPerWave) / G;
  const float c = a.scale_log2;
  constexpr uint32_t kOnePair = 0x3F803F80u;  // two bf16 1.0
  float lrnd = 0.f;  // row sum of the bf16-rounded probabilities

  // With B == 64 a stage is one block, and the memory system writes it
  // straight into the padded LDS layout (global_load_lds_dwordx4: lane l's 16
  // bytes land at its wave's 1 KiB segment base + 16 l, from an address the
  // lane picks), so no staging registers are held across the stage.  Segment
  // sg of a stage is written by wave sg % 4; lane l fills stage unit
  // u = 64 sg + l, i.e. row u / U, column unit u % U of the padded rows
  // (U = D/8 + 1 units per K row, 9 per V^T row); a lane whose unit is row
  // padding loads the row's last data unit again.  Each thread's offsets
  // inside a block are fixed, so they are computed once.  V slots past kv_len
  // are zeroed in LDS afterwards by the lane that loaded them (they may hold
  // anything).  Other block sizes stage through registers (load_stage /
  // store_stage above).
  constexpr int KU = L::KS / 8, VU = L::VS / 8;
  constexpr int K_SEGS = L::KT / 512, V_SEGS = L::VT / 512;
  static_assert(K_SEGS * 512 == L::KT && V_SEGS * 512 == L::VT, "stage regions in whole KiB");
  constexpr int KSEG_W = (K_SEGS + kWaves - 1) / kWaves, VSEG_W = (V_SEGS + kWaves - 1) / kWaves;
  int koff[KSEG_W], voff[VSEG_W];
  if constexpr (B == kKvTile) {
#pragma unroll
    for (int i = 0; i < KSEG_W; ++i) {
      const int u = 64 * (i * kWaves + wave) + lane;
      const int rr = u / KU, tok = (rr & 32) | perm32(rr & 31);
      koff[i] = tok * D + 8 * min(u % KU, D / 8 - 1);
    }
#pragma unroll
    for (int i = 0; i < VSEG_W; ++i) {
      const int u = 64 * (i * kWaves + wave) + lane;
      voff[i] = vt_off<D, B>(u / VU, 8 * min(u % VU, kKvTile / 8 - 1));
    }
  }
  BlockWindow win{bt, sq.nblk, 0, 0};
  if constexpr (B == kKvTile) win.load(it.kv0 / B);
  // This pass's own tokens (positions >= ctx), when read from k_new / v_new:
  // their K rows are DMA'd from k_new (each lane picks its token's row), and
  // their V, token-major there, goes through registers and is transposed into
  // the V^T stage: thread u < 16 * D / 8 takes tokens 4 (u / (D/8)) .. +3 of
  // dims 8 (u % (D/8)) .. +7 (four 16-byte loads, issued a stage ahead like the
  // DMA) and writes 8 dims x 4 tokens.  A stage wholly past ctx skips the V DMA;
  // the one stage holding ctx takes its V DMA from the pool and overwrites the
  // positions >= ctx once every wave's DMA has landed (one extra barrier).
  constexpr bool direct = DIRECT;
  constexpr int VN_DG = D / 8;
  const int vn_tg = tid / VN_DG, vn_dg = tid % VN_DG;
  const bool vn_thread = tid < 16 * VN_DG;
  u32x4 vnew[4];
  auto load_vnew = [&](int tb) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int p = tb + 4 * vn_tg + k;
      vnew[k] = u32x4{0u, 0u, 0u, 0u};
      if (vn_thread && p >= sq.ctx && p < kv_valid) vnew[k] = ld16(a.v_new + new_row(a, sq, p, g) * D + 8 * vn_dg);
    }
  };
  auto store_vnew = [&](int tb, int buf) {
    if (!vn_thread) return;
    uint16_t* vt = lds + buf * L::STAGE + L::KT;
    const int p0 = tb + 4 * vn_tg;
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const uint32_t w0 = (d & 1) ? pick_hi(vnew[0][d >> 1], vnew[1][d >> 1]) : pick_lo(vnew[0][d >> 1], vnew[1][d >> 1]);
      const uint32_t w1 = (d & 1) ? pick_hi(vnew[2][d >> 1], vnew[3][d >> 1]) : pick_lo(vnew[2][d >> 1], vnew[3][d >> 1]);
      uint16_t* dst = vt + (8 * vn_dg + d) * L::VS + 4 * vn_tg;
      if (p0 >= sq.ctx) {
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        *reinterpret_cast<u32x2*>(dst) = u32x2{w0, w1};
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (p0 + k >= sq.ctx) dst[k] = uint16_t(((k < 2 ? w0 : w1) >> (16 * (k & 1))) & 0xffffu);
      }
    }
  };
  auto dma_stage = [&](int tb, int buf) {
    const size_t tile = (size_t(win.get(tb / B)) * a.hkv + kv_head_base) * (size_t(B) * D);
    uint16_t* kt = lds + buf * L::STAGE;
    uint16_t* vt = kt + L::KT;
    const bool has_new = direct && tb + kKvTile > sq.ctx;
#pragma unroll
    for (int i = 0; i < KSEG_W; ++i) {
      if (i * kWaves + wave < K_SEGS) {
        const uint16_t* src = a.kpool + tile + koff[i];
        if (has_new) {
          const int p = tb + koff[i] / D;
          if (p >= sq.ctx && p < kv_valid) src = a.k_new + new_row(a, sq, p, g) * D + koff[i] % D;
        }
        lds_dma16(src, kt + (i * kWaves + wave) * 512);
      }
    }
    if (!(has_new && tb >= sq.ctx)) {
#pragma unroll
      for (int i = 0; i < VSEG_W; ++i)
        if (i * kWaves + wave < V_SEGS) lds_dma16(a.vpool + tile + voff[i], vt + (i * kWaves + wave) * 512);
    }
    if (has_new) load_vnew(tb);
  };

  auto fix_v_tail = [&](int tb, int buf) {
    if (tb + kKvTile <= kv_valid) return;
    uint16_t* vt = lds + buf * L::STAGE + L::KT;
#pragma unroll
    for (int i = 0; i < VSEG_W; ++i) {
      const int u = 64 * (i * kWaves + wave) + lane;
      const int col = u % VU;
      if (i * kWaves + wave < V_SEGS && col < kKvTile / 8 && tb + 8 * col + 8 > kv_valid) {
        uint16_t* dst = vt + 8 * u;
        st16(dst, zero_tail(ld16(dst), tb + 8 * col, kv_valid));
      }
    }
  };
  // After this wave's DMA of stage tb has landed: zero DMA'd V past kv_len and
  // put this pass's V into the positions >= ctx.
  auto finish_stage = [&](int tb, int buf) {
    if (!(direct && tb >= sq.ctx)) fix_v_tail(tb, buf);
    if (direct && tb + kKvTile > sq.ctx) {
      if (tb < sq.ctx) __syncthreads();
      store_vnew(tb, buf);
    }
  };  if constexpr (B == kKvTile) {
    dma_stage(it.kv0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    finish_stage(it.kv0, 0);
  } else {
    load_stage(it.kv0);
    store_stage(0);
  }
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int tb = it.kv0 + t * kKvTile;
    if (t + 1 < ntiles) {
      if constexpr (B == kKvTile)
        dma_stage(tb + kKvTile, (t + 1) & 1);
      else
        load_stage(tb + kKvTile);
    }
    if (active) {
      const uint16_t* kt = lds + (t & 1) * L::STAGE;
      const uint16_t* vt = kt + L::KT;
      // S^T for both 32-token halves; consecutive MFMAs alternate between the
      // two accumulators so no MFMA waits on the one just issued.
      f32x16 sacc[2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int v = 0; v < 16; ++v) sacc[h2][v] = 0.f;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const bf16x8 ka = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const u32x4*>(kt + (32 * h2 + l32) * L::KS + 16 * kk + 8 * hf));
          sacc[h2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qb[kk], sacc[h2], 0, 0, 0);
        }
      }
      // Schedule: the 16 K-fragment reads run four ahead of the 16 MFMAs
      // (LDS reads 0x100, MFMA 0x008), so no MFMA waits on its own read.
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      for (int i = 0; i < 12; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      // raw scores; masked ones become -inf (only in boundary stages)
      float mt = -INFINITY;
      if (tb + kKvTile > it.kv1 || tb + kKvTile - 1 > lim_lo) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int tok = tb + 32 * h2 + 16 * (v >> 3) + 8 * hf + (v & 7);
            const float x = (tok < it.kv1 && tok <= lim) ? sacc[h2][v] : -INFINITY;
            sacc[h2][v] = x;
            mt = fmaxf(mt, x);
          }
      } else {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int v = 0; v < 16; ++v) mt = fmaxf(mt, sacc[h2][v]);
      }
      mt = fmaxf(mt, __shfl_xor(mt, 32)) * c;
      // Lazy rescale: the reference max m moves only when a row's stage max
      // exceeds it by more than kRescaleSlack (log2 units), so probabilities
      // stay <= 2^kRescaleSlack and most stages skip the O rescale.
      if (__any(mt > m + kRescaleSlack)) {
        const float mn = fmaxf(m, mt);
        const float alpha = (mn == -INFINITY) ? 1.f : fast_exp2(m - mn);
        lsum *= alpha;
        lrnd *= alpha;
#pragma unroll
        for (int dd = 0; dd < D / 32; ++dd) o[dd] *= alpha;
        m = mn;
      }
      const float mref = (m == -INFINITY) ? 0.f : m;
      // Probabilities: the fp32 row sum feeds the LSE; the bf16-rounded P^T
      // operand of the P V product is summed as well (v_dot2 against 1.0), and
      // O is normalised by that sum, so it is an exact convex combination of V
      // rows under the weights actually used.
      bf16x8 pb[2][2];
      float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = fast_exp2(fmaf(sacc[h2][v], c, -mref));
          if (v & 1) ps1 += p; else ps0 += p;
          pb[h2][v >> 3][v & 7] = __bf16(p);
        }
      lsum += ps0 + ps1;
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const u32x4 w = __builtin_bit_cast(u32x4, pb[h2][ks]);
#pragma unroll
          for (int e = 0; e < 4; ++e) lrnd = dot2(w[e], kOnePair, lrnd);
        }
      // O^T += V^T P^T; the dims loop is innermost so consecutive MFMAs use
      // different accumulators.
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int dd = 0; dd < D / 32; ++dd) {
            const bf16x8 va = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const u32x4*>(vt + (32 * dd + l32) * L::VS + 32 * h2 + 16 * ks + 8 * hf));
            o[dd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[h2][ks], o[dd], 0, 0, 0);
          }
    }
    if (t + 1 < ntiles) {
      if constexpr (B == kKvTile) {
        __builtin_amdgcn_s_waitcnt(0);
        finish_stage(tb + kKvTile, (t + 1) & 1);
      } else {
        store_stage((t + 1) & 1);
      }
    }
    __syncthreads();
  }

  if (active) {
    const float lt = lsum + __shfl_xor(lsum, 32);
    const float lr = lrnd + __shfl_xor(lrnd, 32);
    const float inv = lr > 0.f ? 1.f / lr : 0.f;
    const float lse_val = lt > 0.f ? (m + fast_log2(lt)) * kLn2 : -INFINITY;
    if (row_ok) {
#pragma unroll
      for (int dd = 0; dd < D / 32; ++dd)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          float vals[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) vals[e] = o[dd][4 * qd + e] * inv;
          store_result(a, sq, it, D, r, 32 * dd + 8 * qd + 4 * hf, vals, 4,
                       hf == 0 && dd == 0 && qd == 0, lse_val);
        }
    }
  }
}

template <int D, int ST>
constexpr int valu_lds_bytes() {
  return (kWaves * kValuMaxRows * ST + 2 * kWaves * kValuMaxRows + kWaves * kValuMaxRows * D) * 4;
}

// Log-sum-exp merge of one split group (every row, every split), by the whole
// work-group, all rows at once: first one thread per row finds the row's
// largest partial lse and the sum of the weights e^(lse_i - max) and writes
// the final lse = max + ln(sum); then every thread takes independent (row,
// 4-dim) units and sums the weighted, normalised partial rows.  Same formula
// as the pages' merge step.  `red` is LDS for 2 * nrows floats.  Inside the
// attention launch (COHERENT) partial values are read with device-coherent
// loads.
template <int D, bool COHERENT>
__device__ void merge_group(const AttnArgs& a, const MergeRec& g, float* red) {
  constexpr int CH = D / 4;
  const int tid = threadIdx.x;
  const SeqRec sq = a.seqs[g.seq];
  ItemRec fin;
  fin.seq = g.seq;
  fin.kv_head = g.kv_head;
  fin.row0 = g.row0;
  fin.nrows = g.nrows;
  fin.slot = -1;
  for (int r = tid; r < g.nrows; r += kThreads) {
    const float* ls = a.ws_lse + g.slot0 + r;
    float mx = -INFINITY;
    for (int i = 0; i < g.nsplit; ++i) mx = fmaxf(mx, load_partial<COHERENT>(ls + size_t(i) * g.nrows));
    float wsum = 0.f;
    for (int i = 0; i < g.nsplit; ++i) {
      const float li = load_partial<COHERENT>(ls + size_t(i) * g.nrows);
      wsum += (li == -INFINITY) ? 0.f : fast_exp2((li - mx) * kLog2e);
    }
    red[r] = mx;
    red[g.nrows + r] = wsum > 0.f ? 1.f / wsum : 0.f;
    store_result(a, sq, fin, D, r, 0, nullptr, 0, true,
                 wsum > 0.f ? mx + fast_log2(wsum) * kLn2 : -INFINITY);
  }
  __syncthreads();
  // Four (row, 4-dim) units per thread per pass, their loads issued together.
  constexpr int UPT = 4;
  const int units = g.nrows * CH;
  for (int u0 = tid; u0 < units; u0 += UPT * kThreads) {
    float acc[UPT][4];
    int rr[UPT], cc[UPT];
    bool ok[UPT];
#pragma unroll
    for (int j = 0; j < UPT; ++j) {
      const int u = u0 + j * kThreads;
      ok[j] = u < units;
      rr[j] = ok[j] ? u / CH : 0;
      cc[j] = ok[j] ? u % CH : 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[j][e] = 0.f;
    }
    for (int i = 0; i < g.nsplit; ++i) {
      float li[UPT], ov[UPT][4];
#pragma unroll
      for (int j = 0; j < UPT; ++j) {
        const size_t pr = size_t(g.slot0) + size_t(i) * g.nrows + rr[j];
        li[j] = ok[j] ? load_partial<COHERENT>(a.ws_lse + pr) : -INFINITY;
        const float* o = a.ws_o + pr * D + 4 * cc[j];
        if constexpr (COHERENT) {
#pragma unroll
          for (int e = 0; e < 4; ++e) ov[j][e] = ok[j] ? load_partial<true>(o + e) : 0.f;
        } else {
          const f32x4 v = ok[j] ? *reinterpret_cast<const f32x4*>(o) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int e = 0; e < 4; ++e) ov[j][e] = v[e];
        }
      }
#pragma unroll
      for (int j = 0; j < UPT; ++j) {
        const float mx = red[rr[j]], inv = red[g.nrows + rr[j]];
        const float w = (li[j] == -INFINITY) ? 0.f : fast_exp2((li[j] - mx) * kLog2e) * inv;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[j][e] = fmaf(w, ov[j][e], acc[j][e]);
      }
    }
#pragma unroll
    for (int j = 0; j < UPT; ++j)
      if (ok[j]) store_result(a, sq, fin, D, rr[j], 4 * cc[j], acc[j], 4, false, 0.f);
  }
}

// End of a split item: its partial rows are in the workspace, written with
// device-coherent stores.  Wait until they have completed, count the split in
// with one device-scope atomic, and if this work-group brought the count to
// nsplit, merge the group (device-coherent loads see every split's rows: each
// split's stores completed before its count) and re-arm the counter for the
// next call.  Counters start at zero (the uploaded metadata holds zeros).  No
// whole-cache writeback or invalidation is involved, so the KV that other
// work-groups keep in L2 stays there.
// `last_flag` is the first word of the item's LDS (the merge uses the LDS
// from 16 bytes on); the barrier before thread 0 writes it follows every LDS
// access of the item.
// The ordering argument above rests on gfx950's memory model (scoped sc1
// accesses, stores counted by vmcnt): build the device code for gfx950 only.
#if defined(__HIP_DEVICE_COMPILE__) && !defined(__gfx950__)
#error "the in-launch split merge is written for gfx950's memory model"
#endif
template <int D>
__device__ void finish_split(const AttnArgs& a, const ItemRec& it, int* last_flag) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const int prev = __hip_atomic_fetch_add(a.counters + it.group, 1, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
    *last_flag = prev == a.groups[it.group].nsplit - 1;
  }
  __syncthreads();
  if (!*last_flag) return;
  merge_group<D, true>(a, a.groups[it.group], reinterpret_cast<float*>(last_flag) + 4);
  if (threadIdx.x == 0)
    __hip_atomic_store(a.counters + it.group, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Append of one run (up to B consecutive new tokens of one sequence in one
// block) for one kv head.  K rows are copied with 16-byte loads and stores.
// V is written transposed: a thread takes an aligned group of 8 block slots
// and 8 dims, loads the 8 token rows' 16-byte dim chunks, transposes the 8x8
// bf16 tile in registers (v_perm_b32 picks 16-bit halves) and stores 8
// contiguous 16-byte slot runs, one per dim; groups the run only partly covers
// store their valid slots with 2-byte stores, so no byte outside the run is
// written.

template <int D, int B>
__device__ __forceinline__ void append_run(const RunRec run, const int g, const uint16_t* k_new,
                                           const uint16_t* v_new, uint16_t* kpool, uint16_t* vpool,
                                           int hkv) {
  constexpr int CPR = D / 8;
  uint16_t* kdst = kpool + ((size_t(run.block) * hkv + g) * B + run.slot0) * D;
  for (int c = threadIdx.x; c < run.count * CPR; c += kThreads) {
    const int i = c / CPR, dc = c % CPR;
    st16(kdst + i * D + 8 * dc, ld16(k_new + (size_t(run.tok0 + i) * hkv + g) * D + 8 * dc));
  }
  uint16_t* vblk = vpool + (size_t(run.block) * hkv + g) * D * B;
  const int first = run.slot0 / 8;
  const int groups = (run.slot0 + run.count - 1) / 8 - first + 1;
  for (int e = threadIdx.x; e < groups * CPR; e += kThreads) {
    const int cg = e % groups, dg = e / groups;   // slot group fastest: coalesced stores
    const int s0 = 8 * (first + cg);
    u32x4 r[8];
    bool full = true;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = s0 + u - run.slot0;
      const bool ok = i >= 0 && i < run.count;
      full = full && ok;
      r[u] = ok ? ld16(v_new + (size_t(run.tok0 + i) * hkv + g) * D + 8 * dg) : u32x4{0u, 0u, 0u, 0u};
    }
    // out[d] holds slots s0..s0+7 of dim 8*dg + d
    u32x4 out[8];
#pragma unroll
    for (int w = 0; w < 4; ++w)          // word w of a row holds dims 2w, 2w+1
#pragma unroll
      for (int k = 0; k < 4; ++k) {      // output word k holds slots 2k, 2k+1
        out[2 * w][k] = pick_lo(r[2 * k][w], r[2 * k + 1][w]);
        out[2 * w + 1][k] = pick_hi(r[2 * k][w], r[2 * k + 1][w]);
      }
    if (full) {
#pragma unroll
      for (int d = 0; d < 8; ++d) st16(vblk + vt_off<D, B>(8 * dg + d, s0), out[d]);
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = s0 + u - run.slot0;
        if (i < 0 || i >= run.count) continue;
#pragma unroll
        for (int d = 0; d < 8; ++d) {
          const uint32_t w = out[d][u >> 1];
          vblk[vt_off<D, B>(8 * dg + d, s0 + u)] = uint16_t((u & 1) ? (w >> 16) : (w & 0xffffu));
        }
      }
    }
  }
}

// The decode loop's step: in the kernel that also runs matrix-core tiles the
// tile path sets the register budget, and 64-token steps (twice the loads in
// flight per wavefront) fit inside it; the decode-only kernel keeps 32-token
// steps, whose smaller register count lets a CU hold a third work-group.
template <int D, int B, bool MFMA, bool DIRECT>
__global__ __launch_bounds__(kThreads, 2) void attn_kernel(AttnArgs a) {
  constexpr int kStep = MFMA ? 2 * kValuSubTile : kValuSubTile;
  constexpr int kLds = MFMA ? (MfmaLds<D>::BYTES > valu_lds_bytes<D, kStep>() ? MfmaLds<D>::BYTES
                                                                               : valu_lds_bytes<D, kStep>())
                            : valu_lds_bytes<D, kStep>();
  __shared__ __attribute__((aligned(16))) unsigned char smem[kLds];
  if constexpr (DIRECT) {
    if (int(blockIdx.x) >= a.n_items) {
      // fused append: reads k_new / v_new and writes pool slots at positions
      // >= ctx, which no attention item of this launch reads from the pools
      const unsigned w = blockIdx.x - unsigned(a.n_items);
      append_run<D, B>(a.runs[w / unsigned(a.hkv)], int(w % unsigned(a.hkv)), a.k_new, a.v_new,
                       a.kpool_w, a.vpool_w, a.hkv);
      return;
    }
  }
  const ItemRec it = a.items[blockIdx.x];
  if constexpr (MFMA) {
    if (it.waves > 0) {
      mfma_item<D, B, DIRECT>(a, it, reinterpret_cast<uint16_t*>(smem));
      if (it.group >= 0 && it.group < a.n_inlaunch) finish_split<D>(a, it, reinterpret_cast<int*>(smem));
      return;
    }
  }
  if (it.nrows == 1)
    valu_item<D, B, 1, kStep, DIRECT>(a, it, reinterpret_cast<float*>(smem));
  else
    valu_item<D, B, kValuMaxRows, kStep, DIRECT>(a, it, reinterpret_cast<float*>(smem));
  if (it.group >= 0 && it.group < a.n_inlaunch) finish_split<D>(a, it, reinterpret_cast<int*>(smem));
}

// Merge launch for split prefill tiles: one work-group per group, after the
// attention launch (so plain loads see the partial rows).
template <int D>
__global__ __launch_bounds__(kThreads) void merge_kernel(AttnArgs a) {
  __shared__ float red[2 * kMfmaTileRows];
  merge_group<D, false>(a, a.groups[a.n_inlaunch + blockIdx.x], red);
}

// One work-group per (append run, kv head).
template <int D, int B>
__global__ __launch_bounds__(kThreads) void append_kernel(const RunRec* runs, const uint16_t* k_new,
                                                           const uint16_t* v_new, uint16_t* kpool,
                                                           uint16_t* vpool, int hkv) {
  append_run<D, B>(runs[blockIdx.x], blockIdx.y, k_new, v_new, kpool, vpool, hkv);
}

// Plan upload and append in one launch.  Work-groups below n_copy copy the
// metadata blob from the pinned host slot into the device buffer (for the
// attention launch that follows); the others append run (i / hkv) of kv head
// (i % hkv), reading their run record straight from the pinned slot, so they
// do not depend on the copy.
template <int D, int B>
__global__ __launch_bounds__(kThreads) void upload_append_kernel(
    const u32x4* __restrict__ blob_host, u32x4* __restrict__ blob_dev, unsigned chunks,
    unsigned n_copy, const RunRec* runs_host, const uint16_t* k_new, const uint16_t* v_new,
    uint16_t* kpool, uint16_t* vpool, int hkv) {
  if (blockIdx.x < n_copy) {
    const unsigned i = blockIdx.x * kThreads + threadIdx.x;
    if (i < chunks) blob_dev[i] = blob_host[i];
    return;
  }
  const unsigned w = blockIdx.x - n_copy;
  append_run<D, B>(runs_host[w / unsigned(hkv)], int(w % unsigned(hkv)), k_new, v_new, kpool, vpool,
                   hkv);
}

// ---------------------------------------------------------------- profiling
struct ProfRec {
  int kind;
  hipEvent_t start, stop;
};
std::mutex g_prof_mu;
uint32_t g_prof_mask = 0;  // bit k: bracket launches of FG_KERNEL k
std::vector<ProfRec> g_prof_recs;
std::vector<hipEvent_t> g_prof_pool;

hipEvent_t prof_event() {
  if (!g_prof_pool.empty()) {
    hipEvent_t e = g_prof_pool.back();
    g_prof_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

struct ProfScope {
  int kind;
  hipStream_t stream;
  hipEvent_t start = nullptr;
  // kind FG_KERNEL_COUNT (or above): never bracketed, no event is created
  ProfScope(int k, hipStream_t s) : kind(k), stream(s) {
    if (kind < 0 || kind >= FG_KERNEL_COUNT || ((g_prof_mask >> kind) & 1u) == 0) return;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    start = prof_event();
    if (start && hipEventRecord(start, stream) != hipSuccess) {
      g_prof_pool.push_back(start);  // not recorded: no measurement for this launch
      start = nullptr;
    }
  }
  ~ProfScope() {
    if (!start) return;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    hipEvent_t stop = prof_event();
    if (!stop || hipEventRecord(stop, stream) != hipSuccess) {
      g_prof_pool.push_back(start);
      if (stop) g_prof_pool.push_back(stop);
      return;
    }
    g_prof_recs.push_back({kind, start, stop});
  }
};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ---------------------------------------------------------------- metadata upload
// Plans are uploaded by a small kernel that reads a pinned host staging slot
// over the host link and writes the device buffer, so the whole pass stays on
// the caller's compute queue (a copy-engine transfer costs a cross-engine
// hand-off before the next kernel).  A ring of kStageSlots pinned slots is
// allocated on first use and held until the process ends; a slot is reused
// only after the event recorded behind its last upload has completed.
// Plans larger than a slot fall back to hipMemcpyAsync.
constexpr int kStageSlots = 8;
constexpr size_t kStageSlotBytes = size_t(2) << 20;

struct StageSlot {
  void* host = nullptr;
  hipEvent_t done = nullptr;
  bool pending = false;
};
std::mutex g_stage_mu;
StageSlot g_stage[kStageSlots];
int g_stage_next = 0;
int g_stage_state = 0;  // 0 untried, 1 ready, -1 unavailable (fall back to copies)

bool stage_ready() {
  if (g_stage_state == 0) {
    g_stage_state = 1;
    for (StageSlot& slot : g_stage) {
      if (hipHostMalloc(&slot.host, kStageSlotBytes, hipHostMallocDefault) != hipSuccess ||
          hipEventCreateWithFlags(&slot.done, hipEventDisableTiming) != hipSuccess) {
        g_stage_state = -1;
        break;
      }
    }
  }
  return g_stage_state == 1;
}

__global__ __launch_bounds__(kThreads) void upload_kernel(const u32x4* __restrict__ src,
                                                          u32x4* __restrict__ dst, unsigned n) {
  const unsigned i = blockIdx.x * kThreads + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

#define FG_SWITCH_DB(D_, B_, MACRO)                 \
  do {                                              \
    if ((D_) == 64 && (B_) == 16) MACRO(64, 16);    \
    else if ((D_) == 64 && (B_) == 32) MACRO(64, 32); \
    else if ((D_) == 64 && (B_) == 64) MACRO(64, 64); \
    else if ((D_) == 128 && (B_) == 16) MACRO(128, 16); \
    else if ((D_) == 128 && (B_) == 32) MACRO(128, 32); \
    else if ((D_) == 128 && (B_) == 64) MACRO(128, 64); \
    else return FG_E_UNSUPPORTED;                   \
  } while (0)

}  // namespace
}  // namespace fg

using namespace fg;

extern "C" int fg_internal_device_cu_count(void) {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  return n;
}

extern "C" fg_status fg_plan_upload(const fg_plan* plan, void* d_meta, void* stream) {
  if (!plan || !d_meta || !aligned16(d_meta)) return FG_E_INVALID;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t bytes = plan->blob.size();
  std::lock_guard<std::mutex> lk(g_stage_mu);
  if (bytes <= kStageSlotBytes && stage_ready()) {
    StageSlot& slot = g_stage[g_stage_next];
    g_stage_next = (g_stage_next + 1) % kStageSlots;
    if (slot.pending) {
      // the slot's previous upload was kStageSlots uploads ago; normally done
      if (hipEventSynchronize(slot.done) != hipSuccess) return FG_E_HIP;
      slot.pending = false;
    }
    memcpy(slot.host, plan->blob.data(), bytes);
    const unsigned chunks = unsigned((bytes + 15) / 16);
    hipLaunchKernelGGL(upload_kernel, dim3((chunks + kThreads - 1) / kThreads), dim3(kThreads), 0, s,
                       reinterpret_cast<const u32x4*>(slot.host), static_cast<u32x4*>(d_meta), chunks);
    if (hipGetLastError() != hipSuccess) return FG_E_HIP;
    if (hipEventRecord(slot.done, s) != hipSuccess) return FG_E_HIP;
    slot.pending = true;
    return FG_OK;
  }
  if (hipMemcpyAsync(d_meta, plan->blob.data(), bytes, hipMemcpyHostToDevice, s) != hipSuccess)
    return FG_E_HIP;
  return FG_OK;
}

extern "C" fg_status fg_kv_append(const fg_plan* plan, const void* d_meta, const void* k_new,
                                  const void* v_new, void* k_pool, void* v_pool, void* stream) {
  if (!plan) return FG_E_INVALID;
  if (plan->n_runs == 0) return FG_OK;
  if (!d_meta || !k_new || !v_new || !k_pool || !v_pool) return FG_E_INVALID;
  if (!aligned16(d_meta) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) ||
      !aligned16(v_pool))
    return FG_E_INVALID;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const RunRec* runs =
      reinterpret_cast<const RunRec*>(static_cast<const uint8_t*>(d_meta) + plan->off_runs);
  ProfScope prof(FG_KERNEL_APPEND, s);
  const dim3 grid(unsigned(plan->n_runs), unsigned(plan->hkv));
#define FG_LAUNCH_APPEND(D_, B_)                                                              \
  hipLaunchKernelGGL((append_kernel<D_, B_>), grid, dim3(kThreads), 0, s, runs,              \
                     static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new), \
                     static_cast<uint16_t*>(k_pool), static_cast<uint16_t*>(v_pool), plan->hkv)
  FG_SWITCH_DB(plan->head_dim, plan->block_size, FG_LAUNCH_APPEND);
#undef FG_LAUNCH_APPEND
  return hipGetLastError() == hipSuccess ? FG_OK : FG_E_HIP;
}

extern "C" fg_status fg_upload_append(const fg_plan* plan, void* d_meta, const void* k_new,
                                     const void* v_new, void* k_pool, void* v_pool, void* stream) {
  if (!plan || !d_meta || !aligned16(d_meta)) return FG_E_INVALID;
  if (plan->n_runs > 0 && (!k_new || !v_new || !k_pool || !v_pool || !aligned16(k_new) ||
                           !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool)))
    return FG_E_INVALID;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t bytes = plan->blob.size();
  {
    std::lock_guard<std::mutex> lk(g_stage_mu);
    if (plan->n_runs > 0 && bytes <= kStageSlotBytes && stage_ready()) {
      StageSlot& slot = g_stage[g_stage_next];
      g_stage_next = (g_stage_next + 1) % kStageSlots;
      if (slot.pending) {
        if (hipEventSynchronize(slot.done) != hipSuccess) return FG_E_HIP;
        slot.pending = false;
      }
      memcpy(slot.host, plan->blob.data(), bytes);
      const unsigned chunks = unsigned((bytes + 15) / 16);
      const unsigned n_copy = (chunks + kThreads - 1) / kThreads;
      const RunRec* runs_host =
          reinterpret_cast<const RunRec*>(static_cast<const uint8_t*>(slot.host) + plan->off_runs);
      {
        ProfScope prof(FG_KERNEL_APPEND, s);
        const dim3 grid(n_copy + unsigned(plan->n_runs) * unsigned(plan->hkv));
#define FG_LAUNCH_UPAPP(D_, B_)                                                                  \
  hipLaunchKernelGGL((upload_append_kernel<D_, B_>), grid, dim3(kThreads), 0, s,                 \
                     reinterpret_cast<const u32x4*>(slot.host), static_cast<u32x4*>(d_meta),      \
                     chunks, n_copy, runs_host, static_cast<const uint16_t*>(k_new),              \
                     static_cast<const uint16_t*>(v_new), static_cast<uint16_t*>(k_pool),          \
                     static_cast<uint16_t*>(v_pool), plan->hkv)
        FG_SWITCH_DB(plan->head_dim, plan->block_size, FG_LAUNCH_UPAPP);
#undef FG_LAUNCH_UPAPP
      }
      if (hipGetLastError() != hipSuccess) return FG_E_HIP;
      if (hipEventRecord(slot.done, s) != hipSuccess) return FG_E_HIP;
      slot.pending = true;
      return FG_OK;
    }
  }
  // no staging (or an empty pass): the two separate steps
  fg_status st = fg_plan_upload(plan, d_meta, stream);
  if (st != FG_OK) return st;
  return fg_kv_append(plan, d_meta, k_new, v_new, k_pool, v_pool, stream);
}

namespace fg {
namespace {

// The attention launch (and the merge launch when the plan splits prefill
// tiles) with the workspace at d_ws, which must already be checked against
// the plan.  `profile` allows the per-launch HIP events of fg_profile_enable.
fg_status launch_attention(const fg_plan* plan, void* d_meta, const void* q, const void* k_pool,
                           const void* v_pool, void* out, int32_t out_dtype, float* lse, void* d_ws,
                           hipStream_t s, bool profile, const void* k_new = nullptr,
                           const void* v_new = nullptr, bool fused_append = false) {
  uint8_t* meta = static_cast<uint8_t*>(d_meta);
  AttnArgs a;
  a.seqs = reinterpret_cast<const SeqRec*>(meta + plan->off_seqs);
  a.bt = reinterpret_cast<const int32_t*>(meta + plan->off_bt);
  a.items = reinterpret_cast<const ItemRec*>(meta + plan->off_items);
  a.groups = reinterpret_cast<const MergeRec*>(meta + plan->off_merges);
  a.counters = reinterpret_cast<int32_t*>(meta + plan->off_counters);
  a.q = static_cast<const uint16_t*>(q);
  a.kpool = static_cast<const uint16_t*>(k_pool);
  a.vpool = static_cast<const uint16_t*>(v_pool);
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.runs = reinterpret_cast<const RunRec*>(meta + plan->off_runs);
  a.kpool_w = static_cast<uint16_t*>(const_cast<void*>(k_pool));
  a.vpool_w = static_cast<uint16_t*>(const_cast<void*>(v_pool));
  a.n_items = plan->n_items;
  a.out = out;
  a.lse = lse;
  a.ws_o = plan->ws_bytes ? reinterpret_cast<float*>(static_cast<uint8_t*>(d_ws) + plan->ws_o_off) : nullptr;
  a.ws_lse = plan->ws_bytes ? reinterpret_cast<float*>(static_cast<uint8_t*>(d_ws) + plan->ws_lse_off) : nullptr;
  a.hq = plan->hq;
  a.hkv = plan->hkv;
  a.group = plan->group;
  a.n_mfma = plan->n_mfma;
  a.n_inlaunch = plan->n_inlaunch_groups;
  a.scale_log2 = plan->scale * kLog2e;
  a.out_bf16 = out_dtype == FG_DTYPE_BF16;

  {
    ProfScope prof(profile ? FG_KERNEL_ATTENTION : FG_KERNEL_COUNT, s);
    const unsigned n_append = fused_append ? unsigned(plan->n_runs) * unsigned(plan->hkv) : 0u;
    const dim3 grid(unsigned(plan->n_items) + n_append);
#define FG_LAUNCH_ATTN(D_, B_)                                                                 \
  do {                                                                                         \
    if (a.k_new) {                                                                             \
      if (plan->n_mfma > 0)                                                                    \
        hipLaunchKernelGGL((attn_kernel<D_, B_, true, true>), grid, dim3(kThreads), 0, s, a);  \
      else                                                                                     \
        hipLaunchKernelGGL((attn_kernel<D_, B_, false, true>), grid, dim3(kThreads), 0, s, a); \
    } else {                                                                                   \
      if (plan->n_mfma > 0)                                                                    \
        hipLaunchKernelGGL((attn_kernel<D_, B_, true, false>), grid, dim3(kThreads), 0, s, a); \
      else                                                                                     \
        hipLaunchKernelGGL((attn_kernel<D_, B_, false, false>), grid, dim3(kThreads), 0, s, a);\
    }                                                                                          \
  } while (0)
    FG_SWITCH_DB(plan->head_dim, plan->block_size, FG_LAUNCH_ATTN);
#undef FG_LAUNCH_ATTN
    if (hipGetLastError() != hipSuccess) return FG_E_HIP;
  }
  const int32_t n_late = plan->n_merge_groups - plan->n_inlaunch_groups;
  if (n_late > 0) {
    ProfScope prof(profile ? FG_KERNEL_MERGE : FG_KERNEL_COUNT, s);
    if (plan->head_dim == 64)
      hipLaunchKernelGGL((merge_kernel<64>), dim3(unsigned(n_late)), dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((merge_kernel<128>), dim3(unsigned(n_late)), dim3(kThreads), 0, s, a);
    if (hipGetLastError() != hipSuccess) return FG_E_HIP;
  }
  return FG_OK;
}

fg_status check_attention_args(const fg_plan* plan, int32_t out_dtype, const void* d_meta,
                               const void* q, const void* k_pool, const void* v_pool,
                               const void* out, const float* lse) {
  if (out_dtype != FG_DTYPE_F32 && out_dtype != FG_DTYPE_BF16) return FG_E_UNSUPPORTED;
  if (!d_meta || !q || !k_pool || !v_pool || !out) return FG_E_INVALID;
  if (!aligned16(d_meta) || !aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) ||
      !aligned16(out) || (lse && !aligned16(lse)))
    return FG_E_INVALID;
  return FG_OK;
}

// ---------------------------------------------------------------- library scratch
// Workspace of fg_attention_ragged_noalloc: one array per device in the code
// object, allocated when the library is loaded onto the device and held until
// the process ends.  In host code `scratch` names a host-side stand-in, not
// device memory: its device address is looked up once per device with
// hipGetSymbolAddress (that device current) and only that address is used.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

fg_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FG_E_HIP;
  if (dev >= kMaxDevices) return FG_E_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return FG_E_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return FG_OK;
}

}  // namespace
}  // namespace fg

extern "C" fg_status fg_attention_ragged(const fg_plan* plan, void* d_meta, const void* q,
                                         const void* k_pool, const void* v_pool, void* out,
                                         int32_t out_dtype, float* lse, void* d_ws,
                                         size_t ws_bytes, void* stream) {
  if (!plan) return FG_E_INVALID;
  if (out_dtype != FG_DTYPE_F32 && out_dtype != FG_DTYPE_BF16) return FG_E_UNSUPPORTED;
  if (plan->n_items == 0) return FG_OK;
  const fg_status st = check_attention_args(plan, out_dtype, d_meta, q, k_pool, v_pool, out, lse);
  if (st != FG_OK) return st;
  if (plan->ws_bytes > 0 && (!d_ws || ws_bytes < plan->ws_bytes || !aligned16(d_ws)))
    return FG_E_WORKSPACE;
  return launch_attention(plan, d_meta, q, k_pool, v_pool, out, out_dtype, lse, d_ws,
                          static_cast<hipStream_t>(stream), true);
}

extern "C" fg_status fg_attention_ragged_noalloc(const fg_plan* plan, void* d_meta, const void* q,
                                                 const void* k_pool, const void* v_pool, void* out,
                                                 int32_t out_dtype, float* lse, void* stream) {
  if (!plan) return FG_E_INVALID;
  if (out_dtype != FG_DTYPE_F32 && out_dtype != FG_DTYPE_BF16) return FG_E_UNSUPPORTED;
  if (plan->n_items == 0) return FG_OK;
  fg_status st = check_attention_args(plan, out_dtype, d_meta, q, k_pool, v_pool, out, lse);
  if (st != FG_OK) return st;
  if (plan->ws_bytes > kScratchBytes) return FG_E_WORKSPACE;
  void* ws = nullptr;
  if (plan->ws_bytes > 0) {
    st = scratch_of_current_device(&ws);
    if (st != FG_OK) return st;
  }
  return launch_attention(plan, d_meta, q, k_pool, v_pool, out, out_dtype, lse, ws,
                          static_cast<hipStream_t>(stream), false);
}

extern "C" size_t fg_noalloc_scratch_bytes(void) { return kScratchBytes; }

extern "C" fg_status fg_attention_ragged_direct(const fg_plan* plan, void* d_meta, const void* q,
                                                const void* k_new, const void* v_new,
                                                const void* k_pool, const void* v_pool, void* out,
                                                int32_t out_dtype, float* lse, void* d_ws,
                                                size_t ws_bytes, void* stream) {
  if (!plan) return FG_E_INVALID;
  if (out_dtype != FG_DTYPE_F32 && out_dtype != FG_DTYPE_BF16) return FG_E_UNSUPPORTED;
  if (plan->n_items == 0) return FG_OK;
  const fg_status st = check_attention_args(plan, out_dtype, d_meta, q, k_pool, v_pool, out, lse);
  if (st != FG_OK) return st;
  if (!k_new || !v_new || !aligned16(k_new) || !aligned16(v_new)) return FG_E_INVALID;
  if (plan->ws_bytes > 0 && (!d_ws || ws_bytes < plan->ws_bytes || !aligned16(d_ws)))
    return FG_E_WORKSPACE;
  return launch_attention(plan, d_meta, q, k_pool, v_pool, out, out_dtype, lse, d_ws,
                          static_cast<hipStream_t>(stream), true, k_new, v_new, false);
}

extern "C" fg_status fg_pass(const fg_plan* plan, void* d_meta, const void* q, const void* k_new,
                             const void* v_new, void* k_pool, void* v_pool, void* out,
                             int32_t out_dtype, float* lse, void* d_ws, size_t ws_bytes, void* stream) {
  if (!plan) return FG_E_INVALID;
  if (out_dtype != FG_DTYPE_F32 && out_dtype != FG_DTYPE_BF16) return FG_E_UNSUPPORTED;
  if (plan->n_items == 0) return FG_OK;
  fg_status st = check_attention_args(plan, out_dtype, d_meta, q, k_pool, v_pool, out, lse);
  if (st != FG_OK) return st;
  if (!k_new || !v_new || !aligned16(k_new) || !aligned16(v_new)) return FG_E_INVALID;
  if (plan->ws_bytes > 0 && (!d_ws || ws_bytes < plan->ws_bytes || !aligned16(d_ws)))
    return FG_E_WORKSPACE;
  if (plan->n_tiles > 0) {
    // Prefill tiles: their stages over the pass's own tokens measured slower
    // when staged from k_new / v_new than from the pool (the V transpose goes
    // through registers), so the append runs first, fused with the upload.
    st = fg_upload_append(plan, d_meta, k_new, v_new, k_pool, v_pool, stream);
    if (st != FG_OK) return st;
    return launch_attention(plan, d_meta, q, k_pool, v_pool, out, out_dtype, lse, d_ws,
                            static_cast<hipStream_t>(stream), true);
  }
  st = fg_plan_upload(plan, d_meta, stream);
  if (st != FG_OK) return st;
  return launch_attention(plan, d_meta, q, k_pool, v_pool, out, out_dtype, lse, d_ws,
                          static_cast<hipStream_t>(stream), true, k_new, v_new, true);
}

extern "C" fg_status fg_plan_resident_slots(const fg_plan* plan, int32_t* planned, int32_t* device) {
  if (!plan || !planned || !device) return FG_E_INVALID;
  *planned = plan->resident_slots;
  *device = -1;
  int pool = 0, direct = 0;
  hipError_t e0 = hipSuccess, e1 = hipSuccess;
#define FG_OCCUPANCY(D_, B_)                                                                       \
  do {                                                                                             \
    if (plan->n_mfma > 0) {                                                                        \
      e0 = hipOccupancyMaxActiveBlocksPerMultiprocessor(&pool, attn_kernel<D_, B_, true, false>,   \
                                                        kThreads, 0);                              \
      e1 = hipOccupancyMaxActiveBlocksPerMultiprocessor(&direct, attn_kernel<D_, B_, true, true>,  \
                                                        kThreads, 0);                              \
    } else {                                                                                       \
      e0 = hipOccupancyMaxActiveBlocksPerMultiprocessor(&pool, attn_kernel<D_, B_, false, false>,  \
                                                        kThreads, 0);                              \
      e1 = hipOccupancyMaxActiveBlocksPerMultiprocessor(&direct, attn_kernel<D_, B_, false, true>, \
                                                        kThreads, 0);                              \
    }                                                                                              \
  } while (0)
  FG_SWITCH_DB(plan->head_dim, plan->block_size, FG_OCCUPANCY);
#undef FG_OCCUPANCY
  if (e0 != hipSuccess || e1 != hipSuccess) {
    (void)hipGetLastError();   // no device: leave *device at -1
    return FG_OK;
  }
  *device = pool < direct ? pool : direct;
  return FG_OK;
}

extern "C" fg_status fg_profile_enable(int32_t mask) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_mask = static_cast<uint32_t>(mask);
  return FG_OK;
}

extern "C" fg_status fg_profile_read(double* total_ms, int32_t* launches, int32_t n_kernels) {
  if (n_kernels < 0 || (n_kernels > 0 && (!total_ms || !launches))) return FG_E_INVALID;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (int i = 0; i < n_kernels; ++i) {
    total_ms[i] = 0.0;
    launches[i] = 0;
  }
  fg_status st = FG_OK;
  for (const ProfRec& r : g_prof_recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.stop) != hipSuccess ||
        hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess)
      st = FG_E_HIP;
    if (r.kind < n_kernels) {
      total_ms[r.kind] += ms;
      launches[r.kind] += 1;
    }
    g_prof_pool.push_back(r.start);
    g_prof_pool.push_back(r.stop);
  }
  g_prof_recs.clear();
  return st;
}

extern "C" const char* fg_kernel_name(int32_t id) {
  switch (id) {
    case FG_KERNEL_APPEND: return "append_kernel";
    case FG_KERNEL_ATTENTION: return "attn_kernel";
    case FG_KERNEL_MERGE: return "merge_kernel";
    default: return "unknown";
  }
}
