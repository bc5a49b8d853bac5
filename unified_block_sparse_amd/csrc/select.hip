// select_pages: query-aware page scores and top-k page selection for one decode
// step (blog "LServe -- Decode Phase" and Figure 2; LServe abstract: hierarchical,
// query-centric page selection under a constant page budget).
//
// Scoring. For sub-page u with channel-wise key bounds kmin/kmax and query head h,
// the Quest bound sum_c max(q_c kmin_c, q_c kmax_c) equals, term by term,
// q-_c kmin_c + q+_c kmax_c with q+ = max(q, 0) and q- = min(q, 0). Written over the
// 2D-long record [kmin | kmax] that is one dot product with [q- | q+], so a group of
// 16 sub-page records times the G query heads of a KV head is one 16x16x(2D)
// product. bf16 x bf16 products are exact in fp32, and the kernel streams the bounds
// straight from HBM into the MFMA B operand (16-byte loads, 64 contiguous bytes per
// record per lane group).
//
// Top-k. One work-group per (sequence, KV head) finds the k-th largest score by a
// bitwise binary search over order-preserving 32-bit keys (counts by wave ballots),
// breaks ties toward the lower page index and compacts the kept indices in
// ascending order with block-wide prefix sums.
#include "common.h"
#include "launch.h"

#include <cstdlib>

namespace ubs {

__device__ __forceinline__ uint32_t neg_part_bf16x2(uint32_t w) {
  // keep each bf16 half whose sign bit is set (min(x, 0)), zero the others
  uint32_t lo = (w & 0x8000u) ? (w & 0xffffu) : 0u;
  uint32_t hi = (w & 0x80000000u) ? (w & 0xffff0000u) : 0u;
  return lo | hi;
}
__device__ __forceinline__ uint32_t pos_part_bf16x2(uint32_t w) {
  uint32_t lo = (w & 0x8000u) ? 0u : (w & 0xffffu);
  uint32_t hi = (w & 0x80000000u) ? 0u : (w & 0xffff0000u);
  return lo | hi;
}

// Grid: one work-group per (b, chunk, dense index), in the order `order` names below, wpg
// waves a work-group (one, unless a measurement override says otherwise). Each wave scores
// `gpw` groups of 16 consecutive sub-pages of its (b, g); with U = P/Lp sub-pages per
// page a group covers 16/U whole pages. At most 128 registers a lane: the allocator then
// keeps the D = 128 kernel in 81 vector registers (5 waves per SIMD) instead of 95 plus 4
// accumulation registers (4 waves); more waves keep more record loads in flight.
template <int D, int U, int G>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4)))
void score_kernel(const uint16_t* __restrict__ q,
                  const uint16_t* __restrict__ bounds,
                  const int32_t* __restrict__ page_table,
                  const int32_t* __restrict__ seq_lens,
                  int max_pages, int Hq, int Hkv, int P, int Lp,
                  HeadList dense, int chunks, int wpg, int gpw, int order,
                  float* __restrict__ scores) {
  constexpr int KK = D / 16;  // MFMA steps over the 2D-long record (K = 32 each)
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  // order 1 (the default): the dense heads of one (b, chunk) on consecutive work-groups,
  // so that the records of one page for all dense heads (adjacent in the bounds) are read
  // at about the same time, and the waves of one work-group round have rows of one length
  // (ragged batch: selection 128.7-130.0 against 131.6-132.7 us); order 0: the chunks of
  // one (b, g) row on consecutive work-groups
  int chunk, di, b;
  if (order == 0) {
    chunk = blockIdx.x % chunks;
    const int bd = blockIdx.x / chunks;
    di = bd % dense.n;
    b = bd / dense.n;
  } else {
    di = blockIdx.x % dense.n;
    const int bc = blockIdx.x / dense.n;
    chunk = bc % chunks;
    b = bc / chunks;
  }
  const int g = dense.h[di];
  const int L = seq_lens[b];
  const int n_pages = (L + P - 1) / P;
  const int n_sub = n_pages * U;
  const int first_group = (chunk * wpg + wave) * gpw;
  if (first_group * 16 >= n_sub) return;

  // A operand: row m = query head of the group, k-slot (l/16)*8 + i of step kk maps
  // to record element kk*32 + (l/16)*8 + i.
  const int m = lane & 15;
  const int qg = lane >> 4;
  bf16x8 a[KK];
  {
    u32x4 qv[D / 32];
    const uint16_t* qrow = q + ((int64_t)b * Hq + (int64_t)g * G + m) * D + qg * 8;
#pragma unroll
    for (int t = 0; t < D / 32; ++t) qv[t] = (m < G) ? ld16(qrow + t * 32) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4 w;
      if (kk < D / 32) {
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = neg_part_bf16x2(qv[kk][e]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = pos_part_bf16x2(qv[kk - D / 32][e]);
      }
      a[kk] = as_bf16x8(w);
    }
  }

  const int32_t* pt = page_table + (int64_t)b * max_pages;
  float* out = scores + ((int64_t)b * Hkv + g) * max_pages;
  // the page-table entries of all the wave's groups first, so that each group's record
  // loads do not wait on a page-table load of their own (gpw <= 2)
  int32_t pg[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int s = (first_group + t) * 16 + m;
    pg[t] = (t < gpw && s < n_sub) ? pt[s / U] : 0;
  }
  for (int t = 0; t < gpw; ++t) {
    const int grp = first_group + t;
    if (grp * 16 >= n_sub) break;  // wave-uniform
    const int s = grp * 16 + m;   // this lane's sub-page (B column)
    const int j = s / U;
    const int u = s % U;
    const bool ok = (s < n_sub) && (j * P + u * Lp < L);
    u32x4 bv[KK];
    if (ok) {
      const uint16_t* rec = bounds + (((int64_t)(t == 0 ? pg[0] : pg[1]) * Hkv + g) * U + u) * (2 * D) + qg * 8;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) bv[kk] = ld16(rec + kk * 32);
    } else {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) bv[kk] = u32x4{0, 0, 0, 0};
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[kk], as_bf16x8(bv[kk]), acc, 0, 0, 0);
    // acc[i] = bound of query head 4*(l/16)+i on sub-page l%16
    float v = kNegInf;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (qg * 4 + i < G) v = fmaxf(v, acc[i]);
    if (G > 4) v = fmaxf(v, shfl_xor(v, 16));
    if (G > 8) v = fmaxf(v, shfl_xor(v, 32));
    if (!ok) v = kNegInf;
#pragma unroll
    for (int o = 1; o < U; o <<= 1) v = fmaxf(v, shfl_xor(v, o));
    if (lane < 16 && (u == 0) && j < n_pages) out[j] = v;
  }
}

// ----------------------------------------------------------------------------- top-k

// Block-wide exclusive prefix sum of a count v in [0, 128) per thread (4 waves): the wave
// prefix from ballots, then the four wave totals through LDS.
__device__ __forceinline__ int block_exclusive_scan(int v, int* tmp, int& total) {
  const int lane = lane_id(), w = threadIdx.x >> 6;
  int wt;
  const int pre = wave_prefix_small<7>(v, wt);
  if (lane == 0) tmp[w] = wt;
  __syncthreads();
  int base = 0;
  total = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = tmp[i];
    base += (i < w) ? t : 0;
    total += t;
  }
  __syncthreads();
  return base + pre;
}

// One 256-thread work-group per (b, KV head). Thread t owns pages t*EPT .. t*EPT+EPT-1,
// so thread order is page order.
template <int EPT>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ scores,
                                                   const int32_t* __restrict__ seq_lens,
                                                   int max_pages, int Hkv, int P, int k,
                                                   uint64_t streaming_mask,
                                                   int32_t* __restrict__ selected,
                                                   int32_t* __restrict__ num_selected) {
  __shared__ int tmp[4];
  __shared__ int cnt[2][4];
  __shared__ uint32_t rng[2][4];
  const int bg = blockIdx.x;
  const int g = bg % Hkv;
  const int b = bg / Hkv;
  const int tid = threadIdx.x;
  int32_t* sel = selected + (int64_t)bg * k;
  const bool streaming = (streaming_mask >> g) & 1ull;
  const int L = seq_lens[b];
  const int n = streaming ? 0 : (L + P - 1) / P;
  if (n <= k) {
    for (int i = tid; i < k; i += 256) sel[i] = (i < n) ? i : -1;
    if (tid == 0) num_selected[bg] = n;
    return;
  }
  const float* sc = scores + (int64_t)bg * max_pages;
  uint32_t key[EPT];
  uint32_t kmin = ~0u, kmax = 0u;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int j = tid * EPT + e;
    key[e] = (j < n) ? float_order_key(sc[j]) : 0u;  // valid keys are > 0
    if (j < n) {
      kmin = min(kmin, key[e]);
      kmax = max(kmax, key[e]);
    }
  }
  // k-th largest key: the largest tau with #(key >= tau) >= k. A candidate with exactly
  // k keys at or above it ends the search early: those keys are the k largest, with no
  // tie at the threshold (it falls between the k-th and the (k+1)-th key, whose bits
  // first differ at this round), and the selection below takes exactly them. (total
  // is the same in every thread, so the exit is uniform.)
  const int w = tid >> 6, lane = lane_id();
  // every key, and so the k-th largest, shares the bits above the first bit where the
  // smallest and the largest key differ: the search starts there
  wave_min_max_u32(kmin, kmax);
  if (lane == 0) {
    rng[0][w] = kmin;
    rng[1][w] = kmax;
  }
  __syncthreads();
  kmin = min(min(rng[0][0], rng[0][1]), min(rng[0][2], rng[0][3]));
  kmax = max(max(rng[1][0], rng[1][1]), max(rng[1][2], rng[1][3]));
  const int top = kmin == kmax ? -1 : 31 - __builtin_clz(kmin ^ kmax);
  uint32_t tau = kmin == kmax ? kmax : (top == 31 ? 0u : (kmax & ~((2u << top) - 1u)));
  for (int bit = top; bit >= 0; --bit) {
    const uint32_t cand = tau | (1u << bit);
    int c = 0;
#pragma unroll
    for (int e = 0; e < EPT; ++e) c += __popcll(__ballot(key[e] >= cand));
    const int slot = bit & 1;
    if (lane == 0) cnt[slot][w] = c;
    __syncthreads();
    const int total = cnt[slot][0] + cnt[slot][1] + cnt[slot][2] + cnt[slot][3];
    if (total >= k) tau = cand;
    if (total == k) break;
  }
  // #(key > tau) < k <= #(key >= tau) (after an early exit: #(key >= tau) = k and every
  // key equal to tau is taken): take all keys above tau and the lowest-index ties.
  int gt = 0, ties = 0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    gt += key[e] > tau;
    ties += key[e] == tau;
  }
  int n_gt;
  {
    int tot;
    block_exclusive_scan(gt, tmp, tot);
    n_gt = tot;
  }
  int tie_total;
  int tie_rank = block_exclusive_scan(ties, tmp, tie_total);
  const int take_ties = k - n_gt;
  bool keep[EPT];
  int kept = 0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    bool kp = key[e] > tau;
    if (key[e] == tau) {
      kp = tie_rank < take_ties;
      ++tie_rank;
    }
    keep[e] = kp;
    kept += kp;
  }
  int kept_total;
  int pos = block_exclusive_scan(kept, tmp, kept_total);
#pragma unroll
  for (int e = 0; e < EPT; ++e)
    if (keep[e]) sel[pos++] = tid * EPT + e;
  if (tid == 0) num_selected[bg] = k;
}

template <int D, int U>
static hipError_t launch_score_du(const SelectArgs& a, int G, int chunks, int wpg, int gpw, int order,
                                  hipStream_t s) {
  const dim3 grid((unsigned)(a.B * a.dense.n * chunks));
#define UBS_SCORE_G(GG)                                                                          \
  if (G == GG) {                                                                                 \
    hipLaunchKernelGGL((score_kernel<D, U, GG>), grid, dim3(64 * wpg), 0, s, a.q, a.bounds,      \
                       a.page_table, a.seq_lens, a.max_pages, a.Hq, a.Hkv, a.P, a.Lp, a.dense,   \
                       chunks, wpg, gpw, order, a.scores);                                       \
    return hipGetLastError();                                                                    \
  }
  UBS_SCORE_G(1) UBS_SCORE_G(2) UBS_SCORE_G(4) UBS_SCORE_G(8) UBS_SCORE_G(16)
#undef UBS_SCORE_G
  return hipErrorInvalidValue;
}

hipError_t launch_select(const SelectArgs& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  const int G = a.Hq / a.Hkv;
  const int U = a.P / a.Lp;
  if (a.dense.n > 0) {
    // groups of 16 sub-pages per (b, dense g); a wave takes gpw groups. One wave a
    // work-group (wpg = 1): the waves past a short row's end then leave the CU at once
    // instead of holding a 4-wave group's slot while its other waves stream, and small
    // launches reach every CU (ragged batch: selection 132-133 against 142 us with 4-wave
    // groups; Llama-3-8B decode step 27.2 against 27.7 us).
    // One group a wave: with the head-inner work-group order, 1 group (4 pages at Lp = 16)
    // a wave beat 2 on the ragged batch (selection 127.8-128.9 against 131.6-132.4 us, two
    // alternations on one box; 2 groups with 2-wave work-groups 128.6-129.6).
    const int64_t groups = ((int64_t)a.max_pages * U + 15) / 16;
    int gpw = 1;
    // (measurement overrides: UBS_SCORE_GPW sets the groups per wave, 1 or 2, and
    // UBS_SCORE_WPG the waves per work-group, 1, 2 or 4; the scores do not depend on them)
    if (const char* env = getenv("UBS_SCORE_GPW")) {
      const int v = atoi(env);
      if (v == 1 || v == 2) gpw = v;
    }
    int wpg = 1;
    if (const char* env = getenv("UBS_SCORE_WPG")) {
      const int v = atoi(env);
      if (v == 1 || v == 2 || v == 4) wpg = v;
    }
    int order = 1;
    if (const char* env = getenv("UBS_SCORE_ORDER")) {   // (measurement override: 0 or 1)
      const int v = atoi(env);
      if (v == 0 || v == 1) order = v;
    }
    const int chunks = (int)((groups + wpg * gpw - 1) / (wpg * gpw));
    hipError_t e = hipErrorInvalidValue;
#define UBS_SCORE_DU(DD, UU) \
    if (a.D == DD && U == UU) e = launch_score_du<DD, UU>(a, G, chunks, wpg, gpw, order, s);
    UBS_SCORE_DU(64, 1) UBS_SCORE_DU(64, 2) UBS_SCORE_DU(64, 4) UBS_SCORE_DU(64, 8) UBS_SCORE_DU(64, 16)
    UBS_SCORE_DU(128, 1) UBS_SCORE_DU(128, 2) UBS_SCORE_DU(128, 4) UBS_SCORE_DU(128, 8) UBS_SCORE_DU(128, 16)
#undef UBS_SCORE_DU
    if (e != hipSuccess) return e;
  }
  if (a.score_only) return hipSuccess;
  const dim3 grid((unsigned)(a.B * a.Hkv));
  const int need = (a.max_pages + 255) / 256;
#define UBS_TOPK(E)                                                                               \
  if (need <= E) {                                                                                \
    hipLaunchKernelGGL((topk_kernel<E>), grid, dim3(256), 0, s, a.scores, a.seq_lens, a.max_pages, \
                       a.Hkv, a.P, a.k, a.streaming_mask, a.selected, a.num_selected);            \
    return hipGetLastError();                                                                     \
  }
  UBS_TOPK(1) UBS_TOPK(2) UBS_TOPK(4) UBS_TOPK(8) UBS_TOPK(16) UBS_TOPK(32) UBS_TOPK(64)
#undef UBS_TOPK
  return hipErrorInvalidValue;
}

}  // namespace ubs
