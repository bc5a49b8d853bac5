// build_page_bounds: per-page, per-channel key min/max over the valid tokens of
// every Lp-token sub-page (the page summary of the LServe decode selector; blog
// "LServe -- Decode Phase", Figure 2). HBM-bound: each (page, dense head) pair is
// one wave that streams its P x D keys once with 16-byte coalesced loads.
#include "common.h"
#include "launch.h"

namespace ubs {

// min and max of v with its partner lane l ^ m for m = 8, 16, 32: a DPP rotate by 8
// inside each 16-lane row, or the row-pair / half-wave swap (one vector instruction each,
// where a shuffle is an LDS round trip)
template <int M>
__device__ __forceinline__ void min_max_xor(float& mn, float& mx) {
  if constexpr (M == 8) {
    mn = fminf(mn, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(mn), 0x128, 0xF, 0xF, false)));
    mx = fmaxf(mx, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(mx), 0x128, 0xF, 0xF, false)));
  } else if constexpr (M == 16) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(mn), __float_as_uint(mn), false, false);
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    mn = fminf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    mx = fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
  } else {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(mn), __float_as_uint(mn), false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    mn = fminf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    mx = fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
  }
}

// One wave per (sequence b, page index j, dense KV head); after an append of n_new
// tokens, one wave per (b, page holding new tokens, dense KV head), recomputing only the
// sub-pages that received new tokens (over all their valid tokens, old and new). Lane layout: CH = D/8
// lanes cover one key row (8 channels = 16 bytes each), RG = 64/CH row groups
// take rows rg, rg + RG, ... The whole page is loaded up front (rows past the
// sequence end are inside the page, so the loads stay in bounds) and only valid
// rows enter the reduction.
template <int D, int P>
__global__ __launch_bounds__(256) void bounds_kernel(const uint16_t* __restrict__ k_cache,
                                                     const int32_t* __restrict__ page_table,
                                                     const int32_t* __restrict__ seq_lens,
                                                     int max_pages, int Hkv, int Lp, HeadList dense,
                                                     int n_new, int page_span, int64_t n_items,
                                                     uint16_t* __restrict__ bounds) {
  constexpr int CH = D / 8;
  constexpr int RG = 64 / CH;
  constexpr int NR = P / RG;  // rows per lane
  const int lane = lane_id();
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= n_items) return;
  const int nd = dense.n;
  const int di = (int)(item % nd);
  const int64_t bj = item / nd;
  const int b = (int)(bj / page_span);
  // an update after an append covers the pages from the one holding the first new token
  const int from = n_new > 0 ? seq_lens[b] : 0;
  const int j = (int)(bj % page_span) + from / P;
  const int L = seq_lens[b] + n_new;
  if (j >= max_pages) return;
  const int valid = min(P, L - j * P);
  if (valid <= 0) return;
  const int g = dense.h[di];
  const int p = page_table[(int64_t)b * max_pages + j];
  const int c = lane % CH;
  const int rg = lane / CH;
  const uint16_t* src = k_cache + (((int64_t)p * Hkv + g) * P) * D + c * 8;

  u32x4 rows[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) rows[i] = ld16(src + (int64_t)(rg + RG * i) * D);

  const int U = P / Lp;
  uint16_t* dst_base = bounds + (((int64_t)p * Hkv + g) * U) * 2 * D + c * 8;
  for (int u = 0; u < U; ++u) {
    const int lo = u * Lp;
    if (lo >= valid) break;
    if (j * P + lo + Lp <= from) continue;   // no new token in this sub-page (updates only)
    const int hi = min(lo + Lp, valid);
    // (an empty asm that claims to change the rows: the rows do not change over the
    // sub-page loop, so the compiler would convert all NR x 8 values to fp32 once, ahead
    // of it, and keep them live beside the raw rows, 192 registers at D = 128, P = 64 and
    // two waves per SIMD instead of 118 and four)
#pragma unroll
    for (int i = 0; i < NR; ++i) asm volatile("" : "+v"(rows[i]));
    float mn[8], mx[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) { mn[e] = __builtin_inff(); mx[e] = -__builtin_inff(); }
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int r = rg + RG * i;
      if (r >= lo && r < hi) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float a = bf16_lo(rows[i][e]), bb = bf16_hi(rows[i][e]);
          mn[2 * e] = fminf(mn[2 * e], a);
          mx[2 * e] = fmaxf(mx[2 * e], a);
          mn[2 * e + 1] = fminf(mn[2 * e + 1], bb);
          mx[2 * e + 1] = fmaxf(mx[2 * e + 1], bb);
        }
      }
    }
    // across the RG row groups (lanes CH, 2 CH, ... apart)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if constexpr (CH <= 8) min_max_xor<8>(mn[e], mx[e]);
      min_max_xor<16>(mn[e], mx[e]);
      min_max_xor<32>(mn[e], mx[e]);
    }
    if (rg == 0) {
      u32x4 vmin, vmax;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // min/max of bf16 values are bf16 values: the truncation below is exact.
        vmin[e] = (__float_as_uint(mn[2 * e]) >> 16) | (__float_as_uint(mn[2 * e + 1]) & 0xffff0000u);
        vmax[e] = (__float_as_uint(mx[2 * e]) >> 16) | (__float_as_uint(mx[2 * e + 1]) & 0xffff0000u);
      }
      uint16_t* dst = dst_base + (int64_t)u * 2 * D;
      st16(dst, vmin);
      st16(dst + D, vmax);
    }
  }
}

template <int D, int P>
static hipError_t launch_bounds_t(const BoundsArgs& a, hipStream_t s) {
  const int64_t n_items = (int64_t)a.B * a.page_span * a.dense.n;
  if (n_items == 0) return hipSuccess;
  const int64_t blocks = (n_items + 3) / 4;
  hipLaunchKernelGGL((bounds_kernel<D, P>), dim3((unsigned)blocks), dim3(256), 0, s, a.k_cache,
                     a.page_table, a.seq_lens, a.max_pages, a.Hkv, a.Lp, a.dense, a.n_new, a.page_span,
                     n_items, a.bounds);
  return hipGetLastError();
}

hipError_t launch_bounds(const BoundsArgs& a, hipStream_t s) {
#define UBS_BOUNDS_CASE(DD, PP) \
  if (a.D == DD && a.P == PP) return launch_bounds_t<DD, PP>(a, s);
  UBS_BOUNDS_CASE(64, 16) UBS_BOUNDS_CASE(64, 32) UBS_BOUNDS_CASE(64, 64) UBS_BOUNDS_CASE(64, 128)
  UBS_BOUNDS_CASE(128, 16) UBS_BOUNDS_CASE(128, 32) UBS_BOUNDS_CASE(128, 64) UBS_BOUNDS_CASE(128, 128)
#undef UBS_BOUNDS_CASE
  return hipErrorInvalidValue;
}

}  // namespace ubs
