// build_page_bounds: per-page, per-channel key min/max over the valid tokens of
// every Lp-token sub-page (the page summary of the LServe decode selector; blog
// "LServe -- Decode Phase", Figure 2). HBM-bound: each (page, dense head) pair is
// one wave that streams its P x D keys once, one whole key row per load instruction.
#include "common.h"
#include "launch.h"

namespace ubs {

__device__ __forceinline__ float vmin(float a, float b) { return __builtin_elementwise_minimum(a, b); }
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// min and max of v with its partner lane l ^ 32 (the half-wave swap, one vector
// instruction where a shuffle is an LDS round trip). The minimum / maximum used here
// propagate NaN and need no operand canonicalisation (fminf / fmaxf cost an extra
// instruction per operand); on the finite keys of a cache they are the same min and max.
template <int M>
__device__ __forceinline__ void min_max_xor(float& mn, float& mx) {
  static_assert(M == 32, "half-wave swap only");
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(mn), __float_as_uint(mn), false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
  mn = vmin(__uint_as_float(a[0]), __uint_as_float(a[1]));
  mx = vmax(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// One wave per (sequence b, page index j, dense KV head); after an append of n_new
// tokens, one wave per (b, page holding new tokens, dense KV head), recomputing only the
// sub-pages that received new tokens (over all their valid tokens, old and new). Lane
// layout: CH = D/2 lanes cover one key row, a 32-bit word (two channels) each, so one
// load instruction reads whole rows (256 contiguous bytes at D = 128); RG = 64/CH row
// groups (1 at D = 128, 2 at D = 64) take rows rg, rg + RG, ... The whole page is loaded
// up front (rows past the sequence end are inside the page, so the loads stay in bounds)
// and only valid rows enter the reduction, which runs inside each lane over its rows: at
// D = 128 no value crosses lanes, at D = 64 one half-wave swap.
// LPC: the sub-page size Lp fixed at compile time (0: taken from the argument). With it,
// the rows of a whole sub-page are the same register slots in every lane (i in
// [u Lp / RG, (u + 1) Lp / RG)), so a full sub-page reduces without a per-row test, two
// rows per three-input min / max; the sub-page holding the sequence end (and every
// sub-page when LPC = 0) takes the per-row test.
template <int D, int P, int LPC>
__global__ __launch_bounds__(256) void bounds_kernel(const uint16_t* __restrict__ k_cache,
                                                     const int32_t* __restrict__ page_table,
                                                     const int32_t* __restrict__ seq_lens,
                                                     int max_pages, int Hkv, int Lp_arg, HeadList dense,
                                                     int n_new, int page_span, int64_t n_items,
                                                     uint16_t* __restrict__ bounds) {
  constexpr int CH = D / 2;
  constexpr int RG = 64 / CH;
  constexpr int NR = P / RG;  // rows per lane
  static_assert(LPC == 0 || (LPC % RG == 0 && P % LPC == 0), "compile-time sub-page size");
  const int Lp = LPC > 0 ? LPC : Lp_arg;
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
  const int c = lane % CH;   // channels 2c, 2c + 1
  const int rg = lane / CH;
  const uint32_t* src = reinterpret_cast<const uint32_t*>(k_cache + (((int64_t)p * Hkv + g) * P) * D) + c;

  uint32_t rows[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) rows[i] = src[(rg + RG * i) * (D / 2)];

  const int U = P / Lp;
  // sub-page u's record: D/2 words of minima, then D/2 words of maxima
  uint32_t* dst_base = reinterpret_cast<uint32_t*>(bounds + (((int64_t)p * Hkv + g) * U) * 2 * D) + c;
#pragma unroll
  for (int u = 0; u < (LPC > 0 ? P / LPC : U); ++u) {
    const int lo = u * Lp;
    if (lo >= valid) break;
    if (j * P + lo + Lp <= from) continue;   // no new token in this sub-page (updates only)
    const int hi = min(lo + Lp, valid);
    // (an empty asm that claims to change the rows: the rows do not change over the
    // sub-page loop, so the compiler would otherwise convert every value to fp32 once,
    // ahead of it, and keep them all live beside the raw rows)
#pragma unroll
    for (int i = 0; i < NR; ++i) asm volatile("" : "+v"(rows[i]));
    float mn0 = __builtin_inff(), mn1 = __builtin_inff(), mx0 = -__builtin_inff(), mx1 = -__builtin_inff();
    if (LPC > 0 && hi == lo + Lp) {
      // a whole sub-page: rows i in [u LPC / RG, (u + 1) LPC / RG) of every lane
#pragma unroll
      for (int i = (LPC > 0 ? u * LPC / RG : 0); i < (LPC > 0 ? (u + 1) * LPC / RG : 0); ++i) {
        const float a = bf16_lo(rows[i]), bb = bf16_hi(rows[i]);
        mn0 = vmin(mn0, a);
        mx0 = vmax(mx0, a);
        mn1 = vmin(mn1, bb);
        mx1 = vmax(mx1, bb);
      }
    } else {
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        const int r = rg + RG * i;
        if (r >= lo && r < hi) {
          const float a = bf16_lo(rows[i]), bb = bf16_hi(rows[i]);
          mn0 = vmin(mn0, a);
          mx0 = vmax(mx0, a);
          mn1 = vmin(mn1, bb);
          mx1 = vmax(mx1, bb);
        }
      }
    }
    if constexpr (RG == 2) {   // the two row groups (half-waves)
      min_max_xor<32>(mn0, mx0);
      min_max_xor<32>(mn1, mx1);
    }
    if (rg == 0) {
      // min/max of bf16 values are bf16 values: the truncation below is exact.
      uint32_t* dst = dst_base + (int64_t)u * D;
      dst[0] = (__float_as_uint(mn0) >> 16) | (__float_as_uint(mn1) & 0xffff0000u);
      dst[D / 2] = (__float_as_uint(mx0) >> 16) | (__float_as_uint(mx1) & 0xffff0000u);
    }
  }
}

template <int D, int P, int LPC>
static hipError_t launch_bounds_t(const BoundsArgs& a, hipStream_t s) {
  const int64_t n_items = (int64_t)a.B * a.page_span * a.dense.n;
  if (n_items == 0) return hipSuccess;
  const int64_t blocks = (n_items + 3) / 4;
  hipLaunchKernelGGL((bounds_kernel<D, P, LPC>), dim3((unsigned)blocks), dim3(256), 0, s, a.k_cache,
                     a.page_table, a.seq_lens, a.max_pages, a.Hkv, a.Lp, a.dense, a.n_new, a.page_span,
                     n_items, a.bounds);
  return hipGetLastError();
}

hipError_t launch_bounds(const BoundsArgs& a, hipStream_t s) {
  // a compile-time sub-page size for whole pages (Lp = P) and for 16-token sub-pages
#define UBS_BOUNDS_CASE(DD, PP)                                                \
  if (a.D == DD && a.P == PP) {                                                \
    if (a.Lp == PP) return launch_bounds_t<DD, PP, PP>(a, s);                  \
    if (a.Lp == 16 && PP > 16) return launch_bounds_t<DD, PP, (PP > 16 ? 16 : PP)>(a, s); \
    return launch_bounds_t<DD, PP, 0>(a, s);                                   \
  }
  UBS_BOUNDS_CASE(64, 16) UBS_BOUNDS_CASE(64, 32) UBS_BOUNDS_CASE(64, 64) UBS_BOUNDS_CASE(64, 128)
  UBS_BOUNDS_CASE(128, 16) UBS_BOUNDS_CASE(128, 32) UBS_BOUNDS_CASE(128, 64) UBS_BOUNDS_CASE(128, 128)
#undef UBS_BOUNDS_CASE
  return hipErrorInvalidValue;
}

}  // namespace ubs
