// Device helpers shared by the gfx950 kernels of libubs.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ubs {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

// Largest KV-head count a head-kind bitmask can describe.
constexpr int kMaxKvHeads = 64;
constexpr int kMaxQHeads = 256;
// Longest kept-tile list one prefill work-group holds (query tiles per sequence).
constexpr int kMaxTileList = 4096;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round-to-nearest-even fp32 -> bf16 bits (inputs here are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two fp32 -> packed bf16x2 (lo in bits 0..15), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16-byte global load / store helpers.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }
__device__ __forceinline__ int shfl_xor(int v, int m) { return __shfl_xor(v, m, 64); }

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Online-softmax helpers in the log2 domain. A running max of -inf means "no key yet".
__device__ __forceinline__ float rescale_factor(float m_old, float m_new) {
  return (m_new == kNegInf) ? 1.0f : fast_exp2(m_old - m_new);
}
__device__ __forceinline__ float softmax_weight(float s, float m) {
  return (m == kNegInf) ? 0.0f : fast_exp2(s - m);
}

// Order-preserving map from fp32 to uint32 (larger float -> larger key). NaN is not expected.
__device__ __forceinline__ uint32_t float_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum over the wave of a count v in [0, 2^BITS), and its total, from
// BITS ballots (bit b of every lane's count) and the count of set bits in the lanes below:
// no LDS round trip, where a shuffle scan takes six.
template <int BITS>
__device__ __forceinline__ int wave_prefix_small(int v, int& total) {
  int pre = 0;
  total = 0;
#pragma unroll
  for (int bit = 0; bit < BITS; ++bit) {
    const uint64_t m = __ballot((v >> bit) & 1);
    const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    pre += below << bit;
    total += __popcll(m) << bit;
  }
  return pre;
}
// min and max of v over the wave: DPP row permutes (neighbours, pairs, half-row and row
// mirrors) within each 16-lane row, then the row-pair and half-wave swaps
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v, int sel) {
  switch (sel) {
    case 0: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
    case 1: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);
    case 2: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false);
    default: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false);
  }
}
__device__ __forceinline__ void wave_min_max_u32(uint32_t& lo, uint32_t& hi) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    lo = min(lo, dpp_u32(lo, k));
    hi = max(hi, dpp_u32(hi, k));
  }
  auto a16 = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
  auto b16 = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
  lo = min(a16[0], a16[1]);
  hi = max(b16[0], b16[1]);
  auto a32 = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
  auto b32 = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
  lo = min(a32[0], a32[1]);
  hi = max(b32[0], b32[1]);
}
}  // namespace ubs
