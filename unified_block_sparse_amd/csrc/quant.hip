// quantize_kv_int4: INT4 pages of the K/V cache for decode (blog "LServe -- Decode
// Phase" and the Figure 2 caption: INT4 KV quantization cuts the bytes of every page
// that decode reads, on top of the pages that page selection skips). The pages give no
// format; each (token, KV head) row of D channels is quantized on its own, asymmetric,
// to codes n in [0, 15]: scale = fp16((max - min) / 15), zero = fp16(min),
// n = clamp(rint((x - zero) / scale), 0, 15) in fp32 (all codes 0 when scale is 0).
// Codes sit 8 to a 32-bit word, code k in nibble k/2 of the low half (k even) or of the
// high half (k odd). K rows keep channel order (words of 8 channels); V is channel-major
// per page (for each channel, words of 8 tokens), the operand layout of decode's P.V.
//
// One work-group per (sequence, page). Per KV head: D/8 lanes share a row (16 bytes
// each), min and max by xor shuffles inside the row; K words go straight out, V codes
// go to LDS (P * D bytes) and leave as channel-major words. A V word holding no valid
// token is not written; the invalid tokens of a word that is written get code 0.
#include "common.h"
#include "launch.h"

namespace ubs {

// position of code k (0..7) in its 32-bit word
__device__ __forceinline__ int code_shift(int k) { return (k & 1) ? 16 + 4 * (k >> 1) : 4 * (k >> 1); }

template <int D>
__global__ __launch_bounds__(256) void quant_kernel(const QuantArgs a) {
  constexpr int CH = D / 8;       // lanes per row
  constexpr int RPP = 256 / CH;   // rows per pass
  constexpr int UN = 4;           // passes whose loads are issued together
  // V codes of one head's page, [row][channel]: P * D bytes of dynamic LDS, so that small
  // pages leave room for more work-groups per CU
  extern __shared__ __attribute__((aligned(16))) uint8_t vcodes[];
  const int b = blockIdx.x / a.max_pages;
  const int j = blockIdx.x % a.max_pages;
  const int n = min(a.P, a.seq_lens[b] - j * a.P);   // valid rows of the page
  if (n <= 0) return;
  const int page = a.page_table[(int64_t)b * a.max_pages + j];
  const int c = threadIdx.x % CH;
  for (int g = 0; g < a.Hkv; ++g) {
    const int64_t slab = (int64_t)page * a.Hkv + g;   // (page, KV head)
    // rows idx < n are K rows, n <= idx < 2n the V rows; UN passes' loads go out before
    // any of them is used (the lanes of a row agree on every branch)
    for (int idx0 = threadIdx.x / CH; idx0 < 2 * n; idx0 += UN * RPP) {
      u32x4 wu[UN];
#pragma unroll
      for (int u = 0; u < UN; ++u) {
        const int idx = idx0 + u * RPP;
        const int kv = idx >= n;
        const int64_t rid = slab * a.P + (idx - kv * n);
        wu[u] = idx < 2 * n ? ld16((kv ? a.v_cache : a.k_cache) + rid * D + c * 8) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < UN; ++u) {
        const int idx = idx0 + u * RPP;
        if (idx >= 2 * n) break;
        const int kv = idx >= n;
        const int row = idx - kv * n;
        const int64_t rid = slab * a.P + row;
        const u32x4 w = wu[u];
        float x[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[2 * e] = bf16_lo(w[e]);
          x[2 * e + 1] = bf16_hi(w[e]);
        }
        float lo = x[0], hi = x[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) {
          lo = fminf(lo, x[e]);
          hi = fmaxf(hi, x[e]);
        }
#pragma unroll
        for (int o = 1; o < CH; o <<= 1) {
          lo = fminf(lo, shfl_xor(lo, o));
          hi = fmaxf(hi, shfl_xor(hi, o));
        }
        const _Float16 s16 = (_Float16)__fdiv_rn(hi - lo, 15.0f);
        const _Float16 z16 = (_Float16)lo;
        const float s = (float)s16, z = (float)z16;
        // n = rint((x - z) / s) with the division correctly rounded. The quotient by the
        // correctly rounded reciprocal, q' = RN((x - z) RN(1/s)), is within 1.5 * 2^-23
        // |q| of the exact one, so rint gives the same integer unless q' lies within
        // 2^-17 of a half-integer (a bound for |q| < 16; quotients outside [-0.5, 15.5]
        // clamp whatever their last bits). A wave with such a lane divides exactly.
        const float rs = s == 0.f ? 0.f : __fdiv_rn(1.0f, s);
        float q[8];
        bool near = false;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          q[e] = (x[e] - z) * rs;
          near |= fabsf(q[e] - floorf(q[e]) - 0.5f) < 0x1p-17f;
        }
        if (__ballot(near)) {
#pragma unroll
          for (int e = 0; e < 8; ++e) q[e] = s == 0.f ? 0.f : __fdiv_rn(x[e] - z, s);
        }
        uint32_t code[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          code[e] = (uint32_t)(s == 0.f ? 0.f : fminf(fmaxf(__builtin_rintf(q[e]), 0.f), 15.f));
        if (kv == 0) {
          uint32_t word = 0;
#pragma unroll
          for (int e = 0; e < 8; ++e) word |= code[e] << code_shift(e);
          *reinterpret_cast<uint32_t*>(a.k_codes + rid * (D / 2) + c * 4) = word;
        } else {
          *reinterpret_cast<uint32_t*>(&vcodes[row * D + c * 8]) = code[0] | code[1] << 8 | code[2] << 16 | code[3] << 24;
          *reinterpret_cast<uint32_t*>(&vcodes[row * D + c * 8 + 4]) = code[4] | code[5] << 8 | code[6] << 16 | code[7] << 24;
        }
        if (c == 0) {
          uint16_t* params = kv ? a.v_params : a.k_params;
          *reinterpret_cast<uint32_t*>(params + rid * 2) =
              (uint32_t)__builtin_bit_cast(uint16_t, s16) | ((uint32_t)__builtin_bit_cast(uint16_t, z16) << 16);
        }
      }
    }
    __syncthreads();
    // V words: channel ch, tokens 8r .. 8r+7 (code 0 past the valid rows)
    const int ngr = (n + 7) / 8;
    for (int idx = threadIdx.x; idx < D * ngr; idx += 256) {
      const int ch = idx / ngr, r = idx % ngr;
      uint32_t word = 0;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int t = 8 * r + k;
        word |= (t < n ? (uint32_t)vcodes[t * D + ch] : 0u) << code_shift(k);
      }
      *reinterpret_cast<uint32_t*>(a.v_codes + (slab * D + ch) * (a.P / 2) + r * 4) = word;
    }
    __syncthreads();
  }
}

hipError_t launch_quant_int4(const QuantArgs& a, hipStream_t s) {
  const int64_t blocks = (int64_t)a.B * a.max_pages;
  if (blocks == 0) return hipSuccess;
#define UBS_QUANT(DD)                                                                   \
  if (a.D == DD) {                                                                      \
    hipLaunchKernelGGL((quant_kernel<DD>), dim3((unsigned)blocks), dim3(256), (size_t)a.P * DD, s, a); \
    return hipGetLastError();                                                           \
  }
  UBS_QUANT(64) UBS_QUANT(128)
#undef UBS_QUANT
  return hipErrorInvalidValue;
}

}  // namespace ubs
