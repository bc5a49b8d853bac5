// quantize_kv_int4: INT4 pages of the K/V cache for decode (blog "LServe -- Decode
// Phase" and the Figure 2 caption: INT4 KV quantization cuts the bytes of every page
// that decode reads, on top of the pages that page selection skips). The pages give no
// format; each (token, KV head) row of D channels is quantized on its own, asymmetric,
// to codes n in [0, 15]: scale = fp16((max - min) / 15), zero = fp16(min),
// n = clamp(rint((x - zero) / scale), 0, 15) in fp32 (all codes 0 when scale is 0);
// two codes per byte, channel 2i in the low nibble.
//
// One work-group per (sequence, page): the valid rows of the page, every KV head, K and
// V. D/8 lanes share a row (16 bytes each); min and max by xor shuffles inside the row.
#include "common.h"
#include "launch.h"

namespace ubs {

template <int D>
__global__ __launch_bounds__(256) void quant_kernel(const QuantArgs a) {
  constexpr int CH = D / 8;       // lanes per row
  constexpr int RPP = 256 / CH;   // rows per pass
  const int b = blockIdx.x / a.max_pages;
  const int j = blockIdx.x % a.max_pages;
  const int n = min(a.P, a.seq_lens[b] - j * a.P);   // valid rows of the page
  if (n <= 0) return;
  const int page = a.page_table[(int64_t)b * a.max_pages + j];
  const int c = threadIdx.x % CH;
  const int per_kv = a.Hkv * n;
  for (int idx = threadIdx.x / CH; idx < 2 * per_kv; idx += RPP) {   // (the lanes of a row agree)
    const int kv = idx / per_kv;
    const int g = (idx % per_kv) / n;
    const int row = (idx % per_kv) % n;
    const int64_t rid = ((int64_t)page * a.Hkv + g) * a.P + row;
    const u32x4 w = ld16((kv ? a.v_cache : a.k_cache) + rid * D + c * 8);
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
    uint32_t packed = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float t = s == 0.f ? 0.f : fminf(fmaxf(__builtin_rintf(__fdiv_rn(x[e] - z, s)), 0.f), 15.f);
      packed |= (uint32_t)t << (4 * e);
    }
    uint8_t* codes = kv ? a.v_codes : a.k_codes;
    *reinterpret_cast<uint32_t*>(codes + rid * (D / 2) + c * 4) = packed;
    if (c == 0) {
      uint16_t* params = kv ? a.v_params : a.k_params;
      *reinterpret_cast<uint32_t*>(params + rid * 2) =
          (uint32_t)__builtin_bit_cast(uint16_t, s16) | ((uint32_t)__builtin_bit_cast(uint16_t, z16) << 16);
    }
  }
}

hipError_t launch_quant_int4(const QuantArgs& a, hipStream_t s) {
  const int64_t blocks = (int64_t)a.B * a.max_pages;
  if (blocks == 0) return hipSuccess;
#define UBS_QUANT(DD)                                                                   \
  if (a.D == DD) {                                                                      \
    hipLaunchKernelGGL((quant_kernel<DD>), dim3((unsigned)blocks), dim3(256), 0, s, a); \
    return hipGetLastError();                                                           \
  }
  UBS_QUANT(64) UBS_QUANT(128)
#undef UBS_QUANT
  return hipErrorInvalidValue;
}

}  // namespace ubs
