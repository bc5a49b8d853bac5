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
// One work-group per (sequence, page). Per KV head: D/16 lanes share a row (16 channels,
// 32 bytes each), min and max by xor shuffles inside the row; K words go straight out, V
// codes go to LDS (P * D bytes) and leave as channel-major words. A V word holding no
// valid token is not written; the invalid tokens of a word that is written get code 0.
//
// The kernel is bound by vector instructions, not bytes, so the common case spends few
// per code: x - zero, then fma(x - zero, RN(1/scale), 1.5 * 2^23), whose low mantissa
// bits hold the rounded quotient (ulp 1 there), clamped to [0, 15] as an integer; a
// second fma gives the distance of the unrounded product from that integer, and a wave
// where some lane's distance comes within 2^-17 of 1/2 redoes its codes with correctly
// rounded division.
#include "common.h"
#include "launch.h"

namespace ubs {

// position of code k (0..7) in its 32-bit word
__device__ __forceinline__ int code_shift(int k) { return (k & 1) ? 16 + 4 * (k >> 1) : 4 * (k >> 1); }

template <int D>
__global__ __launch_bounds__(256) void quant_kernel(const QuantArgs a) {
  constexpr int EPL = 16;         // channels per lane
  constexpr int CH = D / EPL;     // lanes per row
  constexpr int RPP = 256 / CH;   // rows per round
  constexpr float kMagic = 0x1.8p23f;           // 1.5 * 2^23: sums in [2^23, 2^24) have ulp 1
  constexpr int32_t kMagicBits = 0x4B400000;    // its bit pattern; code n is kMagicBits + n
  // the nibble words built by shift-and-add from kMagicBits + n carry this constant
  constexpr uint32_t kWordBias = [] {
    uint32_t w = 0;
    for (int k = 0; k < 8; ++k) w += (uint32_t)kMagicBits << ((k & 1) ? 16 + 4 * (k >> 1) : 4 * (k >> 1));
    return w;
  }();
  // V codes of one head's page, [row][channel]: P * D bytes of dynamic LDS, so that small
  // pages leave room for more work-groups per CU
  extern __shared__ __attribute__((aligned(16))) uint8_t vcodes[];
  const int b = blockIdx.x / a.max_pages;
  const int j = blockIdx.x % a.max_pages;
  const int n = min(a.P, a.seq_lens[b] - j * a.P);   // valid rows of the page
  if (n <= 0) return;
  const int page = a.page_table[(int64_t)b * a.max_pages + j];
  const int c = threadIdx.x % CH;
  const int row0 = threadIdx.x / CH;
  // Rounds of RPP rows, one row a lane group: per KV head RK rounds of K rows, then RK of
  // V rows, so that a round's tensor and (page, head) base are uniform and lanes address
  // with 32-bit offsets. One round's loads at a time keeps the kernel at 7 waves per SIMD
  // (two rounds' loads in flight: 79 registers, 6 waves, 5% slower; four: 4 waves, 9%).
  const int RK = (n + RPP - 1) / RPP;
  const int R = 2 * RK;
  const int total = a.Hkv * R;
  for (int kr = 0; kr < total; ++kr) {
    const int g = kr / R, h = kr - g * R;
    const bool kv = h >= RK;
    const int row = (kv ? h - RK : h) * RPP + row0;
    const int64_t slab = (int64_t)page * a.Hkv + g;   // (page, KV head)
    const int64_t first = slab * a.P;                 // its first row
    if (row < n) {   // the lanes of a row agree on every branch
      const char* src = reinterpret_cast<const char*>((kv ? a.v_cache : a.k_cache) + first * D);
      const uint32_t off = (uint32_t)(row * D + c * EPL) * 2u;   // bytes
      const u32x4 w0 = ld16(src + off), w1 = ld16(src + off + 16);
      float x[EPL];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[2 * e] = bf16_lo(w0[e]);
        x[2 * e + 1] = bf16_hi(w0[e]);
        x[8 + 2 * e] = bf16_lo(w1[e]);
        x[9 + 2 * e] = bf16_hi(w1[e]);
      }
      float lo = x[0], hi = x[0];
#pragma unroll
      for (int e = 1; e < EPL; ++e) {
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
      const float rs = s == 0.f ? 0.f : __fdiv_rn(1.0f, s);
      // Common case. With p = RN(x - z) RN(1/s) (exact inside the fma), t = RN(p + kMagic)
      // is kMagic + rint(p) for |p| < 2^22 and far = |p - rint(p)| to within 2^-25. p is
      // within 2^-23 |q| of the exact quotient q (two roundings), under 2^-19 for q in
      // [-1/2, 31/2], the only range where the code is not a clamp bound; so when far
      // stays 2^-17 below 1/2, q rounds to the same integer as p. Outside that range the
      // clamp gives 0 or 15 for q and p alike (also when |p| >= 2^22: far then exceeds
      // the bound or the bits clamp). s == 0 gives rs = 0, p = 0, code 0 as required; an
      // infinite zero (|min| past the fp16 range) takes the exact path. t grows with x
      // (rs >= 0), so when the row's min and max land in [0, 15] every code does and the
      // wave skips the clamp (the usual case: zero = min exactly for bf16 values in
      // fp16's normal range, and max rounds to 15).
      const bool in_range = (int32_t)__float_as_uint(fmaf(lo - z, rs, kMagic)) >= kMagicBits &&
                            (int32_t)__float_as_uint(fmaf(hi - z, rs, kMagic)) <= kMagicBits + 15;
      int32_t r[EPL];
      float far = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float d = x[e] - z;
        const float t = fmaf(d, rs, kMagic);
        far = fmaxf(far, fabsf(fmaf(d, rs, -(t - kMagic))));
        r[e] = (int32_t)__float_as_uint(t);
      }
      if (__ballot(far > 0.5f - 0x1p-17f || !__builtin_isfinite(z))) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          const float q = s == 0.f ? 0.f : __fdiv_rn(x[e] - z, s);
          r[e] = kMagicBits + (int32_t)(s == 0.f ? 0.f : fminf(fmaxf(__builtin_rintf(q), 0.f), 15.f));
        }
      } else if (__ballot(!in_range)) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) r[e] = min(max(r[e], kMagicBits), kMagicBits + 15);
      }
      if (!kv) {
        uint32_t w[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          uint32_t acc = 0;
#pragma unroll
          for (int k = 0; k < 8; ++k) acc += (uint32_t)r[8 * hh + k] << code_shift(k);
          w[hh] = acc - kWordBias;
        }
        uint32_t* dst = reinterpret_cast<uint32_t*>(a.k_codes + first * (D / 2) + (uint32_t)(row * (D / 2) + c * (EPL / 2)));
        dst[0] = w[0];
        dst[1] = w[1];
      } else {
        // the low byte of kMagicBits + n is n
        u32x4 cb;
#pragma unroll
        for (int m = 0; m < 4; ++m)
          cb[m] = __builtin_amdgcn_perm((uint32_t)r[4 * m + 1], (uint32_t)r[4 * m], 0x0c0c0400u) |
                  __builtin_amdgcn_perm((uint32_t)r[4 * m + 3], (uint32_t)r[4 * m + 2], 0x04000c0cu);
        *reinterpret_cast<u32x4*>(&vcodes[row * D + c * EPL]) = cb;
      }
      if (c == 0) {
        char* params = reinterpret_cast<char*>((kv ? a.v_params : a.k_params) + first * 2);
        *reinterpret_cast<uint32_t*>(params + (uint32_t)row * 4u) =
            (uint32_t)__builtin_bit_cast(uint16_t, s16) | ((uint32_t)__builtin_bit_cast(uint16_t, z16) << 16);
      }
    }
    if (h == R - 1) {   // the head's last round: its V words
      const int ngr = (n + 7) / 8;   // words of 8 tokens a channel
      // rows n .. 8 ngr - 1 of the last word hold code 0
      for (int i = threadIdx.x; i < (8 * ngr - n) * (D / 16); i += 256)
        *reinterpret_cast<u32x4*>(&vcodes[n * D + i * 16]) = u32x4{0, 0, 0, 0};
      __syncthreads();
      // One task per 4 channels and word: the 8 tokens' codes of channels 4q .. 4q+3 as 8
      // LDS words (byte i = channel 4q + i), regrouped by byte permutes into the 4
      // channels' words (n0|n2<<4, n4|n6<<4, n1|n3<<4, n5|n7<<4).
      constexpr int NQ = D / 4;
      const uint32_t* vw = reinterpret_cast<const uint32_t*>(vcodes);
      const int q = threadIdx.x % NQ;
      for (int r = threadIdx.x / NQ; r < ngr; r += 256 / NQ) {
        uint32_t w8[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) w8[k] = vw[(8 * r + k) * NQ + q];
        // [w_a.b0, w_b.b0, w_a.b1, w_b.b1] and [w_a.b2, w_b.b2, w_a.b3, w_b.b3]
        auto lo_pair = [](uint32_t wb, uint32_t wa) { return __builtin_amdgcn_perm(wb, wa, 0x05010400u); };
        auto hi_pair = [](uint32_t wb, uint32_t wa) { return __builtin_amdgcn_perm(wb, wa, 0x07030602u); };
        const uint32_t p04 = lo_pair(w8[4], w8[0]), q04 = hi_pair(w8[4], w8[0]);
        const uint32_t p15 = lo_pair(w8[5], w8[1]), q15 = hi_pair(w8[5], w8[1]);
        const uint32_t p26 = lo_pair(w8[6], w8[2]), q26 = hi_pair(w8[6], w8[2]);
        const uint32_t p37 = lo_pair(w8[7], w8[3]), q37 = hi_pair(w8[7], w8[3]);
        // channel i: A = bytes (n0, n4, n1, n5), B = bytes (n2, n6, n3, n7), word = A | B << 4
        uint32_t word[4];
        word[0] = __builtin_amdgcn_perm(p15, p04, 0x05040100u) | __builtin_amdgcn_perm(p37, p26, 0x05040100u) << 4;
        word[1] = __builtin_amdgcn_perm(p15, p04, 0x07060302u) | __builtin_amdgcn_perm(p37, p26, 0x07060302u) << 4;
        word[2] = __builtin_amdgcn_perm(q15, q04, 0x05040100u) | __builtin_amdgcn_perm(q37, q26, 0x05040100u) << 4;
        word[3] = __builtin_amdgcn_perm(q15, q04, 0x07060302u) | __builtin_amdgcn_perm(q37, q26, 0x07060302u) << 4;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *reinterpret_cast<uint32_t*>(a.v_codes + (slab * D + 4 * q + i) * (a.P / 2) + r * 4) = word[i];
      }
      __syncthreads();
    }
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
