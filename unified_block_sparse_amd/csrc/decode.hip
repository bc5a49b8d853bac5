// sparse_decode: GQA decode attention over the kept pages of dense KV heads, or the
// sink + local tokens of streaming KV heads (blog "LServe -- Decode Phase" and
// Figure 2: token-level attention only inside the selected pages; LServe abstract:
// streaming heads in decode as well).
//
// Work split: (sequence b, KV head g, split s) per 256-thread work-group. The key set
// of (b, g) is a list of 32-token chunks, each inside one physical page (a part of a
// selected page, or of a page of the sink / local window); wave w of split s streams
// chunks (s*4 + w)*cpw ... + cpw - 1. It first resolves all their pages (one round
// trip through the selection and the page table for up to 64 chunks), then keeps the
// K/V loads of chunk t+1 in flight while it computes chunk t:
//   S = Q_g K^T  : bf16 MFMA 16x16x32 (rows = the G query heads, columns = 16 keys),
//                  K rows read straight from HBM, each load instruction 64 contiguous
//                  bytes of each of 16 rows;
//   online softmax in the log2 domain (fp32);
//   O += P V     : fp32 FMAs, each lane owning 8 channels of one key row, V read with
//                  16-byte loads that cover whole rows, P broadcast through LDS.
// INT4 pages (same kernel, Q4 = true): rows come as 4-bit codes n with a per-row fp16
// (scale s, zero z), x = n s + z. Codes enter the MFMA as the value 16 + n (exact: the
// code fills the top mantissa bits of 16), so S = s (Q.(16 + n)) + (z - 16 s) sum(Q).
// P.V runs on the fp16 MFMA, O^T = V^T (P s)^T: V pages are channel-major, so a lane's A
// operand (8 tokens of one channel) is one word; the weights p s, rounded to fp16, go
// through LDS as the B operand, and sum p z - 16 sum fp16(p s) joins every channel at the
// end. (fp16 rather than bf16 for P.V: its 11-bit weights keep the rounding of p s well
// inside the attention tolerance.)
// Partial (max, sum, output) triples of the 4 waves are merged through LDS; the
// work-group writes one partial per split (or the output when the key set has one
// split), and a second launch merges the splits of each (b, g) with a log-sum-exp
// combine staged in LDS.
#include "common.h"
#include "launch.h"

#include <algorithm>

namespace ubs {

typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;

constexpr int kMaxSplits = 128;
constexpr int kChunkTokens = 32;   // tokens per chunk

// K and V of one chunk in registers, per lane: bf16 rows, or INT4 codes and row params
template <int D, bool Q4>
struct ChunkRegs {
  u32x4 k[kChunkTokens / 16][D / 32];
  u32x4 v[D / 16];
};
template <int D>
struct ChunkRegs<D, true> {
  uint32_t k[kChunkTokens / 16][D / 32];   // K codes of the lane's key rows, 8 per word
  uint32_t kp[kChunkTokens / 16];          // fp16 (scale, zero) of those K rows
  uint32_t vp[kChunkTokens / 16];          // ... and of the same V rows
  uint32_t v[D / 16];                      // V codes: channel cb*16 + m, tokens 8*qg + [0, 8)
};

__device__ __forceinline__ float half_lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu)); }
__device__ __forceinline__ float half_hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

// The 8 INT4 codes of a word (code k in nibble k/2 of the low half if k is even, of the
// high half if odd) in code order, as the values 16 + n: exponent 4 and the code as the
// top 4 mantissa bits (bf16 bits 0x4180 | n << 3, fp16 bits 0x4C00 | n << 6). Pair j
// takes nibble j of both halves: one shift and one and-or.
template <int J, int POS>
__device__ __forceinline__ uint32_t nibble_pair(uint32_t w) {
  constexpr int sh = 4 * J - POS;   // nibble J of each half to bit POS of that half
  return sh >= 0 ? w >> sh : w << -sh;
}
// (x & m) | c in one instruction. The three-operand form takes no literal and at most one
// scalar operand on this architecture: m goes in a scalar register, c in a vector register
// (loop-invariant, so set once); written with literals, the compiler emits an and and an
// or, a third more vector instructions for the codes of a chunk.
__device__ __forceinline__ uint32_t and_or_sv(uint32_t x, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(m), "v"(c));
  return r;
}
__device__ __forceinline__ bf16x8 codes_bf16(uint32_t w) {
  constexpr uint32_t m = 0x00780078u, c = 0x41804180u;
  const u32x4 r = {and_or_sv(nibble_pair<0, 3>(w), m, c), and_or_sv(nibble_pair<1, 3>(w), m, c),
                   and_or_sv(nibble_pair<2, 3>(w), m, c), and_or_sv(nibble_pair<3, 3>(w), m, c)};
  return as_bf16x8(r);
}
__device__ __forceinline__ f16x8 codes_f16(uint32_t w) {
  constexpr uint32_t m = 0x03C003C0u, c = 0x4C004C00u;
  const u32x4 r = {and_or_sv(nibble_pair<0, 6>(w), m, c), and_or_sv(nibble_pair<1, 6>(w), m, c),
                   and_or_sv(nibble_pair<2, 6>(w), m, c), and_or_sv(nibble_pair<3, 6>(w), m, c)};
  return __builtin_bit_cast(f16x8, r);
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

struct Chunk {
  int page;        // physical page id, -1 if none
  int t0, t1;      // valid token range [t0, t1) in sequence positions
  int row_base;    // sequence position of row 0 of the page
};

__device__ __forceinline__ Chunk decode_chunk(const DecodeArgs& a, bool streaming, int b, int g, int c,
                                              int L, int nsel) {
  Chunk ch{-1, 0, 0, 0};
  const int P = a.P;
  const int32_t* pt = a.page_table + (int64_t)b * a.max_pages;
  if (!streaming) {
    if (c >= nsel) return ch;
    const int j = a.selected[((int64_t)b * a.Hkv + g) * a.max_selected + c];
    if (j < 0 || (int64_t)j * P >= L) return ch;
    ch.page = pt[j];
    ch.row_base = j * P;
    ch.t0 = j * P;
    ch.t1 = min(j * P + P, L);
    return ch;
  }
  const int A = min(a.sink, L);
  const int Bs = max(A, L - a.local);
  const int nsc = (A + P - 1) / P;
  if (c < nsc) {
    ch.page = pt[c];
    ch.row_base = c * P;
    ch.t0 = c * P;
    ch.t1 = min(c * P + P, A);
    return ch;
  }
  if (L <= Bs) return ch;
  const int fl = Bs / P;
  const int nlc = (L - 1) / P - fl + 1;
  const int cl = c - nsc;
  if (cl >= nlc) return ch;
  const int j = fl + cl;
  ch.page = pt[j];
  ch.row_base = j * P;
  ch.t0 = max(j * P, Bs);
  ch.t1 = min(j * P + P, L);
  return ch;
}

// At most 256 registers a lane (two waves per SIMD or more) wherever that costs no spill:
// the allocator then keeps the INT4 kernel (about 166 registers) in the vector file alone,
// three waves per SIMD (measured on MI355X: about 10% faster than two), and the bf16
// kernel at G = 8, D = 128 at two waves instead of one. At G = 16 the bf16 kernel's
// double-buffered K/V rows and G-wide accumulators need more than 256.
template <int D, int G, bool Q4>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu((Q4 || G <= 8) ? 2 : 1)))
void decode_kernel(const DecodeArgs a) {
  constexpr int KK = D / 32;   // QK MFMA steps (16x16x32)
  constexpr int CH = D / 8;    // lanes per V row (16-byte pieces)
  constexpr int TG = 64 / CH;  // token groups in P.V
  constexpr int CT = kChunkTokens;
  constexpr int NB = CT / 16;  // 16-key MFMA blocks per chunk
  constexpr int VR = CT / TG;  // V rows per lane and chunk
  __shared__ float p_lds[Q4 ? 1 : 4][CT][G];
  __shared__ __attribute__((aligned(16))) float p_t[Q4 ? 4 : 1][16][CT + 4];   // INT4: fp16(p s) [head][token]
  __shared__ float a_lds[4][16];                                                // INT4: per-head factors
  __shared__ float w_m[4][G], w_l[4][G];
  __shared__ float w_o[4][G][D];

  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int tid = threadIdx.x;

  // ---- which (b, g, split)
  const int per_b = a.dense.n * a.splits_dense + a.streaming.n * a.splits_stream;
  const int b = blockIdx.x / per_b;
  int r = blockIdx.x % per_b;
  bool streaming;
  int g, split, n_splits;
  if (r < a.dense.n * a.splits_dense) {
    streaming = false;
    g = a.dense.h[r / a.splits_dense];
    split = r % a.splits_dense;
    n_splits = a.splits_dense;
  } else {
    r -= a.dense.n * a.splits_dense;
    streaming = true;
    g = a.streaming.h[r / a.splits_stream];
    split = r % a.splits_stream;
    n_splits = a.splits_stream;
  }
  const int L = a.seq_lens[b];
  const int nsel = streaming ? 0 : min(a.num_selected[(int64_t)b * a.Hkv + g], a.max_selected);
  const float scale_log2 = a.sm_scale * kLog2e;

  // ---- this wave's chunks c0 .. c0 + cpw - 1 (chunk c: part c % CPP of page-level
  // chunk c / CPP, CT tokens)
  const int P = a.P;
  const int CPP = (P + CT - 1) / CT;
  const int cpw = a.chunks_per_wave;
  const int c0 = (split * 4 + wave) * cpw;

  // ---- Q as the MFMA A operand: row m = query head (zero rows past G); k-slot group
  // qg = l/16 holds channels kk*32 + qg*8 + [0, 8) for step kk (so that one K load
  // instruction reads 64 contiguous bytes of each of its 16 rows); with INT4 pages,
  // channels qg*D/4 + kk*8 + [0, 8) (one load brings a lane's codes for every step).
  const int m = lane & 15;
  const int qg = lane >> 4;
  bf16x8 qa[KK];
  {
    const uint16_t* qrow = a.q + ((int64_t)b * a.Hq + (int64_t)g * G + m) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qa[kk] = as_bf16x8((m < G) ? ld16(qrow + (Q4 ? qg * (D / 4) + kk * 8 : kk * 32 + qg * 8))
                                 : u32x4{0, 0, 0, 0});
  }
  // INT4: sum of the channels of query heads 4*qg + i (the rows of this lane's scores)
  float qsum[4] = {0.f, 0.f, 0.f, 0.f};
  if constexpr (Q4) {
    float sq = 0.f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const u32x4 w = __builtin_bit_cast(u32x4, qa[kk]);
#pragma unroll
      for (int e = 0; e < 4; ++e) sq += bf16_lo(w[e]) + bf16_hi(w[e]);
    }
    sq += shfl_xor(sq, 16);
    sq += shfl_xor(sq, 32);   // all channels of head m
#pragma unroll
    for (int i = 0; i < 4; ++i) qsum[i] = __shfl(sq, 4 * qg + i, 64);
  }

  float m_run[4];   // running max of heads 4*qg + i (lane-replicated within a 16-lane group)
#pragma unroll
  for (int i = 0; i < 4; ++i) m_run[i] = kNegInf;
  float o[G][8];
  float lsum[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    lsum[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[h][e] = 0.f;
  }
  // INT4: O^T blocks (lane: channels cb*16 + 4*qg + i of head m), and the lane's sums
  // over its key rows of p and of p z - 16 fp16(p s) for heads 4*qg + i
  f32x4 oT[Q4 ? D / 16 : 1];
  float lsum4[4], zacc4[4];
#pragma unroll
  for (int cb = 0; cb < (Q4 ? D / 16 : 1); ++cb) oT[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) lsum4[i] = zacc4[i] = 0.f;
  const int cc = lane % CH;
  const int tg = lane / CH;
  const int64_t head_stride = (int64_t)P * D;  // one (page, KV head) slab
  int d_page = -1, d_r0 = 0, d_lo = 0, d_hi = 0;   // chunk descriptors, one chunk per lane

  // ---- K and V of one chunk into registers, branch-free: each tensor through a buffer
  // resource over its (page, KV head) slab, of size zero for an empty chunk (the loads
  // then read nothing and return zeros). Without a branch the compiler can count the
  // loads in flight and wait for chunk t alone while chunk t+1's are outstanding. Rows
  // are clamped into the page; rows outside [lo, hi) are loaded but never weighted.
  auto slab_rsrc = [&](const uint16_t* cache, int page) __attribute__((always_inline)) {
    const uint64_t addr = (uint64_t)(cache + ((int64_t)max(page, 0) * a.Hkv + g) * head_stride);
    const uint64_t addr_u = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(addr >> 32)) << 32) |
                            (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)addr);
    return __builtin_amdgcn_make_buffer_rsrc((void*)addr_u, 0, page >= 0 ? P * D * 2 : 0, 0x00020000);
  };
  // (INT4: the same over a slab of row_bytes-byte rows of codes or of params)
  auto slab_rsrc4 = [&](const void* base, int page, int row_bytes) __attribute__((always_inline)) {
    const uint64_t addr =
        (uint64_t)((const uint8_t*)base + ((int64_t)max(page, 0) * a.Hkv + g) * (int64_t)P * row_bytes);
    const uint64_t addr_u = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(addr >> 32)) << 32) |
                            (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)addr);
    return __builtin_amdgcn_make_buffer_rsrc((void*)addr_u, 0, page >= 0 ? P * row_bytes : 0, 0x00020000);
  };
  auto load = [&](int t, int nt, ChunkRegs<D, Q4>& R) __attribute__((always_inline)) {
    const int page = t < nt ? __builtin_amdgcn_readlane(d_page, min(t, 63)) : -1;
    const int r0 = __builtin_amdgcn_readlane(d_r0, min(t, 63));
    if constexpr (Q4) {
      const __amdgpu_buffer_rsrc_t rk = slab_rsrc4(a.k_codes, page, D / 2);
      const __amdgpu_buffer_rsrc_t rkp = slab_rsrc4(a.k_params, page, 4);
      const __amdgpu_buffer_rsrc_t rv = slab_rsrc4(a.v_codes, page, D / 2);
      const __amdgpu_buffer_rsrc_t rvp = slab_rsrc4(a.v_params, page, 4);
#pragma unroll
      for (int blk = 0; blk < NB; ++blk) {
        const int row = min(r0 + blk * 16 + m, P - 1);
        if constexpr (D == 128) {
          const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(rk, row * 64 + qg * 16, 0, 0);
#pragma unroll
          for (int kk = 0; kk < KK; ++kk) R.k[blk][kk] = w[kk];
        } else {
          const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(rk, row * (D / 2) + qg * (D / 8), 0, 0);
#pragma unroll
          for (int kk = 0; kk < KK; ++kk) R.k[blk][kk] = w[kk];
        }
        R.kp[blk] = __builtin_amdgcn_raw_buffer_load_b32(rkp, row * 4, 0, 0);
      }
#pragma unroll
      for (int blk = 0; blk < NB; ++blk)
        R.vp[blk] = __builtin_amdgcn_raw_buffer_load_b32(rvp, min(r0 + blk * 16 + m, P - 1) * 4, 0, 0);
      // (tokens past the page read the next channel's word, or zeros past the slab; their
      // weights are zero)
#pragma unroll
      for (int cb = 0; cb < D / 16; ++cb)
        R.v[cb] = __builtin_amdgcn_raw_buffer_load_b32(rv, (cb * 16 + m) * (P / 2) + (r0 + 8 * qg) / 2, 0, 0);
    } else {
      const __amdgpu_buffer_rsrc_t rk = slab_rsrc(a.k_cache, page);
      const __amdgpu_buffer_rsrc_t rv = slab_rsrc(a.v_cache, page);
#pragma unroll
      for (int blk = 0; blk < NB; ++blk) {
        const int row = min(r0 + blk * 16 + m, P - 1);
        const int off = (row * D + qg * 8) * 2;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) R.k[blk][kk] = __builtin_amdgcn_raw_buffer_load_b128(rk, off + kk * 64, 0, 0);
      }
#pragma unroll
      for (int x = 0; x < VR; ++x) {
        const int row = min(r0 + tg + TG * x, P - 1);
        R.v[x] = __builtin_amdgcn_raw_buffer_load_b128(rv, (row * D + cc * 8) * 2, 0, 0);
      }
    }
  };
  // ---- online softmax and P.V over one chunk already in registers
  auto compute = [&](int t, int nt, const ChunkRegs<D, Q4>& R) __attribute__((always_inline)) {
    const int page = t < nt ? __builtin_amdgcn_readlane(d_page, min(t, 63)) : -1;
    if (page < 0) return;
    const int r0 = __builtin_amdgcn_readlane(d_r0, t);
    const int lo = __builtin_amdgcn_readlane(d_lo, t), hi = __builtin_amdgcn_readlane(d_hi, t);
    // S for NB blocks of 16 rows
    f32x4 s[NB];
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const int row = r0 + blk * 16 + m;
      const bool ok = row >= lo && row < hi;
      if constexpr (Q4) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[kk], codes_bf16(R.k[blk][kk]), acc, 0, 0, 0);
        const float sk = half_lo(R.kp[blk]), zk = half_hi(R.kp[blk]) - 16.f * sk;
#pragma unroll
        for (int i = 0; i < 4; ++i) s[blk][i] = ok ? fmaf(sk, acc[i], zk * qsum[i]) * scale_log2 : kNegInf;
      } else {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[kk], as_bf16x8(R.k[blk][kk]), acc, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) s[blk][i] = ok ? acc[i] * scale_log2 : kNegInf;
      }
    }
    // chunk max per head (heads 4*qg + i), then running max and weights
    float alpha_i[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float mx = s[0][i];
#pragma unroll
      for (int blk = 1; blk < NB; ++blk) mx = fmaxf(mx, s[blk][i]);
#pragma unroll
      for (int o2 = 1; o2 < 16; o2 <<= 1) mx = fmaxf(mx, shfl_xor(mx, o2));
      const float mn = fmaxf(m_run[i], mx);
      alpha_i[i] = rescale_factor(m_run[i], mn);
      m_run[i] = mn;
    }
    if constexpr (Q4) {
      // weights: p_t[head][token] = fp16(p s_v) (exact as fp32), and the lane's sums
#pragma unroll
      for (int blk = 0; blk < NB; ++blk) {
        const int row = r0 + blk * 16 + m;
        const bool ok = row >= lo && row < hi;   // (params of other rows are not trusted)
        const float sv = ok ? half_lo(R.vp[blk]) : 0.f, zv = ok ? half_hi(R.vp[blk]) : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = softmax_weight(s[blk][i], m_run[i]);
          const float pr = (float)(_Float16)(p * sv);
          p_t[wave][qg * 4 + i][blk * 16 + m] = pr;
          lsum4[i] = blk == 0 ? fmaf(lsum4[i], alpha_i[i], p) : lsum4[i] + p;
          zacc4[i] = fmaf(-16.f, pr, fmaf(p, zv, blk == 0 ? zacc4[i] * alpha_i[i] : zacc4[i]));
        }
      }
      if (m == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) a_lds[wave][qg * 4 + i] = alpha_i[i];
      }
      wave_sync_lds();
      // B operand: head m, tokens 8*qg + [0, 8); (heads past G give columns never read)
      const f32x4 p0 = *reinterpret_cast<const f32x4*>(&p_t[wave][m][8 * qg]);
      const f32x4 p1 = *reinterpret_cast<const f32x4*>(&p_t[wave][m][8 * qg + 4]);
      u32x4 pw;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        pw[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{p0[2 * e], p0[2 * e + 1]}), f16x2));
        pw[2 + e] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{p1[2 * e], p1[2 * e + 1]}), f16x2));
      }
      const f16x8 pb = __builtin_bit_cast(f16x8, pw);
      const float al = a_lds[wave][m];
      if (__ballot(al != 1.f)) {   // (a head's max grew: rare after the first chunks)
#pragma unroll
        for (int cb = 0; cb < D / 16; ++cb) oT[cb] *= al;
      }
#pragma unroll
      for (int cb = 0; cb < D / 16; ++cb)
        oT[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(codes_f16(R.v[cb]), pb, oT[cb], 0, 0, 0);
    } else {
#pragma unroll
      for (int blk = 0; blk < NB; ++blk)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int h = qg * 4 + i;
          if (h < G) p_lds[wave][blk * 16 + m][h] = softmax_weight(s[blk][i], m_run[i]);
        }
      wave_sync_lds();
      float alpha[G];
#pragma unroll
      for (int h = 0; h < G; ++h) alpha[h] = readlane_f(alpha_i[h & 3], 16 * (h >> 2));
#pragma unroll
      for (int h = 0; h < G; ++h) {
        lsum[h] *= alpha[h];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[h][e] *= alpha[h];
      }
      // O += P V over the chunk's rows tg, tg + TG, ... (weights of rows outside [lo, hi)
      // are zero and their V values are replaced by zero)
#pragma unroll
      for (int x = 0; x < VR; ++x) {
        const int rr = tg + TG * x;
        const int row = r0 + rr;
        const bool ok = row >= lo && row < hi;
        float vf[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vf[2 * e] = ok ? bf16_lo(R.v[x][e]) : 0.f;
          vf[2 * e + 1] = ok ? bf16_hi(R.v[x][e]) : 0.f;
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float p = p_lds[wave][rr][h];
          lsum[h] += p;
#pragma unroll
          for (int e = 0; e < 8; ++e) o[h][e] = fmaf(p, vf[e], o[h][e]);
        }
      }
    }
    wave_sync_lds();
  };
  // ---- the wave's chunks, 64 at a time. Lane t resolves chunk c0 + t0 + t to its
  // physical page and valid rows [lo, hi) of the page, so the index chain (selection ->
  // page table) costs one round trip per 64 chunks, before any of their K/V loads. Then
  // the loads of chunk t+1 are in flight while chunk t is computed (register double
  // buffer; unrolled by two so each buffer is a fixed register set).
  ChunkRegs<D, Q4> ra, rb;
  for (int t0 = 0; t0 < cpw; t0 += 64) {
    const int nt = min(64, cpw - t0);
    d_page = -1;
    if (lane < nt) {
      const int c = c0 + t0 + lane;
      const Chunk ch = decode_chunk(a, streaming, b, g, c / CPP, L, nsel);
      const int r0 = (c % CPP) * CT;                    // first row of the part in the page
      const int lo = max(ch.t0 - ch.row_base, r0), hi = min(ch.t1 - ch.row_base, r0 + CT);
      if (ch.page >= 0 && lo < hi) {
        d_page = ch.page;
        d_r0 = r0;
        d_lo = lo;
        d_hi = hi;
      }
    }
    // (chunks past nt are empty: their loads read nothing and their compute is skipped;
    // the scheduling barriers keep each chunk's loads after the previous compute, so
    // at most two chunks' registers are live)
    load(0, nt, ra);
    for (int t = 0; t < nt; t += 2) {
      load(t + 1, nt, rb);
      __builtin_amdgcn_sched_barrier(0);
      compute(t, nt, ra);
      __builtin_amdgcn_sched_barrier(0);
      load(t + 2, nt, ra);
      __builtin_amdgcn_sched_barrier(0);
      compute(t + 1, nt, rb);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if constexpr (Q4) {
    // ---- the wave's partial: sums over the 16 key lanes of each head group; O^T plus
    // the zero term of its head
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int o2 = 1; o2 < 16; o2 <<= 1) {
        lsum4[i] += shfl_xor(lsum4[i], o2);
        zacc4[i] += shfl_xor(zacc4[i], o2);
      }
    if (m == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = qg * 4 + i;
        if (h < G) {
          w_m[wave][h] = m_run[i];
          w_l[wave][h] = lsum4[i];
        }
        a_lds[wave][h] = zacc4[i];
      }
    }
    wave_sync_lds();
    if (m < G) {
      const float z = a_lds[wave][m];
#pragma unroll
      for (int cb = 0; cb < D / 16; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i) w_o[wave][m][cb * 16 + 4 * qg + i] = oT[cb][i] + z;
    }
    __syncthreads();
  } else {
    // ---- reduce the token groups of the wave
#pragma unroll
    for (int x = CH; x < 64; x <<= 1) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        lsum[h] += shfl_xor(lsum[h], x);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[h][e] += shfl_xor(o[h][e], x);
      }
    }
    // ---- stage the wave's partial in LDS
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mh = readlane_f(m_run[h & 3], 16 * (h >> 2));
      if (lane == 0) {
        w_m[wave][h] = mh;
        w_l[wave][h] = lsum[h];
      }
      if (tg == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) w_o[wave][h][cc * 8 + e] = o[h][e];
      }
    }
    __syncthreads();
  }

  // ---- merge the 4 waves: element (h, c) per thread
  const bool single = (n_splits == 1);
  float* part = a.partials;
  for (int idx = tid; idx < G * D; idx += 256) {
    const int h = idx / D, c = idx % D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, w_m[w][h]);
    float O = 0.f, S = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f = fast_exp2(w_m[w][h] - M);
        O = fmaf(f, w_o[w][h][c], O);
        S = fmaf(f, w_l[w][h], S);
      }
    }
    const int64_t qh = (int64_t)b * a.Hq + (int64_t)g * G + h;
    if (single) {
      a.out[qh * D + c] = (S > 0.f) ? O / S : 0.f;
      if (c == 0 && a.lse) a.lse[qh] = (S > 0.f) ? (M + __log2f(S)) * kLn2 : kNegInf;
    } else {
      float* pp = part + (qh * a.max_splits + split) * (D + 2);
      pp[c] = O;
      if (c == 0) {
        pp[D] = M;
        pp[D + 1] = S;
      }
    }
  }
}

// Merge of the split partials of one (b, KV head): log-sum-exp combine staged in LDS.
// A separate launch (rather than a last-arriving work-group) so that no work-group has
// to publish its partials with a device-scope fence, which on this GPU writes back and
// invalidates a whole L2.
template <int D, int G>
__global__ __launch_bounds__(256) void decode_merge_kernel(const DecodeArgs a) {
  __shared__ float c_m[G][kMaxSplits], c_w[G][kMaxSplits];
  const int tid = threadIdx.x;
  // blocks: (b, dense KV head) if dense heads are split, then (b, streaming KV head)
  const int nd = a.splits_dense > 1 ? a.dense.n : 0;
  const int ns = a.splits_stream > 1 ? a.streaming.n : 0;
  const int b = blockIdx.x / (nd + ns);
  const int r = blockIdx.x % (nd + ns);
  const int g = r < nd ? a.dense.h[r] : a.streaming.h[r - nd];
  const int n_splits = r < nd ? a.splits_dense : a.splits_stream;
  const float* part = a.partials;
  for (int idx = tid; idx < G * n_splits; idx += 256) {
    const int h = idx / n_splits, sp = idx % n_splits;
    const int64_t qh = (int64_t)b * a.Hq + (int64_t)g * G + h;
    const float* pp = part + (qh * a.max_splits + sp) * (D + 2);
    c_m[h][sp] = pp[D];
    c_w[h][sp] = pp[D + 1];
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += 256) {
    const int h = idx / D, c = idx % D;
    const int64_t qh = (int64_t)b * a.Hq + (int64_t)g * G + h;
    float M = kNegInf;
    for (int sp = 0; sp < n_splits; ++sp) M = fmaxf(M, c_m[h][sp]);
    float O = 0.f, S = 0.f;
    if (M != kNegInf) {
      // 8 splits at a time, their loads issued before any is used (one at a time, each
      // load waited for by its FMA, the splits cost one cache round trip each)
      const float* pc = part + qh * a.max_splits * (D + 2) + c;
      for (int sp0 = 0; sp0 < n_splits; sp0 += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = sp0 + u < n_splits ? pc[(int64_t)(sp0 + u) * (D + 2)] : 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (sp0 + u < n_splits) {
            const float f = fast_exp2(c_m[h][sp0 + u] - M);
            O = fmaf(f, v[u], O);
            S = fmaf(f, c_w[h][sp0 + u], S);
          }
        }
      }
    }
    a.out[qh * D + c] = (S > 0.f) ? O / S : 0.f;
    if (c == 0 && a.lse) a.lse[qh] = (S > 0.f) ? (M + __log2f(S)) * kLn2 : kNegInf;
  }
}

DecodePlan plan_decode(int B, int Hkv, int n_dense, int P, int max_selected, int sink, int local) {
  DecodePlan pl{};
  const int cpp = (P + 31) / 32;   // 32-token chunks per page
  pl.chunks_dense = max_selected * cpp;
  pl.chunks_stream = ((sink + P - 1) / P + (local + P - 1) / P + 1) * cpp;
  // Chunks per wave: 4 to 8, so that each wave streams several chunks (the loads of the
  // next overlap the compute of this one and the index chain is paid once per wave);
  // 8 once the batch fills two work-groups per CU with 4 (measured on MI355X: 4 is best
  // for 4 x 32K-token sequences, 8 for 64 sequences of 16K-128K tokens). More if the split
  // count would exceed what the merge can combine.
  const int64_t total = (int64_t)B * ((int64_t)n_dense * pl.chunks_dense + (int64_t)(Hkv - n_dense) * pl.chunks_stream);
  constexpr int64_t kWaveSlots = 4 * 2 * 256;
  int cpw = (int)std::min<int64_t>(8, std::max<int64_t>(4, (total + kWaveSlots - 1) / kWaveSlots));
  for (;;) {
    const int sd = n_dense > 0 ? (pl.chunks_dense + 4 * cpw - 1) / (4 * cpw) : 1;
    const int ss = (Hkv - n_dense) > 0 ? (pl.chunks_stream + 4 * cpw - 1) / (4 * cpw) : 1;
    if ((sd <= kMaxSplits && ss <= kMaxSplits) || cpw >= (1 << 20)) {
      pl.chunks_per_wave = cpw;
      pl.splits_dense = sd < 1 ? 1 : sd;
      pl.splits_stream = ss < 1 ? 1 : ss;
      break;
    }
    cpw *= 2;
  }
  pl.max_splits = pl.splits_dense > pl.splits_stream ? pl.splits_dense : pl.splits_stream;
  return pl;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  const int per_b = a.dense.n * a.splits_dense + a.streaming.n * a.splits_stream;
  const int64_t blocks = (int64_t)a.B * per_b;
  if (blocks == 0) return hipSuccess;
  const int G = a.Hq / a.Hkv;
  const int merge_per_b = (a.splits_dense > 1 ? a.dense.n : 0) + (a.splits_stream > 1 ? a.streaming.n : 0);
  const int64_t merge_blocks = (int64_t)a.B * merge_per_b;
#define UBS_DECODE(DD, GG)                                                                            \
  if (a.D == DD && G == GG) {                                                                         \
    if (a.int4)                                                                                       \
      hipLaunchKernelGGL((decode_kernel<DD, GG, true>), dim3((unsigned)blocks), dim3(256), 0, s, a);  \
    else                                                                                              \
      hipLaunchKernelGGL((decode_kernel<DD, GG, false>), dim3((unsigned)blocks), dim3(256), 0, s, a); \
    hipError_t e = hipGetLastError();                                                                 \
    if (e != hipSuccess || merge_blocks == 0) return e;                                               \
    hipLaunchKernelGGL((decode_merge_kernel<DD, GG>), dim3((unsigned)merge_blocks), dim3(256), 0, s, a); \
    return hipGetLastError();                                                                         \
  }
  UBS_DECODE(64, 1) UBS_DECODE(64, 2) UBS_DECODE(64, 4) UBS_DECODE(64, 8) UBS_DECODE(64, 16)
  UBS_DECODE(128, 1) UBS_DECODE(128, 2) UBS_DECODE(128, 4) UBS_DECODE(128, 8) UBS_DECODE(128, 16)
#undef UBS_DECODE
  return hipErrorInvalidValue;
}

}  // namespace ubs
