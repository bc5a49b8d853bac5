// sparse_prefill: block-sparse / streaming causal attention over a paged GQA KV
// cache (blog "LServe -- Prefill Phase" and Figure 1: every KV tile is computed or
// skipped whole at the kernel's tile granularity; streaming heads keep sink tiles
// plus a local window and never visit the tiles in between; one kernel serves both
// head kinds).
//
// One work-group per (query head h, query tile i) with T/32 waves of 32 query rows.
// The kept-tile list is never materialised: dense heads walk their mask row 64
// entries at a time with a wave ballot, streaming heads enumerate the Lambda set
// arithmetically. For each kept KV tile j:
//   K_j  -> LDS row-major (16-byte rows padded),
//   V_j  -> LDS transposed (8x8 register transposes, so that the P.V operand reads
//           8 contiguous bytes),
//   S^T  = K_j Q^T  on bf16 MFMA 32x32x16 (Q stays in registers as the B operand),
//   online softmax per query row in the log2 domain (row = lane % 32; the two lanes
//   of a row exchange with one xor-32 shuffle), causal cut only on the diagonal tile,
//   O^T += V_j^T P^T on bf16 MFMA 32x32x16, P rounded to bf16.
// The S^T accumulator layout (lane = query, 16 keys per lane) is exactly the B
// operand layout that P^T needs, so P never leaves registers.
#include "common.h"
#include "launch.h"

namespace ubs {

template <int T, int D>
struct PrefillSmem {
  static constexpr int KSTR = D + 8;  // bf16 elements per K row in LDS
  static constexpr int VSTR = T + 4;  // bf16 elements per V^T row in LDS
  uint16_t k[T * KSTR];
  uint16_t vt[D * VSTR];
};

template <int T, int D>
__global__ __launch_bounds__(2 * T, 2) void prefill_kernel(const PrefillArgs a) {
  constexpr int NW = T / 32;
  constexpr int NT = 64 * NW;
  constexpr int KSTR = PrefillSmem<T, D>::KSTR;
  constexpr int VSTR = PrefillSmem<T, D>::VSTR;
  constexpr int QK = D / 16;   // MFMA steps over channels
  constexpr int TB = T / 32;   // 32-key blocks per tile
  constexpr int CB = D / 32;   // 32-channel blocks of the output
  __shared__ PrefillSmem<T, D> sm;

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  const int L = a.L;
  const int G = a.Hq / a.Hkv;
  const int nT = (L + T - 1) / T;

  // ---- (head, query tile): dense heads first, longest rows (largest i) first
  int idx = blockIdx.x;
  const int nd = a.order.n_dense;
  bool streaming;
  int h, i;
  if (idx < nd * nT) {
    streaming = false;
    i = nT - 1 - idx / nd;
    h = a.order.h[idx % nd];
  } else {
    idx -= nd * nT;
    const int ns = a.order.n_total - nd;
    streaming = true;
    i = nT - 1 - idx / ns;
    h = a.order.h[nd + idx % ns];
  }
  const int g = h / G;

  // ---- Q rows of this wave as the B operand: query n = lane % 32, k-slot group
  // lane / 32 holds channels (lane/32)*D/2 + kk*8 + [0, 8) for step kk.
  const int qn = lane & 31;
  const int qg = lane >> 5;
  const int qrow = i * T + wave * 32 + qn;
  bf16x8 qb[QK];
  {
    const uint16_t* qp = a.q + ((int64_t)qrow * a.Hq + h) * D + qg * (D / 2);
#pragma unroll
    for (int kk = 0; kk < QK; ++kk) qb[kk] = as_bf16x8(qrow < L ? ld16(qp + kk * 8) : u32x4{0, 0, 0, 0});
  }
  const float scale_log2 = a.sm_scale * kLog2e;
  const int qi = wave * 32 + qn;  // query index inside the tile

  f32x16 oacc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[cb][e] = 0.f;
  float m_run = kNegInf, l_run = 0.f;

  const int64_t head_stride = (int64_t)a.P * D;
  auto process = [&](int j) {
    __syncthreads();  // the previous tile is no longer read
    // ---- K_j -> LDS (row-major)
#pragma unroll
    for (int it = 0; it < D / 16; ++it) {
      const int x = tid + it * NT;
      const int r = x / (D / 8), c8 = x % (D / 8);
      const int t = j * T + r;
      u32x4 v = {0, 0, 0, 0};
      if (t < L) {
        const int pg = a.page_table[t / a.P];
        v = ld16(a.k_cache + ((int64_t)pg * a.Hkv + g) * head_stride + (int64_t)(t % a.P) * D + c8 * 8);
      }
      *reinterpret_cast<u32x4*>(&sm.k[r * KSTR + c8 * 8]) = v;
    }
    // ---- V_j -> LDS transposed: thread takes an 8 (keys) x 8 (channels) block
    if (tid < T * D / 64) {
      const int kb = tid / (D / 8), cbk = tid % (D / 8);
      u32x4 vr[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int t = j * T + kb * 8 + r;
        vr[r] = u32x4{0, 0, 0, 0};
        if (t < L) {
          const int pg = a.page_table[t / a.P];
          vr[r] = ld16(a.v_cache + ((int64_t)pg * a.Hkv + g) * head_stride + (int64_t)(t % a.P) * D + cbk * 8);
        }
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        u32x4 w;
#pragma unroll
        for (int k2 = 0; k2 < 4; ++k2) {
          const uint32_t lo = vr[2 * k2][c >> 1], hi = vr[2 * k2 + 1][c >> 1];
          w[k2] = (c & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
        }
        *reinterpret_cast<u32x4*>(&sm.vt[(cbk * 8 + c) * VSTR + kb * 8]) = w;
      }
    }
    __syncthreads();

    // ---- S^T = K_j Q^T: lane holds query qn, keys tb*32 + 8*jj + 4*qg + ii (reg 4*jj + ii)
    f32x16 st[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) st[tb][e] = 0.f;
      const uint16_t* kr = &sm.k[(tb * 32 + qn) * KSTR + qg * (D / 2)];
#pragma unroll
      for (int kk = 0; kk < QK; ++kk) {
        const bf16x8 ka = as_bf16x8(*reinterpret_cast<const u32x4*>(kr + kk * 8));
        st[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qb[kk], st[tb], 0, 0, 0);
      }
    }
    // ---- scale, causal cut on the diagonal tile, online softmax
    const bool diag = (j == i);
    float mx = kNegInf;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = tb * 32 + 8 * (e >> 2) + 4 * qg + (e & 3);
        float v = st[tb][e] * scale_log2;
        if (diag && key > qi) v = kNegInf;
        st[tb][e] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = rescale_factor(m_run, m_new);
    m_run = m_new;
    float psum = 0.f;
    bf16x8 pb[TB][2];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        u32x4 w;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const float p0 = softmax_weight(st[tb][8 * s2 + 2 * e2], m_new);
          const float p1 = softmax_weight(st[tb][8 * s2 + 2 * e2 + 1], m_new);
          psum += p0 + p1;
          w[e2] = pack_bf16x2(p0, p1);
        }
        pb[tb][s2] = as_bf16x8(w);
      }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[cb][e] *= alpha;
    // ---- O^T += V_j^T P^T: A = V^T rows (channels), k-slots = keys
    //      tb*32 + 16*s2 + 4*qg + [0,4) and tb*32 + 16*s2 + 8 + 4*qg + [0,4)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const uint16_t* vr = &sm.vt[(cb * 32 + qn) * VSTR + 4 * qg];
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vr + tb * 32 + 16 * s2);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(vr + tb * 32 + 16 * s2 + 8);
          const bf16x8 va = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
          oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[tb][s2], oacc[cb], 0, 0, 0);
        }
    }
  };

  if (!streaming) {
    const uint8_t* mrow = a.block_mask + ((int64_t)h * nT + i) * nT;
    for (int base = 0; base <= i; base += 64) {
      const int jj = base + lane;
      const bool kept = (jj <= i) && mrow[jj] != 0;
      uint64_t bits = __ballot(kept);
      while (bits) {
        const int j = base + __builtin_ctzll(bits);
        bits &= bits - 1;
        process(j);
      }
    }
  } else {
    const int s_end = min(a.sink_tiles, i + 1);
    for (int j = 0; j < s_end; ++j) process(j);
    for (int j = max(a.sink_tiles, i - a.local_tiles + 1); j <= i; ++j) process(j);
  }

  // ---- epilogue: O / l, lse
  const float l_tot = l_run + shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (qrow < L) {
    float* op = a.out + ((int64_t)qrow * a.Hq + h) * D + 4 * qg;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        f32x4 v = {oacc[cb][4 * jj] * inv, oacc[cb][4 * jj + 1] * inv, oacc[cb][4 * jj + 2] * inv,
                   oacc[cb][4 * jj + 3] * inv};
        *reinterpret_cast<f32x4*>(op + cb * 32 + 8 * jj) = v;
      }
    if (qg == 0 && a.lse) a.lse[(int64_t)h * L + qrow] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : kNegInf;
  }
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s) {
  const int nT = (a.L + a.T - 1) / a.T;
  const int64_t blocks = (int64_t)nT * a.order.n_total;
  if (blocks == 0) return hipSuccess;
#define UBS_PREFILL(TT, DD)                                                                    \
  if (a.T == TT && a.D == DD) {                                                                \
    hipLaunchKernelGGL((prefill_kernel<TT, DD>), dim3((unsigned)blocks), dim3(2 * TT), 0, s, a); \
    return hipGetLastError();                                                                  \
  }
  UBS_PREFILL(64, 64) UBS_PREFILL(64, 128) UBS_PREFILL(128, 64) UBS_PREFILL(128, 128)
#undef UBS_PREFILL
  return hipErrorInvalidValue;
}

}  // namespace ubs
