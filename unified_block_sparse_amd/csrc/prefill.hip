// sparse_prefill: block-sparse / streaming causal attention over a paged GQA KV
// cache (blog "LServe -- Prefill Phase" and Figure 1: every KV tile is computed or
// skipped whole at the kernel's tile granularity; streaming heads keep sink tiles
// plus a local window and never visit the tiles in between; one kernel serves both
// head kinds).
//
// One work-group per (query head h, query tile i), T/32 waves of 32 query rows each,
// two work-groups resident per CU. Dense heads compact their mask row into an LDS list
// of kept tiles once (block-wide scan); streaming heads enumerate the Lambda set
// arithmetically. Skipped tiles are never loaded.
//
// Data movement per kept KV tile j (K and V each have one T x D bf16 LDS buffer):
//   V_j    global -> LDS by direct-to-LDS 16-byte loads, issued before S is computed
//   S^T    = K_j Q^T on bf16 MFMA 32x32x16 (Q resident in registers as the B operand)
//   softmax per query row in the log2 domain; causal cut on the diagonal tile only
//   K_next global -> LDS, issued once every wave has finished reading K_j
//   O^T   += V_j^T P^T on bf16 MFMA 32x32x16; V_j^T is read from the row-major tile
//            with the LDS transpose read (ds_read_b64_tr_b16), P stays in registers
// so each tile's loads overlap the other half of the previous tile's math. Rows of
// both buffers are XOR-swizzled at 16-byte granularity so the MFMA operand reads are
// free of bank conflicts; the direct-to-LDS loads write the swizzled layout by
// choosing which global chunk each lane fetches.
#include "common.h"
#include "launch.h"

namespace ubs {

typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

template <int D>
__device__ __forceinline__ int k_swz(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int v_swz(int r) {
  return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
}

__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0f70); }  // vmcnt(0)

// Block-wide exclusive scan of one int per thread (NT threads, NT/64 waves).
template <int NT>
__device__ __forceinline__ int block_scan(int v, int* tmp, int& total) {
  const int lane = lane_id(), w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) tmp[w] = x;
  __syncthreads();
  int base = 0;
  total = 0;
#pragma unroll
  for (int k = 0; k < NT / 64; ++k) {
    base += (k < w) ? tmp[k] : 0;
    total += tmp[k];
  }
  __syncthreads();
  return base + x - v;
}

template <int T, int D>
__global__ __launch_bounds__(2 * T, 2) void prefill_kernel(const PrefillArgs a) {
  constexpr int NW = T / 32;          // waves
  constexpr int CPR = D / 8;          // 16-byte chunks per row
  constexpr int IT = D / 16;          // direct-to-LDS loads per lane per tile
  constexpr int QK = D / 16;          // MFMA steps over channels
  constexpr int TB = T / 32;          // 32-key blocks per tile
  constexpr int CB = D / 32;          // 32-channel blocks of the output
  constexpr int NT = 64 * NW;         // threads
  constexpr int MB = kMaxTileList / NT;  // mask bytes scanned per thread
  __shared__ __attribute__((aligned(1024))) uint16_t ks[T * D];
  __shared__ __attribute__((aligned(1024))) uint16_t vs[T * D];
  __shared__ int16_t tlist[kMaxTileList];
  __shared__ int scan_tmp[NW];

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

  // ---- direct-to-LDS tile loader: slot s = (wave*IT + it)*64 + lane holds row s/CPR,
  // physical chunk s%CPR, i.e. logical chunk (s%CPR) ^ swizzle(row). The 64/CPR rows of
  // one load instruction never straddle a page (P >= 16), so the page id is wave-uniform
  // and comes from a scalar load; the loads issued never wait on a vector memory result.
  typedef const int32_t __attribute__((address_space(4)))* const_i32p;
  const const_i32p ptab = (const_i32p)a.page_table;
  const int lp = a.log2_P;
  const int pmask = (1 << lp) - 1;
  constexpr int RPI = 64 / CPR;  // rows per load instruction
  auto lookup_pages = [&](int j, int32_t (&pg)[IT]) {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int r0 = (wave * IT + it) * RPI;
      const int pidx = __builtin_amdgcn_readfirstlane(min(j * T + r0, L - 1) >> lp);
      pg[it] = ptab[pidx];
    }
  };
  auto issue_tile = [&](const uint16_t* cache, uint16_t* buf, int j, const int32_t (&pg)[IT], bool is_k) {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int r = (wave * IT + it) * RPI + lane / CPR;
      const int c = (lane % CPR) ^ (is_k ? k_swz<D>(r) : v_swz<D>(r));
      const int t = min(j * T + r, L - 1);  // rows past the end: any valid row (never weighted)
      const uint32_t row = (((uint32_t)pg[it] * (uint32_t)a.Hkv + (uint32_t)g) << lp) + (uint32_t)(t & pmask);
      const uint16_t* src = cache + (uint64_t)row * D + c * 8;
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(buf + (wave * IT + it) * 512),
                                       16, 0, 0);
    }
  };

  // ---- kept KV tiles, ascending. Dense heads: compact the mask row into LDS once
  // (each thread scans MB bytes, block-wide scan for the positions). Streaming heads:
  // sink tiles, then the local window ending at the diagonal.
  int n_tiles;
  const int lo_local = max(a.sink_tiles, i - a.local_tiles + 1);
  const int n_sink = min(a.sink_tiles, i + 1);
  if (!streaming) {
    const uint8_t* mrow = a.block_mask + ((int64_t)h * nT + i) * nT;
    uint8_t flag[MB];
    int cnt = 0;
#pragma unroll
    for (int e = 0; e < MB; ++e) {
      const int jj = tid * MB + e;
      flag[e] = (jj <= i) ? mrow[jj] : 0;
    }
#pragma unroll
    for (int e = 0; e < MB; ++e) cnt += flag[e] != 0;
    int pos = block_scan<NT>(cnt, scan_tmp, n_tiles);
#pragma unroll
    for (int e = 0; e < MB; ++e)
      if (flag[e]) tlist[pos++] = (int16_t)(tid * MB + e);
    __syncthreads();
  } else {
    n_tiles = n_sink + max(0, i + 1 - lo_local);
  }
  auto tile_at = [&](int n) -> int {
    if (!streaming) return tlist[n];
    return n < n_sink ? n : lo_local + (n - n_sink);
  };

  // ---- Q rows of this wave as the B operand: query n = lane % 32, k-slot group
  // qg = lane / 32 holds channels qg*D/2 + kk*8 + [0, 8) for step kk.
  const int qn = lane & 31;
  const int qg = lane >> 5;
  const int qrow = i * T + wave * 32 + qn;
  bf16x8 qb[QK];
  {
    const uint16_t* qp = a.q + ((int64_t)qrow * a.Hq + h) * D + qg * (D / 2);
#pragma unroll
    for (int kk = 0; kk < QK; ++kk) qb[kk] = as_bf16x8(qrow < L ? ld16(qp + kk * 8) : u32x4{0, 0, 0, 0});
  }
  const float c2 = a.sm_scale * kLog2e;  // scores -> log2 domain
  const int qi = wave * 32 + qn;         // query index inside the tile

  f32x16 oacc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[cb][e] = 0.f;
  float m_run = kNegInf, l_run = 0.f;  // m_run: running max of raw scores

  int32_t pg_cur[IT], pg_next[IT];
  if (n_tiles > 0) {
    const int j0 = tile_at(0);
    lookup_pages(j0, pg_cur);
    issue_tile(a.k_cache, ks, j0, pg_cur, true);
    wait_vm_all();
    __syncthreads();
  }
  for (int n = 0; n < n_tiles; ++n) {
    const int j = tile_at(n);
    issue_tile(a.v_cache, vs, j, pg_cur, false);
    const int jn = (n + 1 < n_tiles) ? tile_at(n + 1) : -1;
    if (jn >= 0) lookup_pages(jn, pg_next);

    // ---- S^T = K_j Q^T: lane holds query qn, keys tb*32 + 8*jj + 4*qg + ii (reg 4*jj + ii)
    f32x16 st[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) st[tb][e] = 0.f;
      const int r = tb * 32 + qn;
      const uint16_t* kr = ks + r * D;
      const int sw = k_swz<D>(r);
      u32x4 kf[QK];
#pragma unroll
      for (int kk = 0; kk < QK; ++kk)
        kf[kk] = *reinterpret_cast<const u32x4*>(kr + (((qg * (D / 16) + kk) ^ sw) * 8));
#pragma unroll
      for (int kk = 0; kk < QK; ++kk)
        st[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf[kk]), qb[kk], st[tb], 0, 0, 0);
    }
    // ---- causal cut on the diagonal tile, online softmax (row max on raw scores)
    if (j == i) {
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = tb * 32 + 8 * (e >> 2) + 4 * qg + (e & 3);
          if (key > qi) st[tb][e] = kNegInf;
        }
    }
    float mx = kNegInf;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int e = 0; e < 16; e += 2) mx = fmaxf(mx, fmaxf(st[tb][e], st[tb][e + 1]));
    mx = fmaxf(mx, shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    if (__ballot(m_new != m_run)) {  // rescale only when some row's max moved
      const float alpha = (m_new == kNegInf) ? 1.0f : fast_exp2((m_run - m_new) * c2);
      l_run *= alpha;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[cb][e] *= alpha;
      m_run = m_new;
    }
    const float mofs = (m_run == kNegInf) ? 0.f : -m_run * c2;
    float psum = 0.f;
    bf16x8 pb[TB][2];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        u32x4 w;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const float p0 = fast_exp2(fmaf(st[tb][8 * s2 + 2 * e2], c2, mofs));
          const float p1 = fast_exp2(fmaf(st[tb][8 * s2 + 2 * e2 + 1], c2, mofs));
          psum += p0 + p1;
          w[e2] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{p0, p1}), bf16x2));
        }
        pb[tb][s2] = as_bf16x8(w);
      }
    l_run += psum;

    // ---- V_j has landed and every wave is done with K_j: prefetch the next K tile
    wait_vm_all();
    __syncthreads();
    if (jn >= 0) issue_tile(a.k_cache, ks, jn, pg_next, true);

    // ---- O^T += V_j^T P^T. A operand (row = channel, k-slots = keys
    //      tb*32 + 16*s2 + 4*qg + [0,4) and the same + 8) by two transpose reads:
    //      lane (group G16 = lane/16, j16 = lane%16) fetches key tok0 + j16/4,
    //      channels chb + 4*(j16%4) + [0,4); it receives channel chb + j16, keys tok0 + [0,4).
    const int G16 = lane >> 4, j16 = lane & 15;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int ch = cb * 32 + 16 * (G16 & 1) + 4 * (j16 & 3);
      u32x4 vf[TB][2];
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const int r1 = tb * 32 + 16 * s2 + 4 * (G16 >> 1) + (j16 >> 2);
          const int r2 = r1 + 8;
          const uint16_t* p1 = vs + r1 * D + (((ch >> 3) ^ v_swz<D>(r1)) * 8) + (ch & 7);
          const uint16_t* p2 = vs + r2 * D + (((ch >> 3) ^ v_swz<D>(r2)) * 8) + (ch & 7);
          const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p1);
          const i16x4 t2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p2);
          vf[tb][s2] = u32x4{__builtin_bit_cast(u32x2, t1)[0], __builtin_bit_cast(u32x2, t1)[1],
                             __builtin_bit_cast(u32x2, t2)[0], __builtin_bit_cast(u32x2, t2)[1]};
        }
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
          oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf[tb][s2]), pb[tb][s2], oacc[cb], 0, 0, 0);
    }
    // ---- the next K tile has landed and every wave is done with V_j
    wait_vm_all();
    __syncthreads();
#pragma unroll
    for (int it = 0; it < IT; ++it) pg_cur[it] = pg_next[it];
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
    if (qg == 0 && a.lse)
      a.lse[(int64_t)h * L + qrow] = l_tot > 0.f ? (m_run * c2 + __log2f(l_tot)) * kLn2 : kNegInf;
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
