// sparse_prefill: block-sparse / streaming causal attention over a paged GQA KV
// cache (blog "LServe -- Prefill Phase" and Figure 1: every KV tile is computed or
// skipped whole at the kernel's tile granularity; streaming heads keep sink tiles
// plus a local window and never visit the tiles in between; one kernel serves both
// head kinds).
//
// One work-group per (query head h, query tile i), one work-group per CU. Its 2T/32
// waves form T/32 query groups of 32 rows times 2 key halves: wave (qg, kh) owns
// query rows qg*32..+32 against keys kh*T/2..+T/2 of every kept tile, with its own
// running (max, sum, O); the two halves merge through LDS at the end.
//
// Kept tiles: dense heads compact their mask row into an LDS list once (block-wide
// scan); streaming heads enumerate the Lambda set arithmetically. Skipped tiles are
// never loaded.
//
// Per kept tile (K and V are double-buffered in LDS, T x D bf16 each):
//   K, V:  global -> LDS with direct-to-LDS 16-byte buffer loads (scalar resource per
//          group of rows, per-lane offsets fixed for the whole loop), issued one tile
//          ahead so they stream in while the current tile is computed
//   S^T  = K Q^T on bf16 MFMA 32x32x16 (Q resident in registers as the B operand)
//   online softmax per query row in the log2 domain; causal cut on the diagonal tile
//   O^T += V^T P^T on bf16 MFMA 32x32x16; V^T comes from the row-major tile through
//          the LDS transpose read (ds_read_b64_tr_b16); P stays in registers
// The two waves that share a SIMD overlap each other's softmax and matrix work
// through the hardware's wave interleaving; within a wave, independent MFMA chains
// are interleaved with the LDS operand reads (sched_group_barrier).
// Rows of both buffers are XOR-swizzled at 16-byte granularity so the operand reads
// are free of bank conflicts; the direct-to-LDS loads write the swizzled layout by
// choosing which global chunk each lane fetches.
//
// Work order: dense heads first, query tiles from the last (longest rows) to the
// first; blocks are renumbered so that the G heads of one KV group at one query tile
// run back to back on the same XCD and share its L2 for their K/V tiles.
#include "common.h"
#include "launch.h"

#include <type_traits>

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

// Largest growth of the row max (log2 domain) absorbed without rescaling O: weights
// stay below 2^8, far inside the range of fp32 sums and of the bf16 weights.
constexpr float kRescaleLog2 = 8.0f;

// max of x over lanes l and l ^ 32: one swap of the wave's halves, then the max of
// the two swapped registers (each lane holds its own value in one and the partner's
// in the other)
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0f70); }  // vmcnt(0)

// Block-wide exclusive scan of one int per thread (NT threads).
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
__global__ __launch_bounds__(4 * T, 1) void prefill_kernel(const PrefillArgs a) {
  constexpr int QG = T / 32;          // query groups of 32 rows
  constexpr int NW = 2 * QG;          // waves: query group x key half
  constexpr int NT = 64 * NW;         // threads
  constexpr int KH = T / 2;           // keys per half tile
  constexpr int TBH = KH / 32;        // 32-key blocks per half
  constexpr int CPR = D / 8;          // 16-byte chunks per row
  constexpr int IT = T * CPR / NT;    // direct-to-LDS loads per lane per tile and tensor
  constexpr int RPI = 64 / CPR;       // rows per load instruction
  constexpr int QK = D / 16;          // MFMA steps over channels
  constexpr int CB = D / 32;          // 32-channel blocks of the output
  constexpr int MB = kMaxTileList / NT;  // mask bytes scanned per thread
  // K and V tiles, double-buffered; every buffer is its own LDS object and the buffer
  // of each access is known at compile time (the tile loop is unrolled by parity).
  // The compiler can then tell the direct-to-LDS loads into one buffer from the reads
  // of the other, and does not make those reads wait for the loads in flight.
  __shared__ __attribute__((aligned(1024))) uint16_t lds_k0[T * D];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_k1[T * D];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_v0[T * D];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_v1[T * D];
  __shared__ __attribute__((aligned(16))) int16_t lds_tlist[kMaxTileList];
  __shared__ int lds_scan[16];

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (and known to be)
  const int qgrp = wave % QG;
  const int kh = wave / QG;
  const int L = a.L;
  const int G = a.Hq / a.Hkv;
  const int nT = (L + T - 1) / T;

  // ---- work item: XCD-aware renumbering of the block index (blocks go to XCDs
  // round-robin), then dense heads first, query tiles from the last to the first,
  // the G heads of a KV group adjacent.
  const int nblk = gridDim.x;
  int w;
  {
    const int b = blockIdx.x;
    const int span = (nblk / (8 * G)) * (8 * G);   // whole rounds of 8 chunks of G items
    if (b < span) {
      const int x = b % 8, r = b / 8;  // XCD x, its r-th block
      w = ((r / G) * 8 + x) * G + r % G;
    } else {
      w = b;
    }
  }
  // query heads in order: the G heads of each dense KV head (ascending), then those of
  // each streaming KV head; the k-th KV head of a kind is the k-th set bit of its mask
  const uint64_t dmask = a.dense_kv_mask;
  const uint64_t smask = ~dmask & (a.Hkv == 64 ? ~0ull : ((1ull << a.Hkv) - 1));
  auto nth_bit = [](uint64_t m, int k) __attribute__((always_inline)) {
    for (; k > 0; --k) m &= m - 1;
    return __builtin_ctzll(m);
  };
  const int nd = a.n_dense_kv * G;
  bool streaming;
  int h, i;
  if (w < nd * nT) {
    streaming = false;
    i = nT - 1 - w / nd;
    const int x = w % nd;
    h = nth_bit(dmask, x / G) * G + x % G;
  } else {
    const int w2 = w - nd * nT;
    const int ns = a.Hq - nd;
    streaming = true;
    i = nT - 1 - w2 / ns;
    const int x = w2 % ns;
    h = nth_bit(smask, x / G) * G + x % G;
  }
  const int g = h / G;

  // ---- direct-to-LDS tile loader. Slot s = (wave*IT + it)*64 + lane holds row s/CPR,
  // physical chunk s%CPR, i.e. logical chunk (s%CPR) ^ swizzle(row). One instruction's
  // RPI rows never straddle a page (P >= 16), so page ids are wave-uniform scalar loads.
  typedef const int32_t __attribute__((address_space(4)))* const_i32p;
  const const_i32p ptab = (const_i32p)a.page_table;
  const int lp = a.log2_P;
  const int pmask = (1 << lp) - 1;
  // Each wave loads 16 consecutive rows of a tile (IT * RPI == 16), which lie in one page
  // (P >= 16), so one page-table entry per wave and tile serves its K and V loads; in the
  // last, partial tile the rows past L-1 are redirected to row L-1 (valid data, never
  // weighted), which lies in the same 16-row block and hence the same page.
  static_assert(IT * RPI == 16, "a wave's share of a tile must be 16 rows");
  // Loads are issued in 16-row blocks (one page: P >= 16). Wave (qg, kh) owns block
  // rb = qg + (1 - kh) * QG: key-half-1 waves load rows 0..T/2-1 (used first, by key
  // half 0), key-half-0 waves load rows T/2..T-1.
  const int rb = qgrp + (1 - kh) * QG;
  auto slot_of = [&](int j) __attribute__((always_inline)) { return min(j * T + rb * 16, L - 1) >> lp; };
  // Loads go through a buffer resource per 16-row block (wave-uniform base: the block's
  // first row in its page; size: the rows of the block below L), with per-lane byte
  // offsets that are constant over the loop (row it*RPI + lane/CPR of the block,
  // logical chunk (lane % CPR) ^ swizzle; the swizzle depends on the row only through
  // its place in the block, which starts at a multiple of 16). No vector ALU work per
  // load; rows at or past L read as zeros (the resource's bounds check), which the
  // causal cut never weights.
  // (valid = false: an empty resource, the loads write zeros and read nothing; lets the
  // caller issue branch-free)
  auto issue = [&](const uint16_t* cache, uint16_t* dst, int j, int32_t page, int is_k, bool valid = true)
      __attribute__((always_inline)) {
    const int t0 = j * T + rb * 16;
    const uint64_t row = (((uint64_t)(uint32_t)page * (uint32_t)a.Hkv + (uint32_t)g) << lp) + (uint32_t)(t0 & pmask);
    // one resource for the 16-row block: base = its first row, size = its rows below L
    // (every input made explicitly wave-uniform: otherwise the compiler may loop over
    // the lanes to build the resource)
    const int nr = __builtin_amdgcn_readfirstlane(valid ? min(max(L - t0, 0), 16) : 0);
    const uint64_t addr = (uint64_t)(cache + row * D);
    const uint64_t addr_u = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(addr >> 32)) << 32) |
                            (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)addr);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)addr_u, 0, nr * D * 2, 0x00020000);
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      // lane offset: row rr = it*RPI + lane/CPR of the block, logical chunk
      // (lane % CPR) ^ swizzle (written out here: a helper lambda called from this one
      // makes the host compilation pass drop the kernel's launch stub)
      const int rr = it * RPI + lane / CPR;
      const int r = rb * 16 + rr;
      const int sw = is_k ? (D == 128 ? (r & 15) : ((r >> 1) & 7)) : (D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1));
      const uint32_t lo = (uint32_t)(rr * D + ((lane % CPR) ^ sw) * 8) * 2;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst + (rb * IT + it) * 512),
                                               16, lo, 0, 0, 0);
    }
  };

  // ---- kept KV tiles, ascending
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
    int pos = block_scan<NT>(cnt, lds_scan, n_tiles);
#pragma unroll
    for (int e = 0; e < MB; ++e)
      if (flag[e]) lds_tlist[pos++] = (int16_t)(tid * MB + e);
  } else {
    n_tiles = n_sink + max(0, i + 1 - lo_local);
    for (int e = tid; e < n_tiles; e += NT) lds_tlist[e] = (int16_t)(e < n_sink ? e : lo_local + (e - n_sink));
  }
  // (the tile index is wave-uniform; saying so keeps the address and buffer-resource
  // arithmetic that depends on it on the scalar unit)
  auto tile_at = [&](int n) __attribute__((always_inline)) -> int {
    return __builtin_amdgcn_readfirstlane(lds_tlist[n]);
  };
  __syncthreads();
  // K and V of tile 0 (every wave its 16-row block) before the loop
  if (n_tiles > 0) {
    const int j0 = tile_at(0);
    const int32_t p0 = ptab[__builtin_amdgcn_readfirstlane(slot_of(j0))];
    issue(a.k_cache, lds_k0, j0, p0, 1);
    issue(a.v_cache, lds_v0, j0, p0, 0);
  }
  const int32_t* __restrict__ ptab_v = a.page_table;

  // ---- Q rows of this wave as the B operand: query n = lane % 32, k-slot group
  // q2 = lane / 32 holds channels q2*D/2 + kk*8 + [0, 8) for step kk.
  const int qn = lane & 31;
  const int q2 = lane >> 5;
  const int qrow = i * T + qgrp * 32 + qn;
  bf16x8 qb[QK];
  {
    const uint16_t* qp = a.q + ((int64_t)qrow * a.Hq + h) * D + q2 * (D / 2);
#pragma unroll
    for (int kk = 0; kk < QK; ++kk) qb[kk] = as_bf16x8(qrow < L ? ld16(qp + kk * 8) : u32x4{0, 0, 0, 0});
  }
  const float c2 = a.sm_scale * kLog2e;  // scores -> log2 domain
  const int qi = qgrp * 32 + qn;         // query index inside the tile

  f32x16 oacc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[cb][e] = 0.f;
  float m_run = kNegInf, l_run = 0.f;  // m_run: the max in use (raw scores)
  const int G16 = lane >> 4, j16 = lane & 15;

  // ---- the pieces of work on one tile
  f32x16 s0[TBH], s1[TBH];  // scores of two consecutive tiles (by parity)
  bf16x8 pb[TBH][2];        // bf16 weights of the tile being finished
  float alpha = 1.f;        // its rescale factor of O (1 where the max in use stayed)
  bool grow = false;
  // S^T = K Q^T over this wave's key half into st: lane holds query qn, keys
  // kh*KH + tb*32 + 8*jj + 4*q2 + ii (reg 4*jj + ii). Emits the LDS reads and the
  // MFMAs only; the caller's scheduling pattern orders them.
  auto qk_emit = [&](const uint16_t* ks, f32x16 (&st)[TBH]) __attribute__((always_inline)) {
    const uint16_t* kr[TBH];
    int sw[TBH];
#pragma unroll
    for (int tb = 0; tb < TBH; ++tb) {
      const int r = kh * KH + tb * 32 + qn;
      kr[tb] = ks + r * D;
      sw[tb] = k_swz<D>(r);
    }
    u32x4 kf[QK][TBH];
#pragma unroll
    for (int kk = 0; kk < QK; ++kk)
#pragma unroll
      for (int tb = 0; tb < TBH; ++tb)
        kf[kk][tb] = *reinterpret_cast<const u32x4*>(kr[tb] + (((q2 * (D / 16) + kk) ^ sw[tb]) * 8));
#pragma unroll
    for (int tb = 0; tb < TBH; ++tb)
#pragma unroll
      for (int e = 0; e < 16; ++e) st[tb][e] = 0.f;
#pragma unroll
    for (int kk = 0; kk < QK; ++kk)
#pragma unroll
      for (int tb = 0; tb < TBH; ++tb)
        st[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf[kk][tb]), qb[kk], st[tb], 0, 0, 0);
  };
  // Online softmax of one tile's scores in two parts. softmax_max: row max, then lazy
  // rescaling: the max in use, m_run, moves only when the tile max exceeds it by more
  // than kRescaleLog2 in the log2 domain, so weights stay below 2^kRescaleLog2 and
  // most tiles leave O alone (m_run = -inf: any finite max moves it; a row max of -inf
  // never does, the difference being NaN or -inf); rescale_o applies the factor to O.
  // softmax_p: bf16 weights into pb and the row sum of the rounded weights (two per
  // dot2) into l_run; branch-free, so that it can share a basic block with MFMA work.
  float mofs = 0.f;
  auto softmax_max = [&](f32x16 (&st)[TBH]) __attribute__((always_inline)) {
    // (scores are finite or -inf: the NaN-propagating maximum needs no operand
    // canonicalisation and folds into three-input max instructions)
    float mx = kNegInf;
#pragma unroll
    for (int tb = 0; tb < TBH; ++tb)
#pragma unroll
      for (int e = 0; e < 16; e += 2)
        mx = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mx, st[tb][e]), st[tb][e + 1]);
    mx = max_xor32(mx);
    grow = (mx - m_run) * c2 > kRescaleLog2;
    alpha = grow ? fast_exp2((m_run - mx) * c2) : 1.0f;
    m_run = grow ? mx : m_run;
    mofs = (m_run == kNegInf) ? 0.f : -m_run * c2;
  };
  auto rescale_o = [&]() __attribute__((always_inline)) {
    if (__ballot(grow)) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[cb][e] *= alpha;
    }
  };
  auto softmax_p = [&](f32x16 (&st)[TBH]) __attribute__((always_inline)) {
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    float psum = 0.f;
#pragma unroll
    for (int tb = 0; tb < TBH; ++tb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        u32x4 wv;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const float p0 = fast_exp2(fmaf(st[tb][8 * s2 + 2 * e2], c2, mofs));
          const float p1 = fast_exp2(fmaf(st[tb][8 * s2 + 2 * e2 + 1], c2, mofs));
          const bf16x2 pp = __builtin_convertvector((f32x2{p0, p1}), bf16x2);
          psum = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, psum, false);
          wv[e2] = __builtin_bit_cast(uint32_t, pp);
        }
        pb[tb][s2] = as_bf16x8(wv);
      }
    l_run = fmaf(l_run, alpha, psum);
  };
  auto qk_only = [&](const uint16_t* ks, f32x16 (&sn)[TBH]) __attribute__((always_inline)) {
    qk_emit(ks, sn);
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * TBH, 0);
#pragma unroll
    for (int x = 0; x < QK * TBH - 2 * TBH; ++x) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * TBH, 0);
  };
  auto pv_emit = [&](const uint16_t* vs) __attribute__((always_inline)) {
    // O^T += V^T P^T. A operand (row = channel, k-slots = keys
    // kh*KH + tb*32 + 16*s2 + 4*q2 + [0,4) and the same + 8) by two transpose reads:
    // lane (G16, j16) fetches key tok0 + j16/4, channels chb + 4*(j16%4) + [0,4)
    // and receives channel chb + j16, keys tok0 + [0,4). The CB output accumulators
    // are advanced in turn; the reads stay one key step ahead of the MFMAs.
    u32x4 vf[TBH * 2][CB];
#pragma unroll
    for (int tb = 0; tb < TBH; ++tb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int r1 = kh * KH + tb * 32 + 16 * s2 + 4 * (G16 >> 1) + (j16 >> 2);
        const int r2 = r1 + 8;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          const int ch = cb * 32 + 16 * (G16 & 1) + 4 * (j16 & 3);
          const uint16_t* p1 = vs + r1 * D + (((ch >> 3) ^ v_swz<D>(r1)) * 8) + (ch & 7);
          const uint16_t* p2 = vs + r2 * D + (((ch >> 3) ^ v_swz<D>(r2)) * 8) + (ch & 7);
          const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p1);
          const i16x4 t2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p2);
          vf[tb * 2 + s2][cb] = u32x4{__builtin_bit_cast(u32x2, t1)[0], __builtin_bit_cast(u32x2, t1)[1],
                                      __builtin_bit_cast(u32x2, t2)[0], __builtin_bit_cast(u32x2, t2)[1]};
        }
      }
#pragma unroll
    for (int tb = 0; tb < TBH; ++tb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
          oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf[tb * 2 + s2][cb]), pb[tb][s2], oacc[cb], 0, 0, 0);
  };
  constexpr int NQ = QK * TBH;       // QK MFMAs (one LDS read each)
  constexpr int NM = TBH * 2 * CB;   // PV MFMAs (two transpose reads each)
  auto pv = [&](const uint16_t* vs) __attribute__((always_inline)) {
    pv_emit(vs);
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * CB, 0);
#pragma unroll
    for (int x = 0; x < NM - CB; ++x) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, CB, 0);
  };
  // One basic block: the step's tile loads (emitted by the caller just before), S(n+1)
  // = K_{n+1} Q^T on the matrix cores while the vector ALUs turn S(n) into bf16
  // weights, then O += P(n) V_n. Scheduled as rounds of 1 QK MFMA, 1 LDS read, NV
  // vector instructions and (in the first NVM rounds) 1 global load, the last rounds
  // starting the V reads; then rounds of 1 PV MFMA and 2 transpose reads. The loads
  // leave one by one between the MFMAs: issued back to back by every wave at once they
  // queue in the texture unit and stall each wave until its last one is accepted.
  constexpr int NVM = 2 * IT + 1;   // tile loads (K and V) + the page-table load
  auto qk_p_pv = [&](const uint16_t* ks, f32x16 (&sn)[TBH], f32x16 (&sc)[TBH], const uint16_t* vs)
      __attribute__((always_inline)) {
    qk_emit(ks, sn);
    softmax_p(sc);
    pv_emit(vs);
    constexpr int NV = 7;
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * TBH, 0);
#pragma unroll
    for (int x = 0; x < NQ; ++x) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (x < NVM) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
      if (x < NQ - 2 * TBH) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      else __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x402, NV, 0);
    }
#pragma unroll
    for (int x = 0; x < NM; ++x) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (NQ + x < NVM) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
  };

  // ---- software-pipelined loop over the kept tiles. Step n (after a barrier):
  //   issue K of tile n+2 (into tile n's K buffer) and V of tile n+1 (into tile n-1's
  //   V buffer); S(n+1) = K_{n+1} Q^T interleaved with the softmax of S(n); rescale O;
  //   O += P(n) V_n.
  // The barrier of step n follows every wave's reads of K_n (step n-1's QK) and V_{n-1}
  // (step n-1's PV), and every wave's wait for its loads of K_{n+1} and V_n. The last
  // step has no next tile: softmax (with the causal cut if it is the diagonal tile,
  // which when kept is always the last) and PV only. The loop is unrolled by two so
  // that buffer and score-register parities are compile-time constants (tag par).
  auto kbuf = [&](auto par) __attribute__((always_inline)) -> uint16_t* {
    if constexpr (decltype(par)::value == 0) return lds_k0; else return lds_k1;
  };
  auto vbuf = [&](auto par) __attribute__((always_inline)) -> uint16_t* {
    if constexpr (decltype(par)::value == 0) return lds_v0; else return lds_v1;
  };
  auto sbuf = [&](auto par) __attribute__((always_inline)) -> f32x16 (&)[TBH] {
    if constexpr (decltype(par)::value == 0) return s0; else return s1;
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  // page of tile n+1 (scalar) and a lane copy of the page of tile n+2 (loaded one step
  // ahead of its use)
  int32_t pg1 = 0, pg2_lane = 0;
  wait_vm_all();
  __syncthreads();
  if (n_tiles > 1) {
    const int j1 = tile_at(1);
    pg1 = ptab[__builtin_amdgcn_readfirstlane(slot_of(j1))];
    issue(a.k_cache, lds_k1, j1, pg1, 1);
    if (n_tiles > 2) pg2_lane = __builtin_nontemporal_load(ptab_v + slot_of(tile_at(2)));
  }
  if (n_tiles > 0) qk_only(lds_k0, s0);
  auto step = [&](int n, auto par) __attribute__((always_inline)) {
    using Q = std::integral_constant<int, 1 - decltype(par)::value>;
    wait_vm_all();
    __syncthreads();
    const int32_t pgk = __builtin_amdgcn_readfirstlane(pg2_lane);
    const int j1 = tile_at(n + 1);
    const int j2 = tile_at(min(n + 2, n_tiles - 1));
    const int j3 = tile_at(min(n + 3, n_tiles - 1));
    softmax_max(sbuf(par));
    rescale_o();
    // from here one basic block (the loads are issued branch-free: past the last tile,
    // K goes out as an empty load into the free buffer, the page entry is re-read)
    issue(a.k_cache, kbuf(par), j2, pgk, 1, n + 2 < n_tiles);
    issue(a.v_cache, vbuf(Q{}), j1, pg1, 0);
    pg2_lane = __builtin_nontemporal_load(ptab_v + slot_of(j3));
    qk_p_pv(kbuf(Q{}), sbuf(Q{}), sbuf(par), vbuf(par));
    pg1 = pgk;
  };
  auto last = [&](int n, auto par) __attribute__((always_inline)) {
    wait_vm_all();
    __syncthreads();
    if (tile_at(n) == i) {  // causal cut on the diagonal tile
      f32x16(&st)[TBH] = sbuf(par);
#pragma unroll
      for (int tb = 0; tb < TBH; ++tb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = kh * KH + tb * 32 + 8 * (e >> 2) + 4 * q2 + (e & 3);
          if (key > qi) st[tb][e] = kNegInf;
        }
    }
    softmax_max(sbuf(par));
    rescale_o();
    softmax_p(sbuf(par));
    pv(vbuf(par));
  };
  int n = 0;
  for (; n + 2 < n_tiles; n += 2) {
    step(n, P0{});
    step(n + 1, P1{});
  }
  if (n + 1 < n_tiles) {
    step(n, P0{});
    last(n + 1, P1{});
  } else if (n < n_tiles) {
    last(n, P0{});
  }

  // ---- merge the two key halves of each query group through LDS, then O / l, lse.
  // Half 1 parks O in the K buffers (query group g in region g: 16-byte chunk c of
  // lane l at float (c*64 + l)*4) and (max, sum) in the tile-list area; half 0
  // combines and writes out.
  constexpr int RS = 64 * CB * 16;   // floats per region
  constexpr int RPB = T * D * 2 / (RS * 4);  // regions per K buffer
  static_assert(RPB >= 1 && 2 * RPB >= QG, "park regions exceed the K buffers");
  float* rg = reinterpret_cast<float*>(qgrp / RPB == 0 ? lds_k0 : lds_k1) + (qgrp % RPB) * RS;
  float* ml = reinterpret_cast<float*>(lds_tlist) + (qgrp * 64 + lane) * 2;
  __syncthreads();  // every wave is done with the tile buffers and the tile list
  const float l_half = l_run + shfl_xor(l_run, 32);   // both lanes of a row hold the row sum
  if (kh == 1) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int e = 0; e < 16; e += 4)
        *reinterpret_cast<f32x4*>(rg + ((cb * 4 + e / 4) * 64 + lane) * 4) =
            f32x4{oacc[cb][e], oacc[cb][e + 1], oacc[cb][e + 2], oacc[cb][e + 3]};
    ml[0] = m_run;
    ml[1] = l_half;
  }
  __syncthreads();
  if (kh == 0) {
    const float m1 = ml[0], l1 = ml[1];
    const float M = fmaxf(m_run, m1);
    const float f0 = (M == kNegInf) ? 0.f : fast_exp2((m_run - M) * c2);
    const float f1 = (M == kNegInf) ? 0.f : fast_exp2((m1 - M) * c2);
    const float l_tot = f0 * l_half + f1 * l1;
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    if (qrow < L) {
      float* op = a.out + ((int64_t)qrow * a.Hq + h) * D + 4 * q2;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const f32x4 o1 = *reinterpret_cast<const f32x4*>(rg + ((cb * 4 + jj) * 64 + lane) * 4);
          f32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (f0 * oacc[cb][4 * jj + e] + f1 * o1[e]) * inv;
          *reinterpret_cast<f32x4*>(op + cb * 32 + 8 * jj) = v;
        }
      if (q2 == 0 && a.lse)
        a.lse[(int64_t)h * L + qrow] = l_tot > 0.f ? (M * c2 + __log2f(l_tot)) * kLn2 : kNegInf;
    }
  }
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s) {
  const int nT = (a.L + a.T - 1) / a.T;
  const int64_t blocks = (int64_t)nT * a.Hq;
  if (blocks == 0) return hipSuccess;
#define UBS_PREFILL(TT, DD)                                                                    \
  if (a.T == TT && a.D == DD) {                                                                \
    hipLaunchKernelGGL((prefill_kernel<TT, DD>), dim3((unsigned)blocks), dim3(4 * TT), 0, s, a); \
    return hipGetLastError();                                                                  \
  }
  UBS_PREFILL(64, 64) UBS_PREFILL(64, 128) UBS_PREFILL(128, 64) UBS_PREFILL(128, 128)
#undef UBS_PREFILL
  return hipErrorInvalidValue;
}

}  // namespace ubs
