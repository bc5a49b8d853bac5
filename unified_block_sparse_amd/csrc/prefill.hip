// sparse_prefill: block-sparse / streaming causal attention over a paged GQA KV
// cache (blog "LServe -- Prefill Phase" and Figure 1: every KV tile is computed or
// skipped whole at the kernel's tile granularity; streaming heads keep sink tiles
// plus a local window and never visit the tiles in between; one kernel serves both
// head kinds).
//
// One work-group per (query head h, query tile i), two work-groups per CU. Its T/32
// waves each own 32 query rows against every key of the kept tiles, with their own
// running (max, sum, O). Keys go by in steps of 64 (a kept tile is T/64 steps), so the
// K and V of a step take 16 KiB each at D = 128 and two work-groups fit in LDS with
// their buffers doubled; each synchronises only its own waves, so the barrier and
// softmax phases of one overlap the matrix work of the other.
//
// Kept tiles: dense heads compact their mask row into an LDS list once (block-wide
// scan); streaming heads write their Lambda set there arithmetically. Skipped tiles
// are never loaded.
//
// Per step s (software-pipelined; K and V double-buffered in LDS):
//   loads:  K of step s+2 and V of step s+1, global -> LDS with direct-to-LDS 16-byte
//           buffer loads (scalar resource per 16-row block, per-lane offsets fixed for
//           the whole loop), spread one by one between the MFMAs
//   S^T  = K Q^T of step s+1 on bf16 MFMA 32x32x16 (Q resident in registers as the B
//           operand), interleaved with
//   the online softmax of step s per query row in the log2 domain (lazy rescaling of
//           O, bf16 weights, causal cut on the diagonal tile), then
//   O^T += V^T P^T of step s on bf16 MFMA 32x32x16; V^T comes from the row-major tile
//           through the LDS transpose read (ds_read_b64_tr_b16); P stays in registers.
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
__global__ __launch_bounds__(2 * T) __attribute__((amdgpu_waves_per_eu(2))) void prefill_kernel(const PrefillArgs a) {
  constexpr int NW = T / 32;          // waves = query groups of 32 rows
  constexpr int NT = 64 * NW;         // threads
  constexpr int SK = 64;              // keys per step (half a tile at T = 128)
  constexpr int NS = T / SK;          // steps per kept tile
  constexpr int TB = SK / 32;         // 32-key blocks per step
  constexpr int CPR = D / 8;          // 16-byte chunks per row
  constexpr int RW = SK / NW;         // rows of a step each wave loads
  constexpr int RB = RW / 16;         // ... as 16-row blocks
  constexpr int IT = 16 * CPR / 64;   // direct-to-LDS loads per 16-row block and tensor
  constexpr int RPI = 64 / CPR;       // rows per load instruction
  constexpr int QK = D / 16;          // MFMA steps over channels
  constexpr int CB = D / 32;          // 32-channel blocks of the output
  constexpr int MB = kMaxTileList / NT;  // mask bytes scanned per thread
  static_assert(RB >= 1 && RB * 16 == RW && IT * RPI == 16, "a wave loads whole 16-row blocks");
  // K and V of a step, double-buffered; every buffer is its own LDS object and the
  // buffer of each access is known at compile time (the step loop is unrolled by
  // parity). The compiler can then tell the direct-to-LDS loads into one buffer from the
  // reads of the other, and does not make those reads wait for the loads in flight.
  __shared__ __attribute__((aligned(1024))) uint16_t lds_k0[SK * D];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_k1[SK * D];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_v0[SK * D];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_v1[SK * D];
  __shared__ __attribute__((aligned(16))) int16_t lds_tlist[kMaxTileList];
  __shared__ int lds_scan[16];

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (and known to be)
  const int G = a.Hq / a.Hkv;

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
  // ---- the work item (sequence, query head h, query tile i). Query heads in order: the
  // G heads of each dense KV head (ascending), then those of each streaming KV head; the
  // k-th KV head of a kind is the k-th set bit of its mask. One sequence per call: q,
  // out, lse and the mask rows hold query tiles q_tile0 .. nT-1 of it (a chunk); items go
  // dense heads first, query tiles from the last to the first. Several sequences: the
  // same order over the whole batch (dense heads, then tile index from the largest,
  // then sequence, then head), so that every sequence's long rows start early; items
  // past a sequence's own tiles have nothing to do. Sequence b's rows start at row
  // cu_seqlens[b] of q, out and lse.
  const uint64_t dmask = a.dense_kv_mask;
  const uint64_t smask = ~dmask & (a.Hkv == 64 ? ~0ull : ((1ull << a.Hkv) - 1));
  auto nth_bit = [](uint64_t m, int k) __attribute__((always_inline)) {
    for (; k > 0; --k) m &= m - 1;
    return __builtin_ctzll(m);
  };
  const int nd = a.n_dense_kv * G;
  const int ns = a.Hq - nd;
  int L, qt0, q_off, lse_stride, m_rows, m_stride;
  const int32_t* __restrict__ ptab_v;
  const uint8_t* mask_base;
  bool streaming;
  int h, i, x;
  if (a.cu_seqlens) {
    const int nb = a.n_seq;
    int bs;
    if (w < nd * a.nT_max * nb) {
      streaming = false;
      i = a.nT_max - 1 - w / (nd * nb);
      bs = (w % (nd * nb)) / nd;
      x = w % nd;
    } else {
      const int w2 = w - nd * a.nT_max * nb;
      streaming = true;
      i = a.nT_max - 1 - w2 / (ns * nb);
      bs = (w2 % (ns * nb)) / ns;
      x = w2 % ns;
    }
    q_off = a.cu_seqlens[bs];
    // (a length past max_seqlen or past the page-table row is a caller error: clamped, so
    // that no page-table entry outside the row is read)
    L = min(a.cu_seqlens[bs + 1] - q_off, min(a.nT_max * T, a.pt_stride << a.log2_P));
    if (i * T >= L) return;   // (whole work-group, before any barrier)
    qt0 = 0;
    lse_stride = a.total_q;
    m_rows = m_stride = a.nT_max;
    ptab_v = a.page_table + (int64_t)bs * a.pt_stride;
    mask_base = a.block_mask + (int64_t)bs * a.Hq * a.nT_max * a.nT_max;
  } else {
    L = a.L;
    qt0 = a.q_tile0;
    q_off = -qt0 * T;
    const int nT1 = (L + T - 1) / T;
    lse_stride = L - qt0 * T;
    m_rows = nT1 - qt0;
    m_stride = nT1;
    ptab_v = a.page_table;
    mask_base = a.block_mask;
    const int nQ1 = nT1 - qt0;
    if (w < nd * nQ1) {
      streaming = false;
      i = nT1 - 1 - w / nd;
      x = w % nd;
    } else {
      const int w2 = w - nd * nQ1;
      streaming = true;
      i = nT1 - 1 - w2 / ns;
      x = w2 % ns;
    }
  }
  h = nth_bit(streaming ? smask : dmask, x / G) * G + x % G;
  const int nT = (L + T - 1) / T;
  const int g = h / G;

  // ---- direct-to-LDS loader. Wave w loads rows w*RW .. w*RW + RW - 1 of every step's
  // 64-row block of K and V, as RB blocks of 16 rows; 16 consecutive rows lie in one page
  // (P >= 16). Slot s = ((w*RB + b)*IT + it)*64 + lane of a buffer holds row s/CPR,
  // physical chunk s%CPR, i.e. logical chunk (s%CPR) ^ swizzle(row).
  const int lp = a.log2_P;
  const int pmask = (1 << lp) - 1;
  // first row (sequence position) of 16-row block b of step half hf of tile j
  auto row0 = [&](int j, int hf, int b) __attribute__((always_inline)) { return j * T + hf * SK + wave * RW + b * 16; };
  // Each 16-row block goes through its own buffer resource (wave-uniform base: the
  // block's first row in its page; size: the block's rows below L), with per-lane byte
  // offsets that are constant over the loop (row it*RPI + lane/CPR of the block, logical
  // chunk (lane % CPR) ^ swizzle; the swizzle depends on the row only through its place
  // in the block, which starts at a multiple of 16). No vector ALU work per load; rows at
  // or past L read as zeros (the resource's bounds check), which the causal cut never
  // weights. valid = false gives an empty resource: the loads write zeros and read
  // nothing, so that callers can issue branch-free.
  auto issue = [&](const uint16_t* cache, uint16_t* dst, int j, int hf, int b, int32_t page, int is_k, bool valid)
      __attribute__((always_inline)) {
    const int t0 = row0(j, hf, b);
    const uint64_t row = (((uint64_t)(uint32_t)page * (uint32_t)a.Hkv + (uint32_t)g) << lp) + (uint32_t)(t0 & pmask);
    // (every input of the resource made explicitly wave-uniform: otherwise the compiler
    // may loop over the lanes to build it)
    const int nr = __builtin_amdgcn_readfirstlane(valid ? min(max(L - t0, 0), 16) : 0);
    const uint64_t addr = (uint64_t)(cache + row * D);
    const uint64_t addr_u = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(addr >> 32)) << 32) |
                            (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)addr);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)addr_u, 0, nr * D * 2, 0x00020000);
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      // (swizzle written out here: a helper lambda called from this one makes the host
      // compilation pass drop the kernel's launch stub)
      const int rr = it * RPI + lane / CPR;
      const int r = wave * RW + b * 16 + rr;
      const int sw = is_k ? (D == 128 ? (r & 15) : ((r >> 1) & 7)) : (D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1));
      const uint32_t lo = (uint32_t)(rr * D + ((lane % CPR) ^ sw) * 8) * 2;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(dst + ((wave * RB + b) * IT + it) * 512), 16, lo, 0, 0, 0);
    }
  };
  // K or V of one step: the wave's RB blocks; pg_lane holds in lane b the page of block b
  auto issue_step = [&](const uint16_t* cache, uint16_t* dst, int j, int hf, int32_t pg_lane, int is_k, bool valid)
      __attribute__((always_inline)) {
#pragma unroll
    for (int b = 0; b < RB; ++b) issue(cache, dst, j, hf, b, __builtin_amdgcn_readlane(pg_lane, b), is_k, valid);
  };
  // lane b < RB: page-table entry of block b of (tile j, half hf) (rows clamped into the
  // sequence)
  auto page_lanes = [&](int j, int hf) __attribute__((always_inline)) -> int32_t {
    return __builtin_nontemporal_load(ptab_v + (min(row0(j, hf, lane < RB ? lane : 0), L - 1) >> lp));
  };

  // ---- kept KV tiles, ascending, as a list in LDS
  int n_tiles;
  if (!streaming) {
    const uint8_t* mrow = mask_base + ((int64_t)h * m_rows + (i - qt0)) * m_stride;
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
    const int lo_local = max(a.sink_tiles, i - a.local_tiles + 1);
    const int n_sink = min(a.sink_tiles, i + 1);
    n_tiles = n_sink + max(0, i + 1 - lo_local);
    for (int e = tid; e < n_tiles; e += NT) lds_tlist[e] = (int16_t)(e < n_sink ? e : lo_local + (e - n_sink));
  }
  // (the tile index is wave-uniform; saying so keeps the address and buffer-resource
  // arithmetic that depends on it on the scalar unit)
  auto tile_at = [&](int n) __attribute__((always_inline)) -> int {
    return __builtin_amdgcn_readfirstlane(lds_tlist[n]);
  };
  __syncthreads();
  // Steps: NS per kept tile (step s = half s % NS of kept tile s / NS). The diagonal
  // tile, when kept, is the last one.
  const int n_steps = n_tiles * NS;
  const bool diag_last = n_tiles > 0 && tile_at(n_tiles - 1) == i;
  // K and V of step 0 before the loop
  if (n_steps > 0) {
    const int j0 = tile_at(0);
    const int32_t pg0 = page_lanes(j0, 0);
    issue_step(a.k_cache, lds_k0, j0, 0, pg0, 1, true);
    issue_step(a.v_cache, lds_v0, j0, 0, pg0, 0, true);
  }

  // ---- Q rows of this wave as the B operand: query n = lane % 32, k-slot group
  // q2 = lane / 32 holds channels q2*D/2 + kk*8 + [0, 8) for step kk.
  const int qn = lane & 31;
  const int q2 = lane >> 5;
  const int qi = wave * 32 + qn;         // query index inside the tile
  const int qrow = i * T + qi;
  bf16x8 qb[QK];
  {
    const uint16_t* qp = a.q + ((int64_t)(qrow + q_off) * a.Hq + h) * D + q2 * (D / 2);
#pragma unroll
    for (int kk = 0; kk < QK; ++kk) qb[kk] = as_bf16x8(qrow < L ? ld16(qp + kk * 8) : u32x4{0, 0, 0, 0});
  }
  const float c2 = a.sm_scale * kLog2e;  // scores -> log2 domain

  f32x16 oacc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[cb][e] = 0.f;
  float m_run = kNegInf, l_run = 0.f;  // m_run: the max in use (raw scores)
  const int G16 = lane >> 4, j16 = lane & 15;

  // ---- the pieces of work on one step
  f32x16 s0[TB], s1[TB];    // scores of two consecutive steps (by parity)
  bf16x8 pb[TB][2];         // bf16 weights of the step being finished
  float alpha = 1.f;        // its rescale factor of O (1 where the max in use stayed)
  bool grow = false;
  // S^T = K Q^T over the step's 64 keys into st: lane holds query qn, keys
  // tb*32 + 8*jj + 4*q2 + ii (reg 4*jj + ii). Emits the LDS reads and the MFMAs only;
  // the caller's scheduling pattern orders them.
  auto qk_emit = [&](const uint16_t* ks, f32x16 (&st)[TB]) __attribute__((always_inline)) {
    const uint16_t* kr[TB];
    int sw[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const int r = tb * 32 + qn;
      kr[tb] = ks + r * D;
      sw[tb] = k_swz<D>(r);
    }
    u32x4 kf[QK][TB];
#pragma unroll
    for (int kk = 0; kk < QK; ++kk)
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
        kf[kk][tb] = *reinterpret_cast<const u32x4*>(kr[tb] + (((q2 * (D / 16) + kk) ^ sw[tb]) * 8));
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int e = 0; e < 16; ++e) st[tb][e] = 0.f;
#pragma unroll
    for (int kk = 0; kk < QK; ++kk)
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
        st[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf[kk][tb]), qb[kk], st[tb], 0, 0, 0);
  };
  // causal cut on the diagonal tile: keys hf*SK + (the step's key index) past the query
  // (the query index goes through an empty asm first: the comparisons are then made on
  // the diagonal step itself, instead of the compiler precomputing all 32 lane masks
  // ahead of the loop, where their 64 scalar registers spill into vector lanes and the
  // reloads run on every step)
  auto diag_cut = [&](f32x16 (&st)[TB], int hf) __attribute__((always_inline)) {
    int qrel = qi - hf * SK - 4 * q2;
    asm volatile("" : "+v"(qrel));
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = tb * 32 + 8 * (e >> 2) + (e & 3);
        if (key > qrel) st[tb][e] = kNegInf;
      }
  };
  // Online softmax of one step's scores in two parts. softmax_max: row max, then lazy
  // rescaling: the max in use, m_run, moves only when the step max exceeds it by more
  // than kRescaleLog2 in the log2 domain, so weights stay below 2^kRescaleLog2 and
  // most steps leave O alone (m_run = -inf: any finite max moves it; a row max of -inf
  // never does, the difference being NaN or -inf); rescale_o applies the factor to O.
  // softmax_p: bf16 weights into pb and the row sum of the rounded weights (two per
  // dot2) into l_run; branch-free, so that it can share a basic block with MFMA work.
  float mofs = 0.f;
  auto softmax_max = [&](f32x16 (&st)[TB]) __attribute__((always_inline)) {
    // (scores are finite or -inf: the NaN-propagating maximum needs no operand
    // canonicalisation and folds into three-input max instructions)
    float mx = kNegInf;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
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
  auto softmax_p = [&](f32x16 (&st)[TB]) __attribute__((always_inline)) {
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    float psum = 0.f;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
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
  // O^T += V^T P^T. A operand (row = channel, k-slots = keys tb*32 + 16*s2 + 4*q2 +
  // [0,4) and the same + 8) by two transpose reads: lane (G16, j16) fetches key
  // tok0 + j16/4, channels chb + 4*(j16%4) + [0,4) and receives channel chb + j16, keys
  // tok0 + [0,4). Emits the reads and the MFMAs only.
  auto pv_emit = [&](const uint16_t* vs) __attribute__((always_inline)) {
    u32x4 vf[TB * 2][CB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int r1 = tb * 32 + 16 * s2 + 4 * (G16 >> 1) + (j16 >> 2);
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
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
          oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf[tb * 2 + s2][cb]), pb[tb][s2], oacc[cb], 0, 0, 0);
  };
  constexpr int NQ = QK * TB;       // QK MFMAs (one LDS read each)
  constexpr int NM = TB * 2 * CB;   // PV MFMAs (two transpose reads each)
  auto qk_only = [&](const uint16_t* ks, f32x16 (&sn)[TB]) __attribute__((always_inline)) {
    qk_emit(ks, sn);
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * TB, 0);
#pragma unroll
    for (int x = 0; x < NQ - 2 * TB; ++x) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * TB, 0);
  };
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
  // One basic block: the step's loads (emitted by the caller just before), S(s+1) =
  // K_{s+1} Q^T on the matrix cores while the vector ALUs turn S(s) into bf16 weights,
  // then O += P(s) V_s while they take the row max of S(s+1). Scheduled as rounds of
  // 1 QK MFMA, 1 LDS read, NV vector instructions and (in the first NVM rounds) 1
  // global load, the last rounds starting the V reads; then rounds of 1 PV MFMA, 2
  // transpose reads and NVP vector instructions. The loads leave one by one between the
  // MFMAs: issued back to back by every wave at once they queue in the texture unit and
  // stall each wave until its last one is accepted.
  constexpr int NVM = 2 * RB * IT + 1;   // tile loads (K and V) + the page-table load
  auto qk_p_pv = [&](const uint16_t* ks, f32x16 (&sn)[TB], f32x16 (&sc)[TB], const uint16_t* vs)
      __attribute__((always_inline)) {
    qk_emit(ks, sn);
    softmax_p(sc);
    pv_emit(vs);
    softmax_max(sn);   // the next step's row max, in the PV rounds
    // (4 and 3 vector instructions a round: measured best of 3-10 and 1-4 on MI355X,
    // 4.5% faster than 7 and 2)
    constexpr int NV = 4, NVP = 3;
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * TB, 0);
#pragma unroll
    for (int x = 0; x < NQ; ++x) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (x < NVM) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
      if (x < NQ - 2 * TB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      else __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x402, NV, 0);
    }
#pragma unroll
    for (int x = 0; x < NM; ++x) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (NQ + x < NVM) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x402, NVP, 0);
    }
  };

  // ---- software-pipelined loop over the steps. Step s (after a barrier):
  //   issue K of step s+2 (into step s's K buffer) and V of step s+1 (into step s-1's
  //   V buffer); S(s+1) = K_{s+1} Q^T interleaved with the softmax of S(s); rescale O;
  //   O += P(s) V_s.
  // The barrier of step s follows every wave's reads of K_s (step s-1's QK) and V_{s-1}
  // (step s-1's PV), and every wave's wait for its loads of K_{s+1} and V_s. The last
  // step has no next one: softmax and PV only. The loop is unrolled by two so that
  // buffer and score-register parities are compile-time constants (tag par).
  auto kbuf = [&](auto par) __attribute__((always_inline)) -> uint16_t* {
    if constexpr (decltype(par)::value == 0) return lds_k0; else return lds_k1;
  };
  auto vbuf = [&](auto par) __attribute__((always_inline)) -> uint16_t* {
    if constexpr (decltype(par)::value == 0) return lds_v0; else return lds_v1;
  };
  auto sbuf = [&](auto par) __attribute__((always_inline)) -> f32x16 (&)[TB] {
    if constexpr (decltype(par)::value == 0) return s0; else return s1;
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  // lane-held page-table entries of steps s+1 and s+2 (each loaded a step before use),
  // and the kept-tile ids of steps s+1 and s+2 (carried from step to step)
  int32_t pg1 = 0, pg2 = 0;
  int jt1 = 0, jt2 = 0;
  wait_vm_all();
  __syncthreads();
  if (n_steps > 1) {
    jt1 = tile_at(1 / NS);
    jt2 = tile_at(min(2, n_steps - 1) / NS);
    pg1 = page_lanes(jt1, 1 % NS);
    issue_step(a.k_cache, lds_k1, jt1, 1 % NS, pg1, 1, true);
    if (n_steps > 2) pg2 = page_lanes(jt2, 2 % NS);
  }
  // Invariant at the top of step s: S(s) is cut (if diagonal) and its row max taken
  // (m_run, alpha, grow, mofs are those of step s).
  if (n_steps > 0) {
    qk_only(lds_k0, s0);
    if (diag_last && 0 >= n_steps - NS) diag_cut(s0, 0);
    softmax_max(s0);
  }
  auto step = [&](int s, auto par) __attribute__((always_inline)) {
    using Q = std::integral_constant<int, 1 - decltype(par)::value>;
    const int s3c = min(s + 3, n_steps - 1);
    const int jt3 = tile_at(s3c / NS);   // (the tile list is read-only: before the wait)
    wait_vm_all();
    __syncthreads();
    rescale_o();
    // from here one basic block (the loads are issued branch-free: past the last step,
    // K goes out as an empty load into the free buffer, the page entry is re-read)
    issue_step(a.k_cache, kbuf(par), jt2, min(s + 2, n_steps - 1) % NS, pg2, 1, s + 2 < n_steps);
    issue_step(a.v_cache, vbuf(Q{}), jt1, (s + 1) % NS, pg1, 0, true);
    pg1 = pg2;
    pg2 = page_lanes(jt3, s3c % NS);
    const float m_prev = m_run;
    qk_p_pv(kbuf(Q{}), sbuf(Q{}), sbuf(par), vbuf(par));
    jt1 = jt2;
    jt2 = jt3;
    if (diag_last && s + 1 >= n_steps - NS) {  // S(s+1) is on the diagonal tile: cut, then redo its max
      m_run = m_prev;
      diag_cut(sbuf(Q{}), (s + 1) % NS);
      softmax_max(sbuf(Q{}));
    }
  };
  auto last = [&](int s, auto par) __attribute__((always_inline)) {
    wait_vm_all();
    __syncthreads();
    rescale_o();
    softmax_p(sbuf(par));
    pv(vbuf(par));
  };
  int s = 0;
  for (; s + 2 < n_steps; s += 2) {
    step(s, P0{});
    step(s + 1, P1{});
  }
  if (s + 1 < n_steps) {
    step(s, P0{});
    last(s + 1, P1{});
  } else if (s < n_steps) {
    last(s, P0{});
  }

  // ---- O / l and lse (both lanes of a query row hold half of its keys' weight sum)
  const float l_row = l_run + shfl_xor(l_run, 32);
  const float inv = l_row > 0.f ? 1.0f / l_row : 0.f;
  if (qrow < L) {
    float* op = a.out + ((int64_t)(qrow + q_off) * a.Hq + h) * D + 4 * q2;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = oacc[cb][4 * jj + e] * inv;
        *reinterpret_cast<f32x4*>(op + cb * 32 + 8 * jj) = v;
      }
    if (q2 == 0 && a.lse)
      a.lse[(int64_t)h * lse_stride + (qrow + q_off)] = l_row > 0.f ? (m_run * c2 + __log2f(l_row)) * kLn2 : kNegInf;
  }
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s) {
  const int nT = (a.L + a.T - 1) / a.T;
  const int64_t blocks = a.cu_seqlens ? (int64_t)a.n_seq * a.Hq * a.nT_max : (int64_t)(nT - a.q_tile0) * a.Hq;
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
