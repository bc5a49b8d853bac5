// sparse_decode: GQA decode attention over the kept pages of dense KV heads, or the
// sink + local tokens of streaming KV heads (blog "LServe -- Decode Phase" and
// Figure 2: token-level attention only inside the selected pages; LServe abstract:
// streaming heads in decode as well).
//
// Work split: one (sequence b, KV head g, split s) per WAVE, four independent waves per
// work-group (two or one for a launch too small to give every CU two work-groups: a CU
// streams only its share of the bandwidth, so a small launch must reach them all). The
// key set of (b, g) is a list of 16-row units, each inside one
// physical page (a part of a selected page, or of a page of the sink / local window), two
// units a 32-key chunk (INT4 pages: 32-row units, one a chunk), cut into splits of equal
// size. The split size is chosen so that
// every wave of the launch is resident at once (as many waves as the GPU holds of this
// kernel): each wave resolves its pages at the start, while the memory system is idle
// (one round trip through the selection and the page table for up to 64 units; under
// load that chain costs several microseconds a link), then streams to its end with no
// barrier. It keeps the K/V loads of chunk t+1 in flight while it computes chunk t:
//   S^T = K Q_g^T : bf16 MFMA 16x16x32 (rows = 16 keys of a unit, columns = the G query
//                   heads), K rows read straight from HBM, each load instruction 64
//                   contiguous bytes of each of 16 rows; lane (qg, m) then holds head
//                   m's scores of its 8 key slots;
//   online softmax in the log2 domain (fp32), row max by lane swaps;
//   O^T += V^T P^T: bf16 MFMA 16x16x32; the lane's weights (bf16) are its B operand as
//                   they stand, and its A operand (8 keys of one channel) comes from its
//                   own 16-byte V row loads by byte permutes.
// INT4 pages (same kernel, Q4 = true): rows come as 4-bit codes n with a per-row fp16
// (scale s, zero z), x = n s + z. Codes enter the MFMA as the value 16 + n (exact: the
// code fills the top mantissa bits of 16), so S = s (Q.(16 + n)) + (z - 16 s) sum(Q).
// P.V runs on the fp16 MFMA, O^T = V^T (P s)^T: V pages are channel-major, so a lane's A
// operand (8 tokens of one channel) is one word. The scores are computed transposed as
// for bf16 pages, with the K rows of the A operand ordered so that lane (qg, m) ends up
// with head m's scores of tokens 8*qg + [0, 8): the same 8 tokens as its V word, so the
// weights p s, rounded to fp16, are its B operand as they stand, and sum p z -
// 16 sum fp16(p s) joins every channel at the end. (fp16 rather than bf16 for P.V: its
// 11-bit weights keep the rounding of p s well inside the attention tolerance.)
// Each wave writes its split's partial (max, sum, output) triple, and a second launch
// merges the splits of each (b, query head) with a log-sum-exp combine staged in LDS.
#include "common.h"
#include "launch.h"

#include <algorithm>
#include <cstdlib>
#include <mutex>

namespace ubs {

typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// At most 96 splits a key list: the merge stages a query head's partials in at most
// 96 * 130 floats + weights, under 64 KiB of LDS
constexpr int kMaxSplits = 96;
constexpr int kChunkTokens = 32;   // tokens per chunk

// K and V of one chunk in registers, per lane: bf16 rows, or INT4 codes and row params
template <int D, bool Q4>
struct ChunkRegs {
  u32x4 k[kChunkTokens / 16][D / 32];      // K rows of the two 16-row halves (A operand)
  uint32_t v[kChunkTokens / 4][D / 32];    // V: key slot s, the lane's D/16 channels
};
template <int D>
struct ChunkRegs<D, true> {
  uint32_t k[kChunkTokens / 16][D / 32];   // K codes of the lane's two A-operand rows, 8 per word
  uint32_t kp[8];                          // fp16 (scale, zero) of K rows 8*qg + [0, 8)
  uint32_t vp[8];                          // ... and of the same V rows
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
// (x_i & m) | c for the four pairs of a word, one instruction each. The three-operand form
// takes no literal and at most one scalar operand on this architecture: m goes in a
// scalar register, c in a vector register (loop-invariant, so set once); written with
// literals, the compiler emits an and and an or, a third more vector instructions for the
// codes of a chunk. The four results are MFMA operands, and an MFMA may read a register
// only two wait states after a vector instruction has written it: the compiler inserts
// those waits for its own instructions but cannot see into inline assembly, so the block
// ends with them (s_nop 1). Without them, an MFMA placed right after the block has read
// stale operands. (Early-clobber outputs: each is written before the last input is read.)
__device__ __forceinline__ u32x4 and_or4(uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3, uint32_t m,
                                         uint32_t c) {
  uint32_t r0, r1, r2, r3;
  asm("v_and_or_b32 %0, %4, %8, %9\n"
      "v_and_or_b32 %1, %5, %8, %9\n"
      "v_and_or_b32 %2, %6, %8, %9\n"
      "v_and_or_b32 %3, %7, %8, %9\n"
      "s_nop 1"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
      : "v"(x0), "v"(x1), "v"(x2), "v"(x3), "s"(m), "v"(c));
  return u32x4{r0, r1, r2, r3};
}
__device__ __forceinline__ bf16x8 codes_bf16(uint32_t w) {
  return as_bf16x8(and_or4(nibble_pair<0, 3>(w), nibble_pair<1, 3>(w), nibble_pair<2, 3>(w),
                           nibble_pair<3, 3>(w), 0x00780078u, 0x41804180u));
}
__device__ __forceinline__ f16x8 codes_f16(uint32_t w) {
  return __builtin_bit_cast(f16x8, and_or4(nibble_pair<0, 6>(w), nibble_pair<1, 6>(w), nibble_pair<2, 6>(w),
                                           nibble_pair<3, 6>(w), 0x03C003C0u, 0x4C004C00u));
}

// max of v over lanes l and l ^ 16 (rows 2r and 2r + 1 of 16 lanes swapped), and over l
// and l ^ 32 (the two halves of the wave swapped): with both operands v, the two results
// of a swap hold v and its partner, in some order, in every lane
__device__ __forceinline__ float max_swap16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_swap32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_swap16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_swap32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

struct Chunk {
  int page;        // physical page id, -1 if none
  int t0, t1;      // valid token range [t0, t1) in sequence positions
  int row_base;    // sequence position of row 0 of the page
};

__device__ __forceinline__ Chunk decode_chunk(const DecodeArgs& a, bool streaming, int b, int g, int c,
                                              int L, int nsel, const int32_t* sel_row, int sel_cap) {
  Chunk ch{-1, 0, 0, 0};
  const int P = a.P;
  const int32_t* pt = a.page_table + (int64_t)b * a.max_pages;
  if (!streaming) {
    // (the selection entry is read before num_selected is known, so that the two loads,
    // and the sequence length, make one round trip; every slot below sel_cap exists: the
    // `selected` row, or the row the wave ranked into its LDS)
    const int j = c < sel_cap ? sel_row[c] : -1;
    if (c >= nsel) return ch;
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

// Selection inside the decode kernel: the wave's row of page scores (n pages, at most
// kMaxFusedPages) ranked as topk_kernel ranks it (the k-th largest order-preserving key by
// a bitwise search from the first bit where the row's keys differ, ties to the lower page
// index), with every count and every prefix sum taken from the wave's own ballots. The
// kept pages go in ascending order to sel[0, k) (this wave's LDS); with `write` also to
// gsel / gnum (the caller's selection outputs). Lane t owns pages t*EPT .. t*EPT + EPT - 1
// (EPT = 8 or 16 from max_pages), so lane order is page order. Returns the number kept,
// min(n, k).
template <int EPT>
__device__ __forceinline__ int wave_topk(const float* __restrict__ sc, const int* __restrict__ seq_len, int P,
                                         int max_pages, int k, __attribute__((address_space(3))) int32_t* sel,
                                         int32_t* gsel, int32_t* gnum, bool write) {
  const int lane = lane_id();
  // the row's scores are loaded before its length is known (one round trip for both);
  // entries past the row's pages are never ranked
  float raw[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int j = lane * EPT + e;
    raw[e] = j < max_pages ? sc[j] : 0.f;
  }
  const int L = *seq_len;
  const int n = (L + P - 1) / P;
  if (n <= k) {
    for (int i = lane; i < k; i += 64) {
      const int v = i < n ? i : -1;
      sel[i] = v;
      if (write) gsel[i] = v;
    }
    if (write && lane == 0) *gnum = n;
    return n;
  }
  uint32_t key[EPT];
  uint32_t kmin = ~0u, kmax = 0u;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const bool valid = lane * EPT + e < n;
    key[e] = valid ? float_order_key(raw[e]) : 0u;   // valid keys are > 0
    if (valid) {
      kmin = min(kmin, key[e]);
      kmax = max(kmax, key[e]);
    }
  }
  wave_min_max_u32(kmin, kmax);
  const int top = kmin == kmax ? -1 : 31 - __builtin_clz(kmin ^ kmax);
  uint32_t tau = kmin == kmax ? kmax : (top == 31 ? 0u : (kmax & ~((2u << top) - 1u)));
  for (int bit = top; bit >= 0; --bit) {
    const uint32_t cand = tau | (1u << bit);
    int c = 0;
#pragma unroll
    for (int e = 0; e < EPT; ++e) c += __popcll(__ballot(key[e] >= cand));
    if (c >= k) tau = cand;
    if (c == k) break;
  }
  int gt = 0, ties = 0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    gt += key[e] > tau;
    ties += key[e] == tau;
  }
  int n_gt, tie_total, kept_total;
  wave_prefix_small<5>(gt, n_gt);
  int tie_rank = wave_prefix_small<5>(ties, tie_total);
  const int take_ties = k - n_gt;
  uint32_t keep = 0;
  int kept = 0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    bool kp = key[e] > tau;
    if (key[e] == tau) {
      kp = tie_rank < take_ties;
      ++tie_rank;
    }
    keep |= (uint32_t)kp << e;
    kept += kp;
  }
  int pos = wave_prefix_small<5>(kept, kept_total);
#pragma unroll
  for (int e = 0; e < EPT; ++e)
    if ((keep >> e) & 1u) {
      const int j = lane * EPT + e;
      sel[pos] = j;
      if (write) gsel[pos] = j;
      ++pos;
    }
  if (write && lane == 0) *gnum = k;
  return k;
}

// At most 256 registers a lane (two waves per SIMD) wherever that costs no spill: the
// allocator then keeps the INT4 kernel (about 166 registers) in the vector file alone,
// three waves per SIMD (measured on MI355X: about 10% faster than two).
template <int D, int G, bool Q4>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void decode_kernel(const DecodeArgs a) {
  constexpr int KK = D / 32;   // QK MFMA steps (16x16x32)
  constexpr int CT = kChunkTokens;
  constexpr int NB = CT / 16;  // 16-key MFMA blocks per chunk
  constexpr int U = Q4 ? 32 : 16;   // rows per unit (the part of one page a lane resolves)
  constexpr int UPC = CT / U;       // units per chunk
  constexpr int NTR = 64 / UPC;     // chunks resolved per round trip (one unit a lane)
  constexpr int CPL = D / 16;       // bf16: V channels a lane holds of each row
  constexpr int WPR = D / 32;       // ... as words

  const int lane = lane_id();
  // (wave-uniform, and said so: every index derived from it then stays scalar)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // ---- which (b, g, split): one per wave (the last work-group's spare waves return;
  // the kernel has no work-group barrier). The nS streaming-head waves of sequence b are
  // spread evenly among its dense-head ones (slot r is the j-th streaming wave when
  // floor(r nS / per_b) steps up there), so that every work-group, and every XCD (work-
  // groups go to the XCDs in turn), gets the same mix of the two list lengths.
  const int nS = a.streaming.n * a.splits_stream;
  const int per_b = a.dense.n * a.splits_dense + nS;
  const int64_t gw = (int64_t)blockIdx.x * a.waves_per_group + wave;
  if (gw >= (int64_t)a.B * per_b) return;
  const int b = (int)(gw / per_b);
  const int r = (int)(gw % per_b);
  const int s_before = (int)((int64_t)r * nS / per_b), s_through = (int)((int64_t)(r + 1) * nS / per_b);
  const bool streaming = s_through > s_before;
  const int idx = streaming ? s_before : r - s_before;
  const int n_splits = streaming ? a.splits_stream : a.splits_dense;
  const int g = streaming ? a.streaming.h[idx / n_splits] : a.dense.h[idx / n_splits];
  const int split = idx % n_splits;
  const int L = a.seq_lens[b];
  // the (b, g) selection: read from `selected`, or (fused) ranked by this wave into its LDS
  extern __shared__ int32_t fused_lds[];
  const int64_t row = (int64_t)b * a.Hkv + g;
  const int32_t* sel_row = a.selected + row * a.max_selected;
  int sel_cap = a.max_selected;
  int nsel = 0;
  if (a.fused_k > 0) {
    __attribute__((address_space(3))) int32_t* my_sel =
        (__attribute__((address_space(3))) int32_t*)fused_lds + wave * a.fused_k;
    if (!streaming) {
      const float* sc = a.scores + row * a.max_pages;
      nsel = a.max_pages <= 512
                 ? wave_topk<8>(sc, a.seq_lens + b, a.P, a.max_pages, a.fused_k, my_sel, a.sel_out + row * a.fused_k,
                                a.nsel_out + row, split == 0)
                 : wave_topk<16>(sc, a.seq_lens + b, a.P, a.max_pages, a.fused_k, my_sel,
                                 a.sel_out + row * a.fused_k, a.nsel_out + row, split == 0);
      // the list is read below by other lanes than wrote it: every LDS write done
      // (lgkmcnt(0)), and no later load moved above this point
      __builtin_amdgcn_s_waitcnt(0xc07f);
      asm volatile("" ::: "memory");
    } else if (split == 0) {
      // a streaming head's row of the selection outputs: nothing selected
      for (int i = lane; i < a.fused_k; i += 64) a.sel_out[row * a.fused_k + i] = -1;
      if (lane == 0) a.nsel_out[row] = 0;
    }
    sel_row = (const int32_t*)my_sel;
    sel_cap = a.fused_k;
  } else {
    nsel = streaming ? 0 : min(a.num_selected[row], a.max_selected);
  }
  const float scale_log2 = a.sm_scale * kLog2e;

  // ---- this wave's chunks c0 .. c0 + cpw - 1 of the (b, g) list (split s of S takes
  // chunks floor(s C / S) .. floor((s + 1) C / S) - 1, so splits differ by one chunk at
  // most): chunk c is units c*UPC .. c*UPC + UPC - 1, unit u is rows (u % UPP)*U .. + U - 1
  // of the list's page u / UPP
  const int P = a.P;
  const int UPP = (P + U - 1) / U;
  const int n_chunks = streaming ? a.chunks_stream : a.chunks_dense;
  const int c0 = (int)((int64_t)split * n_chunks / n_splits);
  const int cpw = (int)((int64_t)(split + 1) * n_chunks / n_splits) - c0;

  // ---- Q in MFMA operand form: lane (qg, m) holds head m (zero past G), channels
  // kk*32 + qg*8 + [0, 8) for step kk (so that one K load instruction reads 64 contiguous
  // bytes of each of its 16 rows); with INT4 pages, channels qg*D/4 + kk*8 + [0, 8) (one
  // load brings a lane's codes for every step). bf16 pages take it as the B operand of
  // S^T = K Q^T, INT4 pages as the A operand of S = Q K^T.
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
  // INT4: sum of the channels of query head m (the head of this lane's scores)
  float qsum = 0.f;
  if constexpr (Q4) {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const u32x4 w = __builtin_bit_cast(u32x4, qa[kk]);
#pragma unroll
      for (int e = 0; e < 4; ++e) qsum += bf16_lo(w[e]) + bf16_hi(w[e]);
    }
    qsum = sum_swap16(qsum);
    qsum = sum_swap32(qsum);   // all channels of head m
  }

  // INT4: O^T blocks (lane (qg, m): channels cb*16 + 4*qg + i of head m) and the lane's
  // sum over its tokens of p z - 16 fp16(p s)
  f32x4 oT[Q4 ? D / 16 : 1];
#pragma unroll
  for (int cb = 0; cb < (Q4 ? D / 16 : 1); ++cb) oT[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float zh = 0.f;
  // lane (qg, m) runs head m: its running max (replicated over qg), its sum over the
  // lane's key slots, and (bf16) O^T block j = channels CPL*(4*qg + i) + j of head m
  float mh = kNegInf, lh = 0.f;
  f32x4 ov[Q4 ? 1 : CPL];
#pragma unroll
  for (int j = 0; j < (Q4 ? 1 : CPL); ++j) ov[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int64_t head_stride = (int64_t)P * D;  // one (page, KV head) slab
  int d_page = -1, d_r0 = 0, d_lo = 0, d_hi = 0;   // unit descriptors, one unit per lane

  // ---- K and V of one chunk into registers, branch-free: each tensor through a buffer
  // resource over its (page, KV head) slab, of size zero for an empty unit (the loads
  // then read nothing and return zeros). Without a branch the compiler can count the
  // loads in flight and wait for chunk t alone while chunk t+1's are outstanding.
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
  auto unit_page = [&](int t, int nt, int h) __attribute__((always_inline)) {
    return t < nt ? __builtin_amdgcn_readlane(d_page, min(t * UPC + h, 63)) : -1;
  };
  auto load = [&](int t, int nt, ChunkRegs<D, Q4>& R) __attribute__((always_inline)) {
    if constexpr (Q4) {
      // one unit of 32 rows of one page. A-operand row m of block blk is token
      // 8*(m/4) + 4*blk + m%4 (rows clamped into the page), so that the scores of lane
      // (qg, m') are those of tokens 8*qg + 4*blk + i; the row params of those 8 tokens
      // (two 16-byte loads each for K and V: 4-row groups lie wholly inside or wholly
      // past the P*4-byte slab, which reads zeros). Tokens outside [lo, hi) are loaded but
      // never weighted.
      const int page = unit_page(t, nt, 0);
      const int r0 = __builtin_amdgcn_readlane(d_r0, min(t, 63));
      const __amdgpu_buffer_rsrc_t rk = slab_rsrc4(a.k_codes, page, D / 2);
      const __amdgpu_buffer_rsrc_t rkp = slab_rsrc4(a.k_params, page, 4);
      const __amdgpu_buffer_rsrc_t rv = slab_rsrc4(a.v_codes, page, D / 2);
      const __amdgpu_buffer_rsrc_t rvp = slab_rsrc4(a.v_params, page, 4);
#pragma unroll
      for (int blk = 0; blk < NB; ++blk) {
        const int row = min(r0 + 8 * (m >> 2) + 4 * blk + (m & 3), P - 1);
        if constexpr (D == 128) {
          const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(rk, row * 64 + qg * 16, 0, 0);
#pragma unroll
          for (int kk = 0; kk < KK; ++kk) R.k[blk][kk] = w[kk];
        } else {
          const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(rk, row * (D / 2) + qg * (D / 8), 0, 0);
#pragma unroll
          for (int kk = 0; kk < KK; ++kk) R.k[blk][kk] = w[kk];
        }
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int off = (r0 + 8 * qg + 4 * h) * 4;
        const u32x4 wk = __builtin_amdgcn_raw_buffer_load_b128(rkp, off, 0, 0);
        const u32x4 wv = __builtin_amdgcn_raw_buffer_load_b128(rvp, off, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          R.kp[4 * h + e] = wk[e];
          R.vp[4 * h + e] = wv[e];
        }
      }
      // (tokens past the page read the next channel's word, or zeros past the slab; their
      // weights are zero)
#pragma unroll
      for (int cb = 0; cb < D / 16; ++cb)
        R.v[cb] = __builtin_amdgcn_raw_buffer_load_b32(rv, (cb * 16 + m) * (P / 2) + (r0 + 8 * qg) / 2, 0, 0);
    } else {
      // two units of 16 rows (halves h = 0, 1; P is a multiple of 16, so a unit never
      // crosses its page). K: the A operand of half h, row r0_h + m, 16 bytes at channel
      // kk*32 + 8*qg. V: key slot s of the lane holds row r0_h + 4*qg + (s & 3) of half
      // h = s / 4 (the rows of the lane's scores), channels CPL*m .. + CPL - 1, the row
      // clamped into the half's valid rows [lo, hi) so that every value read is one the
      // cache defines (the weights of clamped slots are zero).
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int page = unit_page(t, nt, h);
        const int u = min(t * UPC + h, 63);
        const int r0 = __builtin_amdgcn_readlane(d_r0, u);
        const int lo = __builtin_amdgcn_readlane(d_lo, u), hi = __builtin_amdgcn_readlane(d_hi, u);
        const __amdgpu_buffer_rsrc_t rk = slab_rsrc(a.k_cache, page);
        const __amdgpu_buffer_rsrc_t rv = slab_rsrc(a.v_cache, page);
        const int off = ((r0 + m) * D + qg * 8) * 2;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) R.k[h][kk] = __builtin_amdgcn_raw_buffer_load_b128(rk, off + kk * 64, 0, 0);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int row = min(max(r0 + 4 * qg + s, lo), hi - 1);
          const int voff = (row * D + CPL * m) * 2;
          if constexpr (D == 128) {
            const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(rv, voff, 0, 0);
#pragma unroll
            for (int e = 0; e < WPR; ++e) R.v[4 * h + s][e] = w[e];
          } else {
            const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(rv, voff, 0, 0);
#pragma unroll
            for (int e = 0; e < WPR; ++e) R.v[4 * h + s][e] = w[e];
          }
        }
      }
    }
  };
  // ---- online softmax and P.V over one chunk already in registers
  auto compute = [&](int t, int nt, const ChunkRegs<D, Q4>& R) __attribute__((always_inline)) {
    if constexpr (Q4) {
      const int page = unit_page(t, nt, 0);
      if (page < 0) return;
      const int r0 = __builtin_amdgcn_readlane(d_r0, t);
      const int lo = __builtin_amdgcn_readlane(d_lo, t), hi = __builtin_amdgcn_readlane(d_hi, t);
      // S^T per block: lane (qg, m) holds head m, tokens 8*qg + 4*blk + i (A rows ordered
      // by the load), one score per token j = 4*blk + i of the lane's 8
      const uint32_t n_ok = (uint32_t)(hi - lo);
      const int d0 = r0 + 8 * qg - lo;
      float sj[8];
#pragma unroll
      for (int blk = 0; blk < NB; ++blk) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(codes_bf16(R.k[blk][kk]), qa[kk], acc, 0, 0, 0);
        // (the scores are computed for every token and then masked: left to itself the
        // compiler moves each score into a branch of its own around the mask)
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = 4 * blk + i;
          const float sk = half_lo(R.kp[j]), zk = half_hi(R.kp[j]) - 16.f * sk;
          v[i] = fmaf(sk, acc[i], zk * qsum) * scale_log2;
        }
        asm volatile("" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]));
#pragma unroll
        for (int i = 0; i < 4; ++i) sj[4 * blk + i] = ((uint32_t)(d0 + 4 * blk + i) < n_ok) ? v[i] : kNegInf;
      }
      // chunk max of head m over the lane's 8 tokens and the 4 lane groups, running max
      float mx = fmaxf(fmaxf(fmaxf(sj[0], sj[1]), fmaxf(sj[2], sj[3])), fmaxf(fmaxf(sj[4], sj[5]), fmaxf(sj[6], sj[7])));
      mx = max_swap16(mx);
      mx = max_swap32(mx);
      const float mn = fmaxf(mh, mx);
      // (mr: the max, or 0 while every key so far is masked; the scores are then -inf, so
      // every weight is 0, and so is alpha, applied to a zero state)
      const float mr = (mn == kNegInf) ? 0.f : mn;
      const float alpha = fast_exp2(mh - mr);
      mh = mn;
      // weights: the B operand fp16(p s_v) of token 2e, 2e + 1 in word e, and the lane's
      // sums of p and of p z_v - 16 fp16(p s_v) (params of masked tokens are not trusted)
      float ps = 0.f, pz = 0.f;
      u32x4 pw;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float pr[2];
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          const int j = 2 * e + x;
          const bool ok = (uint32_t)(d0 + j) < n_ok;
          const float sv = ok ? half_lo(R.vp[j]) : 0.f, zv = ok ? half_hi(R.vp[j]) : 0.f;
          const float p = fast_exp2(sj[j] - mr);
          pr[x] = (float)(_Float16)(p * sv);
          ps += p;
          pz = fmaf(-16.f, pr[x], fmaf(p, zv, pz));
        }
        pw[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{pr[0], pr[1]}), f16x2));
      }
      lh = fmaf(lh, alpha, ps);
      zh = fmaf(zh, alpha, pz);
      const f16x8 pb = __builtin_bit_cast(f16x8, pw);
      if (__ballot(alpha != 1.f)) {   // (a head's max grew: rare after the first chunks)
#pragma unroll
        for (int cb = 0; cb < D / 16; ++cb) oT[cb] *= alpha;
      }
#pragma unroll
      for (int cb = 0; cb < D / 16; ++cb)
        oT[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(codes_f16(R.v[cb]), pb, oT[cb], 0, 0, 0);
    } else {
      const int page0 = unit_page(t, nt, 0), page1 = unit_page(t, nt, 1);
      if (page0 < 0 && page1 < 0) return;
      // S^T = K Q^T per half: lane (qg, m) holds head m, keys 4*qg + i of each half
      f32x4 s[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int u = min(t * UPC + h, 63);
        const int r0 = __builtin_amdgcn_readlane(d_r0, u);
        const int lo = __builtin_amdgcn_readlane(d_lo, u), hi = __builtin_amdgcn_readlane(d_hi, u);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(R.k[h][kk]), qa[kk], acc, 0, 0, 0);
        // (row - lo < hi - lo as unsigned: one compare for both bounds)
        const uint32_t n_ok = (uint32_t)(hi - lo);
        const int d0 = 4 * qg + (r0 - lo);
#pragma unroll
        for (int i = 0; i < 4; ++i) s[h][i] = ((uint32_t)(d0 + i) < n_ok) ? acc[i] * scale_log2 : kNegInf;
      }
      // chunk max of head m over the lane's 8 keys and the 4 lane groups (row pairs, then
      // halves of the wave, by lane swaps), running max
      float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                       fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
      mx = max_swap16(mx);
      mx = max_swap32(mx);
      const float mn = fmaxf(mh, mx);
      // (mr: the max, or 0 while every key so far is masked; the scores are then -inf, so
      // every weight is 0, and so is alpha, applied to a zero state)
      const float mr = (mn == kNegInf) ? 0.f : mn;
      const float alpha = fast_exp2(mh - mr);
      mh = mn;
      // weights, rounded to bf16 as the B operand of O^T += V^T P^T: key slot 2e, 2e + 1
      // of word e are the lane's keys (h = e/2, i = 2*(e&1)) and + 1
      float p[2][4];
      float ps = 0.f;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[h][i] = fast_exp2(s[h][i] - mr);
          ps += p[h][i];
        }
      lh = fmaf(lh, alpha, ps);
      u32x4 pw;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        pw[e] = __builtin_bit_cast(uint32_t,
                                   __builtin_convertvector((f32x2{p[e >> 1][2 * (e & 1)], p[e >> 1][2 * (e & 1) + 1]}), bf16x2));
      const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
      if (__ballot(alpha != 1.f)) {   // (a head's max grew: rare after the first chunks)
#pragma unroll
        for (int j = 0; j < CPL; ++j) ov[j] *= alpha;
      }
      // A operand of block j: V^T rows = channels CPL*m' + j (m' the MFMA row), key slots
      // as above; word e pairs slot 2e (low half) with slot 2e + 1 (high half), both the
      // half j & 1 of word j/2 of their V row
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        constexpr uint32_t kSelLo = 0x05040100u, kSelHi = 0x07060302u;
        u32x4 va;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          va[e] = __builtin_amdgcn_perm(R.v[2 * e + 1][j >> 1], R.v[2 * e][j >> 1], (j & 1) ? kSelHi : kSelLo);
        ov[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(va), pb, ov[j], 0, 0, 0);
      }
    }
  };
  // ---- the wave's chunks, NTR at a time. Lane l resolves unit l of them to its physical
  // page and valid rows [lo, hi) of the page, so the index chain (selection -> page
  // table) costs one round trip per NTR chunks, before any of their K/V loads. Then the
  // loads of chunks t+1 .. t+NBUF-1 are in flight while chunk t is computed (a ring of
  // NBUF register buffers, the loop unrolled by NBUF so each buffer is a fixed register
  // set). Two: with INT4 pages a four-deep ring (216 registers, two waves per SIMD) ran
  // 5% slower than two buffers at three waves per SIMD.
  constexpr int NBUF = 2;
  ChunkRegs<D, Q4> rr[NBUF];
  for (int t0 = 0; t0 < cpw; t0 += NTR) {
    const int nt = min(NTR, cpw - t0);
    d_page = -1;
    d_r0 = d_lo = d_hi = 0;
    if (lane < nt * UPC) {
      const int u = (c0 + t0) * UPC + lane;
      const Chunk ch = decode_chunk(a, streaming, b, g, u / UPP, L, nsel, sel_row, sel_cap);
      const int r0 = (u % UPP) * U;                     // first row of the unit in the page
      const int lo = max(ch.t0 - ch.row_base, r0), hi = min(ch.t1 - ch.row_base, r0 + U);
      if (ch.page >= 0 && lo < hi) {
        d_page = ch.page;
        d_r0 = r0;
        d_lo = lo;
        d_hi = hi;
      }
    }
    // (chunks past nt are empty: their loads read nothing and their compute is skipped;
    // the scheduling barriers keep each chunk's loads after the previous compute, so
    // at most NBUF chunks' registers are live)
#pragma unroll
    for (int k = 0; k + 1 < NBUF; ++k) load(k, nt, rr[k]);
    for (int t = 0; t < nt; t += NBUF) {
#pragma unroll
      for (int k = 0; k < NBUF; ++k) {
        load(t + k + NBUF - 1, nt, rr[(k + NBUF - 1) % NBUF]);
        __builtin_amdgcn_sched_barrier(0);
        compute(t + k, nt, rr[k]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  // ---- the wave's split partial (max, sum, output), merged by the second launch
  float* const part = a.partials + ((int64_t)b * a.Hq + (int64_t)g * G) * a.max_splits * (D + 2) +
                      (int64_t)split * (D + 2);
  const int64_t head_pitch = (int64_t)a.max_splits * (D + 2);
  if constexpr (Q4) {
    // head m: the sums over the 4 lane groups; lane (qg, m) holds channels cb*16 + 4*qg
    // + i, each plus the head's zero term
    lh = sum_swap16(lh);
    lh = sum_swap32(lh);
    zh = sum_swap16(zh);
    zh = sum_swap32(zh);
    if (m < G) {
      float* pp = part + m * head_pitch;
#pragma unroll
      for (int cb = 0; cb < D / 16; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i) pp[cb * 16 + 4 * qg + i] = oT[cb][i] + zh;
      if (qg == 0) {
        pp[D] = mh;
        pp[D + 1] = lh;
      }
    }
  } else {
    // head m: the sum over the 4 lane groups; lane (qg, m) holds channels
    // CPL*(4*qg + i) + j, that is 4*CPL contiguous channels from 4*CPL*qg
    lh = sum_swap16(lh);
    lh = sum_swap32(lh);
    if (m < G) {
      float* pp = part + m * head_pitch;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < CPL; ++j) pp[CPL * (4 * qg + i) + j] = ov[j][i];
      if (qg == 0) {
        pp[D] = mh;
        pp[D + 1] = lh;
      }
    }
  }
}

// Merge of the split partials of one (sequence b, query head): log-sum-exp combine. The
// head's partials are one contiguous block of n_splits rows of D + 2 floats; the work-group
// stages the whole block in LDS with every load issued at once (one round trip, however
// many splits), then every channel combines its n_splits values (one split: the partial
// normalised).
template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(const DecodeArgs a) {
  constexpr int RW = D + 2;
  // (dynamic LDS, sized by the launch for the plan's largest split count: whole rounds of
  // 256 floats of partials, then one weight a split)
  extern __shared__ __attribute__((aligned(16))) float merge_lds[];
  float* const blk = merge_lds;
  float* const wgt = merge_lds + (a.max_splits * RW + 255) / 256 * 256;
  const int tid = threadIdx.x;
  const int G = a.Hq / a.Hkv;
  const int b = blockIdx.x / a.Hq, h = blockIdx.x % a.Hq;
  const int g = h / G;
  bool streaming = false;
  for (int i = 0; i < a.streaming.n; ++i) streaming |= (a.streaming.h[i] == g);
  const int n_splits = streaming ? a.splits_stream : a.splits_dense;
  const int64_t qh = (int64_t)b * a.Hq + h;
  const float* src = a.partials + qh * a.max_splits * RW;
  const int n = n_splits * RW;
  {
    // direct-to-LDS loads: instruction k of wave w moves floats (4k + w)*64 .. + 63 of the
    // block, lane l the one at + l; the buffer resource ends at the block, so lanes past it
    // read zeros (and write them inside blk, which holds whole rounds of 256)
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint64_t addr = (uint64_t)src;
    const uint64_t addr_u = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(addr >> 32)) << 32) |
                            (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)addr);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)addr_u, 0, n * 4, 0x00020000);
    const int rounds = (n + 255) / 256;
    for (int k = 0; k < rounds; ++k) {
      const int row = 4 * k + wave;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(blk + row * 64), 4,
                                               (uint32_t)(row * 64 + lane_id()) * 4, 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): this wave's loads have landed
  }
  __syncthreads();
  float M = kNegInf;
  for (int sp = 0; sp < n_splits; ++sp) M = fmaxf(M, blk[sp * RW + D]);
  if (tid < n_splits) wgt[tid] = (M == kNegInf) ? 0.f : fast_exp2(blk[tid * RW + D] - M);
  __syncthreads();
  float S = 0.f;
  for (int sp = 0; sp < n_splits; ++sp) S = fmaf(wgt[sp], blk[sp * RW + D + 1], S);
  for (int c = tid; c < D; c += 256) {
    float O = 0.f;
    for (int sp = 0; sp < n_splits; ++sp) O = fmaf(wgt[sp], blk[sp * RW + c], O);
    a.out[qh * D + c] = (S > 0.f) ? O / S : 0.f;
  }
  if (tid == 0 && a.lse) a.lse[qh] = (S > 0.f) ? (M + __log2f(S)) * kLn2 : kNegInf;
}

// Waves of the decode kernel for (D, G, int4) that the current device holds at once:
// work-groups per CU from the occupancy query (registers and LDS of that instance) x 4
// waves x CUs, at most kMaxWaveSlots; cached per device and instance. 2,048 (two
// work-groups per CU on 256 CUs) if the query fails.
int64_t decode_wave_slots(int D, int G, bool int4) {
  constexpr int64_t kFallback = 2 * 4 * 256;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return kFallback;
  const int gi = 31 - __builtin_clz((unsigned)std::max(G, 1));   // log2 G: 0..4
  if (gi > 4 || (D != 64 && D != 128)) return kFallback;
  const int key = ((D == 128) * 5 + gi) * 2 + (int4 ? 1 : 0);   // 0..19
  static std::mutex mu;
  static int64_t cache[64][20] = {};
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev][key] > 0) return cache[dev][key];
  const void* fn = nullptr;
#define UBS_DECODE_FN(DD, GG)                                                                     \
  if (D == DD && G == GG)                                                                         \
    fn = int4 ? reinterpret_cast<const void*>(&decode_kernel<DD, GG, true>)                        \
              : reinterpret_cast<const void*>(&decode_kernel<DD, GG, false>);
  UBS_DECODE_FN(64, 1) UBS_DECODE_FN(64, 2) UBS_DECODE_FN(64, 4) UBS_DECODE_FN(64, 8) UBS_DECODE_FN(64, 16)
  UBS_DECODE_FN(128, 1) UBS_DECODE_FN(128, 2) UBS_DECODE_FN(128, 4) UBS_DECODE_FN(128, 8) UBS_DECODE_FN(128, 16)
#undef UBS_DECODE_FN
  int n_cu = 0, per_cu = 0;
  if (fn == nullptr || hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 256, 0) != hipSuccess || n_cu <= 0 || per_cu <= 0)
    return kFallback;
  const int64_t slots = std::min<int64_t>((int64_t)per_cu * 4 * n_cu, kMaxWaveSlots);
  cache[dev][key] = slots;
  return slots;
}

DecodePlan plan_decode(int B, int Hkv, int n_dense, int P, int max_selected, int sink, int local, bool int4,
                       int64_t wave_slots, bool ranks_selection) {
  DecodePlan pl{};
  // key lists in units of U rows of one page (16 for bf16 pages, 32 for INT4), two or one
  // units a 32-token chunk
  const int U = int4 ? 32 : 16;
  const int upp = (P + U - 1) / U, upc = kChunkTokens / U;
  const int64_t units_dense = (int64_t)max_selected * upp;
  const int64_t units_stream = ((int64_t)(sink + P - 1) / P + (local + P - 1) / P + 1) * upp;
  pl.chunks_dense = (int)((units_dense + upc - 1) / upc);
  pl.chunks_stream = (int)((units_stream + upc - 1) / upc);
  const int nd = n_dense, ns = Hkv - n_dense;
  const int cd = std::max(pl.chunks_dense, 1), cs = std::max(pl.chunks_stream, 1);
  // Chunks per split: the fewest that keep every wave of the launch resident at once
  // (wave_slots: what the device holds of this kernel): all waves then resolve their
  // pages before the memory system fills up, and none starts its index chain behind the
  // K/V traffic of others; and few enough splits for the merge. The kernel then cuts
  // each list into that many splits of equal size (to one chunk).
  const int64_t kWaves = std::max<int64_t>(1, std::min(wave_slots, kMaxWaveSlots));
  auto waves = [&](int c) {
    return (int64_t)B * ((int64_t)nd * ((cd + c - 1) / c) + (int64_t)ns * ((cs + c - 1) / c));
  };
  const int64_t total = (int64_t)B * ((int64_t)nd * cd + (int64_t)ns * cs);
  int cpw = (int)std::max<int64_t>(1, (total + kWaves - 1) / kWaves);
  while (cpw < std::max(cd, cs) && waves(cpw) > kWaves) ++cpw;
  // At least 4 chunks a split: a wave's fixed part (resolving its pages, writing its
  // partial, its share of the merge) costs about as much as streaming two chunks, so
  // smaller splits lose more than the extra waves gain (Llama-3-8B decode, 4 sequences:
  // a step of 31.4 us at 2 chunks a split, 27.6 at 4, 28.8 at 5, 31.6 at 8). At least 6
  // when the waves also rank their selection, a larger fixed part (the same step with
  // sparse_decode_select: 25.2 us at 3, 23.9-24.0 at 4, 23.5-23.7 at 5, 23.3-23.4 at 6,
  // 23.9-24.1 at 8). (A larger floor only lowers the split count: the workspace bound,
  // planned at the floor of 4, still holds.)
  cpw = std::max(cpw, ranks_selection ? 6 : 4);
  // (measurement override: UBS_DECODE_CPW sets the chunks per split; the result does not
  // depend on it beyond the order of the split merge)
  if (const char* e = getenv("UBS_DECODE_CPW")) {
    const int v = atoi(e);
    if (v >= 1 && v <= 4096) cpw = v;
  }
  while ((cd + cpw - 1) / cpw > kMaxSplits || (cs + cpw - 1) / cpw > kMaxSplits) ++cpw;
  pl.chunks_per_wave = cpw;
  pl.splits_dense = nd > 0 ? (cd + cpw - 1) / cpw : 1;
  pl.splits_stream = ns > 0 ? (cs + cpw - 1) / cpw : 1;
  pl.max_splits = pl.splits_dense > pl.splits_stream ? pl.splits_dense : pl.splits_stream;
  return pl;
}

// ----------------------------------------------------------------------------- static scratch
//
// The split partials of sparse_decode_static: a file-scope device array instead of a
// caller workspace, for callers that cannot allocate. Each GPU the library runs on holds
// its own copy (loaded with the code object) until the process ends. Host code never
// passes the array's name to a kernel (there it names a host-side stand-in): the first
// call on a device resolves the device address with hipGetSymbolAddress, with that device
// current, and keeps it per device; every later use goes through that address.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t static_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

int device_cu_count() {
  constexpr int kFallback = 256;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return kFallback;
  static std::mutex mu;
  static int cache[64] = {};
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev] > 0) return cache[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return kFallback;
  cache[dev] = n;
  return n;
}

int waves_per_group(int64_t waves, const char* env) {
  if (env != nullptr) {
    if (const char* e = getenv(env)) {
      const int v = atoi(e);
      if (v == 1 || v == 2 || v == 4) return v;
    }
  }
  const int64_t cus = device_cu_count();
  int wpg = 4;
  while (wpg > 1 && (waves + wpg - 1) / wpg < 2 * cus) wpg >>= 1;
  return wpg;
}

hipError_t launch_decode(const DecodeArgs& args, hipStream_t s) {
  const int per_b = args.dense.n * args.splits_dense + args.streaming.n * args.splits_stream;
  const int64_t waves = (int64_t)args.B * per_b;   // one split per wave
  if (waves == 0) return hipSuccess;
  DecodeArgs a = args;
  a.waves_per_group = waves_per_group(waves, "UBS_DECODE_WPG");
  const int64_t blocks = (waves + a.waves_per_group - 1) / a.waves_per_group;
  const dim3 block((unsigned)(64 * a.waves_per_group));
  const size_t fused_lds = (size_t)a.waves_per_group * a.fused_k * sizeof(int32_t);
  const int G = a.Hq / a.Hkv;
  const int64_t merge_blocks = (int64_t)a.B * a.Hq;   // one work-group per (b, query head)
  const size_t merge_lds = (size_t)(((int64_t)a.max_splits * (a.D + 2) + 255) / 256 * 256 + a.max_splits) * sizeof(float);
#define UBS_DECODE(DD, GG)                                                                            \
  if (a.D == DD && G == GG) {                                                                         \
    if (a.int4)                                                                                       \
      hipLaunchKernelGGL((decode_kernel<DD, GG, true>), dim3((unsigned)blocks), block, fused_lds, s, a); \
    else                                                                                              \
      hipLaunchKernelGGL((decode_kernel<DD, GG, false>), dim3((unsigned)blocks), block, fused_lds, s, a); \
    hipError_t e = hipGetLastError();                                                                 \
    if (e != hipSuccess || merge_blocks == 0) return e;                                               \
    hipLaunchKernelGGL((decode_merge_kernel<DD>), dim3((unsigned)merge_blocks), dim3(256), merge_lds, s, a); \
    return hipGetLastError();                                                                         \
  }
  UBS_DECODE(64, 1) UBS_DECODE(64, 2) UBS_DECODE(64, 4) UBS_DECODE(64, 8) UBS_DECODE(64, 16)
  UBS_DECODE(128, 1) UBS_DECODE(128, 2) UBS_DECODE(128, 4) UBS_DECODE(128, 8) UBS_DECODE(128, 16)
#undef UBS_DECODE
  return hipErrorInvalidValue;
}

}  // namespace ubs
