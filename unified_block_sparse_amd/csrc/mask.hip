// estimate_block_mask: the dense heads' prefill block mask from mean-pooled tile
// scores, the query-tile-level estimate of block sparsity for the blog's "LServe --
// Prefill Phase" (a KV tile computed or skipped whole per query tile): per query tile
// i, the diagonal and the ceil(keep_num*(i+1)/keep_den) - 1 strictly-lower tiles j of
// largest mean(Q tile i) . mean(K tile j), equal scores to the lower j.
//
// Two launches:
//   tile_mean_kernel  one work-group per (tile, head): the fp32 mean of the tile's rows
//                     of a dense query head (Q) or a dense KV head (K, through the page
//                     table), 16-byte loads, a fixed summation order;
//   mask_row_kernel   one wave per (dense query head, query tile), four consecutive
//                     tiles of one head per work-group sharing LDS-staged chunks of 64
//                     K tile means: lane l scores candidate j = 64e + l into register
//                     e (fp32 dot in channel order), the wave finds the row's threshold
//                     by a bitwise binary search over order-preserving keys (ballot
//                     counts), keeps everything above it and the lowest-index ties, and
//                     writes the row's nT mask bytes.
#include "common.h"
#include "launch.h"

namespace ubs {

template <int D>
__global__ __launch_bounds__(256) void tile_mean_kernel(const MaskArgs a) {
  constexpr int CPR = D / 8;       // threads per row, 8 channels each
  constexpr int RPP = 256 / CPR;   // rows per pass
  __shared__ float part[RPP][D + 1];
  const int nq = a.dense_kv.n * a.G;
  // head slot fastest: the work-groups running together read the dense heads of the same
  // tiles, whole runs of each token's [Hq][D] row of q (and whole K pages), instead of
  // one head's 2*D bytes out of many rows
  const int slot = blockIdx.x % (nq + a.dense_kv.n);
  const int tile = blockIdx.x / (nq + a.dense_kv.n);
  const int tid = threadIdx.x, rr = tid / CPR, cc = tid % CPR;
  const int r0 = tile * a.T, r1 = min(r0 + a.T, a.L);
  const bool isq = slot < nq;
  const int g = isq ? a.dense_kv.h[slot / a.G] : a.dense_kv.h[slot - nq];
  const int h = g * a.G + (isq ? slot % a.G : 0);
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  // all of a thread's rows (at most 128 / RPP) loaded before any is summed
  constexpr int MAXR = 128 / RPP;
  u32x4 v[MAXR];
#pragma unroll
  for (int x = 0; x < MAXR; ++x) {
    // (rows past the tile's end are clamped to its last row for the address, so that no
    // page-table entry past the sequence is read; their values are not used)
    const int r = r0 + rr + x * RPP;
    const int rc = min(r, r1 - 1);
    const uint16_t* src =
        isq ? a.q + ((int64_t)rc * a.Hq + h) * D + cc * 8
            : a.k_cache + (((int64_t)a.page_table[rc >> a.log2_P] * a.Hkv + g) * a.P + (rc & (a.P - 1))) * D + cc * 8;
    v[x] = (r < r1) ? ld16(src) : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int x = 0; x < MAXR; ++x)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += bf16_lo(v[x][e]);
      acc[2 * e + 1] += bf16_hi(v[x][e]);
    }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[rr][cc * 8 + e] = acc[e];
  __syncthreads();
  if (tid < D) {
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < RPP; ++k) s += part[k][tid];
    float* dst = isq ? a.qmean + ((int64_t)slot * a.nT + tile) * D : a.kmean + ((int64_t)(slot - nq) * a.nT + tile) * D;
    dst[tid] = s / (float)(r1 - r0);
  }
}

template <int D, int EPT>
__global__ __launch_bounds__(256) void mask_row_kernel(const MaskArgs a) {
  __shared__ __attribute__((aligned(16))) float kb[64][D + 4];
  __shared__ __attribute__((aligned(16))) float qv[4][D];
  const int rows_per_head = (a.nT + 3) / 4;
  const int slot = blockIdx.x / rows_per_head;          // dense query-head slot
  const int i0 = (blockIdx.x % rows_per_head) * 4;
  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kslot = slot / a.G;                          // its dense KV head's slot
  const int g = a.dense_kv.h[kslot];
  const int h = g * a.G + slot % a.G;
  const int i = i0 + wave;                               // this wave's query tile
  const int i_last = min(i0 + 3, a.nT - 1);
  for (int x = tid; x < 4 * D; x += 256) {
    const int w = x / D, c = x % D;
    qv[w][c] = (i0 + w < a.nT) ? a.qmean[((int64_t)slot * a.nT + i0 + w) * D + c] : 0.f;
  }
  // ---- scores of the candidates j < i: lane l, register e -> j = 64e + l. Chunk e of 64
  // K-tile means goes through LDS; its loads are issued into registers while chunk e-1 is
  // scored (thread tid holds pieces tid + 256u of the chunk).
  constexpr int NPC = 64 * (D / 4) / 256;   // 16-byte pieces per thread and chunk
  uint32_t key[EPT];   // order-preserving key of the score, 0 = not a candidate
  const int nchunks = (i_last + 63) / 64;
  f32x4 nxt[NPC];
  auto load_chunk = [&](int e) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < NPC; ++u) {
      const int x = tid + 256 * u;
      const int t = x / (D / 4), c4 = x % (D / 4);
      const int j = e * 64 + t;
      nxt[u] = j < a.nT ? *reinterpret_cast<const f32x4*>(a.kmean + ((int64_t)kslot * a.nT + j) * D + c4 * 4)
                        : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  if (nchunks > 0) load_chunk(0);
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    key[e] = 0u;
    if (e < nchunks) {   // uniform over the work-group
      __syncthreads();   // the previous chunk is consumed (and qv is written)
#pragma unroll
      for (int u = 0; u < NPC; ++u) {
        const int x = tid + 256 * u;
        *reinterpret_cast<f32x4*>(&kb[x / (D / 4)][(x % (D / 4)) * 4]) = nxt[u];
      }
      if (e + 1 < nchunks) load_chunk(e + 1);
      __syncthreads();
      float s = 0.f;
#pragma unroll 8
      for (int c = 0; c < D; c += 4) {
        const f32x4 kk = *reinterpret_cast<const f32x4*>(&kb[lane][c]);
        const f32x4 qq = *reinterpret_cast<const f32x4*>(&qv[wave][c]);
        s = fmaf(qq[0], kk[0], s);
        s = fmaf(qq[1], kk[1], s);
        s = fmaf(qq[2], kk[2], s);
        s = fmaf(qq[3], kk[3], s);
      }
      const int j = e * 64 + lane;
      key[e] = (j < i) ? float_order_key(s) : 0u;
    }
  }
  if (i >= a.nT) return;   // padding wave of the last work-group of a head (no barrier follows)
  // ---- threshold: the take-th largest key, take = n_i - 1 (the diagonal is kept anyway)
  const int take = (int)(((int64_t)a.keep_num * (i + 1) + a.keep_den - 1) / a.keep_den) - 1;
  uint32_t tau = 0xffffffffu;   // with take <= 0 nothing but the diagonal is kept
  if (take > 0) {
    tau = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = tau | (1u << bit);
      int c = 0;
#pragma unroll
      for (int e = 0; e < EPT; ++e) c += __popcll(__ballot(key[e] >= cand));
      if (c >= take) tau = cand;
      if (c == take) break;   // exactly take keys at or above: the answer, no tie at tau
    }
  }
  // #(key > tau) < take <= #(key >= tau) (after an early exit #(key >= tau) = take, and
  // every key equal to tau is kept): every key above tau, then ties by ascending j
  int n_gt = 0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) n_gt += __popcll(__ballot(key[e] > tau && key[e] != 0u));
  const int take_ties = take - n_gt;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int tie_base = 0;
  uint8_t* row = a.block_mask + ((int64_t)h * a.nT + i) * a.nT;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const bool tie = take > 0 && key[e] == tau && key[e] != 0u;
    const uint64_t tm = __ballot(tie);
    const bool kept = (take > 0 && key[e] > tau && key[e] != 0u) ||
                      (tie && tie_base + __popcll(tm & below) < take_ties);
    tie_base += __popcll(tm);
    const int j = e * 64 + lane;
    if (j < a.nT) row[j] = (uint8_t)((j == i || kept) ? 1 : 0);
  }
}

hipError_t launch_mask(const MaskArgs& a, hipStream_t s) {
  const int nq = a.dense_kv.n * a.G;
  if (a.nT == 0 || nq == 0) return hipSuccess;
  const int64_t b1 = (int64_t)(nq + a.dense_kv.n) * a.nT;
  const int64_t b2 = (int64_t)nq * ((a.nT + 3) / 4);
  const int ept = (a.nT + 63) / 64;
#define UBS_MEAN(DD)                                                                        \
  if (a.D == DD) {                                                                          \
    hipLaunchKernelGGL((tile_mean_kernel<DD>), dim3((unsigned)b1), dim3(256), 0, s, a);      \
    hipError_t e = hipGetLastError();                                                       \
    if (e != hipSuccess) return e;                                                          \
  }
  UBS_MEAN(64) UBS_MEAN(128)
#undef UBS_MEAN
#define UBS_ROWS(DD, E)                                                                     \
  if (a.D == DD && ept <= E) {                                                              \
    hipLaunchKernelGGL((mask_row_kernel<DD, E>), dim3((unsigned)b2), dim3(256), 0, s, a);   \
    return hipGetLastError();                                                               \
  }
  UBS_ROWS(64, 1) UBS_ROWS(64, 2) UBS_ROWS(64, 4) UBS_ROWS(64, 8) UBS_ROWS(64, 16) UBS_ROWS(64, 32)
  UBS_ROWS(64, 64) UBS_ROWS(128, 1) UBS_ROWS(128, 2) UBS_ROWS(128, 4) UBS_ROWS(128, 8) UBS_ROWS(128, 16)
  UBS_ROWS(128, 32) UBS_ROWS(128, 64)
#undef UBS_ROWS
  return hipErrorInvalidValue;
}

}  // namespace ubs
