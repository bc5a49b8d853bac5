// Host-side launch descriptors shared by the C ABI layer and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ubs {

// A small list of head indices passed by value as a kernel argument.
struct HeadList {
  int n;
  int16_t h[64];
};


struct BoundsArgs {
  const uint16_t* k_cache;
  const int32_t* page_table;
  const int32_t* seq_lens;
  int B, max_pages, Hkv, D, P, Lp;
  HeadList dense;
  uint16_t* bounds;
  // n_new > 0: an update after appending n_new tokens to each sequence; the sequence
  // is seq_lens[b] + n_new tokens long and only the sub-pages holding tokens at or
  // past seq_lens[b] are recomputed (page_span pages per sequence from page
  // seq_lens[b] / P). n_new = 0: every sub-page (page_span = max_pages).
  int n_new, page_span;
};

struct AppendArgs {
  const uint16_t* k_new;   // [B][n_new][Hkv][D]
  const uint16_t* v_new;
  const int32_t* page_table;
  const int32_t* seq_lens; // before the append
  int B, max_pages, n_new, Hkv, D, P;
  uint16_t* k_cache;
  uint16_t* v_cache;
};

struct SelectArgs {
  const uint16_t* q;
  const uint16_t* bounds;
  const int32_t* page_table;
  const int32_t* seq_lens;
  int B, max_pages, Hq, Hkv, D, P, Lp, k;
  HeadList dense;
  uint64_t streaming_mask;
  int32_t* selected;
  int32_t* num_selected;
  float* scores;  // workspace [B][Hkv][max_pages]
};

struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* page_table;
  const int32_t* seq_lens;
  const int32_t* selected;
  const int32_t* num_selected;
  int B, max_pages, Hq, Hkv, D, P, max_selected, sink, local;
  float sm_scale;
  HeadList dense, streaming;
  int splits_dense, splits_stream, chunks_per_wave;
  float* out;
  float* lse;
  float* partials;     // workspace [B][Hq][max_splits][D + 2]
  int max_splits;
  // INT4 pages (int4 != 0): codes [NP][Hkv][P][D/2], fp16 (scale, zero) [NP][Hkv][P][2]
  int int4;
  const uint8_t* k_codes;
  const uint8_t* v_codes;
  const uint16_t* k_params;
  const uint16_t* v_params;
};

struct QuantArgs {
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* page_table;
  const int32_t* seq_lens;
  int B, max_pages, Hkv, D, P;
  uint8_t* k_codes;
  uint8_t* v_codes;
  uint16_t* k_params;
  uint16_t* v_params;
};

struct PrefillArgs {
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* page_table;
  const uint8_t* block_mask;
  int L, Hq, Hkv, D, P, T, sink_tiles, local_tiles;
  int q_tile0;             // first query tile of the call (a chunk: tiles q_tile0 .. nT-1)
  // several sequences (cu_seqlens != nullptr): sequence b is rows cu_seqlens[b] ..
  // cu_seqlens[b+1]-1 of q / out / lse, page-table row b (pt_stride entries), mask
  // block b of [Hq][nT_max][nT_max]; L and q_tile0 are unused
  const int32_t* cu_seqlens;
  int n_seq, pt_stride, nT_max, total_q;
  int log2_P;
  float sm_scale;
  uint64_t dense_kv_mask;  // bit g set: KV head g is dense
  int n_dense_kv;
  float* out;
  float* lse;
};

struct MaskArgs {
  const uint16_t* q;
  const uint16_t* k_cache;
  const int32_t* page_table;
  int L, Hq, Hkv, D, P, T, log2_P, nT, G;
  int keep_num, keep_den;
  HeadList dense_kv;     // dense KV heads; their query heads are the dense query heads
  uint8_t* block_mask;
  float* qmean;          // workspace [n_dense_kv * G][nT][D]
  float* kmean;          // workspace [n_dense_kv][nT][D]
};

// Decode split planning (shared by the workspace query and the launch).
struct DecodePlan {
  int chunks_dense, chunks_stream;  // upper bounds of key chunks per (b, KV head)
  int chunks_per_wave;
  int splits_dense, splits_stream, max_splits;
};
DecodePlan plan_decode(int B, int Hkv, int n_dense, int P, int max_selected, int sink, int local);

hipError_t launch_bounds(const BoundsArgs& a, hipStream_t s);
hipError_t launch_select(const SelectArgs& a, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s);
hipError_t launch_mask(const MaskArgs& a, hipStream_t s);
hipError_t launch_append(const AppendArgs& a, hipStream_t s);
hipError_t launch_quant_int4(const QuantArgs& a, hipStream_t s);

}  // namespace ubs
