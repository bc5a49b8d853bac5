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

// Rows a decode wave ranks itself (64 lanes x 16 keys) and the largest budget it keeps
constexpr int kMaxFusedPages = 1024;
constexpr int kMaxFusedK = 1024;

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
  int score_only;  // scores only: the decode kernel ranks them (fused selection)
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
  int chunks_dense, chunks_stream;   // chunks of a (b, g) list, dense / streaming (upper bounds)
  float* out;
  float* lse;
  float* partials;     // workspace [B][Hq][max_splits][D + 2]
  int max_splits;
  int waves_per_group;   // waves of a work-group (1, 2 or 4): set by launch_decode
  // Selection ranked inside the kernel (fused_k > 0, the page budget k; rows of at most
  // kMaxFusedPages pages): each dense-head wave takes its row's top k from the page scores
  // into LDS, and split 0 of each row writes the row to sel_out [B][Hkv][k] / nsel_out
  // [B][Hkv]. fused_k = 0: the selection comes from `selected` / `num_selected`.
  const float* scores;   // [B][Hkv][max_pages]
  int fused_k;
  int32_t* sel_out;
  int32_t* nsel_out;
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

// Checked mode: what ubs_check_paged validates and the status record it fills
// (int32 [kind, b, index, value, head]; kind 0 = no violation).
enum CheckKind : int {
  kCheckSeqLen = 1,         // seq_lens[b] (or a cu_seqlens length) outside [0, max_pages * P]
  kCheckCuSeqlens = 2,      // cu_seqlens not starting at 0 or decreasing
  kCheckPageId = 3,         // page_table[b][j] outside [0, num_pages) for a page of the sequence
  kCheckNumSelected = 4,    // num_selected[b][g] outside [0, min(max_selected, pages of b)]
  kCheckSelected = 5,       // selected[b][g][slot] outside [0, pages of b)
  kCheckSelectedOrder = 6,  // selected[b][g] not strictly ascending
};
struct CheckArgs {
  const int32_t* page_table;
  const int32_t* seq_lens;     // or
  const int32_t* cu_seqlens;   // [B + 1]
  int B, max_pages, num_pages, P, Hkv;
  HeadList dense;
  const int32_t* selected;     // NULL: no selection to check
  const int32_t* num_selected;
  int max_selected;
  int32_t* status;
};
hipError_t launch_check(const CheckArgs& a, hipStream_t s);

// Decode split planning (shared by the workspace query and the launch).
struct DecodePlan {
  int chunks_dense, chunks_stream;  // upper bounds of key chunks per (b, KV head)
  int chunks_per_wave;
  int splits_dense, splits_stream, max_splits;
};
// Largest number of decode waves a plan spreads a launch over (4 waves per SIMD on 256
// CUs); the workspace size is computed for it, an upper bound of every launch's plan.
constexpr int64_t kMaxWaveSlots = 4 * 4 * 256;
int64_t decode_wave_slots(int D, int G, bool int4);
// Compute units of the current device (cached per device; 256 if the query fails).
int device_cu_count();
// Waves a work-group of a wave-independent launch (no work-group barrier) of `waves`
// waves: 4, or fewer while the launch would otherwise have under two work-groups per CU,
// so that a small launch still reaches every CU (each CU streams only its share of the
// bandwidth). `env` names a measurement override (1, 2 or 4).
int waves_per_group(int64_t waves, const char* env);
DecodePlan plan_decode(int B, int Hkv, int n_dense, int P, int max_selected, int sink, int local, bool int4,
                       int64_t wave_slots, bool ranks_selection = false);

// Size of the library-owned scratch of sparse_decode_static (per GPU), and its device
// address on the current device (resolved on the first call there).
constexpr size_t kStaticScratchBytes = size_t(32) << 20;
hipError_t static_scratch(void** ptr);

hipError_t launch_bounds(const BoundsArgs& a, hipStream_t s);
hipError_t launch_select(const SelectArgs& a, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s);
hipError_t launch_mask(const MaskArgs& a, hipStream_t s);
hipError_t launch_append(const AppendArgs& a, hipStream_t s);
hipError_t launch_quant_int4(const QuantArgs& a, hipStream_t s);

}  // namespace ubs
