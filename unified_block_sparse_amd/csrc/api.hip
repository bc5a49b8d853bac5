// C ABI of libubs: argument validation (host only, before any HIP call), workspace
// sizing and dispatch to the gfx950 kernels. See include/ubs.h for the contract.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/ubs.h"
#include "common.h"
#include "launch.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return UBS_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(UBS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define REQUIRE(cond, code, ...) \
  do {                           \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

// Splits head_kind (host) into dense / streaming KV-head lists.
int head_lists(const uint8_t* head_kind, int Hkv, ubs::HeadList* dense, ubs::HeadList* streaming,
               uint64_t* streaming_mask) {
  REQUIRE(head_kind != nullptr, UBS_ERR_INVALID_ARGUMENT, "head_kind is NULL");
  REQUIRE(Hkv >= 1 && Hkv <= ubs::kMaxKvHeads, UBS_ERR_UNSUPPORTED, "Hkv=%d outside [1, %d]", Hkv,
          ubs::kMaxKvHeads);
  dense->n = 0;
  streaming->n = 0;
  *streaming_mask = 0;
  for (int g = 0; g < Hkv; ++g) {
    REQUIRE(head_kind[g] <= 1, UBS_ERR_INVALID_ARGUMENT, "head_kind[%d]=%d is neither 0 nor 1", g,
            (int)head_kind[g]);
    if (head_kind[g]) {
      streaming->h[streaming->n++] = (int16_t)g;
      *streaming_mask |= 1ull << g;
    } else {
      dense->h[dense->n++] = (int16_t)g;
    }
  }
  return UBS_OK;
}

int common_heads(int Hq, int Hkv, int D) {
  REQUIRE(Hq >= 1 && Hkv >= 1, UBS_ERR_INVALID_ARGUMENT, "Hq=%d, Hkv=%d must be positive", Hq, Hkv);
  REQUIRE(Hq % Hkv == 0, UBS_ERR_INVALID_ARGUMENT, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  REQUIRE(D == 64 || D == 128, UBS_ERR_UNSUPPORTED, "D=%d (supported: 64, 128)", D);
  return UBS_OK;
}

int paged_P(int P) {
  REQUIRE(P > 0, UBS_ERR_INVALID_ARGUMENT, "P=%d must be positive", P);
  REQUIRE(P == 16 || P == 32 || P == 64 || P == 128, UBS_ERR_UNSUPPORTED,
          "P=%d (supported: 16, 32, 64, 128)", P);
  return UBS_OK;
}

constexpr int kMaxSelectPages = 16384;
static_assert(UBS_STATIC_SCRATCH_BYTES == ubs::kStaticScratchBytes, "static scratch size in ubs.h and launch.h");

}  // namespace

extern "C" {

const char* ubs_last_error(void) { return g_last_error.c_str(); }

int ubs_version(void) { return 100; }

int sparse_prefill_chunk(const ubs_bf16_t* q, const ubs_bf16_t* k_cache, const ubs_bf16_t* v_cache,
                         const int32_t* page_table, int32_t L, int32_t q_start, int32_t Hq, int32_t Hkv,
                         int32_t D, int32_t P, int32_t T, const uint8_t* head_kind, const uint8_t* block_mask,
                         int32_t sink_tiles, int32_t local_tiles, float sm_scale, float* out, float* lse,
                         hipStream_t stream) {
  int rc = common_heads(Hq, Hkv, D);
  if (rc) return rc;
  REQUIRE(L >= 0, UBS_ERR_INVALID_ARGUMENT, "L=%d is negative", L);
  REQUIRE(T == 64 || T == 128, UBS_ERR_UNSUPPORTED, "T=%d (supported: 64, 128)", T);
  REQUIRE(q_start >= 0 && q_start <= L && q_start % T == 0, UBS_ERR_INVALID_ARGUMENT,
          "q_start=%d must be a multiple of T=%d in [0, L=%d]", q_start, T, L);
  REQUIRE(P > 0, UBS_ERR_INVALID_ARGUMENT, "P=%d must be positive", P);
  REQUIRE(pow2(P) && P >= 16 && P <= 4096, UBS_ERR_UNSUPPORTED, "P=%d (supported: powers of two 16..4096)", P);
  REQUIRE(Hq <= ubs::kMaxQHeads, UBS_ERR_UNSUPPORTED, "Hq=%d above %d", Hq, ubs::kMaxQHeads);
  REQUIRE(sink_tiles >= 0 && local_tiles >= 0, UBS_ERR_INVALID_ARGUMENT,
          "sink_tiles=%d, local_tiles=%d must be >= 0", sink_tiles, local_tiles);
  REQUIRE(std::isfinite(sm_scale) && sm_scale > 0.f, UBS_ERR_INVALID_ARGUMENT,
          "sm_scale=%g must be finite and positive", (double)sm_scale);
  ubs::HeadList dense, streaming;
  uint64_t smask;
  rc = head_lists(head_kind, Hkv, &dense, &streaming, &smask);
  if (rc) return rc;
  if (L == q_start) return ok();
  REQUIRE(q && k_cache && v_cache && page_table && out, UBS_ERR_INVALID_ARGUMENT,
          "q, k_cache, v_cache, page_table and out must be non-NULL");
  REQUIRE(dense.n == 0 || block_mask, UBS_ERR_INVALID_ARGUMENT, "block_mask is NULL but a KV head is dense");
  REQUIRE(aligned16(q) && aligned16(k_cache) && aligned16(v_cache) && aligned16(out), UBS_ERR_INVALID_ARGUMENT,
          "q, k_cache, v_cache and out must be 16-byte aligned");
  const int64_t nT = (L + T - 1) / T;
  REQUIRE(nT <= ubs::kMaxTileList, UBS_ERR_UNSUPPORTED, "L=%d spans %lld tiles of %d (at most %d)", L,
          (long long)nT, T, ubs::kMaxTileList);
  REQUIRE((nT - q_start / T) * Hq < (1ll << 31), UBS_ERR_UNSUPPORTED, "grid of %lld work-groups is too large",
          (long long)((nT - q_start / T) * Hq));
  ubs::PrefillArgs a{};
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.page_table = page_table;
  a.block_mask = block_mask;
  a.L = L;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  a.P = P;
  a.T = T;
  a.q_tile0 = q_start / T;
  a.log2_P = __builtin_ctz((unsigned)P);
  a.sink_tiles = sink_tiles;
  a.local_tiles = local_tiles;
  a.sm_scale = sm_scale;
  a.out = out;
  a.lse = lse;
  a.dense_kv_mask = ~smask & (Hkv == 64 ? ~0ull : ((1ull << Hkv) - 1));
  a.n_dense_kv = dense.n;
  return hip_status(ubs::launch_prefill(a, stream), "sparse_prefill launch");
}

int sparse_prefill_varlen(const ubs_bf16_t* q, const ubs_bf16_t* k_cache, const ubs_bf16_t* v_cache,
                          const int32_t* page_table, int32_t max_pages, const int32_t* cu_seqlens, int32_t B,
                          int32_t max_seqlen, int32_t total_q, int32_t Hq, int32_t Hkv, int32_t D, int32_t P,
                          int32_t T, const uint8_t* head_kind, const uint8_t* block_mask, int32_t sink_tiles,
                          int32_t local_tiles, float sm_scale, float* out, float* lse, hipStream_t stream) {
  int rc = common_heads(Hq, Hkv, D);
  if (rc) return rc;
  REQUIRE(B >= 0 && max_seqlen >= 0 && total_q >= 0 && max_pages >= 0, UBS_ERR_INVALID_ARGUMENT,
          "B=%d, max_seqlen=%d, total_q=%d, max_pages=%d must be >= 0", B, max_seqlen, total_q, max_pages);
  REQUIRE(T == 64 || T == 128, UBS_ERR_UNSUPPORTED, "T=%d (supported: 64, 128)", T);
  REQUIRE(P > 0, UBS_ERR_INVALID_ARGUMENT, "P=%d must be positive", P);
  REQUIRE(pow2(P) && P >= 16 && P <= 4096, UBS_ERR_UNSUPPORTED, "P=%d (supported: powers of two 16..4096)", P);
  REQUIRE(Hq <= ubs::kMaxQHeads, UBS_ERR_UNSUPPORTED, "Hq=%d above %d", Hq, ubs::kMaxQHeads);
  REQUIRE(sink_tiles >= 0 && local_tiles >= 0, UBS_ERR_INVALID_ARGUMENT,
          "sink_tiles=%d, local_tiles=%d must be >= 0", sink_tiles, local_tiles);
  REQUIRE(std::isfinite(sm_scale) && sm_scale > 0.f, UBS_ERR_INVALID_ARGUMENT,
          "sm_scale=%g must be finite and positive", (double)sm_scale);
  REQUIRE((int64_t)max_pages * P >= max_seqlen, UBS_ERR_INVALID_ARGUMENT,
          "max_pages=%d pages of %d tokens cannot hold max_seqlen=%d", max_pages, P, max_seqlen);
  ubs::HeadList dense, streaming;
  uint64_t smask;
  rc = head_lists(head_kind, Hkv, &dense, &streaming, &smask);
  if (rc) return rc;
  if (B == 0 || max_seqlen == 0 || total_q == 0) return ok();
  REQUIRE(q && k_cache && v_cache && page_table && cu_seqlens && out, UBS_ERR_INVALID_ARGUMENT,
          "q, k_cache, v_cache, page_table, cu_seqlens and out must be non-NULL");
  REQUIRE(dense.n == 0 || block_mask, UBS_ERR_INVALID_ARGUMENT, "block_mask is NULL but a KV head is dense");
  REQUIRE(aligned16(q) && aligned16(k_cache) && aligned16(v_cache) && aligned16(out), UBS_ERR_INVALID_ARGUMENT,
          "q, k_cache, v_cache and out must be 16-byte aligned");
  const int64_t nTm = (max_seqlen + T - 1) / T;
  REQUIRE(nTm <= ubs::kMaxTileList, UBS_ERR_UNSUPPORTED, "max_seqlen=%d spans %lld tiles of %d (at most %d)",
          max_seqlen, (long long)nTm, T, ubs::kMaxTileList);
  REQUIRE((int64_t)B * Hq * nTm < (1ll << 31), UBS_ERR_UNSUPPORTED, "grid of %lld work-groups is too large",
          (long long)((int64_t)B * Hq * nTm));
  ubs::PrefillArgs a{};
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.page_table = page_table;
  a.block_mask = block_mask;
  a.L = 0;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  a.P = P;
  a.T = T;
  a.q_tile0 = 0;
  a.cu_seqlens = cu_seqlens;
  a.n_seq = B;
  a.pt_stride = max_pages;
  a.nT_max = (int)nTm;
  a.total_q = total_q;
  a.log2_P = __builtin_ctz((unsigned)P);
  a.sink_tiles = sink_tiles;
  a.local_tiles = local_tiles;
  a.sm_scale = sm_scale;
  a.out = out;
  a.lse = lse;
  a.dense_kv_mask = ~smask & (Hkv == 64 ? ~0ull : ((1ull << Hkv) - 1));
  a.n_dense_kv = dense.n;
  return hip_status(ubs::launch_prefill(a, stream), "sparse_prefill_varlen launch");
}

int sparse_prefill(const ubs_bf16_t* q, const ubs_bf16_t* k_cache, const ubs_bf16_t* v_cache,
                   const int32_t* page_table, int32_t L, int32_t Hq, int32_t Hkv, int32_t D, int32_t P,
                   int32_t T, const uint8_t* head_kind, const uint8_t* block_mask, int32_t sink_tiles,
                   int32_t local_tiles, float sm_scale, float* out, float* lse, hipStream_t stream) {
  return sparse_prefill_chunk(q, k_cache, v_cache, page_table, L, 0, Hq, Hkv, D, P, T, head_kind, block_mask,
                              sink_tiles, local_tiles, sm_scale, out, lse, stream);
}

int build_page_bounds(const ubs_bf16_t* k_cache, const int32_t* page_table, const int32_t* seq_lens,
                      int32_t B, int32_t max_pages, int32_t Hkv, int32_t D, int32_t P, int32_t Lp,
                      const uint8_t* head_kind, ubs_bf16_t* bounds, hipStream_t stream) {
  REQUIRE(B >= 0 && max_pages >= 0, UBS_ERR_INVALID_ARGUMENT, "B=%d, max_pages=%d must be >= 0", B, max_pages);
  REQUIRE(D == 64 || D == 128, UBS_ERR_UNSUPPORTED, "D=%d (supported: 64, 128)", D);
  int rc = paged_P(P);
  if (rc) return rc;
  REQUIRE(Lp > 0 && P % Lp == 0, UBS_ERR_UNSUPPORTED, "Lp=%d must divide P=%d", Lp, P);
  ubs::HeadList dense, streaming;
  uint64_t smask;
  rc = head_lists(head_kind, Hkv, &dense, &streaming, &smask);
  if (rc) return rc;
  if (B == 0 || max_pages == 0 || dense.n == 0) return ok();
  REQUIRE(k_cache && page_table && seq_lens && bounds, UBS_ERR_INVALID_ARGUMENT,
          "k_cache, page_table, seq_lens and bounds must be non-NULL");
  REQUIRE(aligned16(k_cache) && aligned16(bounds), UBS_ERR_INVALID_ARGUMENT,
          "k_cache and bounds must be 16-byte aligned");
  ubs::BoundsArgs a{k_cache, page_table, seq_lens, B, max_pages, Hkv, D, P, Lp, dense, bounds, 0, max_pages};
  return hip_status(ubs::launch_bounds(a, stream), "build_page_bounds launch");
}

size_t ubs_select_workspace_size(int32_t B, int32_t max_pages, int32_t Hkv) {
  if (B <= 0 || max_pages <= 0 || Hkv <= 0) return 256;
  return ((size_t)B * Hkv * max_pages * sizeof(float) + 255) / 256 * 256;
}

// Shared body of select_pages and the selection half of sparse_decode_select: validates
// every argument, then (launch) enqueues the scores and, unless score_only (the decode
// kernel then ranks them), the top-k.
static int select_impl(const ubs_bf16_t* q, const ubs_bf16_t* bounds, const int32_t* page_table,
                       const int32_t* seq_lens, int32_t B, int32_t max_pages, int32_t Hq, int32_t Hkv, int32_t D,
                       int32_t P, int32_t Lp, int32_t token_budget, const uint8_t* head_kind, int32_t* selected,
                       int32_t* num_selected, void* workspace, size_t workspace_bytes, bool score_only,
                       bool launch, hipStream_t stream) {
  int rc = common_heads(Hq, Hkv, D);
  if (rc) return rc;
  REQUIRE(B >= 0 && max_pages >= 0, UBS_ERR_INVALID_ARGUMENT, "B=%d, max_pages=%d must be >= 0", B, max_pages);
  rc = paged_P(P);
  if (rc) return rc;
  REQUIRE(Lp > 0 && P % Lp == 0, UBS_ERR_UNSUPPORTED, "Lp=%d must divide P=%d", Lp, P);
  REQUIRE(pow2(P / Lp) && P / Lp <= 16, UBS_ERR_UNSUPPORTED, "P/Lp=%d (supported: 1, 2, 4, 8, 16)", P / Lp);
  REQUIRE(Hq / Hkv <= 16 && pow2(Hq / Hkv), UBS_ERR_UNSUPPORTED, "Hq/Hkv=%d (supported: 1, 2, 4, 8, 16)",
          Hq / Hkv);
  REQUIRE(token_budget > 0, UBS_ERR_INVALID_ARGUMENT, "token_budget=%d must be positive", token_budget);
  REQUIRE(token_budget % P == 0, UBS_ERR_UNSUPPORTED, "token_budget=%d is not a multiple of P=%d", token_budget, P);
  REQUIRE(max_pages <= kMaxSelectPages, UBS_ERR_UNSUPPORTED, "max_pages=%d above %d", max_pages, kMaxSelectPages);
  ubs::HeadList dense, streaming;
  uint64_t smask;
  rc = head_lists(head_kind, Hkv, &dense, &streaming, &smask);
  if (rc) return rc;
  if (B == 0) return ok();
  REQUIRE(q && page_table && seq_lens && selected && num_selected, UBS_ERR_INVALID_ARGUMENT,
          "q, page_table, seq_lens, selected and num_selected must be non-NULL");
  REQUIRE(dense.n == 0 || bounds, UBS_ERR_INVALID_ARGUMENT, "bounds is NULL but a KV head is dense");
  REQUIRE(aligned16(q) && (bounds == nullptr || aligned16(bounds)), UBS_ERR_INVALID_ARGUMENT,
          "q and bounds must be 16-byte aligned");
  const size_t need = ubs_select_workspace_size(B, max_pages, Hkv);
  REQUIRE(workspace && workspace_bytes >= need, UBS_ERR_WORKSPACE_TOO_SMALL,
          "workspace of %zu bytes, need %zu", workspace_bytes, need);
  ubs::SelectArgs a{};
  a.q = q;
  a.bounds = bounds;
  a.page_table = page_table;
  a.seq_lens = seq_lens;
  a.B = B;
  a.max_pages = max_pages;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  a.P = P;
  a.Lp = Lp;
  a.k = token_budget / P;
  a.dense = dense;
  a.streaming_mask = smask;
  a.selected = selected;
  a.num_selected = num_selected;
  a.scores = static_cast<float*>(workspace);
  a.score_only = score_only ? 1 : 0;
  if (!launch) return ok();
  return hip_status(ubs::launch_select(a, stream), "select_pages launch");
}

int select_pages(const ubs_bf16_t* q, const ubs_bf16_t* bounds, const int32_t* page_table,
                 const int32_t* seq_lens, int32_t B, int32_t max_pages, int32_t Hq, int32_t Hkv, int32_t D,
                 int32_t P, int32_t Lp, int32_t token_budget, const uint8_t* head_kind, int32_t* selected,
                 int32_t* num_selected, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return select_impl(q, bounds, page_table, seq_lens, B, max_pages, Hq, Hkv, D, P, Lp, token_budget, head_kind,
                     selected, num_selected, workspace, workspace_bytes, false, true, stream);
}

size_t ubs_decode_workspace_size(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t P,
                                    int32_t max_selected, int32_t sink_tokens, int32_t local_tokens) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || P <= 0 || max_selected < 0 || sink_tokens < 0 ||
      local_tokens < 0)
    return 256;
  // the split plan depends only on these sizes, the number of dense KV heads, the page
  // format and the waves the device holds at once: take the largest over every count
  // and both formats, at the most waves a plan spreads over
  int ms = 1;
  for (int nd = 0; nd <= Hkv; ++nd)
    for (int q4 = 0; q4 < 2; ++q4) {
      const ubs::DecodePlan pl =
          ubs::plan_decode(B, Hkv, nd, P, max_selected, sink_tokens, local_tokens, q4 != 0, ubs::kMaxWaveSlots);
      ms = pl.max_splits > ms ? pl.max_splits : ms;
    }
  return ((size_t)B * Hq * ms * (D + 2) * sizeof(float) + 255) / 256 * 256;
}

// Shared body of sparse_decode (bf16 pages: k, v are the caches) and sparse_decode_int4
// (k, v are the code arrays, kp, vp the row params).
static int decode_impl(const char* name, bool int4, bool use_static, const ubs_bf16_t* q, const void* k, const void* v,
                       const uint16_t* kp, const uint16_t* vp, const int32_t* page_table, const int32_t* seq_lens,
                       int32_t B, int32_t max_pages, int32_t Hq, int32_t Hkv, int32_t D, int32_t P,
                       const uint8_t* head_kind, const int32_t* selected, const int32_t* num_selected,
                       int32_t max_selected, int32_t sink_tokens, int32_t local_tokens, float sm_scale, float* out,
                       float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream,
                       bool launch = true, const float* fused_scores = nullptr, int32_t* sel_out = nullptr,
                       int32_t* nsel_out = nullptr) {
  // fused (fused_scores != NULL): the kernel ranks the page scores itself and writes the
  // selection to sel_out / nsel_out ([B][Hkv][max_selected], [B][Hkv])
  const bool fused = fused_scores != nullptr;
  int rc = common_heads(Hq, Hkv, D);
  if (rc) return rc;
  REQUIRE(B >= 0 && max_pages >= 0, UBS_ERR_INVALID_ARGUMENT, "B=%d, max_pages=%d must be >= 0", B, max_pages);
  REQUIRE(P > 0 && P % 16 == 0 && P <= 256, UBS_ERR_UNSUPPORTED, "P=%d must be a multiple of 16 up to 256", P);
  REQUIRE(Hq / Hkv <= 16 && pow2(Hq / Hkv), UBS_ERR_UNSUPPORTED, "Hq/Hkv=%d (supported: 1, 2, 4, 8, 16)",
          Hq / Hkv);
  REQUIRE(max_selected >= 0 && sink_tokens >= 0 && local_tokens >= 0, UBS_ERR_INVALID_ARGUMENT,
          "max_selected=%d, sink_tokens=%d, local_tokens=%d must be >= 0", max_selected, sink_tokens,
          local_tokens);
  REQUIRE(std::isfinite(sm_scale) && sm_scale > 0.f, UBS_ERR_INVALID_ARGUMENT,
          "sm_scale=%g must be finite and positive", (double)sm_scale);
  ubs::HeadList dense, streaming;
  uint64_t smask;
  rc = head_lists(head_kind, Hkv, &dense, &streaming, &smask);
  if (rc) return rc;
  if (B == 0) return ok();
  if (int4) {
    REQUIRE(q && k && v && kp && vp && page_table && seq_lens && out, UBS_ERR_INVALID_ARGUMENT,
            "q, k_codes, v_codes, k_params, v_params, page_table, seq_lens and out must be non-NULL");
    REQUIRE(aligned16(q) && aligned16(k) && aligned16(v) && ((uintptr_t)kp % 4 == 0) && ((uintptr_t)vp % 4 == 0),
            UBS_ERR_INVALID_ARGUMENT, "q and the codes must be 16-byte aligned, the params 4-byte aligned");
  } else {
    REQUIRE(q && k && v && page_table && seq_lens && out, UBS_ERR_INVALID_ARGUMENT,
            "q, k_cache, v_cache, page_table, seq_lens and out must be non-NULL");
    REQUIRE(aligned16(q) && aligned16(k) && aligned16(v), UBS_ERR_INVALID_ARGUMENT,
            "q, k_cache and v_cache must be 16-byte aligned");
  }
  if (fused) {
    REQUIRE(sel_out && nsel_out, UBS_ERR_INVALID_ARGUMENT, "selected and num_selected must be non-NULL");
  } else {
    REQUIRE(dense.n == 0 || max_selected == 0 || (selected && num_selected), UBS_ERR_INVALID_ARGUMENT,
            "selected / num_selected are NULL but a KV head is dense");
    REQUIRE(dense.n == 0 || num_selected, UBS_ERR_INVALID_ARGUMENT,
            "num_selected is NULL but a KV head is dense");
  }
  const size_t need = ubs_decode_workspace_size(B, Hq, Hkv, D, P, max_selected, sink_tokens, local_tokens);
  if (use_static) {
    REQUIRE(need <= ubs::kStaticScratchBytes, UBS_ERR_WORKSPACE_TOO_SMALL,
            "%s needs %zu bytes of scratch for B=%d, Hq=%d, D=%d; its static scratch holds %zu "
            "(use sparse_decode with a workspace)", name, need, B, Hq, D, ubs::kStaticScratchBytes);
    const hipError_t e = ubs::static_scratch(&workspace);
    if (e != hipSuccess) return hip_status(e, "static scratch address");
    workspace_bytes = ubs::kStaticScratchBytes;
  }
  REQUIRE(workspace && workspace_bytes >= need, UBS_ERR_WORKSPACE_TOO_SMALL,
          "workspace of %zu bytes, need %zu", workspace_bytes, need);
  const ubs::DecodePlan pl = ubs::plan_decode(B, Hkv, dense.n, P, max_selected, sink_tokens, local_tokens, int4,
                                              ubs::decode_wave_slots(D, Hq / Hkv, int4 != 0), fused);
  const int64_t blocks = (int64_t)B * (dense.n * pl.splits_dense + streaming.n * pl.splits_stream);
  REQUIRE(blocks < (1ll << 31), UBS_ERR_UNSUPPORTED, "grid of %lld work-groups is too large", (long long)blocks);
  ubs::DecodeArgs a{};
  a.q = q;
  if (int4) {
    a.int4 = 1;
    a.k_codes = static_cast<const uint8_t*>(k);
    a.v_codes = static_cast<const uint8_t*>(v);
    a.k_params = kp;
    a.v_params = vp;
  } else {
    a.k_cache = static_cast<const uint16_t*>(k);
    a.v_cache = static_cast<const uint16_t*>(v);
  }
  a.page_table = page_table;
  a.seq_lens = seq_lens;
  a.selected = selected;
  a.num_selected = num_selected;
  a.B = B;
  a.max_pages = max_pages;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  a.P = P;
  a.max_selected = max_selected;
  a.sink = sink_tokens;
  a.local = local_tokens;
  a.sm_scale = sm_scale;
  a.dense = dense;
  a.streaming = streaming;
  a.splits_dense = pl.splits_dense;
  a.splits_stream = pl.splits_stream;
  a.chunks_per_wave = pl.chunks_per_wave;
  a.chunks_dense = pl.chunks_dense;
  a.chunks_stream = pl.chunks_stream;
  a.out = out;
  a.lse = lse;
  a.partials = static_cast<float*>(workspace);
  a.max_splits = pl.max_splits;
  if (fused) {
    a.scores = fused_scores;
    a.fused_k = max_selected;
    a.sel_out = sel_out;
    a.nsel_out = nsel_out;
  }
  if (!launch) return ok();
  std::string what = std::string(name) + " launch";
  return hip_status(ubs::launch_decode(a, stream), what.c_str());
}

int sparse_decode(const ubs_bf16_t* q, const ubs_bf16_t* k_cache, const ubs_bf16_t* v_cache,
                  const int32_t* page_table, const int32_t* seq_lens, int32_t B, int32_t max_pages, int32_t Hq,
                  int32_t Hkv, int32_t D, int32_t P, const uint8_t* head_kind, const int32_t* selected,
                  const int32_t* num_selected, int32_t max_selected, int32_t sink_tokens, int32_t local_tokens,
                  float sm_scale, float* out, float* lse, void* workspace, size_t workspace_bytes,
                  hipStream_t stream) {
  return decode_impl("sparse_decode", false, false, q, k_cache, v_cache, nullptr, nullptr, page_table, seq_lens, B,
                     max_pages, Hq, Hkv, D, P, head_kind, selected, num_selected, max_selected, sink_tokens,
                     local_tokens, sm_scale, out, lse, workspace, workspace_bytes, stream);
}

int sparse_decode_static(const ubs_bf16_t* q, const ubs_bf16_t* k_cache, const ubs_bf16_t* v_cache,
                         const int32_t* page_table, const int32_t* seq_lens, int32_t B, int32_t max_pages,
                         int32_t Hq, int32_t Hkv, int32_t D, int32_t P, const uint8_t* head_kind,
                         const int32_t* selected, const int32_t* num_selected, int32_t max_selected,
                         int32_t sink_tokens, int32_t local_tokens, float sm_scale, float* out, float* lse,
                         hipStream_t stream) {
  return decode_impl("sparse_decode_static", false, true, q, k_cache, v_cache, nullptr, nullptr, page_table,
                     seq_lens, B, max_pages, Hq, Hkv, D, P, head_kind, selected, num_selected, max_selected,
                     sink_tokens, local_tokens, sm_scale, out, lse, nullptr, 0, stream);
}

size_t ubs_decode_select_workspace_size(int32_t B, int32_t max_pages, int32_t Hq, int32_t Hkv, int32_t D,
                                        int32_t P, int32_t token_budget, int32_t sink_tokens,
                                        int32_t local_tokens) {
  if (P <= 0 || token_budget <= 0) return 512;
  // [page scores | split partials], each a multiple of 256 bytes
  return ubs_select_workspace_size(B, max_pages, Hkv) +
         ubs_decode_workspace_size(B, Hq, Hkv, D, P, token_budget / P, sink_tokens, local_tokens);
}

int sparse_decode_select(const ubs_bf16_t* q, const ubs_bf16_t* bounds, const ubs_bf16_t* k_cache,
                         const ubs_bf16_t* v_cache, const int32_t* page_table, const int32_t* seq_lens,
                         int32_t B, int32_t max_pages, int32_t Hq, int32_t Hkv, int32_t D, int32_t P,
                         int32_t Lp, int32_t token_budget, const uint8_t* head_kind, int32_t sink_tokens,
                         int32_t local_tokens, float sm_scale, int32_t* selected, int32_t* num_selected,
                         float* out, float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  // workspace: [page scores (ws_sel bytes) | split partials]; every argument of both
  // halves is checked before anything is enqueued
  const size_t ws_sel = ubs_select_workspace_size(B, max_pages, Hkv);
  void* ws_dec = workspace ? static_cast<void*>(static_cast<char*>(workspace) + ws_sel) : nullptr;
  const size_t ws_dec_bytes = workspace_bytes > ws_sel ? workspace_bytes - ws_sel : 0;
  int rc = select_impl(q, bounds, page_table, seq_lens, B, max_pages, Hq, Hkv, D, P, Lp, token_budget, head_kind,
                       selected, num_selected, workspace, workspace_bytes, false, false, stream);
  if (rc) return rc;
  const int32_t k = token_budget / P;
  const bool fused = max_pages <= ubs::kMaxFusedPages && k <= ubs::kMaxFusedK;
  const float* scores = static_cast<const float*>(workspace);
  rc = decode_impl("sparse_decode_select", false, false, q, k_cache, v_cache, nullptr, nullptr, page_table,
                   seq_lens, B, max_pages, Hq, Hkv, D, P, head_kind, selected, num_selected, k, sink_tokens,
                   local_tokens, sm_scale, out, lse, ws_dec, ws_dec_bytes, stream, false,
                   fused ? scores : nullptr, selected, num_selected);
  if (rc) return rc;
  if (B == 0) return ok();
  rc = select_impl(q, bounds, page_table, seq_lens, B, max_pages, Hq, Hkv, D, P, Lp, token_budget, head_kind,
                   selected, num_selected, workspace, ws_sel, fused, true, stream);
  if (rc) return rc;
  return decode_impl("sparse_decode_select", false, false, q, k_cache, v_cache, nullptr, nullptr, page_table,
                     seq_lens, B, max_pages, Hq, Hkv, D, P, head_kind, selected, num_selected, k, sink_tokens,
                     local_tokens, sm_scale, out, lse, ws_dec, ws_dec_bytes, stream, true,
                     fused ? scores : nullptr, selected, num_selected);
}

int sparse_decode_int4(const ubs_bf16_t* q, const uint8_t* k_codes, const uint8_t* v_codes, const uint16_t* k_params,
                       const uint16_t* v_params, const int32_t* page_table, const int32_t* seq_lens, int32_t B,
                       int32_t max_pages, int32_t Hq, int32_t Hkv, int32_t D, int32_t P, const uint8_t* head_kind,
                       const int32_t* selected, const int32_t* num_selected, int32_t max_selected,
                       int32_t sink_tokens, int32_t local_tokens, float sm_scale, float* out, float* lse,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return decode_impl("sparse_decode_int4", true, false, q, k_codes, v_codes, k_params, v_params, page_table, seq_lens, B,
                     max_pages, Hq, Hkv, D, P, head_kind, selected, num_selected, max_selected, sink_tokens,
                     local_tokens, sm_scale, out, lse, workspace, workspace_bytes, stream);
}

int quantize_kv_int4(const ubs_bf16_t* k_cache, const ubs_bf16_t* v_cache, const int32_t* page_table,
                     const int32_t* seq_lens, int32_t B, int32_t max_pages, int32_t Hkv, int32_t D, int32_t P,
                     uint8_t* k_codes, uint8_t* v_codes, uint16_t* k_params, uint16_t* v_params,
                     hipStream_t stream) {
  REQUIRE(Hkv > 0 && Hkv <= 64, UBS_ERR_INVALID_ARGUMENT, "Hkv=%d must be in 1..64", Hkv);
  REQUIRE(D == 64 || D == 128, UBS_ERR_UNSUPPORTED, "D=%d (supported: 64, 128)", D);
  REQUIRE(B >= 0 && max_pages >= 0, UBS_ERR_INVALID_ARGUMENT, "B=%d, max_pages=%d must be >= 0", B, max_pages);
  REQUIRE(P > 0 && P % 16 == 0 && P <= 256, UBS_ERR_UNSUPPORTED, "P=%d must be a multiple of 16 up to 256", P);
  if (B == 0 || max_pages == 0) return ok();
  REQUIRE((int64_t)B * max_pages < (1ll << 31), UBS_ERR_UNSUPPORTED, "B * max_pages is too large");
  REQUIRE(k_cache && v_cache && page_table && seq_lens && k_codes && v_codes && k_params && v_params,
          UBS_ERR_INVALID_ARGUMENT, "every pointer must be non-NULL");
  REQUIRE(aligned16(k_cache) && aligned16(v_cache) && ((uintptr_t)k_codes % 4 == 0) &&
              ((uintptr_t)v_codes % 4 == 0) && ((uintptr_t)k_params % 4 == 0) && ((uintptr_t)v_params % 4 == 0),
          UBS_ERR_INVALID_ARGUMENT, "the caches must be 16-byte aligned, codes and params 4-byte aligned");
  ubs::QuantArgs a{k_cache, v_cache, page_table, seq_lens, B, max_pages, Hkv, D, P,
                   k_codes, v_codes, k_params, v_params};
  return hip_status(ubs::launch_quant_int4(a, stream), "quantize_kv_int4 launch");
}

size_t ubs_mask_workspace_size(int32_t L, int32_t Hq, int32_t Hkv, int32_t D, int32_t T) {
  if (L <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || T <= 0) return 256;
  // fp32 tile means of every query head and every KV head (an upper bound of the dense ones)
  const size_t nT = ((size_t)L + T - 1) / T;
  return (((size_t)Hq + Hkv) * nT * D * sizeof(float) + 255) / 256 * 256;
}

int estimate_block_mask(const ubs_bf16_t* q, const ubs_bf16_t* k_cache, const int32_t* page_table, int32_t L,
                        int32_t Hq, int32_t Hkv, int32_t D, int32_t P, int32_t T, const uint8_t* head_kind,
                        int32_t keep_num, int32_t keep_den, uint8_t* block_mask, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  int rc = common_heads(Hq, Hkv, D);
  if (rc) return rc;
  REQUIRE(L >= 0, UBS_ERR_INVALID_ARGUMENT, "L=%d is negative", L);
  REQUIRE(T == 64 || T == 128, UBS_ERR_UNSUPPORTED, "T=%d (supported: 64, 128)", T);
  REQUIRE(P > 0, UBS_ERR_INVALID_ARGUMENT, "P=%d must be positive", P);
  REQUIRE(pow2(P) && P >= 16 && P <= 4096, UBS_ERR_UNSUPPORTED, "P=%d (supported: powers of two 16..4096)", P);
  REQUIRE(Hq <= ubs::kMaxQHeads, UBS_ERR_UNSUPPORTED, "Hq=%d above %d", Hq, ubs::kMaxQHeads);
  REQUIRE(keep_num > 0 && keep_num <= keep_den && keep_den <= 1024, UBS_ERR_INVALID_ARGUMENT,
          "keep_num=%d, keep_den=%d must satisfy 0 < keep_num <= keep_den <= 1024", keep_num, keep_den);
  ubs::HeadList dense, streaming;
  uint64_t smask;
  rc = head_lists(head_kind, Hkv, &dense, &streaming, &smask);
  if (rc) return rc;
  if (L == 0 || dense.n == 0) return ok();
  REQUIRE(q && k_cache && page_table && block_mask, UBS_ERR_INVALID_ARGUMENT,
          "q, k_cache, page_table and block_mask must be non-NULL");
  REQUIRE(aligned16(q) && aligned16(k_cache), UBS_ERR_INVALID_ARGUMENT, "q and k_cache must be 16-byte aligned");
  const int64_t nT = (L + T - 1) / T;
  REQUIRE(nT <= ubs::kMaxTileList, UBS_ERR_UNSUPPORTED, "L=%d spans %lld tiles of %d (at most %d)", L,
          (long long)nT, T, ubs::kMaxTileList);
  const size_t need = ubs_mask_workspace_size(L, Hq, Hkv, D, T);
  REQUIRE(workspace && workspace_bytes >= need && aligned16(workspace), UBS_ERR_WORKSPACE_TOO_SMALL,
          "workspace of %zu bytes (16-byte aligned), need %zu", workspace_bytes, need);
  ubs::MaskArgs a{};
  a.q = q;
  a.k_cache = k_cache;
  a.page_table = page_table;
  a.L = L;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  a.P = P;
  a.T = T;
  a.log2_P = __builtin_ctz((unsigned)P);
  a.nT = (int)nT;
  a.G = Hq / Hkv;
  a.keep_num = keep_num;
  a.keep_den = keep_den;
  a.dense_kv = dense;
  a.block_mask = block_mask;
  a.qmean = static_cast<float*>(workspace);
  a.kmean = a.qmean + (size_t)dense.n * a.G * nT * D;
  return hip_status(ubs::launch_mask(a, stream), "estimate_block_mask launch");
}

int append_kv(const ubs_bf16_t* k_new, const ubs_bf16_t* v_new, const int32_t* page_table,
              const int32_t* seq_lens, int32_t B, int32_t max_pages, int32_t n_new, int32_t Hkv, int32_t D,
              int32_t P, int32_t Lp, const uint8_t* head_kind, ubs_bf16_t* k_cache, ubs_bf16_t* v_cache,
              ubs_bf16_t* bounds, hipStream_t stream) {
  REQUIRE(B >= 0 && max_pages >= 0 && n_new >= 0, UBS_ERR_INVALID_ARGUMENT,
          "B=%d, max_pages=%d, n_new=%d must be >= 0", B, max_pages, n_new);
  REQUIRE(Hkv >= 1, UBS_ERR_INVALID_ARGUMENT, "Hkv=%d must be positive", Hkv);
  REQUIRE(D == 64 || D == 128, UBS_ERR_UNSUPPORTED, "D=%d (supported: 64, 128)", D);
  int rc = paged_P(P);
  if (rc) return rc;
  REQUIRE(Lp > 0 && P % Lp == 0, UBS_ERR_UNSUPPORTED, "Lp=%d must divide P=%d", Lp, P);
  ubs::HeadList dense, streaming;
  uint64_t smask;
  rc = head_lists(head_kind, Hkv, &dense, &streaming, &smask);
  if (rc) return rc;
  if (B == 0 || n_new == 0) return ok();
  REQUIRE(k_new && v_new && page_table && seq_lens && k_cache && v_cache, UBS_ERR_INVALID_ARGUMENT,
          "k_new, v_new, page_table, seq_lens, k_cache and v_cache must be non-NULL");
  REQUIRE(aligned16(k_new) && aligned16(v_new) && aligned16(k_cache) && aligned16(v_cache) &&
              (!bounds || aligned16(bounds)),
          UBS_ERR_INVALID_ARGUMENT, "k_new, v_new, k_cache, v_cache and bounds must be 16-byte aligned");
  REQUIRE((int64_t)B * n_new * Hkv * (D / 8) < (1ll << 40), UBS_ERR_UNSUPPORTED, "append too large");
  ubs::AppendArgs a{k_new, v_new, page_table, seq_lens, B, max_pages, n_new, Hkv, D, P, k_cache, v_cache};
  hipError_t e = ubs::launch_append(a, stream);
  if (e != hipSuccess || !bounds || dense.n == 0) return hip_status(e, "append_kv launch");
  const int span = (n_new + P - 1) / P + 1;
  ubs::BoundsArgs b{k_cache, page_table, seq_lens, B, max_pages, Hkv, D, P, Lp, dense, bounds, n_new,
                    span < max_pages ? span : max_pages};
  return hip_status(ubs::launch_bounds(b, stream), "append_kv bounds launch");
}

int ubs_check_paged(const int32_t* page_table, int32_t B, int32_t max_pages, const int32_t* seq_lens,
                    const int32_t* cu_seqlens, int32_t num_pages, int32_t P, const uint8_t* head_kind, int32_t Hkv,
                    const int32_t* selected, const int32_t* num_selected, int32_t max_selected, void* status,
                    hipStream_t stream) {
  REQUIRE(B >= 0 && max_pages >= 0 && num_pages >= 0 && max_selected >= 0, UBS_ERR_INVALID_ARGUMENT,
          "B=%d, max_pages=%d, num_pages=%d, max_selected=%d must be >= 0", B, max_pages, num_pages, max_selected);
  REQUIRE(P > 0, UBS_ERR_INVALID_ARGUMENT, "P=%d must be positive", P);
  REQUIRE((seq_lens == nullptr) != (cu_seqlens == nullptr), UBS_ERR_INVALID_ARGUMENT,
          "exactly one of seq_lens and cu_seqlens must be given");
  REQUIRE(status != nullptr && ((uintptr_t)status % 4) == 0, UBS_ERR_INVALID_ARGUMENT,
          "status must be a 4-byte aligned device buffer of UBS_CHECK_STATUS_BYTES bytes");
  ubs::HeadList dense, streaming;
  uint64_t smask;
  if (selected) {
    REQUIRE(num_selected != nullptr, UBS_ERR_INVALID_ARGUMENT, "num_selected is NULL but selected is given");
    int rc = head_lists(head_kind, Hkv, &dense, &streaming, &smask);
    if (rc) return rc;
  } else {
    dense.n = 0;
  }
  if (B == 0) return ok();
  REQUIRE(page_table != nullptr || max_pages == 0, UBS_ERR_INVALID_ARGUMENT, "page_table is NULL");
  ubs::CheckArgs a{};
  a.page_table = page_table;
  a.seq_lens = seq_lens;
  a.cu_seqlens = cu_seqlens;
  a.B = B;
  a.max_pages = max_pages;
  a.num_pages = num_pages;
  a.P = P;
  a.Hkv = selected ? Hkv : 0;
  a.dense = dense;
  a.selected = (selected && dense.n > 0 && max_selected > 0) ? selected : nullptr;
  a.num_selected = num_selected;
  a.max_selected = max_selected;
  a.status = static_cast<int32_t*>(status);
  return hip_status(ubs::launch_check(a, stream), "ubs_check_paged launch");
}

int ubs_check_status(void* status, hipStream_t stream) {
  REQUIRE(status != nullptr, UBS_ERR_INVALID_ARGUMENT, "status is NULL");
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_status(e, "ubs_check_status: stream synchronisation");
  int32_t st[5] = {0, 0, 0, 0, 0};
  e = hipMemcpy(st, status, sizeof(st), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_status(e, "ubs_check_status: reading the status record");
  if (st[0] == 0) return ok();
  const int32_t zero[5] = {0, 0, 0, 0, 0};
  e = hipMemcpy(status, zero, sizeof(zero), hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_status(e, "ubs_check_status: clearing the status record");
  switch (st[0]) {
    case ubs::kCheckSeqLen:
      return fail(UBS_ERR_OUT_OF_RANGE, "sequence %d: length %d outside [0, max_pages * P]", st[1], st[3]);
    case ubs::kCheckCuSeqlens:
      return fail(UBS_ERR_OUT_OF_RANGE, "cu_seqlens[%d] = %d: offsets must start at 0 and not decrease", st[2],
                  st[3]);
    case ubs::kCheckPageId:
      return fail(UBS_ERR_OUT_OF_RANGE, "page_table[%d][%d] = %d is outside [0, num_pages)", st[1], st[2], st[3]);
    case ubs::kCheckNumSelected:
      return fail(UBS_ERR_OUT_OF_RANGE, "num_selected[%d][%d] = %d exceeds max_selected or the sequence's pages",
                  st[1], st[4], st[3]);
    case ubs::kCheckSelected:
      return fail(UBS_ERR_OUT_OF_RANGE, "selected[%d][%d][%d] = %d is not a page of the sequence", st[1], st[4],
                  st[2], st[3]);
    case ubs::kCheckSelectedOrder:
      return fail(UBS_ERR_OUT_OF_RANGE, "selected[%d][%d] is not strictly ascending at slot %d (%d)", st[1], st[4],
                  st[2], st[3]);
    default:
      return fail(UBS_ERR_OUT_OF_RANGE, "violation of kind %d recorded", st[0]);
  }
}

}  // extern "C"
