/*
 * ubs.h -- unified block-sparse attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libubs.so. Four operations make up the hot path of LServe-style
 * unified sparse attention ("LServe: Efficient Long-sequence LLM Serving with
 * Unified Sparse Attention", arXiv 2502.14866; and the blog "LServe +
 * SampleAttention", sections "LServe -- Prefill Phase" with Figure 1 and
 * "LServe -- Decode Phase" with Figure 2):
 *
 *   sparse_prefill     block-sparse causal attention over a paged GQA KV cache;
 *                      each KV tile is computed whole or skipped whole, and
 *                      streaming heads keep only sink tiles plus a local window
 *                      (sparse_prefill_chunk: a chunk of query tiles;
 *                      sparse_prefill_varlen: several sequences per call).
 *   build_page_bounds  per-page, per-channel key min/max (the page summary).
 *   select_pages       query-aware page scores and top-k selection.
 *   sparse_decode      GQA decode attention over the kept pages (dense heads)
 *                      or the sink and local tokens (streaming heads).
 *   sparse_decode_select  select_pages and sparse_decode in one call.
 *   estimate_block_mask  the dense heads' prefill block mask from mean-pooled
 *                      query/key tile scores.
 *   append_kv          new tokens into the paged cache, with the page summaries
 *                      they change.
 *   quantize_kv_int4, sparse_decode_int4
 *                      INT4 pages of the cache and decode attention over them.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every pointer is a DEVICE pointer unless its comment says "host".
 * - bf16 tensors are passed as raw 16-bit patterns (ubs_bf16_t).
 * - All tensors are dense, row-major (last index fastest) and 16-byte aligned.
 * - Paged KV cache: k_cache / v_cache are [NP][Hkv][P][D]; token t of a
 *   sequence lives in physical page page_table[t / P] at row t % P. Page ids
 *   must be in [0, NP); entries past a sequence's last page are never read.
 * - head_kind is HOST memory, uint8 [Hkv]: 0 = dense (retrieval) KV head,
 *   1 = streaming KV head. Query head h belongs to KV head h / (Hq / Hkv).
 *   Hkv <= 64. The call reads it on the host before it returns and passes the head
 *   lists to its kernels by value, so a call captured into a HIP graph keeps the head
 *   kinds it was captured with (like every other scalar argument): replays ignore later
 *   changes to the array, which may be freed once the call has returned.
 * - sm_scale (attention calls) must be finite and positive.
 * - The library never allocates device memory, never synchronises and keeps
 *   no pointer after it returns. Work is enqueued on `stream`; results are
 *   valid once the stream has reached that point, and inputs must stay alive
 *   until then. Calls that share a workspace must be ordered on one stream.
 * - Return value: UBS_OK (0) or a negative UBS_ERR_* code. Arguments are
 *   validated on the host before any HIP call; on error nothing is enqueued
 *   and ubs_last_error() returns a message for the calling thread.
 */
#ifndef UBS_H
#define UBS_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t ubs_bf16_t; /* raw bfloat16 bits */

#define UBS_OK 0
#define UBS_ERR_INVALID_ARGUMENT (-1) /* null pointer, negative size, Hq % Hkv != 0, ... */
#define UBS_ERR_UNSUPPORTED (-2)      /* a size outside the shapes the kernels implement */
#define UBS_ERR_WORKSPACE_TOO_SMALL (-3)
#define UBS_ERR_HIP (-4)              /* a HIP launch failed; message from the runtime */
#define UBS_ERR_OUT_OF_RANGE (-5)     /* checked mode: an index input outside its range */

/* Thread-local description of the last failing call (empty string if none). */
const char* ubs_last_error(void);
/* Library version: major * 10000 + minor * 100 + patch. */
int ubs_version(void);

/*
 * sparse_prefill -- block-sparse / streaming causal attention of ONE sequence.
 *
 * Defined by the blog's "LServe -- Prefill Phase" section and its Figure 1:
 * every (query head h, query tile i) computes or skips each KV tile j whole.
 * Query row r (tile i = r / T) of head h (KV head g = h / (Hq/Hkv)) attends to
 *     K(r) = { c <= r : c / T is a kept tile of (h, i) }
 * with kept tiles
 *     dense KV head g:     { j <= i : block_mask[h][i][j] != 0 }
 *     streaming KV head g: { j <= i : j < sink_tiles  or  j > i - local_tiles }
 * (the local window counts the diagonal tile; the tiles in between are never
 * loaded). Only the diagonal tile is cut per token (c <= r). Mask entries
 * above the diagonal are ignored, and mask rows of streaming heads are not read.
 *     out[r][h][:] = sum_{c in K(r)} softmax_c(sm_scale * q_r . k_c) * v_c
 *     lse[h][r]    = ln sum_{c in K(r)} exp(sm_scale * q_r . k_c)
 * A row with an empty K(r) gets out = 0 and lse = -inf.
 *
 *   q           bf16 [L][Hq][D]
 *   k_cache,    bf16 [NP][Hkv][P][D]
 *   v_cache
 *   page_table  int32 [ceil(L / P)]
 *   block_mask  uint8 [Hq][nT][nT], nT = ceil(L / T); may be NULL when every
 *               KV head streams
 *   out         fp32 [L][Hq][D]           (fully written)
 *   lse         fp32 [Hq][L] or NULL      (fully written when given)
 * Arithmetic: bf16 MFMA products with fp32 accumulation; the softmax weights
 * are rounded to bf16 before the P.V product.
 * Supported: D in {64, 128}; T in {64, 128}; P a power of two in [16, 4096];
 * nT <= 4096; Hq <= 256; L >= 0 (L = 0 is a no-op); Hq % Hkv == 0.
 */
int sparse_prefill(const ubs_bf16_t* q, const ubs_bf16_t* k_cache, const ubs_bf16_t* v_cache,
                   const int32_t* page_table, int32_t L, int32_t Hq, int32_t Hkv, int32_t D,
                   int32_t P, int32_t T, const uint8_t* head_kind /* host */,
                   const uint8_t* block_mask, int32_t sink_tiles, int32_t local_tiles,
                   float sm_scale, float* out, float* lse, hipStream_t stream);

/*
 * sparse_prefill_chunk -- sparse_prefill for the query rows [q_start, L) of a sequence
 * whose first q_start tokens already sit in the cache (chunked prefill: the LServe
 * paper's serving setting, a long prompt prefilled in pieces over one paged cache).
 *
 * Rows r in [q_start, L) attend exactly as in sparse_prefill over the whole
 * sequence of L tokens (keys c <= r of the kept tiles of (h, r / T)); the rows
 * before q_start are neither read nor written. q_start must be a multiple of T, so
 * the chunk is whole query tiles i in [q_start / T, nT), nT = ceil(L / T).
 *
 *   q           bf16 [L - q_start][Hq][D]          (row r at r - q_start)
 *   k_cache,    bf16 [NP][Hkv][P][D], holding all L tokens
 *   v_cache
 *   page_table  int32 [ceil(L / P)]
 *   block_mask  uint8 [Hq][nT - q_start/T][nT]     (row i at i - q_start/T)
 *   out         fp32 [L - q_start][Hq][D]          (fully written)
 *   lse         fp32 [Hq][L - q_start] or NULL
 * sparse_prefill is this call with q_start = 0. Supported: as sparse_prefill.
 */
int sparse_prefill_chunk(const ubs_bf16_t* q, const ubs_bf16_t* k_cache, const ubs_bf16_t* v_cache,
                         const int32_t* page_table, int32_t L, int32_t q_start, int32_t Hq, int32_t Hkv,
                         int32_t D, int32_t P, int32_t T, const uint8_t* head_kind /* host */,
                         const uint8_t* block_mask, int32_t sink_tiles, int32_t local_tiles,
                         float sm_scale, float* out, float* lse, hipStream_t stream);

/*
 * sparse_prefill_varlen -- sparse_prefill of B sequences in one call (batched
 * prefill, the serving setting of the LServe paper; the variable-length layout
 * of packed query rows).
 *
 * Sequence b has L_b = cu_seqlens[b+1] - cu_seqlens[b] tokens, all in the paged
 * cache through page-table row b, and is computed exactly as sparse_prefill of that
 * sequence alone; its query rows are rows cu_seqlens[b] .. cu_seqlens[b+1]-1 of the
 * packed q, out and lse.
 *
 *   q            bf16 [total_q][Hq][D]                 (packed rows)
 *   k_cache,     bf16 [NP][Hkv][P][D]
 *   v_cache
 *   page_table   int32 [B][max_pages]                  (row b: sequence b)
 *   cu_seqlens   int32 [B + 1], DEVICE memory: 0 = cu_seqlens[0] <= ... <=
 *                cu_seqlens[B] = total_q; every L_b <= max_seqlen (host int)
 *   block_mask   uint8 [B][Hq][nT_max][nT_max], nT_max = ceil(max_seqlen / T):
 *                mask row i of head h of sequence b at [b][h][i][0 .. nT_b)
 *   out          fp32 [total_q][Hq][D]                 (fully written)
 *   lse          fp32 [Hq][total_q] or NULL
 * The grid covers B * Hq * nT_max work-groups; those past a sequence's own tiles
 * return at once. A sequence longer than max_seqlen is a caller error (its last
 * rows are not computed). Supported: as sparse_prefill, with nT_max <= 4096 and
 * max_pages * P >= max_seqlen.
 */
int sparse_prefill_varlen(const ubs_bf16_t* q, const ubs_bf16_t* k_cache, const ubs_bf16_t* v_cache,
                          const int32_t* page_table, int32_t max_pages, const int32_t* cu_seqlens, int32_t B,
                          int32_t max_seqlen, int32_t total_q, int32_t Hq, int32_t Hkv, int32_t D, int32_t P,
                          int32_t T, const uint8_t* head_kind /* host */, const uint8_t* block_mask,
                          int32_t sink_tiles, int32_t local_tiles, float sm_scale, float* out, float* lse,
                          hipStream_t stream);

/*
 * build_page_bounds -- the per-page key summary used to score pages.
 *
 * Defined by the blog's "LServe -- Decode Phase" section ("a summary vector
 * per page") together with the query-aware bound of Quest that the LServe
 * paper cites. For every sequence b, every valid page j < ceil(seq_lens[b]/P)
 * (physical page p = page_table[b][j]), every DENSE KV head g and every
 * logical sub-page u of Lp tokens holding at least one valid token
 * (t < seq_lens[b]):
 *     bounds[p][g][u][0][c] = min over those tokens of k[c]
 *     bounds[p][g][u][1][c] = max over those tokens of k[c]
 * Entries of streaming heads, of unreferenced pages and of sub-pages with no
 * valid token are left untouched. Values are exact (bf16 min/max).
 *
 *   k_cache     bf16 [NP][Hkv][P][D]
 *   page_table  int32 [B][max_pages]
 *   seq_lens    int32 [B], 0 <= seq_lens[b] <= max_pages * P
 *   bounds      bf16 [NP][Hkv][P/Lp][2][D]
 * A physical page referenced by several sequences must hold the same valid
 * tokens in each. Supported: D in {64, 128}; P in {16, 32, 64, 128};
 * Lp divides P.
 */
int build_page_bounds(const ubs_bf16_t* k_cache, const int32_t* page_table, const int32_t* seq_lens,
                      int32_t B, int32_t max_pages, int32_t Hkv, int32_t D, int32_t P, int32_t Lp,
                      const uint8_t* head_kind /* host */, ubs_bf16_t* bounds, hipStream_t stream);

/*
 * select_pages -- query-aware top-k page selection for one decode step.
 *
 * Defined by the blog's "LServe -- Decode Phase" section and Figure 2 (score
 * every page from its summary, keep the top-k) and the LServe abstract
 * (hierarchical, query-centric page selection with a constant page budget).
 * For each sequence b and DENSE KV head g with query heads h of its group:
 *   sub-page bound  s_u = max_h sum_c max(q[b][h][c] * kmin_u[c], q[b][h][c] * kmax_u[c])
 *   page score      s_j = max over the sub-pages u of page j that hold valid tokens
 *   selection       the k = token_budget / P pages first in the order
 *                   (score descending, page index ascending); every page when
 *                   the sequence has at most k pages.
 * Scores are evaluated in fp32 as q+ . kmax + q- . kmin (q+ = max(q, 0),
 * q- = min(q, 0)), which equals the sum above term by term.
 *
 *   q             bf16 [B][Hq][D]
 *   bounds        bf16 [NP][Hkv][P/Lp][2][D], as written by build_page_bounds
 *   page_table    int32 [B][max_pages]
 *   seq_lens      int32 [B]
 *   selected      int32 [B][Hkv][k]: page indices j (into page_table[b]) in
 *                 ascending order, unused slots -1; streaming heads get all -1
 *   num_selected  int32 [B][Hkv]: min(k, ceil(seq_lens[b]/P)); 0 for streaming
 *   workspace     >= ubs_select_workspace_size(...) bytes, any contents
 * Supported: D in {64, 128}; Hq/Hkv in {1, 2, 4, 8, 16}; P in {16, 32, 64, 128};
 * P/Lp in {1, 2, 4, 8, 16}; token_budget a positive multiple of P;
 * max_pages <= 16384.
 */
size_t ubs_select_workspace_size(int32_t B, int32_t max_pages, int32_t Hkv);
int select_pages(const ubs_bf16_t* q, const ubs_bf16_t* bounds, const int32_t* page_table,
                 const int32_t* seq_lens, int32_t B, int32_t max_pages, int32_t Hq, int32_t Hkv,
                 int32_t D, int32_t P, int32_t Lp, int32_t token_budget,
                 const uint8_t* head_kind /* host */, int32_t* selected, int32_t* num_selected,
                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * sparse_decode -- sparse paged GQA decode attention (one query per sequence).
 *
 * Defined by the blog's "LServe -- Decode Phase" section and Figure 2
 * (token-level attention only inside the selected pages) and the LServe
 * abstract (streaming heads in decode too). The query of sequence b sits at
 * position L-1 with L = seq_lens[b]; its key set for KV head g is
 *   dense g:     every valid token (t < L) of the pages selected[b][g][0 .. n)
 *                with n = num_selected[b][g]
 *   streaming g: tokens t < sink_tokens or t >= L - local_tokens
 *     out[b][h][:] = sum_t softmax_t(sm_scale * q[b][h] . k_t) * v_t
 *     lse[b][h]    = ln sum_t exp(sm_scale * q[b][h] . k_t)
 * An empty key set gives out = 0, lse = -inf. The key set is split across
 * waves (split-KV); partial (max, sum, output) triples are merged with a
 * log-sum-exp combine. Scores, softmax and accumulation are fp32 on bf16 inputs;
 * the weights enter the P.V product rounded to bf16, as in sparse_prefill.
 *
 *   q             bf16 [B][Hq][D]
 *   selected      int32 [B][Hkv][max_selected], entries in [0, ceil(L/P)),
 *                 distinct; read for dense heads only (may be NULL if none)
 *   num_selected  int32 [B][Hkv], each <= max_selected
 *   out           fp32 [B][Hq][D]        (fully written)
 *   lse           fp32 [B][Hq] or NULL
 *   workspace     >= ubs_decode_workspace_size(...) bytes, any contents
 *                 (holds the split partials between the two launches)
 * Supported: D in {64, 128}; Hq/Hkv in {1, 2, 4, 8, 16}; P a multiple of 16,
 * <= 256.
 */
size_t ubs_decode_workspace_size(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t P,
                                    int32_t max_selected, int32_t sink_tokens, int32_t local_tokens);
int sparse_decode(const ubs_bf16_t* q, const ubs_bf16_t* k_cache, const ubs_bf16_t* v_cache,
                  const int32_t* page_table, const int32_t* seq_lens, int32_t B, int32_t max_pages,
                  int32_t Hq, int32_t Hkv, int32_t D, int32_t P, const uint8_t* head_kind /* host */,
                  const int32_t* selected, const int32_t* num_selected, int32_t max_selected,
                  int32_t sink_tokens, int32_t local_tokens, float sm_scale, float* out, float* lse,
                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * sparse_decode_select -- select_pages followed by sparse_decode, in one call.
 *
 * The decode step of the blog's "LServe -- Decode Phase" section as one pipeline
 * (Figure 2: page scores from the per-page key bounds, the top pages under the
 * token budget, then token-level attention inside them). Results are those of
 *   select_pages(q, bounds, ..., token_budget, selected, num_selected)
 *   sparse_decode(q, k_cache, v_cache, ..., selected, num_selected,
 *                 max_selected = token_budget / P, ...)
 * The selection is the same bit for bit (ties to the lower page index); out and lse
 * are the same attention within sparse_decode's tolerance (the key lists may be cut
 * into splits differently, and each split rounds its weights to bf16 against its own
 * running max). The work
 * differs: for rows of at most 1,024 pages (max_pages <= 1024) and token_budget / P
 * <= 1,024, each decode wave of a dense head ranks its row's page scores itself, so the
 * separate top-k launch is skipped; longer rows run the two calls' kernels as they are.
 *
 *   q, bounds, page_table, seq_lens, head_kind, P, Lp, token_budget
 *                 as for select_pages; k_cache, v_cache, sink_tokens, local_tokens,
 *                 sm_scale as for sparse_decode
 *   selected      int32 [B][Hkv][token_budget / P]   (output, as select_pages writes it)
 *   num_selected  int32 [B][Hkv]                      (output)
 *   out, lse      as for sparse_decode
 *   workspace     >= ubs_decode_select_workspace_size(...) bytes, any contents
 * Supported: the intersection of select_pages and sparse_decode (D in {64, 128};
 * Hq/Hkv and P/Lp in {1, 2, 4, 8, 16}; P in {16, 32, 64, 128}; max_pages <= 16384).
 * Errors: as for the two calls.
 */
size_t ubs_decode_select_workspace_size(int32_t B, int32_t max_pages, int32_t Hq, int32_t Hkv, int32_t D,
                                        int32_t P, int32_t token_budget, int32_t sink_tokens,
                                        int32_t local_tokens);
int sparse_decode_select(const ubs_bf16_t* q, const ubs_bf16_t* bounds, const ubs_bf16_t* k_cache,
                         const ubs_bf16_t* v_cache, const int32_t* page_table, const int32_t* seq_lens,
                         int32_t B, int32_t max_pages, int32_t Hq, int32_t Hkv, int32_t D, int32_t P,
                         int32_t Lp, int32_t token_budget, const uint8_t* head_kind /* host */,
                         int32_t sink_tokens, int32_t local_tokens, float sm_scale, int32_t* selected,
                         int32_t* num_selected, float* out, float* lse, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

/*
 * sparse_decode_static -- sparse_decode that allocates nothing and takes no workspace.
 *
 * For callers that cannot allocate device memory or manage a workspace: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation. The arguments,
 * key sets, results and supported shapes are those of sparse_decode, minus workspace and
 * workspace_bytes; the same kernels run. The split partials live in a library-owned
 * scratch array of UBS_STATIC_SCRATCH_BYTES in device memory: one copy per GPU, loaded
 * with the library's code and held until the process ends; its device address is looked
 * up on the first call on each device (the calling thread's current device must be the
 * device of `stream` and of the pointers).
 * - A call needing more than UBS_STATIC_SCRATCH_BYTES of partials
 *   (ubs_decode_workspace_size(...) > UBS_STATIC_SCRATCH_BYTES) returns
 *   UBS_ERR_WORKSPACE_TOO_SMALL before any HIP call.
 * - Every call on one GPU shares that GPU's scratch. Calls that may overlap on one GPU
 *   (different streams, or threads enqueueing concurrently) race on it and must be
 *   ordered by the caller. Nothing in the scratch needs clearing: each call writes every
 *   partial it reads.
 */
#define UBS_STATIC_SCRATCH_BYTES (32u << 20)
int sparse_decode_static(const ubs_bf16_t* q, const ubs_bf16_t* k_cache, const ubs_bf16_t* v_cache,
                         const int32_t* page_table, const int32_t* seq_lens, int32_t B, int32_t max_pages,
                         int32_t Hq, int32_t Hkv, int32_t D, int32_t P, const uint8_t* head_kind /* host */,
                         const int32_t* selected, const int32_t* num_selected, int32_t max_selected,
                         int32_t sink_tokens, int32_t local_tokens, float sm_scale, float* out, float* lse,
                         hipStream_t stream);

/*
 * INT4 KV pages -- quantize_kv_int4 and sparse_decode_int4.
 *
 * The blog's "LServe -- Decode Phase" section and its Figure 2 caption: INT4 KV
 * quantization stacks with page sparsity, cutting the bytes of every page decode
 * reads. The pages give no format; this library's format quantizes every
 * (token, KV head) row of D channels on its own, asymmetrically:
 *   scale = fp16((max_c x_c - min_c x_c) / 15), zero = fp16(min_c x_c)
 *   n_c   = clamp(rint((x_c - zero) / scale), 0, 15)  in fp32 (n = 0 if scale == 0)
 *   x_c  ~ n_c * scale + zero
 * Storage (same page indexing as the bf16 cache). Codes sit 8 to a 32-bit
 * little-endian word: code k of the 8 in nibble k/2 of the low half (k even) or of
 * the high half (k odd), i.e. bytes (n0|n2<<4, n4|n6<<4, n1|n3<<4, n5|n7<<4).
 *   k_codes uint8  [NP][Hkv][P][D/2]: each token's row, words of 8 channels
 *   v_codes uint8  [NP][Hkv][D][P/2]: channel-major, for each channel the
 *                                      page's tokens in words of 8 tokens
 *   params  uint16 [NP][Hkv][P][2]:   fp16 bits of (scale, zero), K and V each
 * 68 bytes per row at D = 128 against 256 for bf16.
 *
 * quantize_kv_int4: the codes and params of every valid token (t < seq_lens[b])
 * of every sequence, every KV head, K and V; K rows and params of other tokens are
 * left as they were, and so are V words holding no valid token (the other tokens
 * of a V word that is written get code 0). Inputs are bf16 caches
 * [NP][Hkv][P][D] (16-byte aligned); codes and params 4-byte aligned. Values
 * must be finite and their range / 15 must fit fp16.
 *
 * sparse_decode_int4: sparse_decode with K and V read from INT4 pages instead of
 * the bf16 caches; the key sets, arguments, outputs, workspace and supported
 * shapes are those of sparse_decode. The result is attention over the
 * dequantized rows (fp32 arithmetic). Codes 16-byte aligned, params 4-byte.
 */
int quantize_kv_int4(const ubs_bf16_t* k_cache, const ubs_bf16_t* v_cache, const int32_t* page_table,
                     const int32_t* seq_lens, int32_t B, int32_t max_pages, int32_t Hkv, int32_t D, int32_t P,
                     uint8_t* k_codes, uint8_t* v_codes, uint16_t* k_params, uint16_t* v_params,
                     hipStream_t stream);
int sparse_decode_int4(const ubs_bf16_t* q, const uint8_t* k_codes, const uint8_t* v_codes,
                       const uint16_t* k_params, const uint16_t* v_params, const int32_t* page_table,
                       const int32_t* seq_lens, int32_t B, int32_t max_pages, int32_t Hq, int32_t Hkv,
                       int32_t D, int32_t P, const uint8_t* head_kind /* host */, const int32_t* selected,
                       const int32_t* num_selected, int32_t max_selected, int32_t sink_tokens,
                       int32_t local_tokens, float sm_scale, float* out, float* lse, void* workspace,
                       size_t workspace_bytes, hipStream_t stream);

/*
 * append_kv -- write newly decoded or prefilled tokens into the paged KV cache and
 * refresh the page summaries they change (the steps beside decode in the serving
 * loop of the LServe paper; page layout of the blog's "LServe -- Decode Phase").
 *
 * For every sequence b and x < n_new, token t = seq_lens[b] + x gets
 *     k_cache[page_table[b][t / P]][g][t % P][:] = k_new[b][x][g][:]   (every KV head g)
 * and likewise v_cache. When bounds is not NULL, every DENSE KV head's sub-page (Lp
 * tokens) that received a new token is recomputed over all its valid tokens of the
 * sequence of length seq_lens[b] + n_new, exactly as build_page_bounds would;
 * other sub-pages are left untouched. seq_lens is the length BEFORE the append and
 * is not modified; the caller advances it.
 *
 *   k_new, v_new  bf16 [B][n_new][Hkv][D]
 *   page_table    int32 [B][max_pages], pages for all seq_lens[b] + n_new tokens
 *   seq_lens      int32 [B], seq_lens[b] + n_new <= max_pages * P
 *   k_cache,      bf16 [NP][Hkv][P][D]
 *   v_cache
 *   bounds        bf16 [NP][Hkv][P/Lp][2][D] or NULL
 * Supported: D in {64, 128}; P in {16, 32, 64, 128}; Lp divides P.
 */
int append_kv(const ubs_bf16_t* k_new, const ubs_bf16_t* v_new, const int32_t* page_table,
              const int32_t* seq_lens, int32_t B, int32_t max_pages, int32_t n_new, int32_t Hkv, int32_t D,
              int32_t P, int32_t Lp, const uint8_t* head_kind /* host */, ubs_bf16_t* k_cache,
              ubs_bf16_t* v_cache, ubs_bf16_t* bounds, hipStream_t stream);

/*
 * estimate_block_mask -- the dense heads' prefill block mask from mean-pooled
 * tile scores (the step before sparse_prefill for dense heads).
 *
 * The mask rule of the Llama-3-8B prefill workload: a query-tile-level estimate of
 * the block sparsity that the blog's "LServe -- Prefill Phase" section applies (a
 * KV tile is computed or skipped whole per query tile). For every DENSE query head
 * h (KV head g = h / (Hq/Hkv)) and query tile i (nT = ceil(L / T) tiles, the last
 * one possibly partial):
 *     qbar_i = mean over the rows of tile i of q[.][h][:]
 *     kbar_j = mean over the rows of tile j of the sequence's keys of KV head g
 *     score[i][j] = qbar_i . kbar_j                       (j < i)
 *     n_i = ceil(keep_num * (i + 1) / keep_den)           tiles kept, diagonal included
 *     block_mask[h][i][j] = 1 for j = i and for the n_i - 1 tiles j < i of largest
 *                           score (equal scores: the lower j first), else 0
 *                           (entries above the diagonal are 0)
 * Means and scores are evaluated in fp32 (sums in a fixed order), so tiles whose
 * score is within rounding of the row's threshold may differ from an exact
 * evaluation; everything else is exact. Rows of streaming heads are not written.
 *
 *   q           bf16 [L][Hq][D]
 *   k_cache     bf16 [NP][Hkv][P][D]
 *   page_table  int32 [ceil(L / P)]
 *   block_mask  uint8 [Hq][nT][nT]   (dense heads' rows fully written)
 *   workspace   >= ubs_mask_workspace_size(...) bytes, any contents (the tile means)
 * Supported: D in {64, 128}; T in {64, 128}; P a power of two in [16, 4096];
 * nT <= 4096; Hq <= 256; 0 < keep_num <= keep_den <= 1024; L >= 0 (L = 0 is a
 * no-op).
 */
size_t ubs_mask_workspace_size(int32_t L, int32_t Hq, int32_t Hkv, int32_t D, int32_t T);
int estimate_block_mask(const ubs_bf16_t* q, const ubs_bf16_t* k_cache, const int32_t* page_table,
                        int32_t L, int32_t Hq, int32_t Hkv, int32_t D, int32_t P, int32_t T,
                        const uint8_t* head_kind /* host */, int32_t keep_num, int32_t keep_den,
                        uint8_t* block_mask, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Checked mode -- device-side validation of the index inputs every paged call trusts.
 *
 * The kernels read through page ids, sequence lengths and selected page lists without
 * bounds checks (page ids must lie in [0, NP), which no call can know). A caller that
 * wants them verified enqueues ubs_check_paged on the stream before the calls, and asks
 * ubs_check_status afterwards. What is checked, for every sequence b < B:
 *   - its length L_b (seq_lens[b], or cu_seqlens[b+1] - cu_seqlens[b] with cu_seqlens
 *     starting at 0 and not decreasing) lies in [0, max_pages * P];
 *   - page_table[b][j] lies in [0, num_pages) for every page j < ceil(L_b / P) of it;
 *   - when selected is given: for every DENSE KV head g (head_kind, host), num_selected
 *     [b][g] lies in [0, min(max_selected, ceil(L_b / P))] and selected[b][g][0 .. n) are
 *     pages of the sequence, strictly ascending (as select_pages writes them).
 * The first violation found is recorded in `status` (device memory, at least
 * UBS_CHECK_STATUS_BYTES bytes, 4-byte aligned, zeroed by the caller before its first
 * use; later checks keep a recorded violation until it is reported). Arguments follow the
 * conventions above: page_table int32 [B][max_pages]; exactly one of seq_lens (int32
 * [B]) and cu_seqlens (int32 [B + 1]) non-NULL; selected int32 [B][Hkv][max_selected]
 * and num_selected int32 [B][Hkv], or both NULL.
 *
 * ubs_check_status waits for `stream` (the one call here that synchronises), reads the
 * record and returns UBS_OK, or UBS_ERR_OUT_OF_RANGE with ubs_last_error() naming the
 * violation; it then clears the record.
 */
#define UBS_CHECK_STATUS_BYTES 64
int ubs_check_paged(const int32_t* page_table, int32_t B, int32_t max_pages, const int32_t* seq_lens,
                    const int32_t* cu_seqlens, int32_t num_pages, int32_t P, const uint8_t* head_kind /* host */,
                    int32_t Hkv, const int32_t* selected, const int32_t* num_selected, int32_t max_selected,
                    void* status, hipStream_t stream);
int ubs_check_status(void* status, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* UBS_H */
