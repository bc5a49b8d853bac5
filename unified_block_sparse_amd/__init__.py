"""Unified block-sparse attention (LServe-style) for AMD Instinct MI355X (gfx950).

The four operations of the hot path run as hand-written HIP kernels in
libubs.so, reached through its C ABI (include/ubs.h):

    sparse_prefill     block-sparse + streaming (Lambda) causal prefill attention
                       (sparse_prefill_chunk: a chunk of query tiles over a longer cache;
                        sparse_prefill_varlen: several sequences in one call)
    build_page_bounds  per-page, per-channel key min/max
    select_pages       query-aware top-k page selection under a token budget
    sparse_decode      sparse paged GQA decode with split-KV and LSE combine

and the steps around them in serving:

    estimate_block_mask  dense heads' block mask from mean-pooled tile scores
    append_kv            new tokens into the paged cache, page bounds refreshed
    quantize_kv_int4     INT4 pages of the cache (per-row 4-bit codes, fp16 scale/zero)
    sparse_decode_int4   sparse_decode over the INT4 pages
    sparse_decode_select select_pages + sparse_decode in one call

Build the library with ``python -m unified_block_sparse_amd.build``.
"""
from ._lib import (UBSError, load, sparse_prefill, sparse_prefill_chunk, sparse_prefill_varlen, build_page_bounds,  # noqa: F401
                   select_pages, sparse_decode, sparse_decode_select, estimate_block_mask, append_kv, quantize_kv_int4,
                   sparse_decode_int4, check_paged, check_status, bench_read, bench_mfma, LIB_PATH, EXPORTED)

__all__ = ["UBSError", "load", "sparse_prefill", "sparse_prefill_chunk", "sparse_prefill_varlen", "build_page_bounds",
           "select_pages",
           "sparse_decode", "sparse_decode_select", "estimate_block_mask", "append_kv", "quantize_kv_int4", "sparse_decode_int4",
           "check_paged", "check_status", "bench_read", "bench_mfma"]
