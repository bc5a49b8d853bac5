"""fp64 CPU oracle (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package. It shares no code with the GPU library.
"""
from .reference import (bf16_to_f64, tokens_of_sequence, prefill_kept_tiles, prefill_ref,  # noqa: F401
                        prefill_kept_tile_count, bounds_ref, subpage_bound, page_scores_ref,
                        topk_pages_ref, select_ref, decode_keys_ref, decode_ref, tile_means_ref,
                        keep_count, meanpool_mask_ref, append_ref, quantize_int4_ref, pack_int4,
                        unpack_int4, dequant_int4_ref, quantize_cache_int4_ref, decode_int4_ref)
