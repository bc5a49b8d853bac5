"""GPU parity at the largest sizes the entry points accept.

- sparse_prefill at the longest kept-tile list a work-group holds (4,096 query tiles of 64
  rows: one 262,144-token sequence), dense and streaming heads, sampled rows;
- build_page_bounds + select_pages + sparse_decode on a row of 16,384 pages (the most
  select_pages accepts; its top-k then holds 64 keys per thread) beside a short row.
"""
import numpy as np
import pytest
import torch

import oracle
import unified_block_sparse_amd as ubs
from tests.gpu_cases import assert_attention_close, assert_lse_close, check_selection, sample_rows
from tests.helpers import bits
from workloads import cases

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

MAX_TILE_LIST = 4096        # query tiles of one sequence (prefill)
MAX_SELECT_PAGES = 16384    # pages of one row (select_pages)


def _sync():
    torch.cuda.synchronize(DEV)


def test_prefill_longest_tile_list():
    T = 64
    L = MAX_TILE_LIST * T
    # Hq = 4 over Hkv = 2 (G = 2): KV head 0 dense (random 0.5% of the strictly-lower
    # tiles plus the diagonal), KV head 1 streaming (1 sink tile + 8 local tiles)
    c = cases.make_prefill("limit", L, 4, 2, 64, T, 64, [0, 1], 1, 8, "random", 71, DEV,
                           mask_arg=42000)
    assert c.nT == MAX_TILE_LIST
    out, lse = ubs.sparse_prefill(c.q, c.k_cache, c.v_cache, c.page_table, c.head_kind, c.block_mask,
                                  c.sink_tiles, c.local_tiles, c.T, c.sm_scale, return_lse=True)
    _sync()
    rows = sample_rows(L, T, 24, 7)
    q_host = np.zeros(tuple(c.q.shape), dtype=np.uint16)
    ridx = torch.tensor(rows, device=DEV)
    q_host[rows] = bits(c.q[ridx])
    ref, ref_lse = oracle.prefill_ref(q_host, bits(c.k_cache), bits(c.v_cache), c.page_table.cpu().numpy(),
                                      c.L, c.Hq, c.Hkv, c.D, c.P, c.T, c.head_kind, c.block_mask.cpu().numpy(),
                                      c.sink_tiles, c.local_tiles, c.sm_scale, rows=rows)
    assert_attention_close(out[ridx].cpu().numpy(), ref, "prefill at the longest tile list")
    assert_lse_close(lse[:, ridx].cpu().numpy(), ref_lse, "prefill at the longest tile list lse")


def test_select_and_decode_largest_row():
    P, Lp = 16, 16
    lens = [MAX_SELECT_PAGES * P, 3000]
    hk = [0, 1]
    budget = 100 * P
    sink, local = 32, 500
    c = cases.make_decode("limit", lens, 4, 2, 64, P, Lp, hk, budget, sink, local, 72, DEV, planted=True)
    assert c.max_pages == MAX_SELECT_PAGES
    bnd = ubs.build_page_bounds(c.k_cache, c.page_table, c.seq_lens_t, c.head_kind, Lp)
    sel, num = ubs.select_pages(c.q, bnd, c.page_table, c.seq_lens_t, c.head_kind, P, budget)
    _sync()
    sel_o, scores = oracle.select_ref(bits(c.q), bits(c.k_cache), c.page_table.cpu().numpy(), lens,
                                      c.Hq, c.Hkv, P, Lp, budget, hk)
    check_selection(sel.cpu().numpy(), num.cpu().numpy(), sel_o, scores, hk, budget // P)
    # decode on the oracle's selection
    k = budget // P
    sel_t = torch.full((c.B, c.Hkv, k), -1, dtype=torch.int32)
    num_t = torch.zeros((c.B, c.Hkv), dtype=torch.int32)
    for (b, g), s in sel_o.items():
        sel_t[b, g, :len(s)] = torch.tensor(s, dtype=torch.int32)
        num_t[b, g] = len(s)
    out, lse = ubs.sparse_decode(c.q, c.k_cache, c.v_cache, c.page_table, c.seq_lens_t, hk, sel_t.to(DEV),
                                 num_t.to(DEV), sink, local, c.sm_scale, return_lse=True)
    _sync()
    ref, ref_lse = oracle.decode_ref(bits(c.q), bits(c.k_cache), bits(c.v_cache), c.page_table.cpu().numpy(),
                                     lens, c.Hq, c.Hkv, P, hk, sel_o, sink, local, c.sm_scale)
    assert_attention_close(out.cpu().numpy(), ref, "decode at the largest row")
    assert_lse_close(lse.cpu().numpy(), ref_lse, "decode at the largest row lse")
