"""Checked mode on the GPU: ubs_check_paged accepts valid inputs of a decode batch, a
single-sequence prefill and a packed varlen batch, and reports each kind of out-of-range
index (planted in copies of the index arrays only; no attention kernel reads them) as
OUT_OF_RANGE through ubs_check_status, which then clears the record."""
import pytest
import torch

import unified_block_sparse_amd as ubs
from workloads import cases

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _expect(status, frag):
    with pytest.raises(ubs.UBSError) as ei:
        ubs.check_status(status)
    assert ei.value.code == -5 and frag in str(ei.value), str(ei.value)
    ubs.check_status(status)   # cleared


@pytest.fixture(scope="module")
def dec():
    d = cases.make_decode("chk", [3000, 700, 4096], 16, 4, 128, 64, 16, [0, 0, 1, 1], 8 * 64, 64, 256, 2401, DEV)
    bnd = ubs.build_page_bounds(d.k_cache, d.page_table, d.seq_lens_t, d.head_kind, d.Lp)
    sel, num = ubs.select_pages(d.q, bnd, d.page_table, d.seq_lens_t, d.head_kind, d.P, d.token_budget)
    torch.cuda.synchronize(DEV)
    return d, sel, num


def test_valid_inputs_pass(dec):
    d, sel, num = dec
    NP = d.k_cache.shape[0]
    st = ubs.check_paged(d.page_table, NP, d.P, seq_lens=d.seq_lens_t, head_kind=d.head_kind, selected=sel,
                         num_selected=num)
    ubs.check_status(st)
    c = cases.make_prefill("chkp", 1000, 4, 2, 64, 64, 16, [0, 1], 1, 2, "random", 7, DEV, mask_arg=5)
    st = ubs.check_paged(c.page_table, c.k_cache.shape[0], c.P,
                         seq_lens=torch.tensor([c.L], dtype=torch.int32, device=DEV))
    ubs.check_status(st)
    cu = torch.tensor([0, 100, 100, 1000], dtype=torch.int32, device=DEV)
    pt = torch.zeros((3, 16), dtype=torch.int32, device=DEV)
    ubs.check_status(ubs.check_paged(pt, 1, 64, cu_seqlens=cu))


def test_out_of_range_page_id(dec):
    d, _, _ = dec
    NP = d.k_cache.shape[0]
    pt = d.page_table.clone()
    pt[1, 5] = NP                      # page 5 of a 700-token sequence (11 pages)
    _expect(ubs.check_paged(pt, NP, d.P, seq_lens=d.seq_lens_t), "page_table[1][5]")
    pt = d.page_table.clone()
    pt[1, 20] = NP + 7                 # past the sequence's pages: never read, so accepted
    ubs.check_status(ubs.check_paged(pt, NP, d.P, seq_lens=d.seq_lens_t))
    pt[0, 0] = -1
    _expect(ubs.check_paged(pt, NP, d.P, seq_lens=d.seq_lens_t), "page_table[0][0]")


def test_out_of_range_lengths(dec):
    d, _, _ = dec
    NP = d.k_cache.shape[0]
    lens = d.seq_lens_t.clone()
    lens[2] = d.page_table.shape[1] * d.P + 1
    _expect(ubs.check_paged(d.page_table, NP, d.P, seq_lens=lens), "sequence 2")
    cu = torch.tensor([0, 100, 50, 1000], dtype=torch.int32, device=DEV)
    pt = torch.zeros((3, 16), dtype=torch.int32, device=DEV)
    _expect(ubs.check_paged(pt, 1, 64, cu_seqlens=cu), "cu_seqlens")


def test_bad_selection(dec):
    d, sel, num = dec
    NP = d.k_cache.shape[0]
    kw = dict(seq_lens=d.seq_lens_t, head_kind=d.head_kind)
    s = sel.clone()
    s[0, 1, 3] = (d.seq_lens[0] + d.P - 1) // d.P    # one past the last page
    _expect(ubs.check_paged(d.page_table, NP, d.P, selected=s, num_selected=num, **kw), "selected[0][1][3]")
    s = sel.clone()
    s[2, 0, 4] = s[2, 0, 3]                          # a repeated page
    _expect(ubs.check_paged(d.page_table, NP, d.P, selected=s, num_selected=num, **kw), "ascending")
    n = num.clone()
    n[1, 0] = sel.shape[2] + 1
    _expect(ubs.check_paged(d.page_table, NP, d.P, selected=sel, num_selected=n, **kw), "num_selected[1][0]")
    # streaming heads' rows are not read: junk there is accepted
    s = sel.clone()
    s[0, 3, 0] = 10 ** 6
    ubs.check_status(ubs.check_paged(d.page_table, NP, d.P, selected=s, num_selected=num, **kw))
