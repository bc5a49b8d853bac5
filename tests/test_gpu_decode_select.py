"""sparse_decode_select against select_pages + sparse_decode, bit for bit.

The combined call ranks the page scores inside the decode kernel when a row has at most
1,024 pages (one wave per row, up to 16 keys a lane) and falls back to the two calls'
kernels for longer rows; either way its selection and its outputs must equal those of the
two separate calls (which the other tests compare with the oracle). The cases cover both
paths, rows shorter than the budget, streaming heads, exact score ties and G = 1 .. 16.
"""
import pytest
import torch

import unified_block_sparse_amd as ubs
from workloads import cases

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

CASES = [
    # lens, Hq, Hkv, D, P, Lp, head_kind, budget, sink, local, integer-valued (ties)
    ([37, 16, 1, 50, 0, 300], 8, 2, 128, 16, 4, [0, 1], 4 * 16, 5, 20, False),     # 19 pages: 1 key a lane
    ([2000, 1500, 64], 32, 4, 64, 64, 16, [0, 1, 0, 1], 8 * 64, 64, 100, False),
    ([9000, 2500], 16, 2, 128, 16, 16, [0, 0], 30 * 16, 0, 0, True),                 # 563 pages, ties
    ([16000, 300, 7000], 8, 8, 64, 16, 16, [0, 1] * 4, 64 * 16, 16, 64, False),      # 1,000 pages: 16 a lane
    ([16384, 4000], 16, 1, 128, 16, 8, [0], 1024 * 16, 0, 0, False),                 # 1,024 pages, budget 1,024
    ([20000, 3000], 64, 4, 128, 16, 16, [0, 1, 0, 0], 40 * 16, 32, 256, True),      # 1,250 pages: fallback
    ([32768] * 4, 32, 8, 128, 64, 16, [0, 0, 0, 0, 1, 1, 1, 1], 64 * 64, 128, 512, False),  # Llama-3-8B step
]


@pytest.mark.parametrize("lens,Hq,Hkv,D,P,Lp,hk,budget,sink,local,ties", CASES)
def test_decode_select_equals_separate_calls(lens, Hq, Hkv, D, P, Lp, hk, budget, sink, local, ties):
    c = cases.make_decode("ds", lens, Hq, Hkv, D, P, Lp, hk, budget, sink, local, 81, DEV, planted=not ties)
    if ties:
        for t in (c.k_cache, c.q):
            t.copy_(t.float().mul(0.7).round().clamp(-1, 1).to(torch.bfloat16))
    bnd = ubs.build_page_bounds(c.k_cache, c.page_table, c.seq_lens_t, hk, Lp)
    sel, num = ubs.select_pages(c.q, bnd, c.page_table, c.seq_lens_t, hk, P, budget)
    out, lse = ubs.sparse_decode(c.q, c.k_cache, c.v_cache, c.page_table, c.seq_lens_t, hk, sel, num, sink, local,
                                 c.sm_scale, return_lse=True)
    out2, lse2, sel2, num2 = ubs.sparse_decode_select(c.q, bnd, c.k_cache, c.v_cache, c.page_table, c.seq_lens_t,
                                                      hk, P, budget, sink, local, c.sm_scale, return_lse=True)
    torch.cuda.synchronize(DEV)
    assert torch.equal(num2, num), "num_selected differs"
    assert torch.equal(sel2, sel), "selected differs"
    assert torch.equal(out2, out), "out differs"
    assert torch.equal(lse2, lse), "lse differs"
    # a second call on the same (reused) workspace gives the same bits
    out3, sel3, num3 = ubs.sparse_decode_select(c.q, bnd, c.k_cache, c.v_cache, c.page_table, c.seq_lens_t, hk, P,
                                                budget, sink, local, c.sm_scale)
    torch.cuda.synchronize(DEV)
    assert torch.equal(out3, out) and torch.equal(sel3, sel) and torch.equal(num3, num)
