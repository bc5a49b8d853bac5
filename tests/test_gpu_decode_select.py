"""sparse_decode_select against select_pages + sparse_decode.

The combined call ranks the page scores inside the decode kernel when a row has at most
1,024 pages (one wave per row, up to 16 keys a lane) and falls back to the two calls'
kernels for longer rows. Its selection must equal the two calls' bit for bit. Its outputs
are compared with the oracle's decode on that selection, to the attention tolerance: it may
cut the key lists into splits differently from sparse_decode, and each split rounds its
weights to bf16 against its own running max, so the two calls' outputs agree to that
rounding, not bit for bit. The cases cover both paths, rows shorter than the budget,
streaming heads, exact score ties and G = 1 .. 16.
"""
import pytest
import torch

import oracle
import unified_block_sparse_amd as ubs
from tests.gpu_cases import assert_attention_close, assert_lse_close
from tests.helpers import bits
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
    # both outputs against the oracle's decode on this selection
    sel_h, num_h = sel.cpu().tolist(), num.cpu().tolist()
    sel_d = {(b, g): sel_h[b][g][:num_h[b][g]] for b in range(c.B) for g in range(Hkv) if hk[g] == 0}
    ref, ref_lse = oracle.decode_ref(bits(c.q), bits(c.k_cache), bits(c.v_cache), c.page_table.cpu().numpy(), lens,
                                     Hq, Hkv, P, hk, sel_d, sink, local, c.sm_scale)
    for o, l, what in ((out2, lse2, "sparse_decode_select"), (out, lse, "sparse_decode")):
        assert_attention_close(o.cpu().numpy(), ref, what + " out")
        assert_lse_close(l.cpu().numpy(), ref_lse, what + " lse")
    # a second call on the same (reused) workspace gives the same bits
    out3, sel3, num3 = ubs.sparse_decode_select(c.q, bnd, c.k_cache, c.v_cache, c.page_table, c.seq_lens_t, hk, P,
                                                budget, sink, local, c.sm_scale)
    torch.cuda.synchronize(DEV)
    assert torch.equal(out3, out2) and torch.equal(sel3, sel) and torch.equal(num3, num)
