"""GPU parity on small cases: every kernel against the fp64 oracle on the same seeded
bits, covering several tiles, ragged tails, partial pages, empty sequences, every
supported D / T / G / P / Lp family, exact ties in page scores, determinism and
page-table permutation invariance."""
import numpy as np
import pytest
import torch

import oracle
import unified_block_sparse_amd as ubs
from tests.gpu_cases import assert_attention_close, assert_lse_close, check_selection
from tests.helpers import bits
from workloads import cases

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
SENTINEL = 0x7F7F   # a finite bf16 pattern (about 3.4e38) left where bounds are undefined


def _sync():
    torch.cuda.synchronize(DEV)


# ----------------------------------------------------------------------------- bounds

BOUNDS_CASES = [
    ([37, 16, 1, 50, 0], 16, 4, 128, [0, 1]),
    ([200, 64, 65], 64, 16, 64, [0, 0, 1, 1]),
    ([300], 128, 32, 128, [0]),
    ([1000, 77], 32, 32, 64, [0, 1]),
    ([129], 64, 4, 128, [1, 0]),
    ([70, 3], 64, 1, 128, [0]),
    # the compile-time sub-page sizes (Lp = P, Lp = 16) at every P and both D, and
    # sub-pages smaller than a D = 64 row group (two rows per load)
    ([300, 129], 128, 16, 128, [0, 1]),
    ([130, 64], 128, 128, 64, [0]),
    ([45, 90], 32, 16, 128, [0]),
    ([16, 17], 16, 16, 64, [1, 0]),
    ([33, 64], 64, 2, 64, [0, 1]),
    ([20, 5], 16, 1, 64, [0]),
]


@pytest.mark.parametrize("lens,P,Lp,D,hk", BOUNDS_CASES)
def test_bounds_exact(lens, P, Lp, D, hk):
    Hkv = len(hk)
    c = cases.make_decode("b", lens, Hkv * 2, Hkv, D, P, Lp, hk, 2 * P, 4, 8, 31, DEV, extra_pages=3,
                          planted=True)
    out = torch.full((c.num_physical_pages, Hkv, P // Lp, 2, D), 0, dtype=torch.int16, device=DEV)
    out.fill_(SENTINEL)
    out = out.view(torch.bfloat16)
    ubs.build_page_bounds(c.k_cache, c.page_table, c.seq_lens_t, hk, Lp, bounds=out)
    _sync()
    vals, defined = oracle.bounds_ref(bits(c.k_cache), c.page_table.cpu().numpy(), lens, P, Lp, hk)
    got_bits = bits(out)
    got = oracle.bf16_to_f64(got_bits)
    assert defined.sum() > 0
    assert np.array_equal(got[defined], vals[defined])
    assert np.all(got_bits[~defined] == SENTINEL)


# ----------------------------------------------------------------------------- selection

def _oracle_select(c):
    sel, scores = oracle.select_ref(bits(c.q), bits(c.k_cache), c.page_table.cpu().numpy(), c.seq_lens,
                                    c.Hq, c.Hkv, c.P, c.Lp, c.token_budget, c.head_kind)
    return sel, scores


def _gpu_select(c):
    bnd = ubs.build_page_bounds(c.k_cache, c.page_table, c.seq_lens_t, c.head_kind, c.Lp)
    sel, num = ubs.select_pages(c.q, bnd, c.page_table, c.seq_lens_t, c.head_kind, c.P, c.token_budget)
    _sync()
    return sel.cpu().numpy(), num.cpu().numpy()


SELECT_CASES = [
    # lens, Hq, Hkv, D, P, Lp, head_kind, budget
    ([37, 16, 1, 50, 0, 300], 8, 2, 128, 16, 4, [0, 1], 4 * 16),
    ([2000, 1500, 64], 16, 4, 64, 64, 16, [0, 1, 0, 1], 8 * 64),
    ([500, 4000], 32, 2, 128, 32, 32, [0, 0], 4 * 32),
    ([1000, 129, 5000], 4, 4, 64, 128, 8, [0, 0, 1, 0], 3 * 128),
    ([50000], 8, 1, 128, 64, 64, [0], 600 * 64),
    ([3000, 20], 2, 2, 128, 16, 1, [0, 0], 16 * 16),
]


@pytest.mark.parametrize("lens,Hq,Hkv,D,P,Lp,hk,budget", SELECT_CASES)
def test_select_matches_oracle(lens, Hq, Hkv, D, P, Lp, hk, budget):
    c = cases.make_decode("s", lens, Hq, Hkv, D, P, Lp, hk, budget, 4, 8, 32, DEV, planted=True)
    sel_g, num_g = _gpu_select(c)
    sel_o, scores = _oracle_select(c)
    check_selection(sel_g, num_g, sel_o, scores, hk, budget // P)


@pytest.mark.parametrize("lens,P,Lp,budget", [
    ([3000, 777, 4096], 64, 16, 10 * 64),   # rows of at most 64 pages (one key per thread)
    ([6400, 1000], 16, 16, 25 * 16),        # 400 pages (two keys per thread)
    ([9000, 2500], 16, 16, 30 * 16),        # 563 pages (four keys per thread)
    ([20000, 3000], 16, 16, 40 * 16),       # a row of 1,250 pages (eight keys per thread)
    ([262144, 3000], 16, 16, 100 * 16),     # 16,384 pages, the most select_pages takes (64 keys per thread)
])
def test_select_exact_ties_break_to_lower_index(lens, P, Lp, budget):
    """Integer-valued q and keys make many page scores tie exactly (the sums are exact in
    fp32 and fp64), so the tie-break must match the oracle bit for bit."""
    c = cases.make_decode("t", lens, 8, 2, 128, P, Lp, [0, 0], budget, 4, 8, 33, DEV)
    for t in (c.k_cache, c.q):
        t.copy_(t.float().mul(0.7).round().clamp(-1, 1).to(torch.bfloat16))
    sel_g, num_g = _gpu_select(c)
    sel_o, scores = _oracle_select(c)
    n_ties = sum(len(s) - len(set(s.tolist())) for s in scores.values())
    assert n_ties > 0
    swaps = check_selection(sel_g, num_g, sel_o, scores, c.head_kind, c.k_pages)
    assert swaps == 0


def test_score_work_group_orders_give_the_same_scores(monkeypatch):
    """The page scores (the workspace select_pages leaves behind) and the selection do not
    depend on the order in which the scoring work-groups cover the (sequence, page chunk,
    dense head) items: the measurement override's row order equals the default."""
    lib = ubs.load()
    c = cases.make_decode("o", [9000, 333, 4100, 64], 16, 4, 128, 64, 16, [0, 1, 0, 0], 12 * 64, 4, 8, 34, DEV,
                          planted=True)
    bnd = ubs.build_page_bounds(c.k_cache, c.page_table, c.seq_lens_t, c.head_kind, c.Lp)
    n = lib.ubs_select_workspace_size(c.B, c.page_table.shape[1], c.Hkv)
    got = []
    for order in ("1", "0"):
        monkeypatch.setenv("UBS_SCORE_ORDER", order)
        ws = torch.full((n,), 0x7f, dtype=torch.uint8, device=DEV)
        sel, num = ubs.select_pages(c.q, bnd, c.page_table, c.seq_lens_t, c.head_kind, c.P, c.token_budget,
                                    workspace=ws)
        _sync()
        # the scores of every valid page of every dense row (entries past a row are not written)
        sc = ws[:c.B * c.Hkv * c.page_table.shape[1] * 4].view(torch.float32).view(c.B, c.Hkv, -1).cpu()
        rows = {(b, g): sc[b, g, :(L + c.P - 1) // c.P].clone()
                for b, L in enumerate(c.seq_lens) for g in range(c.Hkv) if not c.head_kind[g]}
        got.append((sel.cpu(), num.cpu(), rows))
    assert torch.equal(got[0][0], got[1][0]) and torch.equal(got[0][1], got[1][1])
    for key in got[0][2]:
        assert torch.equal(got[0][2][key].view(torch.int32), got[1][2][key].view(torch.int32)), key


# ----------------------------------------------------------------------------- decode

DECODE_CASES = [
    # lens, Hq, Hkv, D, P, Lp, head_kind, budget, sink, local
    ([37, 16, 1, 50, 0, 300], 8, 2, 128, 16, 4, [0, 1], 4 * 16, 5, 20),
    ([2000, 1500, 64], 32, 4, 64, 64, 16, [0, 1, 0, 1], 8 * 64, 64, 100),
    ([500, 4000], 32, 2, 128, 32, 32, [1, 0], 4 * 32, 0, 64),
    ([1000, 129, 5000], 4, 4, 64, 128, 8, [0, 0, 1, 0], 3 * 128, 128, 1024),
    ([50000], 8, 1, 128, 64, 64, [0], 600 * 64, 0, 0),
    ([20000, 777], 16, 2, 128, 64, 16, [1, 1], 64, 1000, 3000),
    ([3000, 20], 2, 2, 128, 16, 1 * 16, [0, 1], 16 * 16, 7, 33),
    # 16-row units that straddle pages (P = 48, 80: not powers of two), G = 1 with D = 64,
    # G = 16 over 256-token pages with a long local window
    ([3000, 1234, 77], 16, 4, 128, 48, 16, [0, 1, 1, 0], 10 * 48, 40, 200),
    ([9000, 300], 8, 8, 64, 80, 16, [0, 1, 0, 1, 0, 1, 0, 1], 7 * 80, 16, 500),
    ([40000], 64, 4, 128, 256, 64, [0, 1, 0, 0], 20 * 256, 256, 2048),
]


@pytest.mark.parametrize("lens,Hq,Hkv,D,P,Lp,hk,budget,sink,local", DECODE_CASES)
def test_decode_matches_oracle_on_oracle_selection(lens, Hq, Hkv, D, P, Lp, hk, budget, sink, local):
    c = cases.make_decode("d", lens, Hq, Hkv, D, P, Lp, hk, budget, sink, local, 34, DEV, planted=True)
    sel_o, _ = _oracle_select(c)
    k = budget // P
    sel_t = torch.full((c.B, Hkv, k), -1, dtype=torch.int32)
    num_t = torch.zeros((c.B, Hkv), dtype=torch.int32)
    for (b, g), s in sel_o.items():
        sel_t[b, g, :len(s)] = torch.tensor(s, dtype=torch.int32)
        num_t[b, g] = len(s)
    out, lse = ubs.sparse_decode(c.q, c.k_cache, c.v_cache, c.page_table, c.seq_lens_t, hk, sel_t.to(DEV),
                                 num_t.to(DEV), sink, local, c.sm_scale, return_lse=True)
    _sync()
    ref, ref_lse = oracle.decode_ref(bits(c.q), bits(c.k_cache), bits(c.v_cache), c.page_table.cpu().numpy(),
                                     lens, Hq, Hkv, P, hk, sel_o, sink, local, c.sm_scale)
    assert_attention_close(out.cpu().numpy(), ref, "decode out")
    assert_lse_close(lse.cpu().numpy(), ref_lse, "decode lse")
    # a second call reuses the workspace and gives the same bits
    out2 = ubs.sparse_decode(c.q, c.k_cache, c.v_cache, c.page_table, c.seq_lens_t, hk, sel_t.to(DEV),
                             num_t.to(DEV), sink, local, c.sm_scale)
    _sync()
    assert torch.equal(out, out2)


def test_decode_end_to_end_select_then_attend():
    lens = [6000, 2500, 9000]
    c = cases.make_decode("e", lens, 16, 4, 128, 64, 16, [0, 1, 0, 1], 16 * 64, 64, 256, 35, DEV,
                          planted=True)
    bnd = ubs.build_page_bounds(c.k_cache, c.page_table, c.seq_lens_t, c.head_kind, c.Lp)
    sel, num = ubs.select_pages(c.q, bnd, c.page_table, c.seq_lens_t, c.head_kind, c.P, c.token_budget)
    out = ubs.sparse_decode(c.q, c.k_cache, c.v_cache, c.page_table, c.seq_lens_t, c.head_kind, sel, num,
                            c.sink_tokens, c.local_tokens, c.sm_scale)
    _sync()
    sel_o, scores = _oracle_select(c)
    check_selection(sel.cpu().numpy(), num.cpu().numpy(), sel_o, scores, c.head_kind, c.k_pages)
    ref, _ = oracle.decode_ref(bits(c.q), bits(c.k_cache), bits(c.v_cache), c.page_table.cpu().numpy(), lens,
                               c.Hq, c.Hkv, c.P, c.head_kind, sel_o, c.sink_tokens, c.local_tokens, c.sm_scale)
    sg = sel.cpu().numpy()
    got = out.cpu().numpy()
    for b in range(c.B):
        for g in range(c.Hkv):
            if c.head_kind[g] or sg[b, g, :len(sel_o[(b, g)])].tolist() == sel_o[(b, g)]:
                hs = slice(g * c.G, (g + 1) * c.G)
                assert_attention_close(got[b, hs], ref[b, hs], f"end-to-end b={b} g={g}")


def test_decode_full_budget_equals_dense_attention():
    lens = [3000, 64, 1]
    P = 64
    c = cases.make_decode("f", lens, 8, 2, 128, P, P, [0, 0], 64 * P, 0, 0, 36, DEV, keep_tokens=True)
    bnd = ubs.build_page_bounds(c.k_cache, c.page_table, c.seq_lens_t, c.head_kind, P)
    sel, num = ubs.select_pages(c.q, bnd, c.page_table, c.seq_lens_t, c.head_kind, P, 64 * P)
    out = ubs.sparse_decode(c.q, c.k_cache, c.v_cache, c.page_table, c.seq_lens_t, c.head_kind, sel, num, 0, 0,
                            c.sm_scale)
    _sync()
    for b, L in enumerate(lens):
        q = c.q[b].float()[None, :, None, :]                        # [1, Hq, 1, D]
        k = c.k_tok[b].float().repeat_interleave(4, dim=1).permute(1, 0, 2)[None].contiguous()
        v = c.v_tok[b].float().repeat_interleave(4, dim=1).permute(1, 0, 2)[None].contiguous()
        ref = torch.nn.functional.scaled_dot_product_attention(q.cpu(), k.cpu(), v.cpu(), scale=c.sm_scale)
        assert_attention_close(out[b].cpu().numpy(), ref[0, :, 0].numpy(), f"dense b={b}")


# ----------------------------------------------------------------------------- prefill

PREFILL_CASES = [
    # L, Hq, Hkv, D, T, P, head_kind, mask, mask_arg, sink, local
    (200, 4, 2, 64, 64, 16, [0, 1], "random", 3, 1, 2),
    (333, 8, 2, 128, 128, 64, [1, 0], "random", 1, 1, 1),
    (1000, 2, 1, 128, 64, 32, [0], "all", None, 1, 1),
    (130, 4, 4, 64, 128, 64, [0, 0, 1, 1], "diag", None, 0, 1),
    (700, 16, 2, 128, 128, 64, [0, 1], "random", 6, 1, 2),
    (1100, 4, 1, 64, 64, 128, [1], "all", None, 2, 3),
    (257, 2, 2, 128, 64, 16, [1, 1], "all", None, 0, 0),     # every row empty
]


@pytest.mark.parametrize("L,Hq,Hkv,D,T,P,hk,mask,marg,sink,local", PREFILL_CASES)
def test_prefill_matches_oracle(L, Hq, Hkv, D, T, P, hk, mask, marg, sink, local):
    c = cases.make_prefill("p", L, Hq, Hkv, D, T, P, hk, sink, local, mask, 41, DEV, mask_arg=marg,
                           upper_junk=True, extra_pages=2)
    out, lse = ubs.sparse_prefill(c.q, c.k_cache, c.v_cache, c.page_table, hk, c.block_mask, sink, local, T,
                                  c.sm_scale, return_lse=True)
    _sync()
    ref, ref_lse = oracle.prefill_ref(bits(c.q), bits(c.k_cache), bits(c.v_cache), c.page_table.cpu().numpy(),
                                      L, Hq, Hkv, D, P, T, hk, c.block_mask.cpu().numpy(), sink, local,
                                      c.sm_scale)
    assert_attention_close(out.cpu().numpy(), ref, "prefill out")
    assert_lse_close(lse.cpu().numpy(), ref_lse, "prefill lse")


def test_prefill_empty_tile_row():
    L, T = 64 * 5 + 7, 64
    c = cases.make_prefill("e", L, 2, 1, 128, T, 64, [0], 1, 1, "random", 42, DEV, mask_arg=4)
    c.block_mask[0, 3, :] = 0                   # query tile 3 of head 0 keeps nothing
    out, lse = ubs.sparse_prefill(c.q, c.k_cache, c.v_cache, c.page_table, [0], c.block_mask, 1, 1, T,
                                  c.sm_scale, return_lse=True)
    _sync()
    assert torch.all(out[3 * T:4 * T, 0] == 0)
    assert torch.all(torch.isneginf(lse[0, 3 * T:4 * T]))
    ref, _ = oracle.prefill_ref(bits(c.q), bits(c.k_cache), bits(c.v_cache), c.page_table.cpu().numpy(), L,
                                2, 1, 128, 64, T, [0], c.block_mask.cpu().numpy(), 1, 1, c.sm_scale)
    assert_attention_close(out.cpu().numpy(), ref, "prefill out")


@pytest.mark.parametrize("D,T", [(128, 128), (64, 128), (128, 64)])
def test_prefill_growing_scores_rescale(D, T):
    """Keys scaled up along the sequence, so every row's running max keeps growing by more
    than the kernel's lazy-rescale margin (2^8 in weight) and the stored O is rescaled
    several times per row."""
    from workloads import gen
    L, Hq, Hkv, P = 1000, 4, 2, 64
    c = cases.make_prefill("g", L, Hq, Hkv, D, T, P, [0, 1], 1, 2, "all", 44, DEV, keep_tokens=True)
    gain = (1.0 + torch.arange(L, device=DEV, dtype=torch.float32) / 16.0)[:, None, None]
    k_tok = (c.k_tok.float() * gain).to(torch.bfloat16)
    gen.scatter_pages(k_tok, c.page_table, c.k_cache, P, 44, 7)
    # the inputs do what the test is for: the last row's max over all keys exceeds its max
    # over the first 32 keys by more than 8 in the log2 domain
    qf = c.q[L - 1].float().cpu().double().numpy()
    kf = k_tok.float().cpu().double().numpy()
    s = np.einsum("hd,thd->ht", qf[::Hq // Hkv][:Hkv], kf) * c.sm_scale / np.log(2.0)
    assert np.all(s.max(axis=1) - s[:, :32].max(axis=1) > 8.0)
    out, lse = ubs.sparse_prefill(c.q, c.k_cache, c.v_cache, c.page_table, [0, 1], c.block_mask, 1, 2, T,
                                  c.sm_scale, return_lse=True)
    _sync()
    ref, ref_lse = oracle.prefill_ref(bits(c.q), bits(c.k_cache), bits(c.v_cache), c.page_table.cpu().numpy(),
                                      L, Hq, Hkv, D, P, T, [0, 1], c.block_mask.cpu().numpy(), 1, 2, c.sm_scale)
    assert_attention_close(out.cpu().numpy(), ref, "prefill out")
    assert_lse_close(lse.cpu().numpy(), ref_lse, "prefill lse")


# ----------------------------------------------------------------------------- invariances

def _repermute(cache, page_table, seed):
    """Move every physical page to a new seeded position; remap the page table."""
    NP = cache.shape[0]
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    perm = torch.randperm(NP, generator=g).to(cache.device)
    new = torch.empty_like(cache)
    new[perm] = cache
    return new, perm[page_table.long()].to(torch.int32)


def test_prefill_deterministic_and_page_permutation_invariant():
    c = cases.make_prefill("i", 900, 8, 2, 128, 128, 64, [0, 1], 1, 2, "random", 43, DEV, mask_arg=10)
    args = ([0, 1], c.block_mask, 1, 2, 128, c.sm_scale)
    o1 = ubs.sparse_prefill(c.q, c.k_cache, c.v_cache, c.page_table, *args)
    o2 = ubs.sparse_prefill(c.q, c.k_cache, c.v_cache, c.page_table, *args)
    kc, pt = _repermute(c.k_cache, c.page_table, 7)
    vc, _ = _repermute(c.v_cache, c.page_table, 7)
    o3 = ubs.sparse_prefill(c.q, kc, vc, pt, *args)
    _sync()
    assert torch.equal(o1, o2) and torch.equal(o1, o3)


def test_decode_deterministic_and_page_permutation_invariant():
    c = cases.make_decode("i", [5000, 3000], 16, 4, 128, 64, 16, [0, 0, 1, 1], 16 * 64, 64, 512, 44, DEV,
                          planted=True)
    bnd = ubs.build_page_bounds(c.k_cache, c.page_table, c.seq_lens_t, c.head_kind, c.Lp)
    sel, num = ubs.select_pages(c.q, bnd, c.page_table, c.seq_lens_t, c.head_kind, c.P, c.token_budget)
    run = lambda kc, vc, pt, s, n: ubs.sparse_decode(c.q, kc, vc, pt, c.seq_lens_t, c.head_kind, s, n,  # noqa
                                                     64, 512, c.sm_scale)
    o1 = run(c.k_cache, c.v_cache, c.page_table, sel, num)
    o2 = run(c.k_cache, c.v_cache, c.page_table, sel, num)
    kc, pt = _repermute(c.k_cache, c.page_table, 9)
    vc, _ = _repermute(c.v_cache, c.page_table, 9)
    bnd2 = ubs.build_page_bounds(kc, pt, c.seq_lens_t, c.head_kind, c.Lp)
    sel2, num2 = ubs.select_pages(c.q, bnd2, pt, c.seq_lens_t, c.head_kind, c.P, c.token_budget)
    o3 = run(kc, vc, pt, sel2, num2)
    _sync()
    assert torch.equal(sel, sel2) and torch.equal(num, num2)
    assert torch.equal(o1, o2) and torch.equal(o1, o3)
