"""GPU parity on the five named workloads, in the launch configuration the bench uses.

prefill_tiny and decode_llama8b are compared in full. For the large ones the oracle
evaluates samples: 64 query rows per head of prefill_llama8b ({0, T-1, T, L-1} plus
seeded rows), 32 per head of prefill_extreme; decode_ragged is compared on all 64
sequences (every page of each, every head), 16 per test."""
import numpy as np
import pytest
import torch

import oracle
import unified_block_sparse_amd as ubs
from tests.gpu_cases import (assert_attention_close, assert_lse_close, check_selection, decode_subset,
                             sample_rows)
from tests.helpers import bits
from workloads import cases

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _sync():
    torch.cuda.synchronize(DEV)


def _run_prefill(c):
    out, lse = ubs.sparse_prefill(c.q, c.k_cache, c.v_cache, c.page_table, c.head_kind, c.block_mask,
                                  c.sink_tiles, c.local_tiles, c.T, c.sm_scale, return_lse=True)
    _sync()
    return out, lse


def _prefill_rows_parity(c, rows, what):
    out, lse = _run_prefill(c)
    q_host = np.zeros(tuple(c.q.shape), dtype=np.uint16)          # untouched pages stay unmapped
    ridx = torch.tensor(rows, device=DEV)
    q_host[rows] = bits(c.q[ridx])
    ref, ref_lse = oracle.prefill_ref(q_host, bits(c.k_cache), bits(c.v_cache), c.page_table.cpu().numpy(),
                                      c.L, c.Hq, c.Hkv, c.D, c.P, c.T, c.head_kind, c.block_mask.cpu().numpy(),
                                      c.sink_tiles, c.local_tiles, c.sm_scale, rows=rows)
    mx, mn = assert_attention_close(out[ridx].cpu().numpy(), ref, what)
    assert_lse_close(lse[:, ridx].cpu().numpy(), ref_lse, what + " lse")
    print(f"{what}: {len(rows)} rows x {c.Hq} heads, max-abs {mx:.2e}, mean-abs {mn:.2e}")


def test_prefill_tiny_full():
    c = cases.prefill_tiny(DEV)
    kept = oracle.prefill_kept_tile_count(c.nT, c.Hq, c.Hkv, c.head_kind, c.block_mask.cpu().numpy(),
                                          c.sink_tiles, c.local_tiles)
    assert kept == 276
    out, lse = _run_prefill(c)
    ref, ref_lse = oracle.prefill_ref(bits(c.q), bits(c.k_cache), bits(c.v_cache), c.page_table.cpu().numpy(),
                                      c.L, c.Hq, c.Hkv, c.D, c.P, c.T, c.head_kind, c.block_mask.cpu().numpy(),
                                      c.sink_tiles, c.local_tiles, c.sm_scale)
    assert_attention_close(out.cpu().numpy(), ref, "prefill_tiny")
    assert_lse_close(lse.cpu().numpy(), ref_lse, "prefill_tiny lse")


def test_prefill_llama8b_sampled_rows():
    c = cases.prefill_llama8b(DEV)
    kept = oracle.prefill_kept_tile_count(c.nT, c.Hq, c.Hkv, c.head_kind, c.block_mask.cpu().numpy(),
                                          c.sink_tiles, c.local_tiles)
    assert kept == 707216
    _prefill_rows_parity(c, sample_rows(c.L, c.T, 64, 3), "prefill_llama8b")


def test_prefill_extreme_sampled_rows():
    c = cases.prefill_extreme(DEV)
    _prefill_rows_parity(c, sample_rows(c.L, c.T, 32, 5), "prefill_extreme")


def _decode_parity(c, batches, what):
    """Bounds (bit-exact on the sampled sequences' pages), selection, decode on the oracle's
    selection, and end-to-end output where the selections coincide."""
    bnd = ubs.build_page_bounds(c.k_cache, c.page_table, c.seq_lens_t, c.head_kind, c.Lp)
    sel, num = ubs.select_pages(c.q, bnd, c.page_table, c.seq_lens_t, c.head_kind, c.P, c.token_budget)
    out_e2e = ubs.sparse_decode(c.q, c.k_cache, c.v_cache, c.page_table, c.seq_lens_t, c.head_kind, sel, num,
                                c.sink_tokens, c.local_tokens, c.sm_scale)
    _sync()
    qb, kb, vb, pt, lens = decode_subset(c, batches)
    # bounds of the sampled sequences' pages
    vals, defined = oracle.bounds_ref(kb, pt, lens, c.P, c.Lp, c.head_kind)
    pages = torch.tensor([int(c.page_table[b, j]) for b in batches for j in range((c.seq_lens[b] + c.P - 1) // c.P)],
                         device=DEV)
    got = oracle.bf16_to_f64(bits(bnd[pages]))
    assert np.array_equal(got[defined], vals[defined]), f"{what}: bounds differ"
    # selection
    sel_o, scores = oracle.select_ref(qb, kb, pt, lens, c.Hq, c.Hkv, c.P, c.Lp, c.token_budget, c.head_kind)
    bi = torch.tensor(batches, device=DEV)
    swaps = check_selection(sel[bi].cpu().numpy(), num[bi].cpu().numpy(), sel_o, scores, c.head_kind, c.k_pages)
    # decode on the oracle's selection (same data, all B sequences run on the GPU)
    k = c.k_pages
    sel_t = sel.clone()
    num_t = num.clone()
    for (i, g), s in sel_o.items():
        row = torch.full((k,), -1, dtype=torch.int32)
        row[:len(s)] = torch.tensor(s, dtype=torch.int32)
        sel_t[batches[i], g] = row.to(DEV)
        num_t[batches[i], g] = len(s)
    out, lse = ubs.sparse_decode(c.q, c.k_cache, c.v_cache, c.page_table, c.seq_lens_t, c.head_kind, sel_t, num_t,
                                 c.sink_tokens, c.local_tokens, c.sm_scale, return_lse=True)
    _sync()
    ref, ref_lse = oracle.decode_ref(qb, kb, vb, pt, lens, c.Hq, c.Hkv, c.P, c.head_kind, sel_o, c.sink_tokens,
                                     c.local_tokens, c.sm_scale)
    mx, mn = assert_attention_close(out[bi].cpu().numpy(), ref, what)
    assert_lse_close(lse[bi].cpu().numpy(), ref_lse, what + " lse")
    # end-to-end where the GPU kept exactly the oracle's pages
    sg = sel[bi].cpu().numpy()
    e2e = out_e2e[bi].cpu().numpy()
    for (i, g), s in sel_o.items():
        if sg[i, g, :len(s)].tolist() == s:
            hs = slice(g * c.G, (g + 1) * c.G)
            assert_attention_close(e2e[i, hs], ref[i, hs], f"{what} end-to-end")
    print(f"{what}: {len(batches)} seqs, swaps in band {swaps}, max-abs {mx:.2e}, mean-abs {mn:.2e}")


def test_decode_llama8b_full():
    c = cases.decode_llama8b(DEV)
    _decode_parity(c, list(range(c.B)), "decode_llama8b")


@pytest.fixture(scope="module")
def ragged_case():
    c = cases.decode_ragged(DEV)
    yield c
    del c
    torch.cuda.empty_cache()


RAGGED_PARTS = 4   # the 64 sequences in four groups of 16 (bounded host memory per test)


@pytest.mark.parametrize("part", range(RAGGED_PARTS))
def test_decode_ragged_every_sequence(ragged_case, part):
    """All 64 sequences of decode_ragged (the shortest and the longest among them), a
    group of 16 per test: bounds bit-exact, selection to the threshold band, decode on the
    oracle's selection."""
    c = ragged_case
    n = c.B // RAGGED_PARTS
    batches = list(range(part * n, (part + 1) * n))
    _decode_parity(c, batches, f"decode_ragged sequences {batches[0]}-{batches[-1]}")


def test_decode_reused_selection():
    """Selection reused across decode steps (LServe, Decode Phase: the page selection of
    one step serves the next ones): select with one step's queries, then decode R = 4
    steps, each with fresh queries, against the cached selection. Every step must equal
    the oracle's decode of that step's queries over exactly the cached pages."""
    from workloads import gen
    c = cases.decode_llama8b(DEV)
    bnd = ubs.build_page_bounds(c.k_cache, c.page_table, c.seq_lens_t, c.head_kind, c.Lp)
    sel, num = ubs.select_pages(c.q, bnd, c.page_table, c.seq_lens_t, c.head_kind, c.P, c.token_budget)
    _sync()
    batches = list(range(c.B))
    _, kb, vb, pt, lens = decode_subset(c, batches)
    sel_h, num_h = sel.cpu().numpy(), num.cpu().numpy()
    cached = {(i, g): [int(x) for x in sel_h[i, g, :num_h[i, g]]]
              for i in range(c.B) for g in range(c.Hkv) if not c.head_kind[g]}
    for step in range(4):
        q = gen.normal_bf16((c.B, c.Hq, c.D), 1002, 90 + step, DEV)
        out, lse = ubs.sparse_decode(q, c.k_cache, c.v_cache, c.page_table, c.seq_lens_t, c.head_kind, sel, num,
                                     c.sink_tokens, c.local_tokens, c.sm_scale, return_lse=True)
        _sync()
        ref, ref_lse = oracle.decode_ref(bits(q), kb, vb, pt, lens, c.Hq, c.Hkv, c.P, c.head_kind, cached,
                                         c.sink_tokens, c.local_tokens, c.sm_scale)
        mx, mn = assert_attention_close(out.cpu().numpy(), ref, f"reused selection, step {step}")
        assert_lse_close(lse.cpu().numpy(), ref_lse, f"reused selection, step {step} lse")
