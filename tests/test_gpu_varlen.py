"""Batched prefill (sparse_prefill_varlen): B sequences of different lengths in one
call over one shared paged cache. Every sequence's rows must equal, bit for bit, a
sparse_prefill call on that sequence alone, and match the oracle."""
import numpy as np
import pytest
import torch

import oracle
import unified_block_sparse_amd as ubs
from tests.gpu_cases import assert_attention_close, assert_lse_close
from tests.helpers import bits
from workloads import cases

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

VARLEN_CASES = [
    # lens, Hq, Hkv, D, T, P, head_kind, sink, local, lower tiles per dense row
    ([700, 0, 129, 2000, 64], 8, 2, 128, 128, 64, [0, 1], 1, 2, 3),
    ([333, 1100, 1, 640], 4, 4, 64, 64, 16, [0, 0, 1, 1], 1, 3, 4),
    ([4096], 16, 2, 128, 128, 64, [1, 0], 1, 4, 6),
]


def _pack(seqs, lens, T, P, Hq):
    """One cache holding every sequence's pages (page ids offset per sequence), packed q,
    cu_seqlens, page-table rows and the masks padded to [B, Hq, nT_max, nT_max]."""
    offs, NPs = [], 0
    for c in seqs:
        offs.append(NPs)
        NPs += c.k_cache.shape[0]
    k_all = torch.cat([c.k_cache for c in seqs])
    v_all = torch.cat([c.v_cache for c in seqs])
    max_pages = max(1, max((L + P - 1) // P for L in lens))
    pt = torch.zeros((len(seqs), max_pages), dtype=torch.int32, device=DEV)
    for b, c in enumerate(seqs):
        n = c.page_table.numel()
        pt[b, :n] = c.page_table + offs[b]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=DEV)
    q = torch.cat([c.q for c in seqs])
    nTm = (max(lens) + T - 1) // T
    mask = torch.zeros((len(seqs), Hq, nTm, nTm), dtype=torch.uint8, device=DEV)
    for b, c in enumerate(seqs):
        nT = c.nT
        mask[b, :, :nT, :nT] = c.block_mask
    return q, k_all, v_all, pt, cu, mask


@pytest.mark.parametrize("lens,Hq,Hkv,D,T,P,hk,sink,local,marg", VARLEN_CASES)
def test_varlen_equals_single_sequence_calls_and_oracle(lens, Hq, Hkv, D, T, P, hk, sink, local, marg):
    seqs = [cases.make_prefill(f"v{b}", L, Hq, Hkv, D, T, P, hk, sink, local, "random", 70 + b, DEV, mask_arg=marg,
                               upper_junk=True) for b, L in enumerate(lens)]
    q, k_all, v_all, pt, cu, mask = _pack(seqs, lens, T, P, Hq)
    total = sum(lens)
    out, lse = ubs.sparse_prefill_varlen(q, k_all, v_all, pt, cu, max(lens), hk, mask, sink, local, T,
                                         seqs[0].sm_scale, return_lse=True)
    torch.cuda.synchronize(DEV)
    assert out.shape == (total, Hq, D) and lse.shape == (Hq, total)
    start = 0
    for b, (c, L) in enumerate(zip(seqs, lens)):
        if L > 0:
            o1, l1 = ubs.sparse_prefill(c.q, c.k_cache, c.v_cache, c.page_table, hk, c.block_mask, sink, local, T,
                                        c.sm_scale, return_lse=True)
            torch.cuda.synchronize(DEV)
            assert torch.equal(out[start:start + L], o1), f"sequence {b}: out differs from the single call"
            assert torch.equal(lse[:, start:start + L], l1), f"sequence {b}: lse differs from the single call"
            if L <= 1100:
                ref, ref_lse = oracle.prefill_ref(bits(c.q), bits(c.k_cache), bits(c.v_cache),
                                                  c.page_table.cpu().numpy(), L, Hq, Hkv, D, P, T, hk,
                                                  c.block_mask.cpu().numpy(), sink, local, c.sm_scale)
                assert_attention_close(out[start:start + L].cpu().numpy(), ref, f"varlen seq {b}")
                assert_lse_close(lse[:, start:start + L].cpu().numpy(), ref_lse, f"varlen seq {b} lse")
        start += L
