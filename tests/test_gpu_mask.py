"""GPU parity of estimate_block_mask (dense heads' block mask from mean-pooled tile scores).

The GPU evaluates tile means and scores in fp32, the oracle in fp64. A mask entry j of row i
may differ only when its score lies within rounding of the row's threshold tau (the oracle's
(n_i - 1)-th largest score): |s_j - tau| <= 1e-4 (mag_j + mag_tau) with mag = sum_c |qbar_c
kbar_c|, about four times the fp32 error bound of the means and the dot product. Everything
else is bit-exact, every row keeps exactly n_i tiles, the diagonal always, nothing above it,
and rows of streaming heads are not written."""
import numpy as np
import pytest
import torch

import oracle
import unified_block_sparse_amd as ubs
from tests.helpers import bits
from workloads import cases, gen

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _check(got, o_mask, o_score, o_mag, heads, keep, what):
    flips = 0
    nT = o_mask.shape[-1]
    for n, h in enumerate(heads):
        g = got[h]
        assert not np.triu(g, 1).any(), f"{what}: entries above the diagonal (head {h})"
        assert (np.diag(g) == 1).all(), f"{what}: diagonal not kept (head {h})"
        for i in range(nT):
            n_i = oracle.keep_count(i, *keep)
            assert int(g[i].sum()) == n_i, f"{what}: head {h} row {i} keeps {int(g[i].sum())}, want {n_i}"
            if n_i <= 1:
                continue
            s = o_score[n, i, :i]
            order = np.lexsort((np.arange(i), -s))
            jt = order[n_i - 2]
            tau, mtau = s[jt], o_mag[n, i, jt]
            band = np.abs(s - tau) <= 1e-4 * (o_mag[n, i, :i] + mtau)
            diff = g[i, :i] != o_mask[n, i, :i]
            assert not (diff & ~band).any(), f"{what}: head {h} row {i} differs outside the rounding band"
            flips += int(diff.sum())
    return flips


def _run(c_q, c_k, c_pt, L, Hq, Hkv, D, P, T, kind, keep, what, heads=None, fill=0):
    out = torch.full((Hq, (L + T - 1) // T, (L + T - 1) // T), fill, dtype=torch.uint8, device=DEV)
    m = ubs.estimate_block_mask(c_q, c_k, c_pt, kind, T, keep=keep, out=out)
    torch.cuda.synchronize(DEV)
    got = m.cpu().numpy()
    G = Hq // Hkv
    dense = [h for h in range(Hq) if not kind[h // G]] if heads is None else heads
    o_mask, o_score, o_mag = oracle.meanpool_mask_ref(bits(c_q), bits(c_k), c_pt.cpu().numpy(), L, Hq, Hkv, D, P,
                                                      T, kind, keep[0], keep[1], heads=dense)
    flips = _check(got, o_mask, o_score, o_mag, dense, keep, what)
    for h in range(Hq):
        if kind[h // G]:
            assert (got[h] == fill).all(), f"{what}: streaming head {h} row written"
    print(f"{what}: {len(dense)} heads x {got.shape[1]} rows, {flips} entries flipped inside the band")
    return got


@pytest.mark.parametrize("L,Hq,Hkv,D,P,T,keep", [
    (1000, 4, 2, 64, 16, 64, (3, 10)),      # ragged last tile, one dense and one streaming KV head
    (4096 + 77, 8, 2, 128, 64, 128, (1, 2)),
    (8192, 8, 4, 128, 32, 64, (3, 10)),
])
def test_mask_small_cases(L, Hq, Hkv, D, P, T, keep):
    kind = [0, 1] * (Hkv // 2)
    n = (L + P - 1) // P
    q = gen.normal_bf16((L, Hq, D), 2001, 1, DEV)
    k_cache = gen.normal_bf16((n + 3, Hkv, P, D), 2001, 2, DEV)
    # an exactly sized page table (its own allocation, not a view of a longer one), so that
    # a read past entry n - 1 would leave the table
    pt = gen.randperm(n + 3, 2001, 3, DEV)[:n].to(torch.int32).clone()
    assert pt.numel() == n and pt.untyped_storage().nbytes() == 4 * n
    _run(q, k_cache, pt, L, Hq, Hkv, D, P, T, kind, keep, f"mask L={L} D={D} T={T}", fill=7)


def test_mask_llama8b_dense_heads():
    """The Llama-3-8B prefill workload (65,536 tokens, planted K): all 16 dense heads."""
    c = cases.prefill_llama8b(DEV)
    got = _run(c.q, c.k_cache, c.page_table, c.L, c.Hq, c.Hkv, c.D, c.P, c.T, c.head_kind, (3, 10),
               "mask prefill_llama8b")
    # the workload's own mask (the same rule, fp64 on the harness side) agrees on all but a
    # few near-threshold entries
    dense = [h for h in range(c.Hq) if not c.head_kind[h // c.G]]
    ref = c.block_mask.cpu().numpy()
    d = sum(int((np.tril(got[h]) != np.tril(ref[h])).sum()) for h in dense)
    assert d <= 1e-4 * len(dense) * c.nT * c.nT, d


def test_mask_exact_ties_go_to_lower_tiles():
    """Bit-identical key tiles give bit-identical fp32 scores: the kept tiles must be exactly
    the lowest ones (no rounding band needed)."""
    L, Hq, Hkv, D, P, T = 64 * 40, 4, 1, 128, 64, 64
    n = L // P
    q = gen.normal_bf16((L, Hq, D), 2002, 1, DEV)
    row = gen.normal_bf16((1, 1, 1, D), 2002, 2, DEV)
    k_cache = row.expand(n, Hkv, P, D).contiguous()
    pt = torch.arange(n, dtype=torch.int32, device=DEV)
    m = ubs.estimate_block_mask(q, k_cache, pt, [0], T).cpu().numpy()
    nT = L // T
    for h in range(Hq):
        for i in range(nT):
            want = np.zeros(nT, dtype=np.uint8)
            want[:oracle.keep_count(i, 3, 10) - 1] = 1
            want[i] = 1
            assert np.array_equal(m[h, i], want), (h, i)


def test_mask_feeds_sparse_prefill():
    """The estimated mask drives sparse_prefill; the output equals the oracle's prefill
    under that same mask."""
    c = cases.make_prefill("mask_e2e", 1536, 4, 2, 64, 64, 16, [0, 1], 1, 3, "all", 2003, DEV)
    m = ubs.estimate_block_mask(c.q, c.k_cache, c.page_table, c.head_kind, c.T)
    out = ubs.sparse_prefill(c.q, c.k_cache, c.v_cache, c.page_table, c.head_kind, m, c.sink_tiles,
                             c.local_tiles, c.T, c.sm_scale)
    torch.cuda.synchronize(DEV)
    ref, _ = oracle.prefill_ref(bits(c.q), bits(c.k_cache), bits(c.v_cache), c.page_table.cpu().numpy(), c.L, c.Hq,
                                c.Hkv, c.D, c.P, c.T, c.head_kind, m.cpu().numpy(), c.sink_tiles, c.local_tiles,
                                c.sm_scale)
    err = np.abs(out.cpu().numpy() - ref)
    assert err.max() <= 1e-2 and err.mean() <= 1e-3, (err.max(), err.mean())
