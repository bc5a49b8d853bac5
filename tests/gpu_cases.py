"""Shared GPU-test plumbing: run the library on a case, run the oracle on the same
bits, compare. No attention arithmetic lives here (the oracle and the library do it)."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from tests.helpers import bits

MAX_ABS = 1e-2     # attention outputs from bf16 inputs, fp32 accumulation
MEAN_ABS = 1e-3
SEL_BAND = 1e-3    # relative band around the k-th score inside which swaps are allowed


def assert_attention_close(got, ref, what: str):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    d = np.abs(got - ref)
    mx, mn = float(d.max()), float(d.mean())
    assert mx <= MAX_ABS and mn <= MEAN_ABS, f"{what}: max-abs {mx:.3e} mean-abs {mn:.3e}"
    return mx, mn


def assert_lse_close(got, ref, what: str):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    inf_r = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), inf_r), f"{what}: -inf pattern differs"
    d = np.abs(got[~inf_r] - ref[~inf_r])
    if d.size:
        assert d.max() <= MAX_ABS and d.mean() <= MEAN_ABS, f"{what}: lse max {d.max():.3e} mean {d.mean():.3e}"


def check_selection(sel_gpu, num_gpu, oracle_sel, scores, head_kind, k):
    """GPU selection vs the oracle's: bit-exact except pages whose oracle score lies within
    SEL_BAND (relative) of the oracle's k-th score. Returns the number of exempted swaps."""
    sel_gpu = np.asarray(sel_gpu)
    num_gpu = np.asarray(num_gpu)
    swaps = 0
    B, Hkv, kk = sel_gpu.shape
    assert kk == k
    for (b, g), osel in oracle_sel.items():
        n = int(num_gpu[b, g])
        assert n == len(osel), f"(b={b}, g={g}): num_selected {n} != {len(osel)}"
        row = sel_gpu[b, g]
        assert np.all(row[n:] == -1), f"(b={b}, g={g}): unused slots not -1"
        got = row[:n].tolist()
        assert got == sorted(got) and len(set(got)) == n, f"(b={b}, g={g}): not ascending/distinct"
        diff = set(got) ^ set(osel)
        if diff:
            s = scores[(b, g)]
            order = sorted(range(len(s)), key=lambda j: (-s[j], j))
            tau = s[order[k - 1]]
            for j in diff:
                assert abs(s[j] - tau) <= SEL_BAND * abs(tau), \
                    f"(b={b}, g={g}): page {j} score {s[j]} vs k-th {tau} differs outside the band"
            swaps += len(diff) // 2
    for b in range(B):
        for g in range(Hkv):
            if head_kind[g]:
                assert num_gpu[b, g] == 0 and np.all(sel_gpu[b, g] == -1)
    return swaps


def decode_subset(c, batches):
    """Host bits of the pages that sequences `batches` use, with a remapped page table,
    so the oracle can run on a few sequences of a large batch."""
    P = c.P
    pages, pt_rows, lens = [], [], []
    for b in batches:
        L = c.seq_lens[b]
        n = (L + P - 1) // P
        pt_rows.append(list(range(len(pages), len(pages) + n)))
        pages.extend(c.page_table[b, :n].tolist())
        lens.append(L)
    idx = torch.tensor(pages if pages else [0], dtype=torch.long, device=c.k_cache.device)
    kb = bits(c.k_cache[idx])
    vb = bits(c.v_cache[idx])
    mp = max(1, max(len(r) for r in pt_rows))
    pt = np.zeros((len(batches), mp), dtype=np.int32)
    for i, r in enumerate(pt_rows):
        pt[i, :len(r)] = r
    qb = bits(c.q[list(batches)])
    return qb, kb, vb, pt, lens


def sample_rows(L: int, T: int, n: int, seed: int):
    """{0, T-1, T, L-1} plus seeded distinct rows, n in total, sorted."""
    rng = np.random.default_rng(seed)
    fixed = sorted({r for r in (0, T - 1, T, L - 1) if 0 <= r < L})
    pool = np.setdiff1d(np.arange(L), fixed)
    extra = rng.choice(pool, size=min(len(pool), max(0, n - len(fixed))), replace=False)
    return sorted(fixed + [int(x) for x in extra])
