"""Pins of the fp64 oracle against facts fixed by the mathematics and the pages.

Each test checks the oracle against something other than itself: a library routine
(torch's scaled_dot_product_attention in float64 on the CPU), a closed form, an
explicitly materialised token mask, brute force over tokens, a hand-derived worked
example (tests/golden/select_tiny.json) or an invariant of the Quest bound.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from workloads import cases
from tests.helpers import bits

HERE = os.path.dirname(os.path.abspath(__file__))


def _sdpa_f64(q_tok, k_tok, v_tok, G, scale, mask=None, causal=False):
    """Library attention on token-major tensors: q [L,Hq,D], k/v [Lk,Hkv,D] -> [L,Hq,D]."""
    q = q_tok.double().permute(1, 0, 2)[None]
    k = k_tok.double().repeat_interleave(G, dim=1).permute(1, 0, 2)[None]
    v = v_tok.double().repeat_interleave(G, dim=1).permute(1, 0, 2)[None]
    o = F.scaled_dot_product_attention(q, k, v, attn_mask=mask, is_causal=causal, scale=scale)
    return o[0].permute(1, 0, 2).numpy()


def _prefill(c, **kw):
    return oracle.prefill_ref(bits(c.q), bits(c.k_cache), bits(c.v_cache), c.page_table.numpy(),
                              c.L, c.Hq, c.Hkv, c.D, c.P, c.T, c.head_kind, c.block_mask.numpy(),
                              c.sink_tiles, c.local_tiles, c.sm_scale, **kw)


# ----------------------------------------------------------------------------- prefill pins

@pytest.mark.parametrize("L,T,P,D", [(200, 64, 64, 64), (130, 32, 64, 32), (96, 32, 16, 16)])
def test_prefill_all_kept_equals_causal_sdpa(L, T, P, D):
    c = cases.make_prefill("t", L, 4, 2, D, T, P, [0, 0], 1, 1, "all", 11, "cpu",
                           keep_tokens=True, extra_pages=3)
    out, lse = _prefill(c)
    ref = _sdpa_f64(c.q, c.k_tok, c.v_tok, c.G, c.sm_scale, causal=True)
    assert np.abs(out - ref).max() < 1e-12
    # lse against an explicit log-sum-exp over the causal prefix
    q = c.q.double().numpy()
    k = c.k_tok.double().numpy()
    for r in [0, 1, T - 1, T, L - 1]:
        s = c.sm_scale * (k[:r + 1, 1, :] @ q[r, 3, :])
        assert abs(lse[3, r] - np.log(np.exp(s).sum())) < 1e-10


def _lambda_token_mask(L, T, sink_tiles, local_tiles):
    """Streaming support written per token pair: key c is visible to query r iff c <= r
    and c lies in the first sink_tiles*T tokens or in the local_tiles tiles ending with
    the query's own tile."""
    r = torch.arange(L)[:, None]
    c = torch.arange(L)[None, :]
    local_start = (r // T - local_tiles + 1) * T
    return (c <= r) & ((c < sink_tiles * T) | (c >= local_start))


@pytest.mark.parametrize("sink,local", [(1, 3), (2, 1), (0, 2), (1, 1)])
def test_prefill_lambda_equals_materialised_mask(sink, local):
    L, T = 300, 32
    c = cases.make_prefill("t", L, 2, 1, 32, T, 16, [1], sink, local, "all", 12, "cpu",
                           keep_tokens=True)
    out, _ = _prefill(c)
    m = _lambda_token_mask(L, T, sink, local)
    ref = _sdpa_f64(c.q, c.k_tok, c.v_tok, c.G, c.sm_scale, mask=m[None, None])
    assert np.abs(out - ref).max() < 1e-12


def test_prefill_lambda_wide_window_is_dense():
    L, T = 257, 32
    nT = (L + T - 1) // T
    c = cases.make_prefill("t", L, 2, 1, 32, T, 64, [1], 2, nT - 2, "all", 13, "cpu",
                           keep_tokens=True)
    out, _ = _prefill(c)
    ref = _sdpa_f64(c.q, c.k_tok, c.v_tok, c.G, c.sm_scale, causal=True)
    assert np.abs(out - ref).max() < 1e-12


def test_prefill_row0_is_v0_and_const_v():
    c = cases.make_prefill("t", 150, 4, 2, 32, 32, 64, [0, 1], 1, 2, "random", 14, "cpu",
                           mask_arg=5, keep_tokens=True)
    out, lse = _prefill(c)
    v = c.v_tok.double().numpy()
    for h in range(4):
        assert np.array_equal(out[0, h], v[0, h // 2])
        assert lse[h, 0] == pytest.approx(c.sm_scale * float(
            (c.q[0, h].double() * c.k_tok[0, h // 2].double()).sum()), abs=1e-12)
    c.v_cache[:] = torch.tensor(0.71875, dtype=torch.bfloat16)
    out2, _ = _prefill(c)
    assert np.abs(out2 - 0.71875).max() < 1e-12


def test_prefill_diagonal_only_is_per_tile_causal():
    L, T = 170, 32
    c = cases.make_prefill("t", L, 2, 2, 32, T, 32, [0, 0], 1, 1, "diag", 15, "cpu",
                           keep_tokens=True)
    out, _ = _prefill(c)
    for i in range((L + T - 1) // T):
        sl = slice(i * T, min((i + 1) * T, L))
        ref = _sdpa_f64(c.q[sl], c.k_tok[sl], c.v_tok[sl], 1, c.sm_scale, causal=True)
        assert np.abs(out[sl] - ref).max() < 1e-12


def test_prefill_zero_query_averages_kept_keys():
    """q = 0 gives equal weights, so out[r] is the mean of v over K(r); the key set is
    written here per token from the block mask (ignoring tiles above the diagonal) and
    the Lambda rule."""
    L, T = 333, 32
    nT = (L + T - 1) // T
    c = cases.make_prefill("t", L, 4, 2, 16, T, 64, [0, 1], 1, 3, "random", 16, "cpu",
                           mask_arg=12, keep_tokens=True, upper_junk=True)
    c.q.zero_()
    out, lse = _prefill(c)
    v = c.v_tok.double().numpy()
    mask = c.block_mask.numpy()
    lam = _lambda_token_mask(L, T, 1, 3).numpy()
    for h in range(4):
        g = h // 2
        for r in range(L):
            if c.head_kind[g]:
                keys = np.nonzero(lam[r])[0]
            else:
                keys = np.array([t for t in range(r + 1) if mask[h, r // T, t // T]])
            assert np.abs(out[r, h] - v[keys, g].mean(axis=0)).max() < 1e-12
            assert lse[h, r] == pytest.approx(math.log(len(keys)), abs=1e-12)
    assert nT == 11


def test_prefill_empty_row():
    L, T = 64, 16
    c = cases.make_prefill("t", L, 1, 1, 16, T, 16, [0], 1, 1, "diag", 17, "cpu")
    c.block_mask[0, 2, 2] = 0            # tile 2 keeps nothing
    out, lse = _prefill(c)
    assert np.all(out[32:48, 0] == 0) and np.all(np.isneginf(lse[0, 32:48]))


def test_prefill_kept_tile_count_matches_enumeration():
    c = cases.make_prefill("t", 300, 4, 2, 16, 32, 64, [0, 1], 1, 3, "random", 18, "cpu",
                           mask_arg=9, upper_junk=True)
    n = oracle.prefill_kept_tile_count(c.nT, c.Hq, c.Hkv, c.head_kind, c.block_mask.numpy(),
                                       c.sink_tiles, c.local_tiles)
    lam = _lambda_token_mask(c.nT, 1, 1, 3).numpy()      # tile-level Lambda with T = 1
    m = c.block_mask.numpy()
    brute = sum(int(lam.sum()) if c.head_kind[h // 2] else
                sum(int(m[h, i, j]) for i in range(c.nT) for j in range(i + 1)) for h in range(4))
    assert n == brute


# ----------------------------------------------------------------------------- golden example

def _golden_case():
    gj = json.load(open(os.path.join(HERE, "golden", "select_tiny.json")))
    P, L, D = gj["P"], gj["L"], gj["D"]
    pt = np.array(gj["page_table"], dtype=np.int32)
    NP = len(pt)
    keys = np.array(gj["keys"] + [gj["pad_key"]], dtype=np.float32)
    vals = np.array(gj["values"] + [gj["pad_value"]], dtype=np.float32)
    # KV head 0 dense, KV head 1 streaming; both hold the same tokens
    kc = torch.zeros((NP, 2, P, D), dtype=torch.bfloat16)
    vc = torch.zeros((NP, 2, P, D), dtype=torch.bfloat16)
    for t in range(NP * P):
        kc[pt[t // P], :, t % P] = torch.tensor(keys[t]).to(torch.bfloat16)
        vc[pt[t // P], :, t % P] = torch.tensor(vals[t]).to(torch.bfloat16)
    q = torch.zeros((1, 4, D), dtype=torch.bfloat16)
    q[0, :2] = torch.tensor(gj["q_dense_group"]).to(torch.bfloat16)
    return gj, P, L, pt, kc, vc, q


def test_golden_bounds_scores_selection():
    gj, P, L, pt, kc, vc, q = _golden_case()
    hk = [0, 1]
    vals, defined = oracle.bounds_ref(bits(kc), pt[None], [L], P, gj["Lp"], hk)
    for j in range(4):
        p = pt[j]
        assert defined[p, 0, 0] and not defined[p, 1, 0]
        assert vals[p, 0, 0, 0].tolist() == gj["bounds_min"][j]
        assert vals[p, 0, 0, 1].tolist() == gj["bounds_max"][j]
        qg = bits(q)[0, :2]
        per_head = [oracle.subpage_bound(oracle.bf16_to_f64(qg[h:h + 1]), vals[p, 0, 0, 0],
                                         vals[p, 0, 0, 1]) for h in range(2)]
        assert per_head == gj["per_head_bounds"][j]
    scores = oracle.page_scores_ref(bits(q), vals, defined, pt[None], [L], 4, 2, P, gj["Lp"], hk)
    assert scores[(0, 0)].tolist() == gj["page_scores"]
    for k, exp in gj["selected"].items():
        sel, _ = oracle.select_ref(bits(q), bits(kc), pt[None], [L], 4, 2, P, gj["Lp"],
                                   int(k) * P, hk)
        assert sel[(0, 0)] == exp


def test_golden_decode_key_sets():
    gj, P, L, pt, kc, vc, q = _golden_case()
    zero = torch.zeros_like(q)
    sel = {(0, 0): gj["selected"]["3"]}
    out, lse = oracle.decode_ref(bits(zero), bits(kc), bits(vc), pt[None], [L], 4, 2, P, [0, 1],
                                 sel, 1, 2, 1.0)
    assert oracle.decode_keys_ref(L, P, False, sel[(0, 0)], 1, 2).tolist() == gj["decode_q0_dense_k3_keys"]
    assert oracle.decode_keys_ref(L, P, True, [], 1, 2).tolist() == gj["decode_streaming_sink1_local2_keys"]
    assert np.allclose(out[0, 0], gj["decode_q0_dense_k3_out"], rtol=0, atol=1e-15)
    assert np.allclose(out[0, 3], gj["decode_q0_streaming_out"], rtol=0, atol=1e-15)
    assert lse[0, 0] == pytest.approx(math.log(6)) and lse[0, 2] == pytest.approx(math.log(3))


# ----------------------------------------------------------------------------- bounds pins

@pytest.mark.parametrize("P,Lp", [(16, 4), (16, 16), (8, 1)])
def test_bounds_brute_force(P, Lp):
    lens = [37, 16, 1, 50]
    c = cases.make_decode("t", lens, 4, 2, 8, P, Lp, [0, 1], 4 * P, 4, 8, 21, "cpu",
                          keep_tokens=True, extra_pages=2)
    vals, defined = oracle.bounds_ref(bits(c.k_cache), c.page_table.numpy(), lens, P, Lp, c.head_kind)
    pt = c.page_table.numpy()
    seen = 0
    for b, L in enumerate(lens):
        kt = c.k_tok[b].double().numpy()
        for t0 in range(0, L, Lp):
            j, u = t0 // P, (t0 % P) // Lp
            p = pt[b, j]
            lo = [math.inf] * c.D
            hi = [-math.inf] * c.D
            for t in range(t0, min(t0 + Lp, L)):
                for ch in range(c.D):
                    lo[ch] = min(lo[ch], kt[t, 0, ch])
                    hi[ch] = max(hi[ch], kt[t, 0, ch])
            assert defined[p, 0, u] and not defined[p, 1, u]
            assert vals[p, 0, u, 0].tolist() == lo and vals[p, 0, u, 1].tolist() == hi
            seen += 1
    assert defined.sum() == seen
    if Lp == 1:
        # single-token sub-page: min = max = the key itself
        assert np.array_equal(vals[defined][:, 0], vals[defined][:, 1])


# ----------------------------------------------------------------------------- selection pins

def test_bound_is_upper_bound_and_tight_for_single_tokens():
    lens = [70, 33]
    P = 16
    for Lp in (16, 4, 1):
        c = cases.make_decode("t", lens, 8, 2, 16, P, Lp, [0, 0], 2 * P, 4, 8, 22, "cpu",
                              keep_tokens=True, planted=True)
        vals, defined = oracle.bounds_ref(bits(c.k_cache), c.page_table.numpy(), lens, P, Lp, c.head_kind)
        sc = oracle.page_scores_ref(bits(c.q), vals, defined, c.page_table.numpy(), lens, 8, 2, P, Lp,
                                    c.head_kind)
        q = c.q.double().numpy()
        for b, L in enumerate(lens):
            k = c.k_tok[b].double().numpy()
            for g in range(2):
                dots = q[b, 4 * g:4 * g + 4] @ k[:, g, :].T           # [G, L]
                for j in range((L + P - 1) // P):
                    true = dots[:, j * P:min((j + 1) * P, L)].max()
                    assert sc[(b, g)][j] >= true - 1e-12
                    if Lp == 1:
                        assert sc[(b, g)][j] == pytest.approx(true, abs=1e-12)


def test_subpage_scores_tighter_than_page_summary():
    lens = [90]
    P = 32
    c = cases.make_decode("t", lens, 4, 1, 16, P, 8, [0], 2 * P, 4, 8, 23, "cpu", planted=True)
    kb = bits(c.k_cache)
    fine = oracle.page_scores_ref(bits(c.q), *oracle.bounds_ref(kb, c.page_table.numpy(), lens, P, 8, [0]),
                                  c.page_table.numpy(), lens, 4, 1, P, 8, [0])
    coarse = oracle.page_scores_ref(bits(c.q), *oracle.bounds_ref(kb, c.page_table.numpy(), lens, P, P, [0]),
                                    c.page_table.numpy(), lens, 4, 1, P, P, [0])
    assert np.all(fine[(0, 0)] <= coarse[(0, 0)] + 1e-12)
    assert np.any(fine[(0, 0)] < coarse[(0, 0)])


def test_bound_split_sign_identity():
    """sum_c max(q kmin, q kmax) = q+ . kmax + q- . kmin whenever kmin <= kmax (the form a
    kernel may evaluate as one dot product of length 2D)."""
    rng = np.random.default_rng(5)
    for _ in range(50):
        q = rng.standard_normal((4, 128))
        a, b = rng.standard_normal((2, 128))
        kmin, kmax = np.minimum(a, b), np.maximum(a, b)
        lit = oracle.subpage_bound(q, kmin, kmax)
        alt = (np.maximum(q, 0) @ kmax + np.minimum(q, 0) @ kmin).max()
        assert abs(lit - alt) <= 1e-12 * max(1.0, abs(lit))


def test_topk_matches_lexsort_and_small_n():
    rng = np.random.default_rng(7)
    for n, k in [(100, 10), (64, 64), (10, 64), (500, 64), (33, 1)]:
        s = np.round(rng.standard_normal(n) * 4) / 4         # many ties
        got = oracle.topk_pages_ref(s, k)
        order = np.lexsort((np.arange(n), -s))               # primary: -s, secondary: index
        assert got == sorted(order[:k].tolist())
        if n <= k:
            assert got == list(range(n))


def test_budget_covering_context_selects_everything():
    lens = [100, 64, 5]
    P = 16
    c = cases.make_decode("t", lens, 4, 2, 8, P, 4, [0, 1], 8 * P, 4, 8, 24, "cpu")
    sel, _ = oracle.select_ref(bits(c.q), bits(c.k_cache), c.page_table.numpy(), lens, 4, 2, P, 4,
                               8 * P, c.head_kind)
    for b, L in enumerate(lens):
        assert sel[(b, 0)] == list(range((L + P - 1) // P))


# ----------------------------------------------------------------------------- decode pins

def test_decode_full_budget_equals_dense_and_prefill_last_row():
    lens = [77, 128, 3]
    P = 16
    c = cases.make_decode("t", lens, 4, 2, 32, P, P, [0, 0], 1024, 4, 8, 25, "cpu",
                          keep_tokens=True)
    sel = {(b, g): list(range((L + P - 1) // P)) for b, L in enumerate(lens) for g in range(2)}
    out, lse = oracle.decode_ref(bits(c.q), bits(c.k_cache), bits(c.v_cache), c.page_table.numpy(),
                                 lens, 4, 2, P, c.head_kind, sel, 4, 8, c.sm_scale)
    for b, L in enumerate(lens):
        ref = _sdpa_f64(c.q[b:b + 1], c.k_tok[b], c.v_tok[b], 2, c.sm_scale)
        assert np.abs(out[b] - ref[0]).max() < 1e-12
        # same as row L-1 of an all-kept prefill whose last query is this decode query
        qpf = torch.zeros((L, 4, 32), dtype=torch.bfloat16)
        qpf[L - 1] = c.q[b]
        npg = (L + P - 1) // P
        pout, plse = oracle.prefill_ref(bits(qpf), bits(c.k_cache), bits(c.v_cache),
                                        c.page_table.numpy()[b, :npg], L, 4, 2, 32, P, 16, [0, 0],
                                        np.ones((4, (L + 15) // 16, (L + 15) // 16), np.uint8),
                                        1, 1, c.sm_scale, rows=[L - 1])
        assert np.abs(pout[0] - out[b]).max() < 1e-12
        assert np.abs(plse[:, 0] - lse[b]).max() < 1e-12


def test_decode_streaming_wide_window_is_dense():
    lens = [50, 200]
    c = cases.make_decode("t", lens, 4, 2, 16, 16, 16, [1, 1], 64, 30, 20, 26, "cpu",
                          keep_tokens=True)
    out, _ = oracle.decode_ref(bits(c.q), bits(c.k_cache), bits(c.v_cache), c.page_table.numpy(),
                               [50], 4, 2, 16, c.head_kind, {}, 30, 20, c.sm_scale)
    ref = _sdpa_f64(c.q[0:1], c.k_tok[0], c.v_tok[0], 2, c.sm_scale)
    assert np.abs(out[0] - ref[0]).max() < 1e-12


def test_decode_zero_query_averages_key_set():
    lens = [1000, 77, 64, 1]
    P = 64
    c = cases.make_decode("t", lens, 8, 2, 16, P, 16, [0, 1], 4 * P, 100, 130, 27, "cpu",
                          keep_tokens=True)
    c.q.zero_()
    rng = np.random.default_rng(3)
    sel = {}
    for b, L in enumerate(lens):
        n = (L + P - 1) // P
        sel[(b, 0)] = sorted(rng.choice(n, size=min(n, 4), replace=False).tolist())
    out, lse = oracle.decode_ref(bits(c.q), bits(c.k_cache), bits(c.v_cache), c.page_table.numpy(),
                                 lens, 8, 2, P, c.head_kind, sel, 100, 130, c.sm_scale)
    for b, L in enumerate(lens):
        v = c.v_tok[b].double().numpy()
        dense_keys = [t for t in range(L) if t // P in sel[(b, 0)]]
        stream_keys = [t for t in range(L) if t < 100 or t > L - 1 - 130]
        for h in range(4):
            assert np.abs(out[b, h] - v[dense_keys, 0].mean(0)).max() < 1e-12
        for h in range(4, 8):
            assert np.abs(out[b, h] - v[stream_keys, 1].mean(0)).max() < 1e-12
            assert lse[b, h] == pytest.approx(math.log(len(stream_keys)))


def test_decode_empty_sequence():
    c = cases.make_decode("t", [0, 5], 2, 1, 8, 4, 4, [0], 8, 1, 1, 28, "cpu")
    out, lse = oracle.decode_ref(bits(c.q), bits(c.k_cache), bits(c.v_cache), c.page_table.numpy(),
                                 [0, 5], 2, 1, 4, [0], {(0, 0): [], (1, 0): [0, 1]}, 1, 1, 1.0)
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))


# ----------------------------------------------------------------------------- block-mask estimation pins

def _paged(tok_bits, P, seed):
    """Scatter token-major bits [L, Hkv, D] into a paged cache with a seeded permuted page table."""
    L, Hkv, D = tok_bits.shape
    n = (L + P - 1) // P
    rng = np.random.default_rng(seed)
    pt = rng.permutation(n + 2)[:n].astype(np.int32)
    cache = rng.integers(0, 1 << 16, size=(n + 2, Hkv, P, D), dtype=np.uint16)   # noise elsewhere
    for t in range(L):
        cache[pt[t // P], :, t % P, :] = tok_bits[t]
    return cache, pt


def _bits_of(x):
    return torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("keep", [(3, 10), (1, 2)])
def test_meanpool_mask_brute_force(keep):
    """Plain loops over rows, channels and candidates, with Python's sort on (-score, j)."""
    L, Hq, Hkv, D, P, T = 200, 4, 2, 8, 16, 32        # 7 tiles, the last one 8 rows
    rng = np.random.default_rng(7)
    qb = _bits_of(rng.standard_normal((L, Hq, D)))
    kb_tok = _bits_of(rng.standard_normal((L, Hkv, D)))
    cache, pt = _paged(kb_tok, P, 8)
    mask, score, _ = oracle.meanpool_mask_ref(qb, cache, pt, L, Hq, Hkv, D, P, T, [0, 0], keep[0], keep[1])
    qf = oracle.bf16_to_f64(qb)
    kf = oracle.bf16_to_f64(kb_tok)
    nT = (L + T - 1) // T
    G = Hq // Hkv

    def mean_rows(x, lo, hi):
        out = [0.0] * D
        for r in range(lo, hi):
            for c in range(D):
                out[c] += float(x[r, c])
        return [v / (hi - lo) for v in out]

    for h in range(Hq):
        g = h // G
        km = [mean_rows(kf[:, g, :], j * T, min((j + 1) * T, L)) for j in range(nT)]
        for i in range(nT):
            qm = mean_rows(qf[:, h, :], i * T, min((i + 1) * T, L))
            s = [sum(qm[c] * km[j][c] for c in range(D)) for j in range(i)]
            n_i = -(-(keep[0] * (i + 1)) // keep[1])
            kept = set(sorted(range(i), key=lambda j: (-s[j], j))[:n_i - 1]) | {i}
            want = [1 if j in kept else 0 for j in range(nT)]
            assert mask[h, i].tolist() == want, (h, i)
            for j in range(i):
                assert abs(score[h, i, j] - s[j]) <= 1e-12 * (1 + abs(s[j]))


def test_meanpool_mask_monotone_scores_give_closed_forms():
    """Queries along channel 0 and key tiles whose channel-0 mean is +-(j+1): scores rise
    (or fall) with j, so the kept tiles are the n_i - 1 nearest (or the first) ones."""
    L, Hq, Hkv, D, P, T = 16 * 20, 2, 1, 4, 16, 16
    nT = L // T
    q = np.zeros((L, Hq, D)); q[:, :, 0] = 1.0
    for sign in (1.0, -1.0):
        k = np.zeros((L, Hkv, D))
        for t in range(L):
            k[t, 0, 0] = sign * (t // T + 1)
        cache, pt = _paged(_bits_of(k), P, 3)
        mask, _, _ = oracle.meanpool_mask_ref(_bits_of(q), cache, pt, L, Hq, Hkv, D, P, T, [0])
        for h in range(Hq):
            for i in range(nT):
                n_i = oracle.keep_count(i, 3, 10)
                lower = range(i - n_i + 1, i) if sign > 0 else range(0, n_i - 1)
                want = np.zeros(nT, dtype=np.uint8)
                want[list(lower)] = 1
                want[i] = 1
                assert np.array_equal(mask[h, i], want), (sign, h, i)


def test_meanpool_mask_ties_go_to_lower_tiles_and_counts():
    """Identical key tiles give equal scores: the kept tiles are the lowest ones. On random
    data every row keeps exactly n_i tiles and nothing above the diagonal."""
    L, Hq, Hkv, D, P, T = 32 * 12, 2, 1, 8, 32, 32
    rng = np.random.default_rng(11)
    q = rng.standard_normal((L, Hq, D))
    row = rng.standard_normal(D)
    k = np.tile(row, (L, Hkv, 1))
    cache, pt = _paged(_bits_of(k), P, 5)
    mask, _, _ = oracle.meanpool_mask_ref(_bits_of(q), cache, pt, L, Hq, Hkv, D, P, T, [0])
    nT = L // T
    for h in range(Hq):
        for i in range(nT):
            want = np.zeros(nT, dtype=np.uint8)
            want[:oracle.keep_count(i, 3, 10) - 1] = 1
            want[i] = 1
            assert np.array_equal(mask[h, i], want)
    k = rng.standard_normal((L, Hkv, D))
    cache, pt = _paged(_bits_of(k), P, 6)
    mask, _, _ = oracle.meanpool_mask_ref(_bits_of(q), cache, pt, L, Hq, Hkv, D, P, T, [0])
    for h in range(Hq):
        assert not np.triu(mask[h], 1).any()
        for i in range(nT):
            assert int(mask[h, i].sum()) == oracle.keep_count(i, 3, 10)


# ----------------------------------------------------------------------------- KV append pin

def test_append_then_gather_round_trip():
    """Appending then gathering a sequence token by token returns the old tokens followed by
    the new ones; rows of other sequences and unused rows are untouched."""
    rng = np.random.default_rng(3)
    P, Hkv, D, B, n_new = 16, 2, 8, 3, 21
    lens = [5, 16, 40]
    n_pages = [(L + n_new + P - 1) // P for L in lens]
    NP = sum(n_pages) + 2
    perm = rng.permutation(NP)
    pt = np.zeros((B, max(n_pages)), dtype=np.int32)
    off = 0
    for b, n in enumerate(n_pages):
        pt[b, :n] = perm[off:off + n]
        off += n
    k = rng.integers(0, 1 << 16, size=(NP, Hkv, P, D), dtype=np.uint16)
    v = rng.integers(0, 1 << 16, size=(NP, Hkv, P, D), dtype=np.uint16)
    kn = rng.integers(0, 1 << 16, size=(B, n_new, Hkv, D), dtype=np.uint16)
    vn = rng.integers(0, 1 << 16, size=(B, n_new, Hkv, D), dtype=np.uint16)
    k2, v2 = oracle.append_ref(k, v, pt, lens, kn, vn, P)
    touched = np.zeros((NP, P), dtype=bool)
    for b, L in enumerate(lens):
        old = oracle.tokens_of_sequence(k, pt[b], L, P)
        new = oracle.tokens_of_sequence(k2, pt[b], L + n_new, P)
        assert np.array_equal(new[:L], old)
        assert np.array_equal(new[L:], kn[b])
        assert np.array_equal(oracle.tokens_of_sequence(v2, pt[b], L + n_new, P)[L:], vn[b])
        for t in range(L, L + n_new):
            touched[pt[b, t // P], t % P] = True
    kt, k2t = k.transpose(0, 2, 1, 3), k2.transpose(0, 2, 1, 3)       # [NP, P, Hkv, D]
    vt, v2t = v.transpose(0, 2, 1, 3), v2.transpose(0, 2, 1, 3)
    assert np.array_equal(k2t[~touched], kt[~touched]) and np.array_equal(v2t[~touched], vt[~touched])


# ----------------------------------------------------------------------------- INT4 KV pages

def _f32_to_bf16_bits(x) -> np.ndarray:
    """bf16 bits of values that bf16 holds exactly (the test builds only such values)."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32)
    assert np.all(b & 0xFFFF == 0), "value not exact in bf16"
    return (b >> 16).astype(np.uint16)


def test_int4_hand_example_codes_bytes_and_params():
    """Row 0..15: lo 0, hi 15, scale (15 - 0)/15 = 1 -> fp16 0x3C00, zero fp16(0) = 0x0000;
    codes equal the values; each group of 8 codes n0..n7 is stored as the bytes
    (n0 | n2 << 4, n4 | n6 << 4, n1 | n3 << 4, n5 | n7 << 4): 0x20 0x64 0x31 0x75 for 0..7,
    0xA8 0xEC 0xB9 0xFD for 8..15."""
    x = _f32_to_bf16_bits(np.arange(16, dtype=np.float32))
    codes, params = oracle.quantize_int4_ref(x)
    assert codes.tolist() == list(range(16))
    assert params.tolist() == [0x3C00, 0x0000]
    packed = oracle.pack_int4(codes)
    assert packed.tolist() == [0x20, 0x64, 0x31, 0x75, 0xA8, 0xEC, 0xB9, 0xFD]
    assert np.array_equal(oracle.unpack_int4(packed), codes)
    assert np.array_equal(oracle.dequant_int4_ref(packed, params), np.arange(16, dtype=np.float64))


def test_int4_negative_range_exact_round_trip():
    """x = -3 + 0.5k, k = 0..15 in a shuffled order: scale 7.5/15 = 0.5 and zero -3 are exact
    in fp16, every value sits on a code, so the round trip is exact and code = k."""
    rng = np.random.default_rng(5)
    k = rng.permutation(16)
    xs = (-3.0 + 0.5 * k).astype(np.float32)
    codes, params = oracle.quantize_int4_ref(_f32_to_bf16_bits(xs))
    assert codes.tolist() == k.tolist()
    assert params.view(np.float16).astype(np.float64).tolist() == [0.5, -3.0]
    assert np.array_equal(oracle.dequant_int4_ref(oracle.pack_int4(codes), params), xs.astype(np.float64))


def test_int4_constant_row_has_zero_scale():
    x = _f32_to_bf16_bits(np.full(8, -1.25, dtype=np.float32))
    codes, params = oracle.quantize_int4_ref(x)
    assert codes.tolist() == [0] * 8
    assert params.view(np.float16).astype(np.float64).tolist() == [0.0, -1.25]
    assert np.array_equal(oracle.dequant_int4_ref(oracle.pack_int4(codes), params), np.full(8, -1.25))


def test_int4_codes_are_nearest_and_error_bounded():
    """Brute force over the 16 codes: each chosen code is the nearest grid point
    n*scale + zero to x (within fp32 rounding of the division), and |x - xhat| <= scale/2
    up to the fp16 rounding of the parameters."""
    rng = np.random.default_rng(6)
    xb = (rng.standard_normal((300, 64)).astype(np.float32) * rng.uniform(0.01, 20, (300, 1)).astype(np.float32))
    xb = ((xb.view(np.uint32) + 0x8000) >> 16).astype(np.uint16)          # round to bf16
    x = oracle.bf16_to_f64(xb)
    codes, params = oracle.quantize_int4_ref(xb)
    pr = params.view(np.float16).astype(np.float64)
    s, z = pr[:, 0:1], pr[:, 1:2]
    grid = np.arange(16)[None, None, :] * s[:, :, None] + z[:, :, None]   # [rows, 1, 16]
    dist = np.abs(x[:, :, None] - grid)
    chosen = np.take_along_axis(dist, codes[:, :, None].astype(np.int64), axis=2)[:, :, 0]
    assert np.all(chosen <= dist.min(axis=2) + 1e-6 * s)
    xhat = oracle.dequant_int4_ref(oracle.pack_int4(codes), params)
    assert np.all(np.abs(x - xhat) <= 0.51 * s + 1e-12)
    assert np.all((codes >= 0) & (codes <= 15))


def test_int4_cache_writes_valid_rows_only():
    """K codes and both params exactly for the valid rows; V words (8 tokens of a channel)
    exactly for the token groups holding a valid token, code 0 for the invalid tokens."""
    rng = np.random.default_rng(7)
    P, Hkv, D = 16, 2, 8
    lens = [5, 40]
    pt = np.array([[3, 0, 0], [1, 4, 2]], dtype=np.int32)
    mk = lambda: ((rng.standard_normal((5, Hkv, P, D)).astype(np.float32).view(np.uint32) + 0x8000) >> 16
                  ).astype(np.uint16)
    kb, vb = mk(), mk()
    kq, vq, kp, vp, written = oracle.quantize_cache_int4_ref(kb, vb, pt, lens, P)
    want = np.zeros((5, P), dtype=bool)
    want[3, :5] = True
    want[1, :] = True
    want[4, :] = True
    want[2, :8] = True
    assert np.array_equal(written, want)
    for a in (kq, kp, vp):
        assert not a.transpose(0, 2, 1, 3)[~want].any()
    c, p = oracle.quantize_int4_ref(kb[2, 1, 3])
    assert np.array_equal(kq[2, 1, 3], oracle.pack_int4(c)) and np.array_equal(kp[2, 1, 3], p)
    # V of page 3 (5 valid tokens): channel-major, tokens 5..7 of the first word coded 0,
    # the second word (tokens 8..15) untouched
    c, p = oracle.quantize_int4_ref(vb[3, 0, :5])                       # [5 tokens, D]
    ct = np.zeros((D, 8), dtype=np.uint8)
    ct[:, :5] = c.T
    assert np.array_equal(vq[3, 0, :, :4], oracle.pack_int4(ct)) and not vq[3, 0, :, 4:].any()
    assert np.array_equal(vp[3, 0, :5], p)
    assert np.array_equal(oracle.unpack_int4(vq[3, 0])[:, :5], c.T)


def test_int4_decode_equals_bf16_decode_on_exactly_representable_rows():
    """Rows built on an exact INT4 grid (integers 0..15 times a power of two plus an offset
    that bf16 and fp16 hold exactly, both ends present): dequantization reproduces them, so
    decode over the INT4 pages equals decode over the bf16 pages."""
    rng = np.random.default_rng(8)
    B, Hq, Hkv, D, P = 2, 4, 2, 16, 16
    lens = [40, 23]
    NP = 6
    pt = np.array([[5, 0, 3], [2, 4, 0]], dtype=np.int32)
    codes = rng.integers(0, 16, size=(NP, Hkv, P, 2, D))
    codes[..., 0] = 0
    codes[..., 1] = 15
    step = 2.0 ** rng.integers(-3, 2, size=(NP, Hkv, P, 2, 1))
    off = rng.integers(-8, 8, size=(NP, Hkv, P, 2, 1)) * 0.25
    vals = (codes * step + off).astype(np.float32)
    kb, vb = _f32_to_bf16_bits(vals[:, :, :, 0]), _f32_to_bf16_bits(vals[:, :, :, 1])
    q = ((rng.standard_normal((B, Hq, D)).astype(np.float32).view(np.uint32) + 0x8000) >> 16).astype(np.uint16)
    kq, vq, kp, vp, _ = oracle.quantize_cache_int4_ref(kb, vb, pt, lens, P)
    sel = {(0, 0): [0, 2], (1, 0): [1]}
    args = (pt, lens, Hq, Hkv, P, [0, 1], sel, 3, 7, 0.3)
    o1, l1 = oracle.decode_ref(q, kb, vb, *args)
    o2, l2 = oracle.decode_int4_ref(q, kq, vq, kp, vp, *args)
    assert np.allclose(o1, o2, rtol=0, atol=1e-12) and np.allclose(l1, l2, rtol=0, atol=1e-12)
