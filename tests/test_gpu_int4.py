"""INT4 KV pages on the GPU against the oracle: quantize_kv_int4 bit-exact (codes and
fp16 params of every valid row; other rows untouched), sparse_decode_int4 on the
oracle's codes and selection within the attention tolerance, and both at the ragged
serving shape on all of its sequences."""
import numpy as np
import pytest
import torch

import oracle
import unified_block_sparse_amd as ubs
from tests.gpu_cases import assert_attention_close, assert_lse_close, decode_subset
from tests.helpers import bits
from workloads import cases

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _sync():
    torch.cuda.synchronize(DEV)


def _u8(t):
    return t.cpu().numpy().astype(np.uint8)


def _u16(t):
    return t.cpu().numpy().view(np.uint16)


QUANT_CASES = [
    # lens, Hkv, D, P
    ([37, 16, 1, 50, 0, 300], 2, 128, 16),
    ([2000, 1500, 64], 4, 64, 64),
    ([500, 4000], 2, 128, 32),
    ([1000, 129, 5000], 4, 64, 128),
    ([777], 8, 128, 256),
]


@pytest.mark.parametrize("lens,Hkv,D,P", QUANT_CASES)
def test_quantize_int4_bit_exact(lens, Hkv, D, P):
    c = cases.make_decode("q4", lens, 2 * Hkv, Hkv, D, P, P, [0] * Hkv, P, 1, 1, 51, DEV, planted=True,
                          extra_pages=3)
    NP = c.k_cache.shape[0]
    sentinel = (torch.full((NP, Hkv, P, D // 2), 0xA5, dtype=torch.uint8, device=DEV),
                torch.full((NP, Hkv, D, P // 2), 0x5A, dtype=torch.uint8, device=DEV),
                torch.full(c.k_cache.shape[:3] + (2,), 0x1234, dtype=torch.int16, device=DEV),
                torch.full(c.k_cache.shape[:3] + (2,), 0x4321, dtype=torch.int16, device=DEV))
    kc, vc, kp, vp = ubs.quantize_kv_int4(c.k_cache, c.v_cache, c.page_table, c.seq_lens_t, out=sentinel)
    _sync()
    pt = c.page_table.cpu().numpy()
    rkq, rvq, rkp, rvp, written = oracle.quantize_cache_int4_ref(bits(c.k_cache), bits(c.v_cache), pt, c.seq_lens, P)
    tr = lambda x: x.transpose(0, 2, 1, 3)               # [NP, P, Hkv, ...]
    for got, ref, fill, what in ((_u8(kc), rkq, 0xA5, "k codes"), (_u16(kp), rkp, 0x1234, "k params"),
                                 (_u16(vp), rvp, 0x4321, "v params")):
        assert np.array_equal(tr(got)[written], tr(ref)[written]), f"{what} differ"
        assert np.all(tr(got)[~written] == fill), f"{what}: rows outside the sequences touched"
    # V words: written where a word holds a valid token, untouched elsewhere
    gv = _u8(vc).reshape(NP, Hkv, D, P // 8, 4)
    wv = written.reshape(NP, P // 8, 8).any(axis=2)      # [NP, words]
    rv = rvq.reshape(NP, Hkv, D, P // 8, 4)
    sel = np.broadcast_to(wv[:, None, None, :], gv.shape[:4])
    assert np.array_equal(gv[sel], rv[sel]), "v codes differ"
    assert np.all(gv[~sel] == 0x5A), "v words outside the sequences touched"


def test_quantize_int4_half_integer_quotients():
    """Rows whose quotients (x - zero) / scale fall exactly on half-integers, and just
    beside them: every row spans [0, 15] (scale 1, zero 0) and holds k + 0.5 for every
    k < 15 (exact in bf16) and k + 0.5 -/+ 1/64 (rounded to bf16: beside the tie, or onto
    it), so rint's ties (to even) occur many times a row. Codes and params bit-exact
    against the oracle."""
    P, D, Hkv, L = 16, 128, 2, 16
    k = torch.arange(D, dtype=torch.float32)
    ties = (k % 15) + 0.5                                  # 0.5 .. 14.5
    row = torch.where(k % 3 == 0, ties, torch.where(k % 3 == 1, ties - 1 / 64, ties + 1 / 64))
    row[0], row[1] = 0.0, 15.0                             # the row's range: scale 1, zero 0
    rows = torch.stack([torch.roll(row, int(r)) for r in range(P)])       # [P, D], each a permutation
    cache = rows.to(torch.bfloat16).reshape(1, 1, P, D).repeat(1, Hkv, 1, 1).contiguous().to(DEV)
    pt = torch.zeros((1, 1), dtype=torch.int32, device=DEV)
    lens = torch.tensor([L], dtype=torch.int32, device=DEV)
    kc, vc, kp, vp = ubs.quantize_kv_int4(cache, cache, pt, lens)
    _sync()
    rkq, rvq, rkp, rvp, written = oracle.quantize_cache_int4_ref(bits(cache), bits(cache), pt.cpu().numpy(), [L], P)
    assert written.all()
    assert np.array_equal(_u8(kc), rkq) and np.array_equal(_u8(vc), rvq), "codes differ"
    assert np.array_equal(_u16(kp), rkp) and np.array_equal(_u16(vp), rvp), "params differ"


@pytest.mark.parametrize("D", [64, 128])
def test_quantize_int4_edge_rows(D):
    """Rows at the edges of the format (finite values whose range / 15 fits fp16), codes
    and params bit-exact against the oracle: a minimum below -65504 (zero = -inf, every
    code 15) or above it (zero = +inf, every code 0), constant rows (scale 0, every code
    0) with a finite and an infinite zero, and values in fp16's subnormal range (zero
    rounds above the minimum, so that row's quotient is negative and clamps to 0). The
    first eight rows hold the extreme ones; at D = 128 the next eight, ordinary and
    subnormal rows, fill another wave of their own."""
    P, Hkv, L = 16, 2, 16
    gen = torch.Generator().manual_seed(61)
    u = torch.rand((P, D), generator=gen, dtype=torch.float64)
    z = torch.randn((P, D), generator=gen, dtype=torch.float64)
    rows = torch.stack([
        -70000 + 10000 * u[0], 66000 + 4000 * u[1], torch.full((D,), 70000.0), torch.full((D,), -1.5),
        -80000 + 100 * u[4], 65600 + 10 * u[5], torch.full((D,), -66000.0), z[7],
        1e-7 + 3e-6 * u[8], 1e-7 + 3e-6 * u[9], z[10], 3 * z[11], torch.full((D,), 2.0 ** -24),
        1e-6 * z[13], 0.01 * z[14], z[15]])
    cache = rows.to(torch.bfloat16).reshape(1, 1, P, D).repeat(1, Hkv, 1, 1).contiguous().to(DEV)
    pt = torch.zeros((1, 1), dtype=torch.int32, device=DEV)
    lens = torch.tensor([L], dtype=torch.int32, device=DEV)
    kc, vc, kp, vp = ubs.quantize_kv_int4(cache, cache, pt, lens)
    _sync()
    with np.errstate(over="ignore", invalid="ignore"):
        rkq, rvq, rkp, rvp, written = oracle.quantize_cache_int4_ref(bits(cache), bits(cache), pt.cpu().numpy(),
                                                                     [L], P)
    assert written.all()
    assert np.array_equal(_u8(kc), rkq) and np.array_equal(_u8(vc), rvq), "codes differ"
    assert np.array_equal(_u16(kp), rkp) and np.array_equal(_u16(vp), rvp), "params differ"
    # the rows mean what the docstring says (a check of the inputs)
    codes = oracle.unpack_int4(rkq[0, 0])
    assert (codes[0] == 15).all() and (codes[1] == 0).all() and (codes[2] == 0).all() and (codes[3] == 0).all()


DECODE4_CASES = [
    # lens, Hq, Hkv, D, P, Lp, head_kind, budget, sink, local
    ([37, 16, 1, 50, 0, 300], 8, 2, 128, 16, 4, [0, 1], 4 * 16, 5, 20),
    ([2000, 1500, 64], 32, 4, 64, 64, 16, [0, 1, 0, 1], 8 * 64, 64, 100),
    ([500, 4000], 32, 2, 128, 32, 32, [1, 0], 4 * 32, 0, 64),
    ([1000, 129, 5000], 4, 4, 64, 128, 8, [0, 0, 1, 0], 3 * 128, 128, 1024),
    ([20000, 777], 16, 2, 128, 64, 16, [1, 0], 64 * 64, 100, 3000),
    ([3000, 20], 2, 2, 128, 16, 16, [0, 1], 16 * 16, 7, 33),
    # 16-row units that straddle pages (P = 48, 80: not powers of two), G = 1 with D = 64,
    # G = 16 over 256-token pages with a long local window
    ([3000, 1234, 77], 16, 4, 128, 48, 16, [0, 1, 1, 0], 10 * 48, 40, 200),
    ([9000, 300], 8, 8, 64, 80, 16, [0, 1, 0, 1, 0, 1, 0, 1], 7 * 80, 16, 500),
    ([40000], 64, 4, 128, 256, 64, [0, 1, 0, 0], 20 * 256, 256, 2048),
]


def _sel_tensors(sel_o, B, Hkv, k):
    sel_t = torch.full((B, Hkv, k), -1, dtype=torch.int32)
    num_t = torch.zeros((B, Hkv), dtype=torch.int32)
    for (b, g), s in sel_o.items():
        sel_t[b, g, :len(s)] = torch.tensor(s, dtype=torch.int32)
        num_t[b, g] = len(s)
    return sel_t.to(DEV), num_t.to(DEV)


@pytest.mark.parametrize("lens,Hq,Hkv,D,P,Lp,hk,budget,sink,local", DECODE4_CASES)
def test_decode_int4_matches_oracle(lens, Hq, Hkv, D, P, Lp, hk, budget, sink, local):
    c = cases.make_decode("d4", lens, Hq, Hkv, D, P, Lp, hk, budget, sink, local, 52, DEV, planted=True)
    pt = c.page_table.cpu().numpy()
    kq, vq, kp, vp, _ = oracle.quantize_cache_int4_ref(bits(c.k_cache), bits(c.v_cache), pt, lens, P)
    sel_o, _ = oracle.select_ref(bits(c.q), bits(c.k_cache), pt, lens, Hq, Hkv, P, Lp, budget, hk)
    sel_t, num_t = _sel_tensors(sel_o, c.B, Hkv, budget // P)
    dev = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).view(dt).to(DEV)
    out, lse = ubs.sparse_decode_int4(c.q, dev(kq, torch.uint8), dev(vq, torch.uint8), dev(kp, torch.int16),
                                      dev(vp, torch.int16), c.page_table, c.seq_lens_t, hk, sel_t, num_t, sink,
                                      local, c.sm_scale, return_lse=True)
    _sync()
    ref, ref_lse = oracle.decode_int4_ref(bits(c.q), kq, vq, kp, vp, pt, lens, Hq, Hkv, P, hk, sel_o, sink, local,
                                          c.sm_scale)
    assert_attention_close(out.cpu().numpy(), ref, "decode_int4 out")
    assert_lse_close(lse.cpu().numpy(), ref_lse, "decode_int4 lse")


def test_int4_pipeline_close_to_bf16_decode():
    """Quantize on the GPU, select, decode the INT4 pages, against the bf16 decode on the
    same selection. This measures the format's rounding (per-row 4-bit steps of
    range/15 perturb every score), not parity, which the tests above check; on these
    planted keys the mean difference is about 0.09 and the largest about 1.2."""
    c = cases.make_decode("p4", [3000, 9000, 513], 32, 8, 128, 64, 16, [0, 0, 0, 0, 1, 1, 1, 1], 16 * 64, 64, 512,
                          53, DEV, planted=True)
    kc, vc, kp, vp = ubs.quantize_kv_int4(c.k_cache, c.v_cache, c.page_table, c.seq_lens_t)
    bnd = ubs.build_page_bounds(c.k_cache, c.page_table, c.seq_lens_t, c.head_kind, c.Lp)
    sel, num = ubs.select_pages(c.q, bnd, c.page_table, c.seq_lens_t, c.head_kind, c.P, c.token_budget)
    o16 = ubs.sparse_decode(c.q, c.k_cache, c.v_cache, c.page_table, c.seq_lens_t, c.head_kind, sel, num,
                            c.sink_tokens, c.local_tokens, c.sm_scale)
    o4 = ubs.sparse_decode_int4(c.q, kc, vc, kp, vp, c.page_table, c.seq_lens_t, c.head_kind, sel, num,
                                c.sink_tokens, c.local_tokens, c.sm_scale)
    _sync()
    d = (o4 - o16).abs()
    assert torch.isfinite(o4).all()
    print(f"int4 vs bf16 decode: mean-abs {d.mean().item():.3e}, max-abs {d.max().item():.3e}")
    assert d.mean().item() < 0.2 and d.max().item() < 3.0, (d.mean().item(), d.max().item())


@pytest.fixture(scope="module")
def ragged_int4():
    c = cases.decode_ragged(DEV)
    kc, vc, kp, vp = ubs.quantize_kv_int4(c.k_cache, c.v_cache, c.page_table, c.seq_lens_t)
    _sync()
    yield c, kc, vc, kp, vp
    del c, kc, vc, kp, vp
    torch.cuda.empty_cache()


@pytest.mark.parametrize("part", range(4))
def test_int4_ragged_every_sequence(ragged_int4, part):
    """All 64 sequences of decode_ragged, 16 per test: codes and params bit-exact, decode
    over the oracle's codes and selection within the attention tolerance."""
    c, kc, vc, kp, vp = ragged_int4
    n = c.B // 4
    batches = list(range(part * n, (part + 1) * n))
    qb, kb, vb, pt, lens = decode_subset(c, batches)
    kq, vq, kpr, vpr, written = oracle.quantize_cache_int4_ref(kb, vb, pt, lens, c.P)
    pages = torch.tensor([int(c.page_table[b, j]) for b in batches for j in range((c.seq_lens[b] + c.P - 1) // c.P)],
                         device=DEV)
    assert np.array_equal(_u8(kc[pages]), kq) and np.array_equal(_u16(kp[pages]), kpr.view(np.uint16))
    wv = np.broadcast_to(written.reshape(-1, c.P // 8, 8).any(axis=2)[:, None, None, :],
                         (len(pages), c.Hkv, c.D, c.P // 8))
    gv = _u8(vc[pages]).reshape(len(pages), c.Hkv, c.D, c.P // 8, 4)
    assert np.array_equal(gv[wv], vq.reshape(gv.shape)[wv]) and np.array_equal(_u16(vp[pages]), vpr.view(np.uint16))
    sel_o, _ = oracle.select_ref(qb, kb, pt, lens, c.Hq, c.Hkv, c.P, c.Lp, c.token_budget, c.head_kind)
    sel_t = torch.full((c.B, c.Hkv, c.k_pages), -1, dtype=torch.int32, device=DEV)
    num_t = torch.zeros((c.B, c.Hkv), dtype=torch.int32, device=DEV)
    for (i, g), s in sel_o.items():
        row = torch.full((c.k_pages,), -1, dtype=torch.int32)
        row[:len(s)] = torch.tensor(s, dtype=torch.int32)
        sel_t[batches[i], g] = row.to(DEV)
        num_t[batches[i], g] = len(s)
    out, lse = ubs.sparse_decode_int4(c.q, kc, vc, kp, vp, c.page_table, c.seq_lens_t, c.head_kind, sel_t, num_t,
                                      c.sink_tokens, c.local_tokens, c.sm_scale, return_lse=True)
    _sync()
    ref, ref_lse = oracle.decode_int4_ref(qb, kq, vq, kpr, vpr, pt, lens, c.Hq, c.Hkv, c.P, c.head_kind, sel_o,
                                          c.sink_tokens, c.local_tokens, c.sm_scale)
    bi = torch.tensor(batches, device=DEV)
    assert_attention_close(out[bi].cpu().numpy(), ref, "decode_int4 ragged")
    assert_lse_close(lse[bi].cpu().numpy(), ref_lse, "decode_int4 ragged lse")
