"""GPU parity of append_kv: new tokens land where the paged layout puts them (bit-exact
against the oracle's append), nothing else in the cache changes, and the refreshed page
bounds equal the oracle's bounds of the longer sequences on every sub-page (bit-exact)."""
import numpy as np
import pytest
import torch

import oracle
import unified_block_sparse_amd as ubs
from tests.helpers import bits
from workloads import cases, gen

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _setup(final_lens, n_new, P, Lp, seed):
    kind = [0, 0, 1, 1]
    d = cases.make_decode("append", final_lens, 16, 4, 128, P, Lp, kind, 4 * P, 32, 64, seed, DEV, planted=True)
    old = [L - n_new for L in final_lens]
    return d, kind, old


def _gather_new(cache, d, old, n_new):
    """The rows of tokens old[b] .. old[b] + n_new - 1 of every sequence: [B, n_new, Hkv, D]."""
    rows = []
    for b, L0 in enumerate(old):
        t = torch.arange(L0, L0 + n_new, device=DEV)
        pg = d.page_table[b, (t // d.P).long()].long()
        rows.append(cache[pg, :, (t % d.P).long(), :])
    return torch.stack(rows).contiguous()


@pytest.mark.parametrize("n_new,P,Lp", [(1, 64, 16), (37, 64, 16), (69, 32, 32), (5, 16, 16)])
def test_append_matches_oracle(n_new, P, Lp):
    final = [300, 64 + n_new, 2000]
    d, kind, old = _setup(final, n_new, P, Lp, 2201)
    k_new, v_new = _gather_new(d.k_cache, d, old, n_new), _gather_new(d.v_cache, d, old, n_new)
    # the cache before the append: the new tokens' rows hold other data
    k0, v0 = d.k_cache.clone(), d.v_cache.clone()
    noise = gen.normal_bf16(k0.shape, 2202, 1, DEV)
    for b, L0 in enumerate(old):
        t = torch.arange(L0, L0 + n_new, device=DEV)
        pg = d.page_table[b, (t // d.P).long()].long()
        k0[pg, :, (t % d.P).long(), :] = noise[pg, :, (t % d.P).long(), :]
        v0[pg, :, (t % d.P).long(), :] = noise[pg, :, (t % d.P).long(), :]
    k_cache, v_cache = k0.clone(), v0.clone()
    old_t = torch.tensor(old, dtype=torch.int32, device=DEV)
    bnd = ubs.build_page_bounds(k_cache, d.page_table, old_t, kind, Lp)
    bnd_before = bnd.clone()
    ubs.append_kv(k_new, v_new, d.page_table, old_t, kind, k_cache, v_cache, bounds=bnd, Lp=Lp)
    torch.cuda.synchronize(DEV)
    pt = d.page_table.cpu().numpy()
    ko, vo = oracle.append_ref(bits(k0), bits(v0), pt, old, bits(k_new), bits(v_new), P)
    assert np.array_equal(bits(k_cache), ko) and np.array_equal(bits(v_cache), vo)
    vals, defined = oracle.bounds_ref(ko, pt, final, P, Lp, kind)
    got = oracle.bf16_to_f64(bits(bnd))
    assert np.array_equal(got[defined], vals[defined])
    # sub-pages without a new token keep their old bounds
    _, defined_old = oracle.bounds_ref(bits(k0), pt, old, P, Lp, kind)
    touched = np.zeros_like(defined)
    U = P // Lp
    for b, L0 in enumerate(old):
        for t in range(L0, L0 + n_new):
            touched[pt[b, t // P], :, (t % P) // Lp] = True
    keep = defined_old & ~touched
    assert np.array_equal(bits(bnd)[keep], bits(bnd_before)[keep])


def test_append_decode_loop_keeps_bounds_exact():
    """Twenty single-token appends (a decode loop): the bounds they leave equal the oracle's
    bounds of the final sequences bit for bit (and so equal one full build)."""
    n_steps = 20
    final = [1000, 129, 64 * 7]
    d, kind, old = _setup(final, n_steps, 64, 16, 2203)
    k_full, v_full = d.k_cache.clone(), d.v_cache.clone()
    lens = torch.tensor(old, dtype=torch.int32, device=DEV)
    bnd = ubs.build_page_bounds(d.k_cache, d.page_table, lens, kind, 16)
    for s in range(n_steps):
        cur = [L0 + s for L0 in old]
        kn, vn = _gather_new(k_full, d, cur, 1), _gather_new(v_full, d, cur, 1)
        ubs.append_kv(kn, vn, d.page_table, lens, kind, d.k_cache, d.v_cache, bounds=bnd, Lp=16)
        lens += 1
    torch.cuda.synchronize(DEV)
    assert lens.cpu().tolist() == final
    pt = d.page_table.cpu().numpy()
    assert np.array_equal(bits(d.k_cache), bits(k_full)) and np.array_equal(bits(d.v_cache), bits(v_full))
    vals, defined = oracle.bounds_ref(bits(k_full), pt, final, 64, 16, kind)
    got = oracle.bf16_to_f64(bits(bnd))
    assert defined.any() and np.array_equal(got[defined], vals[defined])
