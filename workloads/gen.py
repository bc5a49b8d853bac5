"""Seeded synthetic inputs for unified block-sparse attention.

This module only draws random numbers and arranges them into the layouts that
the attention calls take: bf16 tensors, a paged KV cache with a page table,
per-(head, query-tile) block masks and per-sequence context lengths. It holds
none of the attention arithmetic (no softmax, no page bounds, no selection);
both the fp64 oracle and the GPU library consume what it produces.

Every tensor is drawn from its own torch.Generator seeded with
``seed * 1000 + stream`` on the requested device, so a case is reproducible on
one device type. CPU and GPU generators give different streams, so a test draws
a case once and hands the same bits to both sides.

Layouts (all contiguous):
  q (prefill)      bf16 [L, Hq, D]
  q (decode)       bf16 [B, Hq, D]
  k_cache/v_cache  bf16 [NP, Hkv, P, D]   physical page, KV head, token, channel
  page_table       int32 [n_pages] (one sequence) or [B, max_pages]
  block_mask       uint8 [Hq, nT, nT]     1 = keep KV tile j for query tile i
  seq_lens         int32 [B]
Tokens of a partially filled last page are drawn too (N(0,1) x 64) so that a
kernel that wrongly reads them is visibly wrong; they are never valid keys.
"""
from __future__ import annotations

import math

import torch

PAD_GAIN = 64.0


def generator(device, seed: int, stream: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1000 + int(stream))
    return g


def normal_bf16(shape, seed: int, stream: int, device) -> torch.Tensor:
    """i.i.d. N(0,1) drawn in fp32, rounded once to bf16 (round to nearest even)."""
    g = generator(device, seed, stream)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


def randperm(n: int, seed: int, stream: int, device) -> torch.Tensor:
    g = generator(device, seed, stream)
    return torch.randperm(n, generator=g, device=device)


def planted_keys(L: int, Hkv: int, D: int, seed: int, stream: int, device, rho: float = 0.9,
                 n_sink: int = 4, sink_gain: float = 8.0, n_col: int = 32,
                 col_gain: float = 4.0) -> torch.Tensor:
    """Keys with planted structure, bf16 [L, Hkv, D].

    Per KV head and channel a stationary AR(1) sequence along the tokens:
    k_0 = e_0 and k_t = rho * k_(t-1) + sqrt(1 - rho^2) * e_t with e i.i.d. N(0,1).
    Tokens 0..n_sink-1 are then scaled by sink_gain, and n_col distinct tokens drawn
    per KV head from [n_sink, L) by col_gain ("column" keys). The recurrence is
    evaluated in fp64 with a doubling scan (sum over s <= t of rho^(t-s) x_s).
    """
    g = generator(device, seed, stream)
    x = torch.randn((L, Hkv, D), generator=g, device=device, dtype=torch.float32).double()
    if L > 1:
        x[1:] *= math.sqrt(1.0 - rho * rho)
    a, shift = rho, 1
    while shift < L:
        x[shift:] += a * x[:-shift]
        a, shift = a * a, shift * 2
    x[:min(n_sink, L)] *= sink_gain
    span = L - n_sink
    if span > 0 and n_col > 0:
        gc = generator(device, seed, stream + 500)
        for h in range(Hkv):
            pos = torch.randperm(span, generator=gc, device=device)[:min(n_col, span)] + n_sink
            x[pos, h, :] *= col_gain
    return x.to(torch.bfloat16)


def scatter_pages(tokens: torch.Tensor, page_ids: torch.Tensor, cache: torch.Tensor, P: int,
                  seed: int, stream: int) -> None:
    """Write token-major rows [L, Hkv, D] into cache[page_ids[t // P], :, t % P, :].

    The unused tail of the last page is filled with N(0,1) x PAD_GAIN values.
    """
    L, Hkv, D = tokens.shape
    n = (L + P - 1) // P
    if n == 0:
        return
    padded = torch.empty((n * P, Hkv, D), dtype=torch.bfloat16, device=tokens.device)
    padded[:L] = tokens
    if n * P > L:
        g = generator(tokens.device, seed, stream)
        padded[L:] = (torch.randn((n * P - L, Hkv, D), generator=g, device=tokens.device)
                      * PAD_GAIN).to(torch.bfloat16)
    cache[page_ids[:n].long()] = padded.view(n, P, Hkv, D).permute(0, 2, 1, 3)


# ----------------------------------------------------------------------------- masks

def random_block_mask(Hq: int, nT: int, dense_q_heads, n_lower: int, seed: int, stream: int,
                      device, upper_junk: bool = False, streaming_fill: int = 1) -> torch.Tensor:
    """Diagonal plus n_lower strictly-lower tiles, uniform without replacement, per dense q head.

    Rows of the other heads are filled with ``streaming_fill`` (they must be ignored).
    With upper_junk, random tiles above the diagonal are set too (they must be ignored).
    """
    mask = torch.full((Hq, nT, nT), streaming_fill, dtype=torch.uint8)
    ii, jj = torch.tril_indices(nT, nT, offset=-1)
    g = generator("cpu", seed, stream)
    for h in dense_q_heads:
        mask[h].zero_()
        pick = torch.randperm(ii.numel(), generator=g)[:min(n_lower, ii.numel())]
        mask[h, ii[pick], jj[pick]] = 1
        mask[h].fill_diagonal_(1)
        if upper_junk and nT > 1:
            ui, uj = torch.triu_indices(nT, nT, offset=1)
            sel = torch.rand(ui.numel(), generator=g) < 0.5
            mask[h, ui[sel], uj[sel]] = 1
    return mask.to(device)


def meanpool_topk_mask(q: torch.Tensor, k_tokens: torch.Tensor, T: int, dense_q_heads,
                       G: int, num: int = 3, den: int = 10) -> torch.Tensor:
    """Per dense q head and query tile i: the diagonal plus the n_i - 1 strictly-lower tiles
    with the largest mean-pooled score, n_i = ceil(num*(i+1)/den).

    score[i, j] = mean over the rows of Q tile i . mean over the rows of K tile j (fp64);
    ties go to the lower j. Other heads' rows are all ones (ignored by the kernels).
    """
    L, Hq, D = q.shape
    nT = (L + T - 1) // T
    mask = torch.ones((Hq, nT, nT), dtype=torch.uint8, device=q.device)
    idx = torch.arange(nT, device=q.device)
    n_keep = (num * (idx + 1) + den - 1) // den            # includes the diagonal
    lower = idx[None, :] < idx[:, None]                     # j < i
    for h in dense_q_heads:
        gk = h // G
        qm = _tile_means(q[:, h, :], T)                     # [nT, D] fp64
        km = _tile_means(k_tokens[:, gk, :], T)
        s = qm @ km.T
        s = torch.where(lower, s, torch.full_like(s, -math.inf))
        order = torch.sort(s, dim=1, descending=True, stable=True).indices
        rank = torch.empty_like(order)
        rank.scatter_(1, order, idx.expand(nT, nT).contiguous())
        keep = (rank < (n_keep - 1)[:, None]) & lower
        keep |= torch.eye(nT, dtype=torch.bool, device=q.device)
        mask[h] = keep.to(torch.uint8)
    return mask


def _tile_means(x: torch.Tensor, T: int) -> torch.Tensor:
    L, D = x.shape
    nT = (L + T - 1) // T
    xd = x.double()
    out = torch.empty((nT, D), dtype=torch.float64, device=x.device)
    full = L // T
    if full:
        out[:full] = xd[:full * T].view(full, T, D).mean(1)
    if full < nT:
        out[full] = xd[full * T:].mean(0)
    return out


def column_slash_mask(Hq: int, nT: int, dense_q_heads, slash_tiles=(0, 1, 8, 64),
                      density_num: int = 1, density_den: int = 10, seed: int = 0,
                      stream: int = 0, device="cpu") -> torch.Tensor:
    """Slash + column block mask per dense q head.

    Every dense head keeps the tiles (i, i - o) for each tile offset o in slash_tiles,
    then whole seeded columns c (tiles (i, c) for all i >= c), drawn uniformly without
    replacement, are added until the head keeps at least round(density * nT(nT+1)/2)
    tiles. Other heads' rows are all ones (ignored by the kernels).
    """
    mask = torch.ones((Hq, nT, nT), dtype=torch.uint8)
    causal = nT * (nT + 1) // 2
    target = (2 * density_num * causal + density_den) // (2 * density_den)   # round half up
    g = generator("cpu", seed, stream)
    idx = torch.arange(nT)
    for h in dense_q_heads:
        m = torch.zeros((nT, nT), dtype=torch.bool)
        for o in slash_tiles:
            i = idx[o:]
            m[i, i - o] = True
        count = int(m.sum())
        for c in torch.randperm(nT, generator=g).tolist():
            if count >= target:
                break
            col = m[c:, c]
            count += int((~col).sum())
            m[c:, c] = True
        mask[h] = m.to(torch.uint8)
    return mask.to(device)
