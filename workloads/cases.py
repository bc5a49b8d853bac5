"""Case builders: the five workload shapes and small unit cases.

A case is a plain dataclass of parameters plus the tensors drawn by ``gen``.
Nothing here computes attention, bounds or selections.

The five named workloads (seed = 1000 + index):
  prefill_tiny      L=1024, Hq=Hkv=4, D=64, T=64; heads 0-1 random 50% block mask
                    (diagonal + 52 of 120 strictly-lower tiles); heads 2-3 streaming,
                    1 sink tile + 4 local tiles; Q/K/V N(0,1); scale 1/8.
  decode_llama8b    B=4, L=32768, Hq=32, Hkv=8, D=128, P=Lp=64, permuted pages;
                    KV heads 0-3 dense (budget 4096 tokens), 4-7 streaming (128 sink +
                    512 local tokens); Q/K/V N(0,1).
  prefill_llama8b   L=65536, Hq=32, Hkv=8, D=128, T=128, P=64; planted K; dense KV heads
                    0-3 use the mean-pooled Q.K top-30% mask, KV heads 4-7 stream with
                    1 sink tile + 8 local tiles.
  decode_ragged     B=64, L_b uniform in [16384, 131072], Hq=32, Hkv=8, D=128, P=64,
                    Lp=16; planted K per sequence; budget 4096; streaming 128 + 1024.
  prefill_extreme   L=262144, Hq=64, Hkv=8, D=128, T=128, P=64; planted K; dense KV
                    heads 0-3 use slash offsets {0,1,8,64} tiles + seeded columns to 10%
                    density; KV heads 4-7 stream with 1 sink tile + 16 local tiles.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import torch

from . import gen


@dataclasses.dataclass
class PrefillCase:
    name: str
    L: int
    Hq: int
    Hkv: int
    D: int
    T: int
    P: int
    head_kind: List[int]            # per KV head: 0 dense, 1 streaming
    sink_tiles: int
    local_tiles: int
    sm_scale: float
    q: Optional[torch.Tensor] = None          # bf16 [L, Hq, D]
    k_cache: Optional[torch.Tensor] = None    # bf16 [NP, Hkv, P, D]
    v_cache: Optional[torch.Tensor] = None
    page_table: Optional[torch.Tensor] = None  # int32 [n_pages]
    block_mask: Optional[torch.Tensor] = None  # uint8 [Hq, nT, nT]
    k_tok: Optional[torch.Tensor] = None       # bf16 [L, Hkv, D] (keep_tokens only)
    v_tok: Optional[torch.Tensor] = None

    @property
    def G(self):
        return self.Hq // self.Hkv

    @property
    def nT(self):
        return (self.L + self.T - 1) // self.T

    @property
    def n_pages(self):
        return (self.L + self.P - 1) // self.P


@dataclasses.dataclass
class DecodeCase:
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    P: int
    Lp: int
    head_kind: List[int]
    token_budget: int
    sink_tokens: int
    local_tokens: int
    sm_scale: float
    seq_lens: List[int]
    max_pages: int
    q: Optional[torch.Tensor] = None           # bf16 [B, Hq, D]
    k_cache: Optional[torch.Tensor] = None     # bf16 [NP, Hkv, P, D]
    v_cache: Optional[torch.Tensor] = None
    page_table: Optional[torch.Tensor] = None  # int32 [B, max_pages]
    seq_lens_t: Optional[torch.Tensor] = None  # int32 [B]
    k_tok: Optional[list] = None               # per sequence bf16 [L_b, Hkv, D] (keep_tokens only)
    v_tok: Optional[list] = None

    @property
    def G(self):
        return self.Hq // self.Hkv

    @property
    def k_pages(self):
        return self.token_budget // self.P

    @property
    def num_physical_pages(self):
        return int(self.k_cache.shape[0])


def _streaming_upper_half(Hkv: int) -> List[int]:
    return [0] * (Hkv // 2) + [1] * (Hkv - Hkv // 2)


# ----------------------------------------------------------------------------- prefill

def make_prefill(name: str, L: int, Hq: int, Hkv: int, D: int, T: int, P: int, head_kind,
                 sink_tiles: int, local_tiles: int, mask: str, seed: int, device,
                 planted: bool = False, mask_arg=None, sm_scale: Optional[float] = None,
                 extra_pages: int = 0, upper_junk: bool = False,
                 keep_tokens: bool = False) -> PrefillCase:
    """Draw a single-sequence prefill case.

    mask: "random" (mask_arg = number of strictly-lower tiles per dense head),
          "all" (every causal tile), "diag" (diagonal only), "meanpool" (top-30% rule),
          "colslash" (slash + columns to 10%).
    extra_pages: unused physical pages appended to the cache (never referenced).
    """
    c = PrefillCase(name, L, Hq, Hkv, D, T, P, list(head_kind), sink_tiles, local_tiles,
                    sm_scale if sm_scale is not None else 1.0 / math.sqrt(D))
    G = c.G
    n_pages = c.n_pages
    NP = n_pages + extra_pages
    c.q = gen.normal_bf16((L, Hq, D), seed, 1, device)
    if planted:
        k_tok = gen.planted_keys(L, Hkv, D, seed, 2, device)
    else:
        k_tok = gen.normal_bf16((L, Hkv, D), seed, 2, device)
    v_tok = gen.normal_bf16((L, Hkv, D), seed, 3, device)
    perm = gen.randperm(NP, seed, 4, device)
    c.page_table = perm[:n_pages].to(torch.int32).contiguous()
    c.k_cache = gen.normal_bf16((NP, Hkv, P, D), seed, 5, device)   # unreferenced pages: noise
    c.v_cache = gen.normal_bf16((NP, Hkv, P, D), seed, 6, device)
    gen.scatter_pages(k_tok, c.page_table, c.k_cache, P, seed, 7)
    gen.scatter_pages(v_tok, c.page_table, c.v_cache, P, seed, 8)
    if keep_tokens:
        c.k_tok, c.v_tok = k_tok, v_tok
    dense_q = [h for h in range(Hq) if head_kind[h // G] == 0]
    nT = c.nT
    if mask == "random":
        c.block_mask = gen.random_block_mask(Hq, nT, dense_q, int(mask_arg), seed, 9, device,
                                             upper_junk=upper_junk)
    elif mask == "all":
        c.block_mask = torch.ones((Hq, nT, nT), dtype=torch.uint8, device=device)
    elif mask == "diag":
        m = torch.eye(nT, dtype=torch.uint8).expand(Hq, nT, nT).contiguous()
        c.block_mask = m.to(device)
    elif mask == "meanpool":
        c.block_mask = gen.meanpool_topk_mask(c.q, k_tok, T, dense_q, G)
    elif mask == "colslash":
        c.block_mask = gen.column_slash_mask(Hq, nT, dense_q, seed=seed, stream=9, device=device)
    else:
        raise ValueError(mask)
    c.block_mask = c.block_mask.contiguous()
    return c


def prefill_tiny(device, seed: int = 1001) -> PrefillCase:
    return make_prefill("prefill_tiny", 1024, 4, 4, 64, 64, 64, [0, 0, 1, 1], 1, 4,
                        "random", seed, device, mask_arg=52, sm_scale=1.0 / 8.0)


def prefill_llama8b(device, seed: int = 1003) -> PrefillCase:
    return make_prefill("prefill_llama8b", 65536, 32, 8, 128, 128, 64, _streaming_upper_half(8),
                        1, 8, "meanpool", seed, device, planted=True)


def prefill_extreme(device, seed: int = 1005) -> PrefillCase:
    return make_prefill("prefill_extreme", 262144, 64, 8, 128, 128, 64, _streaming_upper_half(8),
                        1, 16, "colslash", seed, device, planted=True)


# ----------------------------------------------------------------------------- decode

def make_decode(name: str, seq_lens, Hq: int, Hkv: int, D: int, P: int, Lp: int, head_kind,
                token_budget: int, sink_tokens: int, local_tokens: int, seed: int, device,
                planted: bool = False, sm_scale: Optional[float] = None,
                extra_pages: int = 0, max_pages: Optional[int] = None,
                keep_tokens: bool = False) -> DecodeCase:
    """Draw a batched decode case with a seeded random page table.

    Physical pages are a random permutation of all pages the batch needs (plus
    extra_pages never referenced); sequence b takes the next ceil(L_b/P) of them.
    Unused page-table slots hold 0 (a valid id that must never be read).
    """
    B = len(seq_lens)
    n_b = [(int(L) + P - 1) // P for L in seq_lens]
    mp = max(max(n_b), 1) if max_pages is None else max_pages
    c = DecodeCase(name, B, Hq, Hkv, D, P, Lp, list(head_kind), token_budget, sink_tokens,
                   local_tokens, sm_scale if sm_scale is not None else 1.0 / math.sqrt(D),
                   [int(x) for x in seq_lens], mp)
    NP = sum(n_b) + extra_pages
    c.q = gen.normal_bf16((B, Hq, D), seed, 1, device)
    perm = gen.randperm(max(NP, 1), seed, 4, device).to(torch.int32)
    pt = torch.zeros((B, mp), dtype=torch.int32, device=device)
    off = 0
    for b in range(B):
        pt[b, :n_b[b]] = perm[off:off + n_b[b]]
        off += n_b[b]
    c.page_table = pt.contiguous()
    c.seq_lens_t = torch.tensor(c.seq_lens, dtype=torch.int32, device=device)
    c.k_cache = torch.empty((max(NP, 1), Hkv, P, D), dtype=torch.bfloat16, device=device)
    c.v_cache = torch.empty_like(c.k_cache)
    if extra_pages or NP == 0:
        c.k_cache.copy_(gen.normal_bf16(c.k_cache.shape, seed, 5, device))
        c.v_cache.copy_(gen.normal_bf16(c.v_cache.shape, seed, 6, device))
    if keep_tokens:
        c.k_tok, c.v_tok = [], []
    for b in range(B):
        L = c.seq_lens[b]
        if L == 0:
            if keep_tokens:
                c.k_tok.append(torch.zeros((0, Hkv, D), dtype=torch.bfloat16))
                c.v_tok.append(torch.zeros((0, Hkv, D), dtype=torch.bfloat16))
            continue
        if planted:
            k_tok = gen.planted_keys(L, Hkv, D, seed, 100 + 4 * b, device)
        else:
            k_tok = gen.normal_bf16((L, Hkv, D), seed, 100 + 4 * b, device)
        v_tok = gen.normal_bf16((L, Hkv, D), seed, 101 + 4 * b, device)
        gen.scatter_pages(k_tok, pt[b], c.k_cache, P, seed, 102 + 4 * b)
        gen.scatter_pages(v_tok, pt[b], c.v_cache, P, seed, 103 + 4 * b)
        if keep_tokens:
            c.k_tok.append(k_tok)
            c.v_tok.append(v_tok)
        del k_tok, v_tok
    return c


def decode_llama8b(device, seed: int = 1002) -> DecodeCase:
    return make_decode("decode_llama8b", [32768] * 4, 32, 8, 128, 64, 64, _streaming_upper_half(8),
                       4096, 128, 512, seed, device)


def ragged_lengths(B: int, lo: int, hi: int, seed: int) -> List[int]:
    g = gen.generator("cpu", seed, 50)
    return torch.randint(lo, hi + 1, (B,), generator=g).tolist()


def decode_ragged(device, seed: int = 1004) -> DecodeCase:
    lens = ragged_lengths(64, 16384, 131072, seed)
    return make_decode("decode_ragged", lens, 32, 8, 128, 64, 16, _streaming_upper_half(8),
                       4096, 128, 1024, seed, device, planted=True)
