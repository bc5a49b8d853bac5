"""Plain fp64 CPU oracle for LServe-style unified block-sparse attention.

TEST INFRASTRUCTURE ONLY. Only the tests, ``__graft_entry__.smoke()`` and the
bench's cpu_baseline leg may import this module. The library path never calls
it, and it shares no code with the GPU kernels or their bindings.

Inputs are raw bf16 bit patterns (numpy uint16) and int arrays exactly as the
GPU receives them; bf16 is decoded exactly to fp64 and everything after that is
fp64 NumPy. Sources (the LServe pages):

* "LServe: Efficient Long-sequence LLM Serving with Unified Sparse Attention"
  (arXiv 2502.14866), abstract: half the heads become streaming heads in both
  prefill and decode; a constant number of KV pages suffices; a hierarchical,
  query-centric page selector prunes pages; less important tokens are skipped
  block-wise.
* "LServe + SampleAttention" blog, sections "LServe -- Prefill Phase" (Figure 1)
  and "LServe -- Decode Phase" (Figure 2): a KV tile is computed or skipped whole
  at kernel-tile granularity; a streaming head keeps sink tokens plus a local
  window (the Lambda shape); decode scores every page from a per-page summary,
  keeps the top-k and attends token by token inside the kept pages.

The page bound sum_c max(q_c*kmin_c, q_c*kmax_c) is the query-aware bound of
Quest (cited by the LServe paper); the pages call it only "a summary vector per
page". Readings taken where the pages are silent are listed in each docstring.

Every function here is pinned by a test in tests/test_oracle.py.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np


# ----------------------------------------------------------------------------- helpers

def bf16_to_f64(bits) -> np.ndarray:
    """Exact decode of bf16 bit patterns: the 16 bits are the top half of an fp32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def tokens_of_sequence(cache: np.ndarray, page_row: np.ndarray, L: int, P: int,
                       token_idx: Optional[np.ndarray] = None) -> np.ndarray:
    """Token-major view of one sequence of a paged cache.

    cache is [NP, Hkv, P, D]; token t of the sequence lives at
    cache[page_row[t // P], :, t % P, :] (PagedAttention layout). Returns [n, Hkv, D].
    """
    t = np.arange(L) if token_idx is None else np.asarray(token_idx, dtype=np.int64)
    return cache[np.asarray(page_row, dtype=np.int64)[t // P], :, t % P, :]


def _softmax_attend(s: np.ndarray, v: np.ndarray) -> Tuple[np.ndarray, float]:
    """out = sum_c softmax(s)_c v_c with max subtraction; lse = ln sum_c exp(s_c)."""
    if s.size == 0:
        return np.zeros(v.shape[-1]), -math.inf
    m = s.max()
    p = np.exp(s - m)
    l = p.sum()
    return (p @ v) / l, m + math.log(l)


# ----------------------------------------------------------------------------- prefill

def prefill_kept_tiles(i: int, streaming: bool, mask_row, sink_tiles: int,
                       local_tiles: int) -> List[int]:
    """KV tiles kept for query tile i (blog, Prefill section and Figure 1).

    Dense head: the tiles j <= i whose mask entry is set (entries above the diagonal
    are ignored; causality always holds). Streaming head (Lambda shape): the first
    sink_tiles tiles plus the local_tiles most recent tiles, the diagonal tile counted
    among the local ones; the tiles in between are never visited.
    """
    if streaming:
        return [j for j in range(i + 1) if j < sink_tiles or j > i - local_tiles]
    return [j for j in range(i + 1) if mask_row[j]]


def prefill_ref(q_bits, k_cache_bits, v_cache_bits, page_table, L: int, Hq: int, Hkv: int,
                D: int, P: int, T: int, head_kind, block_mask, sink_tiles: int,
                local_tiles: int, sm_scale: float, rows: Optional[Sequence[int]] = None,
                heads: Optional[Sequence[int]] = None):
    """Block-sparse / Lambda causal attention of one sequence, fp64.

    Query row r of head h (KV head g = h // (Hq/Hkv)) attends to the keys
    K(r) = { c <= r : c // T is a kept tile of (h, r // T) }:
      out[r, h] = sum_{c in K(r)} softmax_c(sm_scale * q_r . k_c) v_c,
      lse[h, r] = ln sum_{c in K(r)} exp(sm_scale * q_r . k_c).
    Only the diagonal tile is cut at token level (c <= r); every other kept tile
    enters whole. A row with no key gets out = 0 and lse = -inf.

    rows/heads restrict the evaluation (default: all). Returns (out, lse) with
    out [n_rows, n_heads, D] and lse [n_heads, n_rows] in the order given.
    """
    G = Hq // Hkv
    rows = list(range(L)) if rows is None else [int(r) for r in rows]
    heads = list(range(Hq)) if heads is None else [int(h) for h in heads]
    # gather the sequence's tokens first, then decode only those (exact either way)
    K = bf16_to_f64(tokens_of_sequence(np.asarray(k_cache_bits), page_table, L, P))  # [L, Hkv, D]
    V = bf16_to_f64(tokens_of_sequence(np.asarray(v_cache_bits), page_table, L, P))
    q_rows = np.asarray(q_bits)[rows]                        # [n_rows, Hq, D] bits
    row_pos = {r: n for n, r in enumerate(rows)}
    mask = np.asarray(block_mask)
    out = np.zeros((len(rows), len(heads), D))
    lse = np.full((len(heads), len(rows)), -math.inf)
    by_tile: Dict[int, List[Tuple[int, int]]] = {}
    for ri, r in enumerate(rows):
        by_tile.setdefault(r // T, []).append((ri, r))
    for hi, h in enumerate(heads):
        g = h // G
        streaming = bool(head_kind[g])
        for i, members in by_tile.items():
            kept = prefill_kept_tiles(i, streaming, mask[h, i], sink_tiles, local_tiles)
            keys = np.concatenate([np.arange(j * T, min((j + 1) * T, L)) for j in kept]) \
                if kept else np.zeros(0, dtype=np.int64)
            rr = np.array([r for _, r in members])
            Qh = bf16_to_f64(q_rows[[row_pos[r] for r in rr], h, :])
            s = sm_scale * (Qh @ K[keys, g, :].T)              # [rows, keys]
            allowed = keys[None, :] <= rr[:, None]
            for (ri, r), srow, arow in zip(members, s, allowed):
                o, z = _softmax_attend(srow[arow], V[keys[arow], g, :])
                out[ri, hi] = o
                lse[hi, ri] = z
    return out, lse


def prefill_kept_tile_count(nT: int, Hq: int, Hkv: int, head_kind, block_mask, sink_tiles: int,
                            local_tiles: int) -> int:
    """Number of kept (head, query tile, KV tile) triples: the unit of prefill work."""
    G = Hq // Hkv
    mask = np.asarray(block_mask)
    total = 0
    for h in range(Hq):
        if head_kind[h // G]:
            for i in range(nT):
                total += min(sink_tiles, i + 1) + min(local_tiles, max(0, i + 1 - sink_tiles))
        else:
            total += int(np.tril(mask[h] != 0).sum())
    return total


# ----------------------------------------------------------------------------- block-mask estimation

def tile_means_ref(x: np.ndarray, T: int) -> np.ndarray:
    """Mean over the rows of every T-row tile of x [L, D] (fp64); a last, partial tile
    averages the rows it has."""
    L, D = x.shape
    nT = (L + T - 1) // T
    out = np.empty((nT, D))
    for i in range(nT):
        out[i] = x[i * T:min((i + 1) * T, L)].mean(axis=0)
    return out


def keep_count(i: int, keep_num: int, keep_den: int) -> int:
    """Tiles kept in query-tile row i, the diagonal included: ceil(keep_num*(i+1)/keep_den)."""
    return (keep_num * (i + 1) + keep_den - 1) // keep_den


def meanpool_mask_ref(q_bits, k_cache_bits, page_table, L: int, Hq: int, Hkv: int, D: int, P: int,
                      T: int, head_kind, keep_num: int = 3, keep_den: int = 10,
                      heads: Optional[Sequence[int]] = None):
    """Block mask of the dense heads from mean-pooled tile scores, fp64.

    The dense heads' mask rule of the Llama-3-8B prefill workload, a query-tile-level
    estimate of the block sparsity that the blog's LServe prefill section applies (a KV
    tile computed or skipped whole per query tile). For dense query head h (KV head
    g = h // (Hq/Hkv)) and query tile i:
        score[i, j] = mean over the rows of Q_h tile i . mean over the rows of K_g tile j
        (j < i), n_i = ceil(keep_num*(i+1)/keep_den) tiles kept, the diagonal included:
        the diagonal and the n_i - 1 strictly-lower tiles of largest score, equal scores
        going to the lower j. Entries above the diagonal are 0.
    A last, partial tile averages the rows it has. heads: the query heads to evaluate
    (default: every dense one). Returns (mask [n, nT, nT] uint8, score [n, nT, nT] with
    -inf outside j < i, mag [n, nT, nT] = sum_c |qbar_c * kbar_c|, the scale of a score's
    rounding error in lower precision), in the order of heads.
    """
    G = Hq // Hkv
    nT = (L + T - 1) // T
    if heads is None:
        heads = [h for h in range(Hq) if not head_kind[h // G]]
    heads = [int(h) for h in heads]
    K = tokens_of_sequence(np.asarray(k_cache_bits), page_table, L, P)        # [L, Hkv, D] bits
    kmeans: Dict[int, np.ndarray] = {}
    mask = np.zeros((len(heads), nT, nT), dtype=np.uint8)
    score = np.full((len(heads), nT, nT), -math.inf)
    mag = np.zeros((len(heads), nT, nT))
    qb = np.asarray(q_bits)
    for n, h in enumerate(heads):
        g = h // G
        if g not in kmeans:
            kmeans[g] = tile_means_ref(bf16_to_f64(K[:, g, :]), T)
        km = kmeans[g]
        qm = tile_means_ref(bf16_to_f64(qb[:, h, :]), T)
        s = qm @ km.T
        m = np.abs(qm) @ np.abs(km).T
        for i in range(nT):
            mask[n, i, i] = 1
            lower = s[i, :i]
            score[n, i, :i] = lower
            mag[n, i, :i] = m[i, :i]
            take = keep_count(i, keep_num, keep_den) - 1
            if take > 0:
                # descending score, then ascending j: lexsort's last key is the primary one
                order = np.lexsort((np.arange(i), -lower))
                mask[n, i, order[:take]] = 1
    return mask, score, mag


# ----------------------------------------------------------------------------- KV append

def append_ref(k_cache_bits, v_cache_bits, page_table, seq_lens, k_new_bits, v_new_bits, P: int):
    """The paged cache after appending n_new tokens to every sequence (the layout of the
    blog's decode section, as in tokens_of_sequence): token t = seq_lens[b] + x of sequence
    b goes to row t % P of physical page page_table[b][t // P], for every KV head.
    k_new/v_new are [B, n_new, Hkv, D] bits. Returns new (k_cache, v_cache) arrays."""
    k = np.array(k_cache_bits, copy=True)
    v = np.array(v_cache_bits, copy=True)
    kn, vn = np.asarray(k_new_bits), np.asarray(v_new_bits)
    pt = np.asarray(page_table)
    for b, L in enumerate(seq_lens):
        for x in range(kn.shape[1]):
            t = int(L) + x
            k[pt[b, t // P], :, t % P, :] = kn[b, x]
            v[pt[b, t // P], :, t % P, :] = vn[b, x]
    return k, v


# ----------------------------------------------------------------------------- page bounds

def bounds_ref(k_cache_bits, page_table, seq_lens, P: int, Lp: int, head_kind,
               pages: Optional[Sequence[Tuple[int, int]]] = None):
    """Per-page key summary (blog, Decode section: "a summary vector per page").

    For every valid page j of sequence b (physical page p = page_table[b, j]), every
    dense KV head g and every logical sub-page u of Lp tokens that holds at least one
    valid token, the channel-wise min and max of the keys over the valid tokens of
    that sub-page. Valid tokens of page j are t < seq_lens[b] - j*P.

    Returns (values, defined): values [NP, Hkv, P/Lp, 2, D] fp64 (index 0 = min,
    1 = max) and a bool [NP, Hkv, P/Lp] marking the entries that are defined.
    pages restricts the work to the given (b, j) pairs.
    """
    Kc = np.asarray(k_cache_bits)                            # bits; decoded per sub-page
    NP, Hkv, _, D = Kc.shape
    U = P // Lp
    values = np.zeros((NP, Hkv, U, 2, D))
    defined = np.zeros((NP, Hkv, U), dtype=bool)
    pt = np.asarray(page_table)
    lens = [int(x) for x in seq_lens]
    if pages is None:
        pages = [(b, j) for b in range(len(lens)) for j in range((lens[b] + P - 1) // P)]
    for b, j in pages:
        p = int(pt[b, j])
        valid = min(P, lens[b] - j * P)
        for g in range(Hkv):
            if head_kind[g]:
                continue
            for u in range(U):
                lo, hi = u * Lp, min((u + 1) * Lp, valid)
                if hi <= lo:
                    continue
                kk = bf16_to_f64(Kc[p, g, lo:hi, :])
                values[p, g, u, 0] = kk.min(axis=0)
                values[p, g, u, 1] = kk.max(axis=0)
                defined[p, g, u] = True
    return values, defined


# ----------------------------------------------------------------------------- selection

def subpage_bound(q_group: np.ndarray, kmin: np.ndarray, kmax: np.ndarray) -> float:
    """Upper bound of max_{h, t} q_h . k_t over the tokens of one sub-page.

    For each query head h of the group: sum over channels c of
    max(q_hc * kmin_c, q_hc * kmax_c) (the Quest bound); the group takes the max over
    its heads, so the result still bounds every head's best dot product.
    """
    per_head = np.maximum(q_group * kmin[None, :], q_group * kmax[None, :]).sum(axis=1)
    return float(per_head.max())


def page_scores_ref(q_bits, bounds_values, bounds_defined, page_table, seq_lens, Hq: int,
                    Hkv: int, P: int, Lp: int, head_kind,
                    pairs: Optional[Sequence[Tuple[int, int]]] = None) -> Dict[Tuple[int, int], np.ndarray]:
    """Score of every valid page of every (sequence b, dense KV head g).

    A page's score is the max of the bounds of its sub-pages that hold valid tokens
    (the hierarchical step: Lp-token summaries reduced to the P-token page that is
    selected). Returns {(b, g): scores[n_b]} with n_b = ceil(seq_lens[b] / P).
    """
    G = Hq // Hkv
    Q = bf16_to_f64(q_bits)                      # [B, Hq, D]
    pt = np.asarray(page_table)
    lens = [int(x) for x in seq_lens]
    if pairs is None:
        pairs = [(b, g) for b in range(len(lens)) for g in range(Hkv) if not head_kind[g]]
    out = {}
    for b, g in pairs:
        L = lens[b]
        n = (L + P - 1) // P
        qg = Q[b, g * G:(g + 1) * G, :]
        sc = np.empty(n)
        for j in range(n):
            p = int(pt[b, j])
            valid = min(P, L - j * P)
            nsub = (valid + Lp - 1) // Lp
            best = -math.inf
            for u in range(nsub):
                assert bounds_defined[p, g, u]
                best = max(best, subpage_bound(qg, bounds_values[p, g, u, 0], bounds_values[p, g, u, 1]))
            sc[j] = best
        out[(b, g)] = sc
    return out


def topk_pages_ref(scores: np.ndarray, k: int) -> List[int]:
    """The k best pages: order by (score descending, page index ascending), keep the
    first k (all pages when there are at most k), return them in ascending order."""
    n = len(scores)
    if n <= k:
        return list(range(n))
    order = sorted(range(n), key=lambda j: (-scores[j], j))
    return sorted(order[:k])


def select_ref(q_bits, k_cache_bits, page_table, seq_lens, Hq: int, Hkv: int, P: int, Lp: int,
               token_budget: int, head_kind, pairs=None):
    """Query-aware page selection for one decode step, end to end (bounds -> scores ->
    top-k with k = token_budget / P). Returns ({(b, g): selected pages}, scores dict)."""
    lens = [int(x) for x in seq_lens]
    if pairs is None:
        pairs = [(b, g) for b in range(len(lens)) for g in range(Hkv) if not head_kind[g]]
    bs = sorted({b for b, _ in pairs})
    pages = [(b, j) for b in bs for j in range((lens[b] + P - 1) // P)]
    vals, defined = bounds_ref(k_cache_bits, page_table, seq_lens, P, Lp, head_kind, pages=pages)
    scores = page_scores_ref(q_bits, vals, defined, page_table, seq_lens, Hq, Hkv, P, Lp,
                             head_kind, pairs=pairs)
    k = token_budget // P
    return {bg: topk_pages_ref(s, k) for bg, s in scores.items()}, scores


# ----------------------------------------------------------------------------- decode

def decode_keys_ref(L: int, P: int, streaming: bool, selected: Sequence[int], sink_tokens: int,
                    local_tokens: int) -> np.ndarray:
    """Token positions one decode query attends to (the query sits at position L-1 and
    the context holds tokens 0..L-1).

    Dense head: every valid token of the selected pages (token-level attention inside
    the kept pages). Streaming head: tokens t < sink_tokens or t >= L - local_tokens.
    """
    if streaming:
        return np.array([t for t in range(L) if t < sink_tokens or t >= L - local_tokens],
                        dtype=np.int64)
    toks = [np.arange(j * P, min((j + 1) * P, L)) for j in sorted(int(x) for x in selected)]
    return np.concatenate(toks).astype(np.int64) if toks else np.zeros(0, dtype=np.int64)


def _decode_over(Q: np.ndarray, rows, D: int, page_table, seq_lens, Hq: int, Hkv: int, P: int,
                 head_kind, selected, sink_tokens: int, local_tokens: int, sm_scale: float,
                 batches: Optional[Sequence[int]]):
    """Decode attention with the key and value rows of a key set supplied by
    rows(b, g, page_row, L, keys) -> (K [n, D], V [n, D]) in fp64."""
    G = Hq // Hkv
    pt = np.asarray(page_table)
    lens = [int(x) for x in seq_lens]
    bl = list(range(len(lens))) if batches is None else [int(b) for b in batches]
    out = np.zeros((len(bl), Hq, D))
    lse = np.full((len(bl), Hq), -math.inf)
    for bi, b in enumerate(bl):
        L = lens[b]
        for g in range(Hkv):
            streaming = bool(head_kind[g])
            keys = decode_keys_ref(L, P, streaming, [] if streaming else selected[(b, g)],
                                   sink_tokens, local_tokens)
            Kt, Vt = rows(b, g, pt[b], L, keys)
            for h in range(g * G, (g + 1) * G):
                o, z = _softmax_attend(sm_scale * (Kt @ Q[b, h]), Vt)
                out[bi, h] = o
                lse[bi, h] = z
    return out, lse


def decode_ref(q_bits, k_cache_bits, v_cache_bits, page_table, seq_lens, Hq: int, Hkv: int,
               P: int, head_kind, selected: Dict[Tuple[int, int], Sequence[int]],
               sink_tokens: int, local_tokens: int, sm_scale: float,
               batches: Optional[Sequence[int]] = None):
    """Sparse decode attention, fp64: out[b, h] = softmax-weighted sum of v over the key
    set of (b, KV head h // G) from decode_keys_ref; lse = ln sum exp(scores); an empty
    key set gives out = 0 and lse = -inf. selected maps (b, g) of dense heads to page
    indices. Returns (out [nb, Hq, D], lse [nb, Hq]) for the batches given."""
    Kc = np.asarray(k_cache_bits)                            # bits; decoded per key set
    Vc = np.asarray(v_cache_bits)

    def rows(b, g, page_row, L, keys):
        return (bf16_to_f64(tokens_of_sequence(Kc, page_row, L, P, keys)[:, g, :]),
                bf16_to_f64(tokens_of_sequence(Vc, page_row, L, P, keys)[:, g, :]))

    return _decode_over(bf16_to_f64(q_bits), rows, Kc.shape[-1], page_table, seq_lens, Hq, Hkv, P,
                        head_kind, selected, sink_tokens, local_tokens, sm_scale, batches)


# ----------------------------------------------------------------------------- INT4 KV pages
#
# Blog "LServe -- Decode Phase" and the Figure 2 caption: INT4 KV quantization stacks
# with page sparsity, cutting the bytes of every page that is read. The pages give no
# format; the reading taken here: every (token, KV head) row of D channels is quantized
# on its own, asymmetrically, to 4-bit codes n in [0, 15] with x ~ n * scale + zero;
# scale and zero are stored as fp16. The code is an integer chosen by floating point, so
# it is taken in fp32, as the GPU takes it:
#   lo, hi = min_c x_c, max_c x_c;  scale16 = fp16((hi - lo) / 15);  zero16 = fp16(lo)
#   n_c = clamp(rint((x_c - zero) / scale), 0, 15), all in fp32 with the fp16 values
#   widened; a row with scale16 == 0 has every code 0 (and dequantizes to zero16).
# Storage of the codes, in 32-bit little-endian words of 8 codes: code k of a group of 8
# goes to nibble k/2 of the word's low half (k even) or of its high half (k odd), so the
# word's bytes are (n0 | n2 << 4, n4 | n6 << 4, n1 | n3 << 4, n5 | n7 << 4). K pages hold
# each token's row as D/8 such words, channels in order ([NP][Hkv][P][D/2] bytes). V pages
# are channel-major: for each channel, the P tokens of the page as P/8 words
# ([NP][Hkv][D][P/2] bytes). Params: [NP][Hkv][P][2] fp16 (scale, zero) for K and for V.

def quantize_int4_ref(x_bits) -> Tuple[np.ndarray, np.ndarray]:
    """Codes [..., D] (uint8 in [0, 15]) and fp16 bit patterns [..., 2] = (scale, zero)
    of bf16 rows x_bits [..., D], by the steps above (fp32 arithmetic, round half to even)."""
    x = (np.ascontiguousarray(x_bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    lo = x.min(axis=-1)
    hi = x.max(axis=-1)
    scale16 = ((hi - lo) / np.float32(15.0)).astype(np.float16)
    zero16 = lo.astype(np.float16)
    sc = scale16.astype(np.float32)[..., None]
    ze = zero16.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.rint((x - ze) / sc)
    codes = np.where(sc == 0, np.float32(0), np.clip(t, 0, 15)).astype(np.uint8)
    params = np.stack([scale16.view(np.uint16), zero16.view(np.uint16)], axis=-1)
    return codes, params


def pack_int4(codes) -> np.ndarray:
    """Codes [..., 8m] -> bytes [..., 4m]: each group of 8 codes n0..n7 as the bytes
    (n0 | n2 << 4, n4 | n6 << 4, n1 | n3 << 4, n5 | n7 << 4)."""
    c = np.asarray(codes, dtype=np.uint8)
    g = c.reshape(c.shape[:-1] + (c.shape[-1] // 8, 8))
    out = np.stack([g[..., 0] | (g[..., 2] << 4), g[..., 4] | (g[..., 6] << 4),
                    g[..., 1] | (g[..., 3] << 4), g[..., 5] | (g[..., 7] << 4)], axis=-1)
    return out.reshape(c.shape[:-1] + (c.shape[-1] // 2,)).astype(np.uint8)


def unpack_int4(packed) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    w = p.reshape(p.shape[:-1] + (p.shape[-1] // 4, 4))
    g = np.stack([w[..., 0] & 0xF, w[..., 2] & 0xF, w[..., 0] >> 4, w[..., 2] >> 4,
                  w[..., 1] & 0xF, w[..., 3] & 0xF, w[..., 1] >> 4, w[..., 3] >> 4], axis=-1)
    return g.reshape(p.shape[:-1] + (2 * p.shape[-1],)).astype(np.uint8)


def dequant_int4_ref(packed, params) -> np.ndarray:
    """x_c = n_c * scale + zero in fp64 from packed codes [..., D/2] and fp16 params [..., 2]."""
    pr = np.ascontiguousarray(params, dtype=np.uint16).view(np.float16).astype(np.float64)
    return unpack_int4(packed).astype(np.float64) * pr[..., 0:1] + pr[..., 1:2]


def quantize_cache_int4_ref(k_bits, v_bits, page_table, seq_lens, P: int):
    """INT4 pages of the valid tokens of every sequence, in the storage above:
    (k_codes [NP, Hkv, P, D/2], v_codes [NP, Hkv, D, P/2], k_params, v_params
    [NP, Hkv, P, 2]) and a mask [NP, P] of the token rows that were written. K codes and
    both params are written for valid tokens only; a V word is written when one of its 8
    tokens is valid, with code 0 for the others. Everything else stays zero."""
    K = np.asarray(k_bits, dtype=np.uint16)
    V = np.asarray(v_bits, dtype=np.uint16)
    NP, Hkv, _, D = K.shape
    kq = np.zeros((NP, Hkv, P, D // 2), dtype=np.uint8)
    vq = np.zeros((NP, Hkv, D, P // 2), dtype=np.uint8)
    kp = np.zeros((NP, Hkv, P, 2), dtype=np.uint16)
    vp = np.zeros((NP, Hkv, P, 2), dtype=np.uint16)
    written = np.zeros((NP, P), dtype=bool)
    pt = np.asarray(page_table)
    for b, L in enumerate(int(x) for x in seq_lens):
        for j in range((L + P - 1) // P):
            pg = int(pt[b, j])
            n = min(P, L - j * P)
            c, pr = quantize_int4_ref(K[pg, :, :n, :])
            kq[pg, :, :n] = pack_int4(c)
            kp[pg, :, :n] = pr
            c, pr = quantize_int4_ref(V[pg, :, :n, :])
            vp[pg, :, :n] = pr
            ct = np.zeros((Hkv, D, P), dtype=np.uint8)
            ct[:, :, :n] = c.transpose(0, 2, 1)
            nw = (n + 7) // 8                                  # words touched per channel
            vq[pg, :, :, :4 * nw] = pack_int4(ct)[:, :, :4 * nw]
            written[pg, :n] = True
    return kq, vq, kp, vp, written


def decode_int4_ref(q_bits, k_codes, v_codes, k_params, v_params, page_table, seq_lens, Hq: int,
                    Hkv: int, P: int, head_kind, selected: Dict[Tuple[int, int], Sequence[int]],
                    sink_tokens: int, local_tokens: int, sm_scale: float,
                    batches: Optional[Sequence[int]] = None):
    """decode_ref over INT4 pages (storage above): the same key sets, with K and V rows the
    fp64 dequantization of their codes."""
    Kq, Vq = np.asarray(k_codes), np.asarray(v_codes)
    Kp, Vp = np.asarray(k_params), np.asarray(v_params)
    Vrows = unpack_int4(Vq).transpose(0, 1, 3, 2)               # [NP, Hkv, P, D] codes

    def rows(b, g, page_row, L, keys):
        vc = tokens_of_sequence(Vrows, page_row, L, P, keys)[:, g, :].astype(np.float64)
        vpr = tokens_of_sequence(Vp, page_row, L, P, keys)[:, g, :].view(np.float16).astype(np.float64)
        return (dequant_int4_ref(tokens_of_sequence(Kq, page_row, L, P, keys)[:, g, :],
                                 tokens_of_sequence(Kp, page_row, L, P, keys)[:, g, :]),
                vc * vpr[:, 0:1] + vpr[:, 1:2])

    return _decode_over(bf16_to_f64(q_bits), rows, 2 * Kq.shape[-1], page_table, seq_lens, Hq, Hkv, P,
                        head_kind, selected, sink_tokens, local_tokens, sm_scale, batches)
