"""Benchmark of the unified block-sparse attention hot path on one MI355X.

A step is one pass of the whole path on the Llama-3-8B layer workload:
  sparse_prefill     on prefill_llama8b (L=65536, Hq=32, Hkv=8, D=128, T=128; dense KV heads
                     0-3 with the mean-pooled top-30% block mask, KV heads 4-7 streaming with
                     1 sink + 8 local tiles; 707,216 kept 128x128 tiles),
  build_page_bounds, select_pages, sparse_decode
                     on decode_llama8b (B=4, L=32768, Hq=32, Hkv=8, D=128, P=64, budget 4096
                     tokens, streaming 128 sink + 512 local tokens).
Inputs are synthetic, seeded and resident in HBM before timing starts. Each step runs
build_page_bounds, sparse_prefill, select_pages, sparse_decode in that order: the prefill
streams > 1.5 GB, which evicts the bounds and K/V pages from L2 and the 256 MB Infinity
Cache, so selection and decode read cold HBM.

value = 100 * (sum over the step's ops of their roofline time) / (measured step time),
i.e. the step's speed as a percentage of the MI355X roofline: prefill counted as
kept-tile flops against dense bf16 MFMA peak, bounds / selection / decode as their
algorithmic HBM bytes against peak HBM bandwidth.

The same line carries, outside `value`, one roofline fraction per named workload
(`per_config`): prefill_tiny, the decode_llama8b step replayed as a HIP graph over 24
cache instances, prefill_llama8b, the decode_ragged step (64 sequences of 16K-128K tokens)
and prefill_extreme (262,144 tokens, Llama-3-70B heads), plus further legs (mask
estimation, batched and chunked prefill, KV append, reused selection, INT4 pages) and the
fp64 oracle timed on the host cores (`cpu_baseline`).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--legs LIST] [--no-cpu-baseline]

--legs selects what runs (default: all): step, tiny, graph, ragged, extreme, mask,
varlen, chunk, append, peaks, cpu. Without `step` the line holds only the selected legs' results; profiling
runs use this to trace one workload at a time.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # 256 CU x 2.4 GHz x 4096 flop/clk/CU, dense
PEAK_HBM_GBPS = 8000.0
METRIC = "sparse prefill TFLOP/s (kept tiles) + decode KV GB/s, as % of MI355X roofline"
LEGS = ("step", "tiny", "graph", "ragged", "extreme", "mask", "varlen", "chunk", "append", "peaks", "cpu")
# The pages' own figures for this method, quoted as context (relative speedups, no hardware
# or absolute numbers given): LServe index page, Abstract.
PAGES_CONTEXT = ("LServe (arXiv 2502.14866) abstract: up to 2.9x prefill and 1.3-2.1x decode speedup over "
                 "vLLM on long-sequence serving; hardware, precision and absolute rates not stated")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_llama8b_traffic.json")
KERNEL_SOURCES = ["unified_block_sparse_amd/csrc/prefill.hip", "unified_block_sparse_amd/csrc/common.h",
                  "unified_block_sparse_amd/csrc/launch.h"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--legs", default=",".join(LEGS),
                    help="comma-separated subset of: " + ", ".join(LEGS))
    ap.add_argument("--no-cpu-baseline", action="store_true", help="same as leaving `cpu` out of --legs")
    ap.add_argument("--cpu-rows-per-head", type=int, default=256)
    ap.add_argument("--no-ragged", action="store_true", help="same as leaving `ragged` out of --legs")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB (5 times) and exit: "
                         "the known-size kernel that scales the HBM byte counters")
    ap.add_argument("--gemm-ceiling", action="store_true",
                    help="only time the vendor library's dense bf16 GEMM (torch.matmul, n = 8192 and "
                         "16384) and exit: the matrix-core rate this GPU sustains in practice")
    return ap.parse_args()


def copy_calibration(mib: int):
    """A plain copy of known size, for scaling FETCH_SIZE / WRITE_SIZE counter readings."""
    import torch
    dev = torch.device("cuda:0")
    n = mib * (1 << 20)
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize(dev)
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}), flush=True)


def gemm_ceiling():
    """Sustained bf16 matrix-core rate of the vendor GEMM (hipBLASLt through torch.matmul):
    a practical ceiling to read the prefill kernel's TFLOP/s against, next to the
    published dense peak."""
    import torch
    dev = torch.device("cuda:0")
    for n, reps in ((8192, 20), (16384, 4)):
        a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
        b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
        for _ in range(3):
            a @ b
        torch.cuda.synchronize(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            a @ b
        e1.record()
        torch.cuda.synchronize(dev)
        ms = e0.elapsed_time(e1) / reps
        print(json.dumps({"gemm_bf16_n": n, "ms": round(ms, 4), "tflops": round(2 * n ** 3 / ms / 1e9, 1),
                          "frac_of_peak": round(2 * n ** 3 / ms / 1e9 / PEAK_BF16_TFLOPS, 4)}), flush=True)


def measured_peaks():
    """What this GPU sustains, measured beside the published peaks:
    - the matrix cores on back-to-back bf16 MFMAs from registers (ubs_bench_mfma: no
      memory traffic, at whatever clock the GPU holds under that load);
    - the vendor bf16 GEMM (hipBLASLt through torch.matmul, n = 16384, compute-bound);
    - a plain HBM read of 8 GiB (ubs_bench_read: 16-byte loads, one contiguous share per
      work-group) and a 4 GiB device copy (torch; read + written bytes).
    The per-workload fractions are also given against the GEMM and the plain read."""
    import torch
    import unified_block_sparse_amd as ubs
    dev = torch.device("cuda:0")

    def timed(f, reps, warm=2):
        for _ in range(warm):
            f()
        torch.cuda.synchronize(dev)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record()
        for i in range(reps):
            f()
            ev[i + 1].record()
        torch.cuda.synchronize(dev)
        t = sorted(ev[i].elapsed_time(ev[i + 1]) * 1e-3 for i in range(reps))
        return t[len(t) // 2]

    out = torch.zeros(4, dtype=torch.float32, device=dev)
    iters = 40000
    flops = ubs.bench_mfma(iters, out)
    t_m = timed(lambda: ubs.bench_mfma(iters, out), 5)
    n = 16384
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    t_g = timed(lambda: a @ b, 5)
    del a, b
    x = torch.ones(8 << 30, dtype=torch.uint8, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    t_r = timed(lambda: ubs.bench_read(x, sink), 10)
    del x
    src = torch.ones(4 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    t_c = timed(lambda: dst.copy_(src), 10)
    del src, dst
    torch.cuda.empty_cache()
    return {"mfma_loop_bf16_tflops": round(flops / t_m / 1e12, 1),
            "gemm_bf16_tflops": round(2 * n ** 3 / t_g / 1e12, 1), "gemm_n": n,
            "hbm_read_gbps": round((8 << 30) / t_r / 1e9, 1), "hbm_copy_gbps": round((8 << 30) / t_c / 1e9, 1),
            "note": "medians of timed calls; copy counts bytes read + written"}


# ----------------------------------------------------------------------------- work accounting

def kept_tile_count(c, first_tile: int = 0) -> int:
    """Kept (query head, query tile, KV tile) triples of query tiles first_tile .. nT-1: the
    tiles the kernel computes."""
    import torch
    nT = c.nT
    total = 0
    i = torch.arange(first_tile, nT)
    lam = (torch.clamp(i + 1, max=c.sink_tiles) +
           torch.clamp(torch.clamp(i + 1 - c.sink_tiles, min=0), max=c.local_tiles)).sum().item()
    for h in range(c.Hq):
        if c.head_kind[h // c.G]:
            total += int(lam)
        else:
            total += int(torch.tril(c.block_mask[h] != 0)[first_tile:].sum().item())
    return total


def prefill_flops(c, kept_tiles: int) -> float:
    return 4.0 * kept_tiles * c.T * c.T * c.D


def decode_bytes(d, sel_pages):
    """Algorithmic HBM bytes of bounds, selection and decode for one decode step.

    bounds:    K rows of dense heads' valid tokens + the bounds written
    selection: bounds of dense heads' valid sub-pages + q + selected indices
    decode:    K and V rows of every attended token + q + out
    """
    G = d.Hq // d.Hkv
    row = d.D * 2
    dense = [g for g in range(d.Hkv) if not d.head_kind[g]]
    stream = [g for g in range(d.Hkv) if d.head_kind[g]]
    U = d.P // d.Lp
    k_dense_tokens = sum(d.seq_lens) * len(dense)
    n_sub = sum(sum(min(U, math.ceil((min(d.P, L - j * d.P)) / d.Lp)) for j in range(math.ceil(L / d.P)))
                for L in d.seq_lens) * len(dense)
    bounds_w = n_sub * 2 * row
    b_bounds = k_dense_tokens * row + bounds_w
    q_bytes = d.B * d.Hq * d.D * 2
    b_select = bounds_w + q_bytes + d.B * d.Hkv * d.k_pages * 4
    attended = 0
    for b, L in enumerate(d.seq_lens):
        for g in dense:
            attended += sum(min(d.P, L - j * d.P) for j in sel_pages[b][g])
        A = min(d.sink_tokens, L)
        attended += len(stream) * (A + L - max(A, L - d.local_tokens))
    b_decode = attended * 2 * row + q_bytes + d.B * d.Hq * d.D * 4
    return b_bounds, b_select, b_decode


# ----------------------------------------------------------------------------- cpu baseline

def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        return os.cpu_count() or 1


def _host_bits(t):
    import numpy as np
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def oracle_prefill_sample(c, rows_per_head: int, seed: int = 11):
    """The fp64 oracle on `rows_per_head` query rows of every head of prefill case c: rows 0,
    T-1, T and L-1 (the first tile's edges and the last row), the others seeded.
    Returns (seconds for the sample, the oracle's fixed per-call part (K/V gather and
    decode), seconds extrapolated to all L rows)."""
    import numpy as np
    import torch
    import oracle
    # the rows at the first tile's edges and the last row, then seeded others
    fixed = sorted({r for r in (0, c.T - 1, c.T, c.L - 1) if 0 <= r < c.L})[:rows_per_head]
    rest = np.setdiff1d(np.arange(c.L), fixed)
    rng = np.random.default_rng(seed)
    extra = rng.choice(rest, size=min(rows_per_head - len(fixed), len(rest)), replace=False).tolist()
    rows = sorted(fixed + [int(x) for x in extra])
    q_host = np.zeros(tuple(c.q.shape), dtype=np.uint16)
    q_host[rows] = _host_bits(c.q[torch.tensor(rows, device=c.q.device)])
    kb, vb = _host_bits(c.k_cache), _host_bits(c.v_cache)
    pt, mask = c.page_table.cpu().numpy(), c.block_mask.cpu().numpy()
    t0 = time.perf_counter()
    oracle.prefill_ref(q_host, kb, vb, pt, c.L, c.Hq, c.Hkv, c.D, c.P, c.T, c.head_kind, mask, c.sink_tiles,
                       c.local_tiles, c.sm_scale, rows=[])
    t_fixed = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.prefill_ref(q_host, kb, vb, pt, c.L, c.Hq, c.Hkv, c.D, c.P, c.T, c.head_kind, mask, c.sink_tiles,
                       c.local_tiles, c.sm_scale, rows=rows)
    t = time.perf_counter() - t0
    return t, t_fixed, t_fixed + max(t - t_fixed, 0.0) * (c.L / len(rows)), len(rows)


def _host_ram_bytes() -> int:
    try:
        return os.sysconf("SC_PAGE_SIZE") * os.sysconf("SC_PHYS_PAGES")
    except (ValueError, OSError, AttributeError):
        return 0


def oracle_decode_sample(d, batches):
    """The fp64 oracle's whole decode step (bounds -> selection -> decode) on sequences
    `batches` of decode case d, timed sequence by sequence (host copies of each sequence's
    pages are made outside the timed part). Returns seconds."""
    import numpy as np
    import oracle
    t_dec = 0.0
    for b in batches:
        dq = _host_bits(d.q[b:b + 1])
        nb = (d.seq_lens[b] + d.P - 1) // d.P
        idx = d.page_table[b, :nb].long()
        dk, dv = _host_bits(d.k_cache[idx]), _host_bits(d.v_cache[idx])
        dpt = np.arange(nb, dtype=np.int32)[None]
        t0 = time.perf_counter()
        sel, _ = oracle.select_ref(dq, dk, dpt, d.seq_lens[b:b + 1], d.Hq, d.Hkv, d.P, d.Lp, d.token_budget,
                                   d.head_kind)
        oracle.decode_ref(dq, dk, dv, dpt, d.seq_lens[b:b + 1], d.Hq, d.Hkv, d.P, d.head_kind, sel,
                          d.sink_tokens, d.local_tokens, d.sm_scale, batches=[0])
        t_dec += time.perf_counter() - t0
    return t_dec


def cpu_baseline(c, d, rows_per_head: int, ideal_s: float, extra: dict):
    """The fp64 oracle as it stands, on the host cores, on a bounded sample of the step's
    workloads (prefill_llama8b rows, every decode_llama8b sequence); per-workload figures
    for the other configurations come in `extra` (measured by their legs while their
    inputs are resident). A one-thread figure of a smaller sample is added."""
    threads = _blas_threads()
    t_pf, t_fixed, pf_full, n_rows = oracle_prefill_sample(c, rows_per_head)
    t_dec = oracle_decode_sample(d, range(d.B))
    step_s = pf_full + t_dec
    per_config = {
        "prefill_llama8b": {"rows_per_s": round(n_rows * c.Hq / max(t_pf - t_fixed, 1e-9), 1),
                            "sample": f"{n_rows} rows (0, T-1, T, L-1, the rest seeded) x {c.Hq} heads, {t_pf:.2f} s",
                            "full_config_s_extrapolated": round(pf_full, 1)},
        "decode_llama8b": {"steps_per_s": round(1.0 / t_dec, 3),
                           "sample": f"all {d.B} sequences (bounds, selection, decode), {t_dec:.2f} s"},
    }
    per_config.update(extra)
    one = {}
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            t1, f1, full1, n1 = oracle_prefill_sample(c, 32, seed=12)
            td1 = oracle_decode_sample(d, range(d.B))
        one = {"cores": 1, "prefill_llama8b_rows_per_s": round(n1 * c.Hq / max(t1 - f1, 1e-9), 1),
               "decode_llama8b_steps_per_s": round(1.0 / td1, 3),
               "step_s_extrapolated": round(full1 + td1, 1),
               "value": 100.0 * ideal_s / (full1 + td1),
               "sample": f"{n1} seeded prefill rows x {c.Hq} heads ({t1:.2f} s) + decode_llama8b "
                         f"({td1:.2f} s) with BLAS limited to one thread"}
    except Exception as e:   # threadpoolctl missing: say so instead
        one = {"error": f"one-thread figure not taken: {e}"}
    return {
        "value": 100.0 * ideal_s / step_s,
        "unit": "% of MI355X roofline",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"fp64 NumPy oracle: {c.name} {n_rows} rows (0, T-1, T, L-1, the rest seeded) x {c.Hq} heads "
                   f"({t_pf:.2f} s incl. {t_fixed:.2f} s K/V gather; per-row part extrapolated "
                   f"x{c.L / n_rows:.1f} to all {c.L} rows) + {d.name} "
                   f"bounds/selection/decode of all {d.B} sequences ({t_dec:.2f} s); "
                   f"extrapolated step {step_s:.1f} s"),
        "step_seconds_extrapolated": step_s,
        "host_cpus": os.cpu_count(),
        "affinity_cpus": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None,
        "cpu_model": _cpu_model(),
        "per_config": per_config,
        "one_thread": one,
    }


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ----------------------------------------------------------------------------- mask estimation

def mask_estimation(c, steps: int, warmup: int):
    """estimate_block_mask on prefill_llama8b (the dense heads' mask the prefill above uses,
    computed on the GPU), timed alone and outside `value`. Algorithmic bytes: the dense
    query heads' Q and the dense KV heads' K read once, the mask rows written."""
    import torch
    import unified_block_sparse_amd as ubs
    dev = c.q.device
    out = torch.empty((c.Hq, c.nT, c.nT), dtype=torch.uint8, device=dev)
    f = lambda: ubs.estimate_block_mask(c.q, c.k_cache, c.page_table, c.head_kind, c.T, keep=(3, 10), out=out)
    for _ in range(warmup):
        f()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    e0.record(stream)
    for _ in range(steps):
        f()
    e1.record(stream)
    torch.cuda.synchronize(dev)
    t = e0.elapsed_time(e1) * 1e-3 / steps
    n_dkv = sum(1 for g in range(c.Hkv) if not c.head_kind[g])
    nq = n_dkv * c.G
    nbytes = c.L * (nq + n_dkv) * c.D * 2 + nq * c.nT * c.nT
    return {"workload": "prefill_llama8b dense heads (16 query heads, 512 query tiles)", "ms": round(t * 1e3, 4),
            "bytes": nbytes, "gbps": round(nbytes / t / 1e9, 1), "frac": round(nbytes / t / 1e9 / PEAK_HBM_GBPS, 4)}


# ----------------------------------------------------------------------------- batched prefill

def varlen_prefill(steps: int, warmup: int):
    """sparse_prefill_varlen on 8 sequences of 4K-16K tokens (seeded lengths) with the
    Llama-3-8B layer's heads and mask rule (planted keys, mean-pooled top-30% rows for the
    dense heads, sink 1 + local 8 tiles for the streaming ones), packed into one call over
    one paged cache. Work = kept tiles x 4 T^2 D, as for the single-sequence prefill."""
    import numpy as np
    import torch
    import unified_block_sparse_amd as ubs
    from workloads import cases
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(1006)
    lens = [int(x) * 128 for x in rng.integers(32, 129, size=8)]
    hk = [0, 0, 0, 0, 1, 1, 1, 1]
    seqs = [cases.make_prefill(f"vb{b}", L, 32, 8, 128, 128, 64, hk, 1, 8, "meanpool", 1100 + b, dev, planted=True)
            for b, L in enumerate(lens)]
    kept = sum(kept_tile_count(c) for c in seqs)
    flops = sum(prefill_flops(c, kept_tile_count(c)) for c in seqs)
    offs, n = [], 0
    for c in seqs:
        offs.append(n)
        n += c.k_cache.shape[0]
    k_all = torch.cat([c.k_cache for c in seqs])
    v_all = torch.cat([c.v_cache for c in seqs])
    max_pages = max((L + 63) // 64 for L in lens)
    pt = torch.zeros((len(seqs), max_pages), dtype=torch.int32, device=dev)
    for b, c in enumerate(seqs):
        pt[b, :c.page_table.numel()] = c.page_table + offs[b]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=dev)
    q = torch.cat([c.q for c in seqs])
    nTm = max(lens) // 128
    mask = torch.zeros((len(seqs), 32, nTm, nTm), dtype=torch.uint8, device=dev)
    for b, c in enumerate(seqs):
        mask[b, :, :c.nT, :c.nT] = c.block_mask
    out = torch.empty((sum(lens), 32, 128), dtype=torch.float32, device=dev)
    del seqs
    f = lambda: ubs.sparse_prefill_varlen(q, k_all, v_all, pt, cu, max(lens), hk, mask, 1, 8, 128,
                                          1.0 / math.sqrt(128), out=out)
    for _ in range(warmup):
        f()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    e0.record(stream)
    for _ in range(steps):
        f()
    e1.record(stream)
    torch.cuda.synchronize(dev)
    t = e0.elapsed_time(e1) * 1e-3 / steps
    return {"workload": f"8 sequences, lengths {lens}, Hq=32, Hkv=8, D=128, T=128, half KV heads streaming",
            "ms": round(t * 1e3, 4), "kept_tiles": kept, "tflop": round(flops / 1e12, 4),
            "tflops": round(flops / t / 1e12, 2), "frac": round(flops / t / 1e12 / PEAK_BF16_TFLOPS, 4)}


# ----------------------------------------------------------------------------- graph-replayed decode

def decode_graph_step(R: int = 24, replays: int = 10):
    """Selection + decode of decode_llama8b (one sparse_decode_select call: page scores,
    then the decode kernel ranking each row's scores itself, then the split merge), cycled
    over R independent cache instances (seeds 1002 + r) captured once as one HIP graph:
    R x ~43 MB > 1 GiB of working set, so each step reads HBM rather than the Infinity Cache,
    and graph replay takes the host launch path out of the step. Time per step = replay
    time / R. Every replay's outputs are checked bitwise against an eager run of the same
    calls before capture.
    """
    import torch
    import unified_block_sparse_amd as ubs
    from workloads import cases
    dev = torch.device("cuda:0")
    lib = ubs.load()
    inst = []
    for r in range(R):
        d = cases.decode_llama8b(dev, seed=1002 + r)
        bnd = torch.zeros((d.num_physical_pages, d.Hkv, d.P // d.Lp, 2, d.D), dtype=torch.bfloat16, device=dev)
        ubs.build_page_bounds(d.k_cache, d.page_table, d.seq_lens_t, d.head_kind, d.Lp, bounds=bnd)
        sel = torch.empty((d.B, d.Hkv, d.k_pages), dtype=torch.int32, device=dev)
        num = torch.empty((d.B, d.Hkv), dtype=torch.int32, device=dev)
        out = torch.empty((d.B, d.Hq, d.D), dtype=torch.float32, device=dev)
        inst.append((d, bnd, sel, num, out))
    d0 = inst[0][0]
    ws = torch.zeros(max(256, lib.ubs_decode_select_workspace_size(d0.B, d0.page_table.shape[1], d0.Hq, d0.Hkv,
                                                                   d0.D, d0.P, d0.token_budget, d0.sink_tokens,
                                                                   d0.local_tokens)),
                     dtype=torch.uint8, device=dev)

    def run_all():
        for d, bnd, sel, num, out in inst:
            ubs.sparse_decode_select(d.q, bnd, d.k_cache, d.v_cache, d.page_table, d.seq_lens_t, d.head_kind, d.P,
                                     d.token_budget, d.sink_tokens, d.local_tokens, d.sm_scale, out=out,
                                     selected=sel, num_selected=num, workspace=ws)

    run_all()
    torch.cuda.synchronize(dev)
    ref = [(sel.clone(), num.clone(), out.clone()) for _, _, sel, num, out in inst]
    nbytes = 0
    for (d, _, _, _, _), (sel_r, num_r, _) in zip(inst, ref):
        sel_h, num_h = sel_r.cpu().tolist(), num_r.cpu().tolist()
        sel_pages = [[sel_h[b][g][:num_h[b][g]] for g in range(d.Hkv)] for b in range(d.B)]
        _, b_select, b_decode = decode_bytes(d, sel_pages)
        nbytes += b_select + b_decode
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        run_all()                     # warm the side stream before capture
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize(dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_all()
    torch.cuda.synchronize(dev)
    for _, _, sel, num, out in inst:  # replays must rewrite every output
        sel.fill_(-7)
        num.fill_(-7)
        out.fill_(float("nan"))
    g.replay()
    g.replay()
    torch.cuda.synchronize(dev)
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(replays):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize(dev)
    for (_, _, sel, num, out), (sel_r, num_r, out_r) in zip(inst, ref):
        if not (torch.equal(sel, sel_r) and torch.equal(num, num_r) and torch.equal(out, out_r)):
            raise RuntimeError("graph replay differs from the eager run")
    t = e0.elapsed_time(e1) * 1e-3 / replays / R
    nb = nbytes / R
    return {"workload": f"decode_llama8b x {R} cache instances, one HIP graph", "ms": round(t * 1e3, 4),
            "bytes": int(nb), "gbps": round(nb / t / 1e9, 1), "frac": round(nb / t / 1e9 / PEAK_HBM_GBPS, 4)}


# ----------------------------------------------------------------------------- ragged decode

def ragged_decode_step(steps: int, warmup: int, cpu: bool = False):
    """Selection + decode on decode_ragged (B=64, L_b in [16384, 131072], Lp=16), timed alone.

    Not part of the step above (and not of `value`): it reports the decode path at a batch
    large enough to amortise launches. Bounds are built once beforehand (they are updated
    when pages fill, not every step). The 19 GB cache and 0.6 GB of bounds exceed the
    Infinity Cache, so every step reads mostly HBM.
    """
    import torch
    import unified_block_sparse_amd as ubs
    from workloads import cases
    dev = torch.device("cuda:0")
    r = cases.decode_ragged(dev)
    bnd = torch.zeros((r.num_physical_pages, r.Hkv, r.P // r.Lp, 2, r.D), dtype=torch.bfloat16, device=dev)
    sel = torch.empty((r.B, r.Hkv, r.k_pages), dtype=torch.int32, device=dev)
    num = torch.empty((r.B, r.Hkv), dtype=torch.int32, device=dev)
    out = torch.empty((r.B, r.Hq, r.D), dtype=torch.float32, device=dev)
    ubs.build_page_bounds(r.k_cache, r.page_table, r.seq_lens_t, r.head_kind, r.Lp, bounds=bnd)

    def op_select():
        ubs.select_pages(r.q, bnd, r.page_table, r.seq_lens_t, r.head_kind, r.P, r.token_budget, selected=sel,
                         num_selected=num)

    def op_decode():
        ubs.sparse_decode(r.q, r.k_cache, r.v_cache, r.page_table, r.seq_lens_t, r.head_kind, sel, num,
                          r.sink_tokens, r.local_tokens, r.sm_scale, out=out)

    for _ in range(warmup):
        op_select()
        op_decode()
    torch.cuda.synchronize(dev)
    sel_h, num_h = sel.cpu().tolist(), num.cpu().tolist()
    sel_pages = [[sel_h[b][g][:num_h[b][g]] for g in range(r.Hkv)] for b in range(r.B)]
    _, b_select, b_decode = decode_bytes(r, sel_pages)
    stream = torch.cuda.current_stream(dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for s_ in range(steps):
        ev[s_][0].record(stream)
        op_select()
        ev[s_][1].record(stream)
        op_decode()
        ev[s_][2].record(stream)
    torch.cuda.synchronize(dev)
    t_sel = sum(e[0].elapsed_time(e[1]) for e in ev) / steps * 1e-3
    t_dec = sum(e[1].elapsed_time(e[2]) for e in ev) / steps * 1e-3
    t = t_sel + t_dec
    # selection reused over R = 4 steps (one select_pages, then four sparse_decode)
    R = 4
    er = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    er[0].record(stream)
    for _ in range(steps):
        op_select()
        for _ in range(R):
            op_decode()
    er[1].record(stream)
    torch.cuda.synchronize(dev)
    t_r = er[0].elapsed_time(er[1]) * 1e-3 / (steps * R)
    b_r = b_select / R + b_decode
    res = {"workload": "decode_ragged (B=64, L_b uniform in [16384, 131072], Hq=32, Hkv=8, D=128, P=64, Lp=16, "
                       "budget 4096, streaming 128 + 1024)",
           "ms": round(t * 1e3, 4), "bytes": b_select + b_decode,
           "gbps": round((b_select + b_decode) / t / 1e9, 1),
           "frac": round((b_select + b_decode) / t / 1e9 / PEAK_HBM_GBPS, 4),
           "select_pages": {"ms": round(t_sel * 1e3, 4), "bytes": b_select, "gbps": round(b_select / t_sel / 1e9, 1)},
           "sparse_decode": {"ms": round(t_dec * 1e3, 4), "bytes": b_decode, "gbps": round(b_decode / t_dec / 1e9, 1)},
           "selection_reused_4_steps": {"ms_per_step": round(t_r * 1e3, 4), "bytes_per_step": int(b_r),
                                        "gbps": round(b_r / t_r / 1e9, 1),
                                        "frac": round(b_r / t_r / 1e9 / PEAK_HBM_GBPS, 4)}}
    # build_page_bounds over the whole cache (once per filled page in serving; timed here
    # as its own pass: 19.3 GB of K/V, far beyond the Infinity Cache)
    b_bounds, _, _ = decode_bytes(r, sel_pages)
    n_b = max(2, steps // 4)
    eb = [torch.cuda.Event(enable_timing=True) for _ in range(n_b + 1)]
    for i in range(n_b):
        eb[i].record(stream)
        ubs.build_page_bounds(r.k_cache, r.page_table, r.seq_lens_t, r.head_kind, r.Lp, bounds=bnd)
    eb[n_b].record(stream)
    torch.cuda.synchronize(dev)
    tb = sorted(eb[i].elapsed_time(eb[i + 1]) * 1e-3 for i in range(n_b))
    t_b = tb[len(tb) // 2]
    res["build_page_bounds"] = {"ms": round(t_b * 1e3, 4), "bytes": int(b_bounds),
                                "gbps": round(b_bounds / t_b / 1e9, 1),
                                "frac": round(b_bounds / t_b / 1e9 / PEAK_HBM_GBPS, 4),
                                "note": f"median of {n_b} calls"}
    res["int4"] = ragged_int4(r, sel, num, sel_pages, b_select, op_select, steps, warmup)
    if cpu:
        # the oracle's whole step (bounds, selection, decode): every sequence when the host
        # has 48 GB or more, else 16 seeded ones (extrapolated by tokens)
        import numpy as np
        ram = _host_ram_bytes()
        if ram >= 48 * 2**30:
            batches = list(range(r.B))
        else:
            batches = sorted(np.random.default_rng(13).choice(r.B, size=16, replace=False).tolist())
        t = oracle_decode_sample(r, batches)
        scale = sum(r.seq_lens) / sum(r.seq_lens[b] for b in batches)
        what = (f"all {r.B} sequences" if len(batches) == r.B else
                f"16 seeded sequences of {r.B} ({sum(r.seq_lens[b] for b in batches)} tokens)")
        res["_oracle"] = {
                          "sample": f"{what}, {t:.2f} s (host RAM {ram / 2**30:.0f} GiB)" +
                                    ("" if len(batches) == r.B else
                                     f"; the step over all {r.B} extrapolated by tokens x {scale:.2f}"),
                          "step_s_extrapolated" if len(batches) < r.B else "step_s": round(t * scale, 2)}
    del r, bnd
    torch.cuda.empty_cache()
    return res


def ragged_int4(r, sel, num, sel_pages, b_select, op_select, steps: int, warmup: int):
    """INT4 pages of decode_ragged: quantize_kv_int4 over every valid token (read K and V
    bf16 rows, write codes and params), then steps of select_pages + sparse_decode_int4,
    timed call by call like the bf16 steps (the selection's 612 MB pass evicts the 184 MB
    of INT4 pages from the Infinity Cache before each decode, as in serving)."""
    import torch
    import unified_block_sparse_amd as ubs
    dev = r.q.device
    kc, vc, kp, vp = ubs.quantize_kv_int4(r.k_cache, r.v_cache, r.page_table, r.seq_lens_t)
    out = torch.empty((r.B, r.Hq, r.D), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def timed(f, n):
        for _ in range(warmup):
            f()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize(dev)
        e0.record(stream)
        for _ in range(n):
            f()
        e1.record(stream)
        torch.cuda.synchronize(dev)
        return e0.elapsed_time(e1) * 1e-3 / n

    t_q = timed(lambda: ubs.quantize_kv_int4(r.k_cache, r.v_cache, r.page_table, r.seq_lens_t,
                                             out=(kc, vc, kp, vp)), max(1, steps // 4))
    def op_decode4():
        ubs.sparse_decode_int4(r.q, kc, vc, kp, vp, r.page_table, r.seq_lens_t, r.head_kind, sel, num,
                               r.sink_tokens, r.local_tokens, r.sm_scale, out=out)

    for _ in range(warmup):
        op_select()
        op_decode4()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize(dev)
    for s_ in range(steps):
        ev[s_][0].record(stream)
        op_select()
        ev[s_][1].record(stream)
        op_decode4()
        ev[s_][2].record(stream)
    torch.cuda.synchronize(dev)
    t_sel = sum(e[0].elapsed_time(e[1]) for e in ev) / steps * 1e-3
    t_d = sum(e[1].elapsed_time(e[2]) for e in ev) / steps * 1e-3
    row4 = r.D // 2 + 4
    tokens = sum(r.seq_lens) * r.Hkv
    b_q = tokens * 2 * (r.D * 2 + row4)
    attended = 0
    for b, L in enumerate(r.seq_lens):
        for g in range(r.Hkv):
            if r.head_kind[g]:
                A = min(r.sink_tokens, L)
                attended += A + L - max(A, L - r.local_tokens)
            else:
                attended += sum(min(r.P, L - j * r.P) for j in sel_pages[b][g])
    q_bytes = r.B * r.Hq * r.D * 2
    b_d = attended * 2 * row4 + q_bytes + r.B * r.Hq * r.D * 4
    t_step = t_sel + t_d
    del kc, vc, kp, vp
    return {"quantize_kv_int4": {"ms": round(t_q * 1e3, 4), "bytes": b_q, "gbps": round(b_q / t_q / 1e9, 1),
                                 "frac": round(b_q / t_q / 1e9 / PEAK_HBM_GBPS, 4)},
            "sparse_decode_int4": {"ms": round(t_d * 1e3, 4), "bytes": b_d, "gbps": round(b_d / t_d / 1e9, 1),
                                   "frac": round(b_d / t_d / 1e9 / PEAK_HBM_GBPS, 4)},
            "step_select_plus_int4_decode": {"ms": round(t_step * 1e3, 4), "bytes": b_select + b_d,
                                             "gbps": round((b_select + b_d) / t_step / 1e9, 1),
                                             "frac": round((b_select + b_d) / t_step / 1e9 / PEAK_HBM_GBPS, 4)}}


# ----------------------------------------------------------------------------- single prefill legs

def time_calls(f, steps: int, warmup: int, stream):
    """Mean seconds per call of f over `steps` calls, HIP events on `stream` around each."""
    import torch
    for _ in range(warmup):
        f()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    torch.cuda.synchronize()
    for e in ev:
        e[0].record(stream)
        f()
        e[1].record(stream)
    torch.cuda.synchronize()
    ts = sorted(e[0].elapsed_time(e[1]) * 1e-3 for e in ev)
    return sum(ts) / len(ts), ts[0], ts[len(ts) // 2]


def prefill_leg(c, steps: int, warmup: int, cpu_rows: int = 0):
    """sparse_prefill of one case timed call by call: kept-tile TFLOP/s against the bf16
    MFMA peak. With cpu_rows > 0 the oracle is timed on that many rows per head while the
    inputs are resident."""
    import torch
    import unified_block_sparse_amd as ubs
    kept = kept_tile_count(c)
    flops = prefill_flops(c, kept)
    out = torch.empty((c.L, c.Hq, c.D), dtype=torch.float32, device=c.q.device)
    f = lambda: ubs.sparse_prefill(c.q, c.k_cache, c.v_cache, c.page_table, c.head_kind, c.block_mask,
                                   c.sink_tiles, c.local_tiles, c.T, c.sm_scale, out=out)
    t, t_min, t_med = time_calls(f, steps, warmup, torch.cuda.current_stream(c.q.device))
    res = {"workload": f"{c.name} (L={c.L}, Hq={c.Hq}, Hkv={c.Hkv}, D={c.D}, T={c.T}, P={c.P}, "
                       f"sink {c.sink_tiles} + local {c.local_tiles} tiles on streaming heads)",
           "calls": steps, "ms": round(t * 1e3, 4), "ms_min": round(t_min * 1e3, 4), "ms_median": round(t_med * 1e3, 4),
           "kept_tiles": kept, "tflop": round(flops / 1e12, 4), "tflops": round(flops / t / 1e12, 2),
           "frac": round(flops / t / 1e12 / PEAK_BF16_TFLOPS, 4)}
    del out
    if cpu_rows:
        t_s, t_fixed, full, n = oracle_prefill_sample(c, cpu_rows, seed=14)
        res["_oracle"] = {"rows_per_s": round(n * c.Hq / max(t_s - t_fixed, 1e-9), 1),
                          "sample": f"{n} rows (0, T-1, T, L-1, the rest seeded) x {c.Hq} heads, {t_s:.2f} s incl. {t_fixed:.2f} s "
                                    f"K/V gather; all {c.L} rows extrapolated",
                          "full_config_s_extrapolated": round(full, 1)}
    return res


# ----------------------------------------------------------------------------- serving-loop legs

def chunk_prefill(c, steps: int, warmup: int):
    """sparse_prefill_chunk: the last 8,192 query rows (64 query tiles) of prefill_llama8b
    over its whole 65,536-token cache, the last chunk of a chunked prefill. Kept-tile
    TFLOP/s of the chunk's query tiles against the bf16 MFMA peak."""
    import torch
    import unified_block_sparse_amd as ubs
    q0 = c.L - 8192
    i0 = q0 // c.T
    kept = kept_tile_count(c, first_tile=i0)
    flops = prefill_flops(c, kept)
    q = c.q[q0:].contiguous()
    mask = c.block_mask[:, i0:, :].contiguous()
    out = torch.empty((c.L - q0, c.Hq, c.D), dtype=torch.float32, device=c.q.device)
    f = lambda: ubs.sparse_prefill_chunk(q, c.k_cache, c.v_cache, c.page_table, c.L, q0, c.head_kind, mask,
                                         c.sink_tiles, c.local_tiles, c.T, c.sm_scale, out=out)
    t, t_min, t_med = time_calls(f, steps, warmup, torch.cuda.current_stream(c.q.device))
    del q, mask, out
    return {"workload": f"{c.name}: query rows {q0}..{c.L - 1} ({c.nT - i0} query tiles) over all {c.L} tokens",
            "calls": steps, "ms": round(t * 1e3, 4), "ms_median": round(t_med * 1e3, 4),
            "kept_tiles": kept, "tflop": round(flops / 1e12, 4), "tflops": round(flops / t / 1e12, 2),
            "frac": round(flops / t / 1e12 / PEAK_BF16_TFLOPS, 4)}


def append_leg(steps: int, warmup: int):
    """append_kv in the serving loop, with the dense heads' page bounds refreshed: one decoded
    token for each of 64 sequences of 2K-8K tokens (Llama-3-8B KV heads, P = 64, Lp = 16),
    and a 4,096-token prefill chunk for each of 4 sequences (P = Lp = 64). Every call writes
    the same tokens at the same positions (the lengths do not change), so repeated calls
    time one append. The calls are captured in a HIP graph and replayed (the binding's
    host work per call is longer than the GPU work of these appends); the chunk appends
    cycle over four cache instances, so that a call does not find the previous one's
    data in the 256 MB Infinity Cache. Algorithmic bytes: the new K and V rows read and
    written, the K rows of the dense heads' sub-pages holding a new token read (their
    valid rows, old and new) and those sub-pages' bounds written."""
    import numpy as np
    import torch
    import unified_block_sparse_amd as ubs
    from workloads import cases, gen
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    kind = [0, 0, 0, 0, 1, 1, 1, 1]
    rng = np.random.default_rng(21)
    res = {}
    for name, lens, n_new, Lp, R in (("decode_token", rng.integers(2048, 8193, size=64).tolist(), 1, 16, 1),
                                     ("prefill_chunk", [32768] * 4, 4096, 64, 4)):
        inst = []
        for r in range(R):
            d = cases.make_decode(f"append_{name}", lens, 32, 8, 128, 64, Lp, kind, 4096, 128, 512,
                                  1700 + n_new + r, dev)
            old_t = torch.tensor([L - n_new for L in lens], dtype=torch.int32, device=dev)
            k_new = gen.normal_bf16((d.B, n_new, d.Hkv, d.D), 1800 + n_new + r, 1, dev)
            v_new = gen.normal_bf16((d.B, n_new, d.Hkv, d.D), 1800 + n_new + r, 2, dev)
            bnd = ubs.build_page_bounds(d.k_cache, d.page_table, old_t, kind, Lp)
            inst.append((d, old_t, k_new, v_new, bnd))

        def run_all(reps):
            for _ in range(reps):
                for d, old_t, k_new, v_new, bnd in inst:
                    ubs.append_kv(k_new, v_new, d.page_table, old_t, kind, d.k_cache, d.v_cache, bounds=bnd, Lp=Lp)

        reps = max(1, 24 // R)
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            run_all(max(1, warmup))
        stream.wait_stream(side)
        torch.cuda.synchronize(dev)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run_all(reps)
        g.replay()
        torch.cuda.synchronize(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize(dev)
        t = e0.elapsed_time(e1) * 1e-3 / (steps * reps * R)
        d = inst[0][0]
        old = [L - n_new for L in lens]
        row = d.D * 2
        nd = kind.count(0)
        sub_rows = sum(L1 - (L0 // Lp) * Lp for L0, L1 in zip(old, lens))
        n_sub = sum((L1 - 1) // Lp - L0 // Lp + 1 for L0, L1 in zip(old, lens))
        nbytes = 2 * d.B * n_new * d.Hkv * 2 * row + nd * (sub_rows * row + n_sub * 2 * row)
        res[name] = {"workload": f"{d.B} sequences, {n_new} new token(s) each, Hkv={d.Hkv} (4 dense), D={d.D}, "
                                 f"P={d.P}, Lp={Lp}",
                     "ms": round(t * 1e3, 4), "bytes": int(nbytes),
                     "gbps": round(nbytes / t / 1e9, 1), "frac": round(nbytes / t / 1e9 / PEAK_HBM_GBPS, 4),
                     "note": f"HIP graph of {reps * R} calls over {R} cache instance(s), {steps} replays"}
        del inst, g
        torch.cuda.empty_cache()
    return res


# ----------------------------------------------------------------------------- main

def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(every workload here is a single-GPU shard).", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib)
        return
    if args.gemm_ceiling:
        gemm_ceiling()
        return
    legs = [x.strip() for x in args.legs.split(",") if x.strip()]
    bad = [x for x in legs if x not in LEGS]
    if bad:
        print(f"unknown legs {bad}; choose from {list(LEGS)}", file=sys.stderr)
        sys.exit(2)
    if args.no_cpu_baseline and "cpu" in legs:
        legs.remove("cpu")
    if args.no_ragged and "ragged" in legs:
        legs.remove("ragged")
    cpu = "cpu" in legs
    import torch
    import unified_block_sparse_amd as ubs
    from workloads import cases

    ubs.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    oracle_extra = {}
    per_config = {}
    legs_out = {}
    result = None

    if "step" in legs:
        c = cases.prefill_llama8b(dev)
        d = cases.decode_llama8b(dev)
        kept = kept_tile_count(c)
        out = torch.empty((c.L, c.Hq, c.D), dtype=torch.float32, device=dev)
        bnd = torch.zeros((d.num_physical_pages, d.Hkv, d.P // d.Lp, 2, d.D), dtype=torch.bfloat16, device=dev)
        sel = torch.empty((d.B, d.Hkv, d.k_pages), dtype=torch.int32, device=dev)
        num = torch.empty((d.B, d.Hkv), dtype=torch.int32, device=dev)
        dout = torch.empty((d.B, d.Hq, d.D), dtype=torch.float32, device=dev)

        def op_prefill():
            ubs.sparse_prefill(c.q, c.k_cache, c.v_cache, c.page_table, c.head_kind, c.block_mask, c.sink_tiles,
                               c.local_tiles, c.T, c.sm_scale, out=out)

        def op_bounds():
            ubs.build_page_bounds(d.k_cache, d.page_table, d.seq_lens_t, d.head_kind, d.Lp, bounds=bnd)

        def op_select():
            ubs.select_pages(d.q, bnd, d.page_table, d.seq_lens_t, d.head_kind, d.P, d.token_budget, selected=sel,
                             num_selected=num)

        def op_decode():
            ubs.sparse_decode(d.q, d.k_cache, d.v_cache, d.page_table, d.seq_lens_t, d.head_kind, sel, num,
                              d.sink_tokens, d.local_tokens, d.sm_scale, out=dout)

        # The bounds are built before the prefill so that the prefill's > 1.5 GB stream evicts
        # the K pages build_page_bounds just read: selection and decode then read cold HBM.
        ops = [("build_page_bounds", op_bounds), ("sparse_prefill", op_prefill), ("select_pages", op_select),
               ("sparse_decode", op_decode)]
        for _ in range(args.warmup):
            for _, f in ops:
                f()
        torch.cuda.synchronize(dev)
        flops = prefill_flops(c, kept)

        # ---- timed region: K whole steps, events between the ops (same stream as the kernels)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(ops) + 1)] for _ in range(args.steps)]
        torch.cuda.synchronize(dev)
        t0 = time.perf_counter()
        for s in range(args.steps):
            ev[s][0].record(stream)
            for i, (_, f) in enumerate(ops):
                f()
                ev[s][i + 1].record(stream)
        torch.cuda.synchronize(dev)
        wall = time.perf_counter() - t0
        per_op = {name: sum(ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(args.steps)) / args.steps * 1e-3
                  for i, (name, _) in enumerate(ops)}
        i_pf = [name for name, _ in ops].index("sparse_prefill")
        t_pf_all = sorted(ev[s][i_pf].elapsed_time(ev[s][i_pf + 1]) for s in range(args.steps))
        # the selection every timed step made (the same in each: same inputs)
        sel_h, num_h = sel.cpu().tolist(), num.cpu().tolist()
        sel_pages = [[sel_h[b][g][:num_h[b][g]] for g in range(d.Hkv)] for b in range(d.B)]
        b_bounds, b_select, b_decode = decode_bytes(d, sel_pages)
        ms_per_step = wall / args.steps * 1e3
        step_s = wall / args.steps

        ideal = {
            "sparse_prefill": flops / (PEAK_BF16_TFLOPS * 1e12),
            "build_page_bounds": b_bounds / (PEAK_HBM_GBPS * 1e9),
            "select_pages": b_select / (PEAK_HBM_GBPS * 1e9),
            "sparse_decode": b_decode / (PEAK_HBM_GBPS * 1e9),
        }
        ideal_s = sum(ideal.values())
        value = 100.0 * ideal_s / step_s

        t_pf = per_op["sparse_prefill"]
        achieved = flops / t_pf / 1e12
        traffic = None
        if os.path.exists(TRAFFIC_FILE):
            tr = json.load(open(TRAFFIC_FILE))
            if tr.get("kernel_source_hash") == kernel_source_hash():
                traffic = tr.get("hbm_bytes_per_launch")
        roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                    "kernel": "prefill_kernel<128,128> (sparse_prefill)", "flops_per_launch": flops,
                    "kept_tiles": kept, "avg_launch_ms": round(t_pf * 1e3, 4)}
        t_dstep = per_op["select_pages"] + per_op["sparse_decode"]
        breakdown = {
            name: {"ms": round(per_op[name] * 1e3, 4), "roofline_ms": round(ideal[name] * 1e3, 4),
                   "frac": round(ideal[name] / per_op[name], 4)} for name, _ in ops}
        breakdown["sparse_prefill"]["tflops"] = round(achieved, 2)
        breakdown["sparse_prefill"]["ms_median"] = round(t_pf_all[len(t_pf_all) // 2], 4)
        breakdown["sparse_prefill"]["ms_min"] = round(t_pf_all[0], 4)
        breakdown["build_page_bounds"]["gbps"] = round(b_bounds / per_op["build_page_bounds"] / 1e9, 1)
        breakdown["select_pages"]["gbps"] = round(b_select / per_op["select_pages"] / 1e9, 1)
        breakdown["sparse_decode"]["gbps"] = round(b_decode / per_op["sparse_decode"] / 1e9, 1)
        breakdown["decode_step"] = {"ms": round(t_dstep * 1e3, 4), "bytes": b_select + b_decode,
                                    "gbps": round((b_select + b_decode) / t_dstep / 1e9, 1),
                                    "frac": round((b_select + b_decode) / t_dstep / 1e9 / PEAK_HBM_GBPS, 4)}
        per_config["prefill_llama8b"] = {"frac": round(achieved / PEAK_BF16_TFLOPS, 4), "bound": "mfma",
                                         "ms": round(t_pf * 1e3, 4), "tflops": round(achieved, 2)}
        result = {
            "metric": METRIC,
            "value": round(value, 3),
            "unit": "% of MI355X roofline",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": round(ms_per_step, 4),
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": "llama3_8b_layer: prefill_llama8b (L=65536, Hq=32, Hkv=8, D=128, T=128, "
                                   "half KV heads streaming) + decode_llama8b (B=4, L=32768, P=64, budget 4096)",
                       "prefill_kept_tiles": kept, "prefill_tflop": round(flops / 1e12, 4),
                       "decode_bytes": b_bounds + b_select + b_decode},
            "roofline": roofline,
            "per_config": per_config,
            "breakdown": breakdown,
            "context": PAGES_CONTEXT,
        }
        legs_out = breakdown
        del out
        if "mask" in legs:
            breakdown["estimate_block_mask"] = mask_estimation(c, args.steps, args.warmup)
        if "chunk" in legs:
            breakdown["sparse_prefill_chunk"] = chunk_prefill(c, max(3, args.steps // 2), min(args.warmup, 2))
        if cpu:
            cpu_args = (c, d, args.cpu_rows_per_head, ideal_s)
        else:
            del c, d
        torch.cuda.empty_cache()
    elif "mask" in legs or "chunk" in legs:
        c = cases.prefill_llama8b(dev)
        if "mask" in legs:
            legs_out["estimate_block_mask"] = mask_estimation(c, args.steps, args.warmup)
        if "chunk" in legs:
            legs_out["sparse_prefill_chunk"] = chunk_prefill(c, max(3, args.steps // 2), min(args.warmup, 2))
        del c
        torch.cuda.empty_cache()

    if "tiny" in legs:
        r = prefill_leg(cases.prefill_tiny(dev), args.steps, args.warmup)
        legs_out["prefill_tiny"] = r
        per_config["prefill_tiny"] = {"frac": r["frac"], "bound": "mfma", "ms": r["ms"], "tflops": r["tflops"],
                                      "note": "276 kept 64x64 tiles, 0.29 GFLOP: launch-bound, parity case"}
    if "graph" in legs:
        r = decode_graph_step()
        legs_out["decode_step_graph"] = r
        per_config["decode_llama8b_step"] = {"frac": r["frac"], "bound": "hbm", "ms": r["ms"], "gbps": r["gbps"],
                                             "note": "sparse_decode_select (scores, decode with in-kernel top-k, merge), HIP graph over 24 instances"}
    if "varlen" in legs:
        legs_out["sparse_prefill_varlen"] = varlen_prefill(max(2, args.steps // 4), 2)
    if "append" in legs:
        legs_out["append_kv"] = append_leg(args.steps, args.warmup)
    if "ragged" in legs:
        r = ragged_decode_step(args.steps, args.warmup, cpu=cpu)
        if "_oracle" in r:
            oracle_extra["decode_ragged"] = r.pop("_oracle")
        legs_out["decode_ragged_step"] = r
        per_config["decode_ragged_step"] = {"frac": r["frac"], "bound": "hbm", "ms": r["ms"], "gbps": r["gbps"],
                                            "note": "select_pages + sparse_decode, 64 sequences"}
    if "extreme" in legs:
        c5 = cases.prefill_extreme(dev)
        r = prefill_leg(c5, max(2, args.steps // 4), min(args.warmup, 1), cpu_rows=32 if cpu else 0)
        del c5
        torch.cuda.empty_cache()
        if "_oracle" in r:
            oracle_extra["prefill_extreme"] = r.pop("_oracle")
        legs_out["prefill_extreme"] = r
        per_config["prefill_extreme"] = {"frac": r["frac"], "bound": "mfma", "ms": r["ms"], "tflops": r["tflops"]}

    if "peaks" in legs:
        pk = measured_peaks()
        legs_out["measured_peaks"] = pk
        for name, pc in per_config.items():
            if pc.get("bound") == "mfma" and "tflops" in pc:
                pc["frac_of_measured"] = round(pc["tflops"] / pk["gemm_bf16_tflops"], 4)
            elif pc.get("bound") == "hbm" and "gbps" in pc:
                pc["frac_of_measured"] = round(pc["gbps"] / pk["hbm_read_gbps"], 4)
        if result is not None:
            result["measured_peaks"] = pk

    if result is None:
        print(json.dumps({"legs": legs_out, "per_config": per_config, "oracle": oracle_extra}), flush=True)
        return
    if cpu:
        result["cpu_baseline"] = cpu_baseline(*cpu_args, oracle_extra)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
