"""ctypes binding of libubs.so (the C ABI in include/ubs.h).

Argument marshalling only: tensors are checked for dtype, device, shape and
contiguity, then their device pointers and the current HIP stream go to the C
entry points, which run every step on the GPU. There is no fallback: if the
library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional, Sequence, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# UBS_LIBRARY names another build of the same library (the host-sanitizer build that the
# CPU-side ABI tests run under); by default the in-tree libubs.so
LIB_PATH = os.environ.get("UBS_LIBRARY") or os.path.join(_HERE, "libubs.so")

UBS_OK = 0
ERR_NAMES = {-1: "INVALID_ARGUMENT", -2: "UNSUPPORTED", -3: "WORKSPACE_TOO_SMALL", -4: "HIP_ERROR",
             -5: "OUT_OF_RANGE"}
CHECK_STATUS_BYTES = 64
EXPORTED = ("sparse_prefill", "sparse_prefill_chunk", "sparse_prefill_varlen", "build_page_bounds", "select_pages", "ubs_select_workspace_size",
            "sparse_decode", "ubs_decode_workspace_size", "estimate_block_mask", "ubs_mask_workspace_size",
            "append_kv", "quantize_kv_int4", "sparse_decode_int4", "sparse_decode_static",
            "sparse_decode_select", "ubs_decode_select_workspace_size",
            "ubs_check_paged", "ubs_check_status",
            "ubs_bench_read", "ubs_bench_mfma", "ubs_bench_mfma_waves",
            "ubs_last_error", "ubs_version")


class UBSError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed with {ERR_NAMES.get(code, code)} ({code}): {msg}")
        self.code = code


_lib = None
_lock = threading.Lock()

_p = ctypes.c_void_p
_i = ctypes.c_int32
_f = ctypes.c_float
_sz = ctypes.c_size_t


def load() -> ctypes.CDLL:
    """Load libubs.so (built by unified_block_sparse_amd.build); raises if it is missing."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -m unified_block_sparse_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        lib.ubs_last_error.restype = ctypes.c_char_p
        lib.ubs_last_error.argtypes = []
        lib.ubs_version.restype = ctypes.c_int
        lib.ubs_version.argtypes = []
        lib.sparse_prefill.restype = ctypes.c_int
        lib.sparse_prefill.argtypes = [_p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _p, _p, _i, _i, _f, _p, _p, _p]
        lib.sparse_prefill_chunk.restype = ctypes.c_int
        lib.sparse_prefill_chunk.argtypes = [_p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _p, _p, _i, _i, _f, _p, _p,
                                             _p]
        lib.sparse_prefill_varlen.restype = ctypes.c_int
        lib.sparse_prefill_varlen.argtypes = [_p, _p, _p, _p, _i, _p, _i, _i, _i, _i, _i, _i, _i, _i, _p, _p, _i, _i,
                                              _f, _p, _p, _p]
        lib.build_page_bounds.restype = ctypes.c_int
        lib.build_page_bounds.argtypes = [_p, _p, _p, _i, _i, _i, _i, _i, _i, _p, _p, _p]
        lib.ubs_select_workspace_size.restype = _sz
        lib.ubs_select_workspace_size.argtypes = [_i, _i, _i]
        lib.select_pages.restype = ctypes.c_int
        lib.select_pages.argtypes = [_p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _sz, _p]
        lib.ubs_decode_workspace_size.restype = _sz
        lib.ubs_decode_workspace_size.argtypes = [_i, _i, _i, _i, _i, _i, _i, _i]
        lib.sparse_decode.restype = ctypes.c_int
        lib.sparse_decode.argtypes = [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _p, _p, _p, _i, _i, _i,
                                      _f, _p, _p, _p, _sz, _p]
        lib.sparse_decode_int4.restype = ctypes.c_int
        lib.sparse_decode_int4.argtypes = [_p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _p, _p, _p, _i, _i,
                                           _i, _f, _p, _p, _p, _sz, _p]
        lib.ubs_decode_select_workspace_size.restype = _sz
        lib.ubs_decode_select_workspace_size.argtypes = [_i, _i, _i, _i, _i, _i, _i, _i, _i]
        lib.sparse_decode_select.restype = ctypes.c_int
        lib.sparse_decode_select.argtypes = [_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _i, _p, _i, _i,
                                             _f, _p, _p, _p, _p, _p, _sz, _p]
        lib.sparse_decode_static.restype = ctypes.c_int
        lib.sparse_decode_static.argtypes = [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _p, _p, _p, _i, _i, _i,
                                             _f, _p, _p, _p]
        lib.quantize_kv_int4.restype = ctypes.c_int
        lib.quantize_kv_int4.argtypes = [_p, _p, _p, _p, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p]
        lib.append_kv.restype = ctypes.c_int
        lib.append_kv.argtypes = [_p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p]
        lib.ubs_mask_workspace_size.restype = _sz
        lib.ubs_mask_workspace_size.argtypes = [_i, _i, _i, _i, _i]
        lib.estimate_block_mask.restype = ctypes.c_int
        lib.estimate_block_mask.argtypes = [_p, _p, _p, _i, _i, _i, _i, _i, _i, _p, _i, _i, _p, _p, _sz, _p]
        lib.ubs_check_paged.restype = ctypes.c_int
        lib.ubs_check_paged.argtypes = [_p, _i, _i, _p, _p, _i, _i, _p, _i, _p, _p, _i, _p, _p]
        lib.ubs_check_status.restype = ctypes.c_int
        lib.ubs_check_status.argtypes = [_p, _p]
        lib.ubs_bench_read.restype = ctypes.c_int
        lib.ubs_bench_read.argtypes = [_p, _sz, _p, _p]
        lib.ubs_bench_mfma.restype = ctypes.c_int
        lib.ubs_bench_mfma.argtypes = [_i, _p, _p]
        lib.ubs_bench_mfma_waves.restype = ctypes.c_int64
        lib.ubs_bench_mfma_waves.argtypes = []
        _lib = lib
        return lib


def _check(fn: str, rc: int):
    if rc != UBS_OK:
        raise UBSError(fn, rc, load().ubs_last_error().decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _kinds(head_kind: Sequence[int]) -> ctypes.Array:
    return (ctypes.c_uint8 * len(head_kind))(*[int(x) for x in head_kind])


def _need(t: torch.Tensor, name: str, dtype, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


# ----------------------------------------------------------------------------- workspaces

_ws_cache = {}


def _workspace(kind: str, device, stream: int, nbytes: int) -> torch.Tensor:
    """Per (kind, device, stream) workspace, grown on demand.

    Calls ordered on one stream may share it; calls on different streams get their own.
    """
    key = (kind, device, stream)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        _ws_cache[key] = buf
    return buf


# ----------------------------------------------------------------------------- entry points

def sparse_prefill(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   page_table: torch.Tensor, head_kind: Sequence[int], block_mask: Optional[torch.Tensor],
                   sink_tiles: int, local_tiles: int, T: int, sm_scale: float,
                   out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                   return_lse: bool = False):
    """Block-sparse / streaming prefill attention of one sequence (see include/ubs.h).

    q bf16 [L, Hq, D]; k_cache, v_cache bf16 [NP, Hkv, P, D]; page_table int32 [>= ceil(L/P)];
    block_mask uint8 [Hq, nT, nT] (None when every KV head streams). Returns out fp32
    [L, Hq, D] (and lse fp32 [Hq, L] with return_lse).
    """
    lib = load()
    L, Hq, D = q.shape
    NP, Hkv, P, D2 = k_cache.shape
    dev = q.device
    _need(q, "q", torch.bfloat16, device=dev)
    _need(k_cache, "k_cache", torch.bfloat16, device=dev)
    _need(v_cache, "v_cache", torch.bfloat16, shape=k_cache.shape, device=dev)
    _need(page_table, "page_table", torch.int32, device=dev)
    if D2 != D:
        raise ValueError("q and k_cache head dims differ")
    if len(head_kind) != Hkv:
        raise ValueError("head_kind must have one entry per KV head")
    nT = (L + T - 1) // T
    if page_table.numel() < (L + P - 1) // P:
        raise ValueError("page_table is shorter than ceil(L / P)")
    if block_mask is not None:
        _need(block_mask, "block_mask", torch.uint8, shape=(Hq, nT, nT), device=dev)
    if out is None:
        out = torch.empty((L, Hq, D), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, shape=(L, Hq, D), device=dev)
    if return_lse and lse is None:
        lse = torch.empty((Hq, L), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, shape=(Hq, L), device=dev)
    rc = lib.sparse_prefill(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table), L, Hq, Hkv, D, P, T,
                            _kinds(head_kind), _ptr(block_mask), sink_tiles, local_tiles, float(sm_scale),
                            _ptr(out), _ptr(lse), _stream(dev))
    _check("sparse_prefill", rc)
    return (out, lse) if return_lse else out


def sparse_prefill_varlen(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                          page_table: torch.Tensor, cu_seqlens: torch.Tensor, max_seqlen: int,
                          head_kind: Sequence[int], block_mask: Optional[torch.Tensor], sink_tiles: int,
                          local_tiles: int, T: int, sm_scale: float, out: Optional[torch.Tensor] = None,
                          lse: Optional[torch.Tensor] = None, return_lse: bool = False):
    """Block-sparse / streaming prefill of B sequences in one call (see include/ubs.h).

    q bf16 [total_q, Hq, D] (packed rows); page_table int32 [B, max_pages]; cu_seqlens int32
    [B + 1] on the GPU; max_seqlen >= every length; block_mask uint8 [B, Hq, nT_max, nT_max]
    with nT_max = ceil(max_seqlen / T). Returns out fp32 [total_q, Hq, D] (and lse fp32
    [Hq, total_q] with return_lse).
    """
    lib = load()
    total_q, Hq, D = q.shape
    NP, Hkv, P, D2 = k_cache.shape
    B, max_pages = page_table.shape
    dev = q.device
    _need(q, "q", torch.bfloat16, device=dev)
    _need(k_cache, "k_cache", torch.bfloat16, device=dev)
    _need(v_cache, "v_cache", torch.bfloat16, shape=k_cache.shape, device=dev)
    _need(page_table, "page_table", torch.int32, device=dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, shape=(B + 1,), device=dev)
    if D2 != D:
        raise ValueError("q and k_cache head dims differ")
    if len(head_kind) != Hkv:
        raise ValueError("head_kind must have one entry per KV head")
    nTm = (max_seqlen + T - 1) // T
    if block_mask is not None:
        _need(block_mask, "block_mask", torch.uint8, shape=(B, Hq, nTm, nTm), device=dev)
    if out is None:
        out = torch.empty((total_q, Hq, D), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, shape=(total_q, Hq, D), device=dev)
    if return_lse and lse is None:
        lse = torch.empty((Hq, total_q), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, shape=(Hq, total_q), device=dev)
    rc = lib.sparse_prefill_varlen(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table), max_pages,
                                   _ptr(cu_seqlens), B, int(max_seqlen), total_q, Hq, Hkv, D, P, T,
                                   _kinds(head_kind), _ptr(block_mask), sink_tiles, local_tiles, float(sm_scale),
                                   _ptr(out), _ptr(lse), _stream(dev))
    _check("sparse_prefill_varlen", rc)
    return (out, lse) if return_lse else out


def build_page_bounds(k_cache: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor,
                      head_kind: Sequence[int], Lp: int, bounds: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Per-page key min/max of dense KV heads: bounds bf16 [NP, Hkv, P/Lp, 2, D]."""
    lib = load()
    NP, Hkv, P, D = k_cache.shape
    B, max_pages = page_table.shape
    dev = k_cache.device
    _need(k_cache, "k_cache", torch.bfloat16, device=dev)
    _need(page_table, "page_table", torch.int32, device=dev)
    _need(seq_lens, "seq_lens", torch.int32, shape=(B,), device=dev)
    if P % Lp:
        raise ValueError("Lp must divide P")
    if bounds is None:
        bounds = torch.zeros((NP, Hkv, P // Lp, 2, D), dtype=torch.bfloat16, device=dev)
    _need(bounds, "bounds", torch.bfloat16, shape=(NP, Hkv, P // Lp, 2, D), device=dev)
    rc = lib.build_page_bounds(_ptr(k_cache), _ptr(page_table), _ptr(seq_lens), B, max_pages, Hkv, D, P, Lp,
                               _kinds(head_kind), _ptr(bounds), _stream(dev))
    _check("build_page_bounds", rc)
    return bounds


def select_pages(q: torch.Tensor, bounds: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor,
                 head_kind: Sequence[int], P: int, token_budget: int,
                 selected: Optional[torch.Tensor] = None, num_selected: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Top-k page selection: returns (selected int32 [B, Hkv, k], num_selected int32 [B, Hkv])."""
    lib = load()
    B, Hq, D = q.shape
    NP, Hkv, U, two, D2 = bounds.shape
    _, max_pages = page_table.shape
    dev = q.device
    _need(q, "q", torch.bfloat16, device=dev)
    _need(bounds, "bounds", torch.bfloat16, device=dev)
    _need(page_table, "page_table", torch.int32, shape=(B, max_pages), device=dev)
    _need(seq_lens, "seq_lens", torch.int32, shape=(B,), device=dev)
    if two != 2 or D2 != D or P % U:
        raise ValueError("bounds must be [NP, Hkv, P/Lp, 2, D]")
    Lp = P // U
    if token_budget <= 0 or token_budget % P:
        raise ValueError("token_budget must be a positive multiple of P")
    k = token_budget // P
    if selected is None:
        selected = torch.empty((B, Hkv, k), dtype=torch.int32, device=dev)
    if num_selected is None:
        num_selected = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
    _need(selected, "selected", torch.int32, shape=(B, Hkv, k), device=dev)
    _need(num_selected, "num_selected", torch.int32, shape=(B, Hkv), device=dev)
    st = _stream(dev)
    need = lib.ubs_select_workspace_size(B, max_pages, Hkv)
    if workspace is None:
        workspace = _workspace("select", dev, st, need)
    rc = lib.select_pages(_ptr(q), _ptr(bounds), _ptr(page_table), _ptr(seq_lens), B, max_pages, Hq, Hkv, D, P,
                          Lp, token_budget, _kinds(head_kind), _ptr(selected), _ptr(num_selected),
                          _ptr(workspace), workspace.numel() * workspace.element_size(), st)
    _check("select_pages", rc)
    return selected, num_selected


def sparse_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, page_table: torch.Tensor,
                  seq_lens: torch.Tensor, head_kind: Sequence[int], selected: Optional[torch.Tensor],
                  num_selected: Optional[torch.Tensor], sink_tokens: int, local_tokens: int, sm_scale: float,
                  out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                  return_lse: bool = False, workspace: Optional[torch.Tensor] = None):
    """Sparse paged GQA decode: out fp32 [B, Hq, D] (and lse fp32 [B, Hq] with return_lse)."""
    lib = load()
    B, Hq, D = q.shape
    NP, Hkv, P, D2 = k_cache.shape
    _, max_pages = page_table.shape
    dev = q.device
    _need(q, "q", torch.bfloat16, device=dev)
    _need(k_cache, "k_cache", torch.bfloat16, device=dev)
    _need(v_cache, "v_cache", torch.bfloat16, shape=k_cache.shape, device=dev)
    _need(page_table, "page_table", torch.int32, shape=(B, max_pages), device=dev)
    _need(seq_lens, "seq_lens", torch.int32, shape=(B,), device=dev)
    if D2 != D:
        raise ValueError("q and k_cache head dims differ")
    if selected is not None:
        _need(selected, "selected", torch.int32, device=dev)
        if selected.dim() != 3 or selected.shape[:2] != (B, Hkv):
            raise ValueError("selected must be [B, Hkv, max_selected]")
        max_selected = selected.shape[2]
    else:
        max_selected = 0
    if num_selected is not None:
        _need(num_selected, "num_selected", torch.int32, shape=(B, Hkv), device=dev)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, shape=(B, Hq, D), device=dev)
    if return_lse and lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, shape=(B, Hq), device=dev)
    st = _stream(dev)
    need = lib.ubs_decode_workspace_size(B, Hq, Hkv, D, P, max_selected, sink_tokens, local_tokens)
    if workspace is None:
        workspace = _workspace("decode", dev, st, need)
    rc = lib.sparse_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table), _ptr(seq_lens), B, max_pages,
                           Hq, Hkv, D, P, _kinds(head_kind), _ptr(selected), _ptr(num_selected), max_selected,
                           sink_tokens, local_tokens, float(sm_scale), _ptr(out), _ptr(lse), _ptr(workspace),
                           workspace.numel() * workspace.element_size(), st)
    _check("sparse_decode", rc)
    return (out, lse) if return_lse else out


def sparse_decode_select(q: torch.Tensor, bounds: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                         page_table: torch.Tensor, seq_lens: torch.Tensor, head_kind: Sequence[int], P: int,
                         token_budget: int, sink_tokens: int, local_tokens: int, sm_scale: float,
                         out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                         return_lse: bool = False, selected: Optional[torch.Tensor] = None,
                         num_selected: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """select_pages then sparse_decode in one call (see include/ubs.h). Returns (out, selected,
    num_selected), and lse after out with return_lse: out fp32 [B, Hq, D], selected int32
    [B, Hkv, token_budget / P], num_selected int32 [B, Hkv]."""
    lib = load()
    B, Hq, D = q.shape
    NP, Hkv, P2, D2 = k_cache.shape
    NPb, Hkv2, U, two, D3 = bounds.shape
    _, max_pages = page_table.shape
    dev = q.device
    _need(q, "q", torch.bfloat16, device=dev)
    _need(bounds, "bounds", torch.bfloat16, device=dev)
    _need(k_cache, "k_cache", torch.bfloat16, device=dev)
    _need(v_cache, "v_cache", torch.bfloat16, shape=k_cache.shape, device=dev)
    _need(page_table, "page_table", torch.int32, shape=(B, max_pages), device=dev)
    _need(seq_lens, "seq_lens", torch.int32, shape=(B,), device=dev)
    if P2 != P or D2 != D or D3 != D or Hkv2 != Hkv or two != 2 or P % U:
        raise ValueError("k_cache must be [NP, Hkv, P, D] and bounds [NP, Hkv, P/Lp, 2, D]")
    Lp = P // U
    if token_budget <= 0 or token_budget % P:
        raise ValueError("token_budget must be a positive multiple of P")
    k = token_budget // P
    if selected is None:
        selected = torch.empty((B, Hkv, k), dtype=torch.int32, device=dev)
    if num_selected is None:
        num_selected = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
    _need(selected, "selected", torch.int32, shape=(B, Hkv, k), device=dev)
    _need(num_selected, "num_selected", torch.int32, shape=(B, Hkv), device=dev)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, shape=(B, Hq, D), device=dev)
    if return_lse and lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, shape=(B, Hq), device=dev)
    st = _stream(dev)
    need = lib.ubs_decode_select_workspace_size(B, max_pages, Hq, Hkv, D, P, token_budget, sink_tokens,
                                                local_tokens)
    if workspace is None:
        workspace = _workspace("decode_select", dev, st, need)
    rc = lib.sparse_decode_select(_ptr(q), _ptr(bounds), _ptr(k_cache), _ptr(v_cache), _ptr(page_table),
                                  _ptr(seq_lens), B, max_pages, Hq, Hkv, D, P, Lp, token_budget, _kinds(head_kind),
                                  sink_tokens, local_tokens, float(sm_scale), _ptr(selected), _ptr(num_selected),
                                  _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                  st)
    _check("sparse_decode_select", rc)
    return (out, lse, selected, num_selected) if return_lse else (out, selected, num_selected)


def quantize_kv_int4(k_cache: torch.Tensor, v_cache: torch.Tensor, page_table: torch.Tensor,
                     seq_lens: torch.Tensor, out: Optional[Tuple[torch.Tensor, ...]] = None):
    """INT4 pages of the valid tokens of every sequence (see include/ubs.h).

    k_cache, v_cache bf16 [NP, Hkv, P, D]; page_table int32 [B, max_pages]; seq_lens int32 [B].
    Returns the tuple (k_codes uint8 [NP, Hkv, P, D/2], v_codes uint8 [NP, Hkv, D, P/2] (channel-
    major), k_params, v_params int16 [NP, Hkv, P, 2] holding fp16 (scale, zero) bits). What is
    not written (rows that are not valid tokens; V words with no valid token) keeps what `out`
    held (zeros when out is None).
    """
    lib = load()
    NP, Hkv, P, D = k_cache.shape
    B, max_pages = page_table.shape
    dev = k_cache.device
    _need(k_cache, "k_cache", torch.bfloat16, device=dev)
    _need(v_cache, "v_cache", torch.bfloat16, shape=k_cache.shape, device=dev)
    _need(page_table, "page_table", torch.int32, shape=(B, max_pages), device=dev)
    _need(seq_lens, "seq_lens", torch.int32, shape=(B,), device=dev)
    if out is None:
        out = (torch.zeros((NP, Hkv, P, D // 2), dtype=torch.uint8, device=dev),
               torch.zeros((NP, Hkv, D, P // 2), dtype=torch.uint8, device=dev),
               torch.zeros((NP, Hkv, P, 2), dtype=torch.int16, device=dev),
               torch.zeros((NP, Hkv, P, 2), dtype=torch.int16, device=dev))
    kc, vc, kp, vp = out
    for t, name, dt, shp in ((kc, "k_codes", torch.uint8, (NP, Hkv, P, D // 2)),
                             (vc, "v_codes", torch.uint8, (NP, Hkv, D, P // 2)),
                             (kp, "k_params", torch.int16, (NP, Hkv, P, 2)),
                             (vp, "v_params", torch.int16, (NP, Hkv, P, 2))):
        _need(t, name, dt, shape=shp, device=dev)
    rc = lib.quantize_kv_int4(_ptr(k_cache), _ptr(v_cache), _ptr(page_table), _ptr(seq_lens), B, max_pages, Hkv,
                              D, P, _ptr(kc), _ptr(vc), _ptr(kp), _ptr(vp), _stream(dev))
    _check("quantize_kv_int4", rc)
    return kc, vc, kp, vp


def sparse_decode_int4(q: torch.Tensor, k_codes: torch.Tensor, v_codes: torch.Tensor, k_params: torch.Tensor,
                       v_params: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor,
                       head_kind: Sequence[int], selected: Optional[torch.Tensor],
                       num_selected: Optional[torch.Tensor], sink_tokens: int, local_tokens: int, sm_scale: float,
                       out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                       return_lse: bool = False, workspace: Optional[torch.Tensor] = None):
    """sparse_decode over INT4 pages (k_codes uint8 [NP, Hkv, P, D/2], v_codes uint8 [NP, Hkv, D, P/2],
    params int16 [NP, Hkv, P, 2]; see include/ubs.h)."""
    lib = load()
    B, Hq, D = q.shape
    NP, Hkv, P, D2 = k_codes.shape
    _, max_pages = page_table.shape
    dev = q.device
    _need(q, "q", torch.bfloat16, device=dev)
    _need(k_codes, "k_codes", torch.uint8, device=dev)
    _need(v_codes, "v_codes", torch.uint8, shape=(NP, Hkv, D2 * 2, P // 2), device=dev)
    _need(k_params, "k_params", torch.int16, shape=(NP, Hkv, P, 2), device=dev)
    _need(v_params, "v_params", torch.int16, shape=(NP, Hkv, P, 2), device=dev)
    _need(page_table, "page_table", torch.int32, shape=(B, max_pages), device=dev)
    _need(seq_lens, "seq_lens", torch.int32, shape=(B,), device=dev)
    if 2 * D2 != D:
        raise ValueError("q's head dim must be twice the codes' last dim")
    if selected is not None:
        _need(selected, "selected", torch.int32, device=dev)
        if selected.dim() != 3 or selected.shape[:2] != (B, Hkv):
            raise ValueError("selected must be [B, Hkv, max_selected]")
        max_selected = selected.shape[2]
    else:
        max_selected = 0
    if num_selected is not None:
        _need(num_selected, "num_selected", torch.int32, shape=(B, Hkv), device=dev)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, shape=(B, Hq, D), device=dev)
    if return_lse and lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, shape=(B, Hq), device=dev)
    st = _stream(dev)
    need = lib.ubs_decode_workspace_size(B, Hq, Hkv, D, P, max_selected, sink_tokens, local_tokens)
    if workspace is None:
        workspace = _workspace("decode", dev, st, need)
    rc = lib.sparse_decode_int4(_ptr(q), _ptr(k_codes), _ptr(v_codes), _ptr(k_params), _ptr(v_params),
                                _ptr(page_table), _ptr(seq_lens), B, max_pages, Hq, Hkv, D, P, _kinds(head_kind),
                                _ptr(selected), _ptr(num_selected), max_selected, sink_tokens, local_tokens,
                                float(sm_scale), _ptr(out), _ptr(lse), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), st)
    _check("sparse_decode_int4", rc)
    return (out, lse) if return_lse else out


def estimate_block_mask(q: torch.Tensor, k_cache: torch.Tensor, page_table: torch.Tensor,
                        head_kind: Sequence[int], T: int, keep: Tuple[int, int] = (3, 10),
                        out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Dense heads' prefill block mask from mean-pooled tile scores (see include/ubs.h).

    q bf16 [L, Hq, D]; k_cache bf16 [NP, Hkv, P, D]; page_table int32 [>= ceil(L/P)];
    keep = (keep_num, keep_den): ceil(keep_num*(i+1)/keep_den) tiles kept in query-tile row
    i, the diagonal included. Returns block_mask uint8 [Hq, nT, nT]; rows of streaming heads
    are left as they were in `out` (zeros when out is None).
    """
    lib = load()
    L, Hq, D = q.shape
    NP, Hkv, P, D2 = k_cache.shape
    dev = q.device
    _need(q, "q", torch.bfloat16, device=dev)
    _need(k_cache, "k_cache", torch.bfloat16, device=dev)
    _need(page_table, "page_table", torch.int32, device=dev)
    if D2 != D:
        raise ValueError("q and k_cache head dims differ")
    if len(head_kind) != Hkv:
        raise ValueError("head_kind must have one entry per KV head")
    if page_table.numel() < (L + P - 1) // P:
        raise ValueError("page_table is shorter than ceil(L / P)")
    nT = (L + T - 1) // T
    if out is None:
        out = torch.zeros((Hq, nT, nT), dtype=torch.uint8, device=dev)
    _need(out, "out", torch.uint8, shape=(Hq, nT, nT), device=dev)
    stream = _stream(dev)
    nbytes = lib.ubs_mask_workspace_size(L, Hq, Hkv, D, T)
    ws = _workspace("mask", dev, stream, nbytes)
    rc = lib.estimate_block_mask(_ptr(q), _ptr(k_cache), _ptr(page_table), L, Hq, Hkv, D, P, T, _kinds(head_kind),
                                 int(keep[0]), int(keep[1]), _ptr(out), _ptr(ws), ws.numel(), stream)
    _check("estimate_block_mask", rc)
    return out


def sparse_prefill_chunk(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                         page_table: torch.Tensor, L: int, q_start: int, head_kind: Sequence[int],
                         block_mask: Optional[torch.Tensor], sink_tiles: int, local_tiles: int, T: int,
                         sm_scale: float, out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                         return_lse: bool = False):
    """Chunked prefill: query rows [q_start, L) over a cache holding all L tokens (see include/ubs.h).

    q bf16 [L - q_start, Hq, D]; block_mask uint8 [Hq, nT - q_start/T, nT] (None when every KV
    head streams). Returns out fp32 [L - q_start, Hq, D] (and lse fp32 [Hq, L - q_start]).
    """
    lib = load()
    Lq, Hq, D = q.shape
    NP, Hkv, P, D2 = k_cache.shape
    dev = q.device
    if Lq != L - q_start:
        raise ValueError("q must hold rows q_start .. L-1")
    _need(q, "q", torch.bfloat16, device=dev)
    _need(k_cache, "k_cache", torch.bfloat16, device=dev)
    _need(v_cache, "v_cache", torch.bfloat16, shape=k_cache.shape, device=dev)
    _need(page_table, "page_table", torch.int32, device=dev)
    if D2 != D:
        raise ValueError("q and k_cache head dims differ")
    if len(head_kind) != Hkv:
        raise ValueError("head_kind must have one entry per KV head")
    nT = (L + T - 1) // T
    if page_table.numel() < (L + P - 1) // P:
        raise ValueError("page_table is shorter than ceil(L / P)")
    if block_mask is not None:
        _need(block_mask, "block_mask", torch.uint8, shape=(Hq, nT - q_start // T, nT), device=dev)
    if out is None:
        out = torch.empty((Lq, Hq, D), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, shape=(Lq, Hq, D), device=dev)
    if return_lse and lse is None:
        lse = torch.empty((Hq, Lq), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, shape=(Hq, Lq), device=dev)
    rc = lib.sparse_prefill_chunk(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table), L, q_start, Hq, Hkv, D,
                                  P, T, _kinds(head_kind), _ptr(block_mask), sink_tiles, local_tiles,
                                  float(sm_scale), _ptr(out), _ptr(lse), _stream(dev))
    _check("sparse_prefill_chunk", rc)
    return (out, lse) if return_lse else out


def append_kv(k_new: torch.Tensor, v_new: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor,
              head_kind: Sequence[int], k_cache: torch.Tensor, v_cache: torch.Tensor,
              bounds: Optional[torch.Tensor] = None, Lp: Optional[int] = None) -> None:
    """Write n_new tokens per sequence into the paged cache after position seq_lens[b], and
    refresh the dense heads' page bounds they change (see include/ubs.h). seq_lens is the
    length before the append; it is not modified.

    k_new, v_new bf16 [B, n_new, Hkv, D]; page_table int32 [B, max_pages]; seq_lens int32 [B];
    k_cache, v_cache bf16 [NP, Hkv, P, D]; bounds bf16 [NP, Hkv, P/Lp, 2, D] or None.
    """
    lib = load()
    B, n_new, Hkv, D = k_new.shape
    NP, Hkv2, P, D2 = k_cache.shape
    dev = k_new.device
    _need(k_new, "k_new", torch.bfloat16, device=dev)
    _need(v_new, "v_new", torch.bfloat16, shape=k_new.shape, device=dev)
    _need(k_cache, "k_cache", torch.bfloat16, device=dev)
    _need(v_cache, "v_cache", torch.bfloat16, shape=k_cache.shape, device=dev)
    _need(page_table, "page_table", torch.int32, device=dev)
    _need(seq_lens, "seq_lens", torch.int32, shape=(B,), device=dev)
    if (Hkv2, D2) != (Hkv, D):
        raise ValueError("k_new and k_cache shapes differ")
    if len(head_kind) != Hkv:
        raise ValueError("head_kind must have one entry per KV head")
    if page_table.dim() != 2 or page_table.shape[0] != B:
        raise ValueError("page_table must be [B, max_pages]")
    if bounds is not None:
        if Lp is None:
            Lp = P // bounds.shape[2]
        _need(bounds, "bounds", torch.bfloat16, shape=(NP, Hkv, P // Lp, 2, D), device=dev)
    rc = lib.append_kv(_ptr(k_new), _ptr(v_new), _ptr(page_table), _ptr(seq_lens), B, page_table.shape[1], n_new,
                       Hkv, D, P, int(Lp if Lp is not None else P), _kinds(head_kind), _ptr(k_cache), _ptr(v_cache),
                       _ptr(bounds), _stream(dev))
    _check("append_kv", rc)


def check_paged(page_table: torch.Tensor, num_pages: int, P: int, seq_lens: Optional[torch.Tensor] = None,
                cu_seqlens: Optional[torch.Tensor] = None, head_kind: Optional[Sequence[int]] = None,
                selected: Optional[torch.Tensor] = None, num_selected: Optional[torch.Tensor] = None,
                status: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Checked mode: enqueue the device-side validation of page ids, lengths and (when
    given) the selection; returns the status record to pass to check_status."""
    lib = load()
    if page_table.dim() == 1:
        page_table = page_table.view(1, -1)
    B, max_pages = page_table.shape
    dev = page_table.device
    _need(page_table, "page_table", torch.int32, device=dev)
    if (seq_lens is None) == (cu_seqlens is None):
        raise ValueError("give exactly one of seq_lens and cu_seqlens")
    if seq_lens is not None:
        _need(seq_lens, "seq_lens", torch.int32, shape=(B,), device=dev)
    else:
        _need(cu_seqlens, "cu_seqlens", torch.int32, shape=(B + 1,), device=dev)
    if status is None:
        status = torch.zeros(CHECK_STATUS_BYTES // 4, dtype=torch.int32, device=dev)
    _need(status, "status", torch.int32, device=dev)
    Hkv, ms, kinds = 0, 0, None
    if selected is not None:
        if head_kind is None or num_selected is None:
            raise ValueError("selected needs head_kind and num_selected")
        _, Hkv, ms = selected.shape
        _need(selected, "selected", torch.int32, shape=(B, Hkv, ms), device=dev)
        _need(num_selected, "num_selected", torch.int32, shape=(B, Hkv), device=dev)
        kinds = _kinds(head_kind)
    rc = lib.ubs_check_paged(_ptr(page_table), B, max_pages, _ptr(seq_lens), _ptr(cu_seqlens), int(num_pages), P,
                             kinds, Hkv, _ptr(selected), _ptr(num_selected), ms, _ptr(status), _stream(dev))
    _check("ubs_check_paged", rc)
    return status


def check_status(status: torch.Tensor) -> None:
    """Wait for the stream, then raise UBSError (OUT_OF_RANGE) if a violation was recorded
    (the record is cleared)."""
    lib = load()
    rc = lib.ubs_check_status(_ptr(status), _stream(status.device))
    _check("ubs_check_status", rc)


# ----------------------------------------------------------------------------- measurement helpers

def bench_read(buf: torch.Tensor, sink: torch.Tensor) -> None:
    """Read all of `buf` once (include/ubs_bench.h: ubs_bench_read); `sink` is a device
    tensor of at least 4 bytes. For timing the plain read rate with events."""
    if not (buf.is_cuda and sink.is_cuda and buf.is_contiguous()):
        raise ValueError("buf and sink must be contiguous GPU tensors")
    lib = load()
    _check("ubs_bench_read", lib.ubs_bench_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                                _stream(buf.device)))


def bench_mfma(iters: int, out: torch.Tensor) -> int:
    """Back-to-back bf16 MFMAs on every SIMD (include/ubs_bench.h: ubs_bench_mfma); returns
    the flops the call performs."""
    lib = load()
    _check("ubs_bench_mfma", lib.ubs_bench_mfma(int(iters), _ptr(out), _stream(out.device)))
    return int(lib.ubs_bench_mfma_waves()) * int(iters) * 4 * 32768

