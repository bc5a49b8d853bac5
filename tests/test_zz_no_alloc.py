"""sparse_decode_static (no allocation, library-owned scratch) against sparse_decode with a
caller workspace: two calls in a row through the C ABI, the second with a smaller batch,
each equal to the workspace call bit for bit (the same kernels and split plan run) and so
within the attention tolerance of it."""
import ctypes

import numpy as np
import pytest
import torch

import unified_block_sparse_amd as ubs
from workloads import cases

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _static_call(lib, d, sel, num, out, lse):
    kinds = (ctypes.c_uint8 * d.Hkv)(*d.head_kind)
    st = torch.cuda.current_stream(DEV).cuda_stream
    return lib.sparse_decode_static(d.q.data_ptr(), d.k_cache.data_ptr(), d.v_cache.data_ptr(),
                                    d.page_table.data_ptr(), d.seq_lens_t.data_ptr(), d.B, d.page_table.shape[1],
                                    d.Hq, d.Hkv, d.D, d.P, kinds, sel.data_ptr(), num.data_ptr(), sel.shape[2],
                                    d.sink_tokens, d.local_tokens, ctypes.c_float(d.sm_scale), out.data_ptr(),
                                    lse.data_ptr(), st)


def test_decode_static_equals_workspace_decode_twice():
    lib = ubs.load()
    torch.cuda.set_device(DEV)
    # first the Llama-3-8B decode batch (4 x 32K tokens), then a smaller, ragged one
    for d in (cases.decode_llama8b(DEV),
              cases.make_decode("static2", [3000, 700, 17], 16, 4, 128, 64, 16, [0, 0, 1, 1], 8 * 64, 64, 256,
                                2301, DEV, planted=True)):
        bnd = ubs.build_page_bounds(d.k_cache, d.page_table, d.seq_lens_t, d.head_kind, d.Lp)
        sel, num = ubs.select_pages(d.q, bnd, d.page_table, d.seq_lens_t, d.head_kind, d.P, d.token_budget)
        ref, ref_lse = ubs.sparse_decode(d.q, d.k_cache, d.v_cache, d.page_table, d.seq_lens_t, d.head_kind, sel,
                                         num, d.sink_tokens, d.local_tokens, d.sm_scale, return_lse=True)
        out = torch.full((d.B, d.Hq, d.D), float("nan"), dtype=torch.float32, device=DEV)
        lse = torch.full((d.B, d.Hq), float("nan"), dtype=torch.float32, device=DEV)
        rc = _static_call(lib, d, sel, num, out, lse)
        assert rc == 0, lib.ubs_last_error().decode()
        torch.cuda.synchronize(DEV)
        assert torch.isfinite(out).all()
        d_out = (out - ref).abs().max().item()
        assert d_out <= 1e-2 and (out - ref).abs().mean().item() <= 1e-3
        assert torch.equal(out, ref) and torch.equal(lse, ref_lse), f"B={d.B}: differs from sparse_decode"
        print(f"sparse_decode_static B={d.B}: equal to the workspace call")
