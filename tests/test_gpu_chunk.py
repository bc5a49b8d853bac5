"""GPU parity of chunked prefill (sparse_prefill_chunk): query tiles [q_start/T, nT) of a
sequence whose whole K/V sits in the paged cache. Each chunk must equal the oracle's
attention of those rows, and be bit-identical to the same rows of a whole-sequence
sparse_prefill (the kernel's work per (head, query tile) does not depend on the chunk)."""
import numpy as np
import pytest
import torch

import oracle
import unified_block_sparse_amd as ubs
from tests.gpu_cases import assert_attention_close, assert_lse_close, sample_rows
from tests.helpers import bits
from workloads import cases

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _chunks(c, starts):
    full, full_lse = ubs.sparse_prefill(c.q, c.k_cache, c.v_cache, c.page_table, c.head_kind, c.block_mask,
                                        c.sink_tiles, c.local_tiles, c.T, c.sm_scale, return_lse=True)
    outs = []
    for q0 in starts:
        i0 = q0 // c.T
        mask = c.block_mask[:, i0:, :].contiguous()
        o, l = ubs.sparse_prefill_chunk(c.q[q0:].contiguous(), c.k_cache, c.v_cache, c.page_table, c.L, q0,
                                        c.head_kind, mask, c.sink_tiles, c.local_tiles, c.T, c.sm_scale,
                                        return_lse=True)
        outs.append((q0, o, l))
    torch.cuda.synchronize(DEV)
    for q0, o, l in outs:
        assert torch.equal(o, full[q0:]), f"chunk at {q0}: differs from the whole-sequence rows"
        assert torch.equal(l, full_lse[:, q0:]), f"chunk at {q0}: lse differs"
    return outs


def test_prefill_chunks_small():
    c = cases.make_prefill("chunks", 2000, 8, 2, 128, 128, 64, [0, 1], 1, 3, "random", 2101, DEV, mask_arg=40)
    outs = _chunks(c, [0, 512, 1024, 1920])
    q0, o, l = outs[2]
    rows = list(range(q0, c.L))
    qh = np.zeros(tuple(c.q.shape), dtype=np.uint16)
    qh[rows] = bits(c.q[q0:])
    ref, ref_lse = oracle.prefill_ref(qh, bits(c.k_cache), bits(c.v_cache), c.page_table.cpu().numpy(), c.L, c.Hq,
                                      c.Hkv, c.D, c.P, c.T, c.head_kind, c.block_mask.cpu().numpy(), c.sink_tiles,
                                      c.local_tiles, c.sm_scale, rows=rows)
    assert_attention_close(o.cpu().numpy(), ref, "chunk at 1024")
    assert_lse_close(l.cpu().numpy(), ref_lse, "chunk at 1024 lse")


def test_prefill_chunk_llama8b_tail():
    """The last 32 query tiles of the 65,536-token Llama-3-8B workload as one chunk."""
    c = cases.prefill_llama8b(DEV)
    q0 = c.L - 32 * c.T
    (q0, o, l), = _chunks(c, [q0])
    rows = sample_rows(c.L - q0, c.T, 24, 7)
    rows = [q0 + r for r in rows]
    qh = np.zeros(tuple(c.q.shape), dtype=np.uint16)
    qh[rows] = bits(c.q[torch.tensor(rows, device=DEV)])
    ref, ref_lse = oracle.prefill_ref(qh, bits(c.k_cache), bits(c.v_cache), c.page_table.cpu().numpy(), c.L, c.Hq,
                                      c.Hkv, c.D, c.P, c.T, c.head_kind, c.block_mask.cpu().numpy(), c.sink_tiles,
                                      c.local_tiles, c.sm_scale, rows=rows)
    ridx = torch.tensor([r - q0 for r in rows], device=DEV)
    assert_attention_close(o[ridx].cpu().numpy(), ref, "llama8b tail chunk")
    assert_lse_close(l[:, ridx].cpu().numpy(), ref_lse, "llama8b tail chunk lse")
