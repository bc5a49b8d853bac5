"""The hot-path calls captured in a HIP graph (torch.cuda.graph) and replayed: every
replay, with eager work and synchronisations in between, must reproduce the eager
results bit for bit (selection, decode output, prefill output)."""
import pytest
import torch

import unified_block_sparse_amd as ubs
from workloads import cases

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def test_select_and_decode_graph_replays_match_eager():
    lib = ubs.load()
    cs = [cases.make_decode(f"g{r}", [3000, 129, 1500], 16, 4, 128, 64, 16, [0, 1, 0, 1], 8 * 64, 64, 256,
                            60 + r, DEV, planted=True) for r in range(3)]
    inst = []
    for c in cs:
        bnd = torch.zeros((c.num_physical_pages, c.Hkv, c.P // c.Lp, 2, c.D), dtype=torch.bfloat16, device=DEV)
        ubs.build_page_bounds(c.k_cache, c.page_table, c.seq_lens_t, c.head_kind, c.Lp, bounds=bnd)
        sel = torch.empty((c.B, c.Hkv, c.k_pages), dtype=torch.int32, device=DEV)
        num = torch.empty((c.B, c.Hkv), dtype=torch.int32, device=DEV)
        out = torch.empty((c.B, c.Hq, c.D), dtype=torch.float32, device=DEV)
        lse = torch.empty((c.B, c.Hq), dtype=torch.float32, device=DEV)
        inst.append((c, bnd, sel, num, out, lse))
    c0 = cs[0]
    ws_sel = torch.zeros(lib.ubs_select_workspace_size(c0.B, c0.page_table.shape[1], c0.Hkv) + 256,
                         dtype=torch.uint8, device=DEV)
    ws_dec = torch.zeros(lib.ubs_decode_workspace_size(c0.B, c0.Hq, c0.Hkv, c0.D, c0.P, c0.k_pages,
                                                       c0.sink_tokens, c0.local_tokens) + 256,
                         dtype=torch.uint8, device=DEV)

    def run_all():
        for c, bnd, sel, num, out, lse in inst:
            ubs.select_pages(c.q, bnd, c.page_table, c.seq_lens_t, c.head_kind, c.P, c.token_budget,
                             selected=sel, num_selected=num, workspace=ws_sel)
            ubs.sparse_decode(c.q, c.k_cache, c.v_cache, c.page_table, c.seq_lens_t, c.head_kind, sel, num,
                              c.sink_tokens, c.local_tokens, c.sm_scale, out=out, lse=lse, workspace=ws_dec)

    run_all()
    torch.cuda.synchronize(DEV)
    ref = [(sel.clone(), num.clone(), out.clone(), lse.clone()) for _, _, sel, num, out, lse in inst]
    side = torch.cuda.Stream(DEV)
    side.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(side):
        run_all()
    torch.cuda.current_stream(DEV).wait_stream(side)
    torch.cuda.synchronize(DEV)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_all()
    torch.cuda.synchronize(DEV)
    for rep in range(4):
        for _, _, sel, num, out, lse in inst:
            sel.fill_(-7)
            num.fill_(-7)
            out.fill_(float("nan"))
            lse.fill_(float("nan"))
        # eager work of the program between replays: another selection + decode into the
        # same workspaces, then a synchronisation
        c, bnd = inst[rep % 3][0], inst[rep % 3][1]
        s2, _ = ubs.select_pages(c.q, bnd, c.page_table, c.seq_lens_t, c.head_kind, c.P, c.token_budget,
                                 workspace=ws_sel)
        torch.cuda.synchronize(DEV)
        g.replay()
        torch.cuda.synchronize(DEV)
        for (_, _, sel, num, out, lse), (sr, nr, orf, lr) in zip(inst, ref):
            assert torch.equal(sel, sr) and torch.equal(num, nr), f"replay {rep}: selection differs"
            assert torch.equal(out, orf) and torch.equal(lse, lr), f"replay {rep}: decode output differs"


def test_decode_select_graph_replays_match_eager():
    """sparse_decode_select (top-k ranked inside the decode kernel) captured and replayed."""
    lib = ubs.load()
    cs = [cases.make_decode(f"gs{r}", [3000, 129, 1500], 16, 4, 128, 64, 16, [0, 1, 0, 1], 8 * 64, 64, 256,
                            70 + r, DEV, planted=True) for r in range(3)]
    inst = []
    for c in cs:
        bnd = ubs.build_page_bounds(c.k_cache, c.page_table, c.seq_lens_t, c.head_kind, c.Lp)
        sel = torch.empty((c.B, c.Hkv, c.k_pages), dtype=torch.int32, device=DEV)
        num = torch.empty((c.B, c.Hkv), dtype=torch.int32, device=DEV)
        out = torch.empty((c.B, c.Hq, c.D), dtype=torch.float32, device=DEV)
        inst.append((c, bnd, sel, num, out))
    c0 = cs[0]
    ws = torch.zeros(lib.ubs_decode_select_workspace_size(c0.B, c0.page_table.shape[1], c0.Hq, c0.Hkv, c0.D, c0.P,
                                                          c0.token_budget, c0.sink_tokens, c0.local_tokens),
                     dtype=torch.uint8, device=DEV)

    def run_all():
        for c, bnd, sel, num, out in inst:
            ubs.sparse_decode_select(c.q, bnd, c.k_cache, c.v_cache, c.page_table, c.seq_lens_t, c.head_kind, c.P,
                                     c.token_budget, c.sink_tokens, c.local_tokens, c.sm_scale, out=out,
                                     selected=sel, num_selected=num, workspace=ws)

    run_all()
    torch.cuda.synchronize(DEV)
    ref = [(sel.clone(), num.clone(), out.clone()) for _, _, sel, num, out in inst]
    side = torch.cuda.Stream(DEV)
    side.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(side):
        run_all()
    torch.cuda.current_stream(DEV).wait_stream(side)
    torch.cuda.synchronize(DEV)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_all()
    torch.cuda.synchronize(DEV)
    for rep in range(4):
        for _, _, sel, num, out in inst:
            sel.fill_(-7)
            num.fill_(-7)
            out.fill_(float("nan"))
        c, bnd = inst[rep % 3][0], inst[rep % 3][1]   # eager work between replays, same workspace
        ubs.sparse_decode_select(c.q, bnd, c.k_cache, c.v_cache, c.page_table, c.seq_lens_t, c.head_kind, c.P,
                                 c.token_budget, c.sink_tokens, c.local_tokens, c.sm_scale, workspace=ws)
        torch.cuda.synchronize(DEV)
        g.replay()
        torch.cuda.synchronize(DEV)
        for (_, _, sel, num, out), (sr, nr, orf) in zip(inst, ref):
            assert torch.equal(sel, sr) and torch.equal(num, nr), f"replay {rep}: selection differs"
            assert torch.equal(out, orf), f"replay {rep}: decode output differs"


def test_prefill_graph_replays_match_eager():
    c = cases.make_prefill("gp", 700, 8, 2, 128, 128, 64, [0, 1], 1, 2, "random", 61, DEV, mask_arg=3)
    out = torch.empty((c.L, c.Hq, c.D), dtype=torch.float32, device=DEV)
    lse = torch.empty((c.Hq, c.L), dtype=torch.float32, device=DEV)

    def run():
        ubs.sparse_prefill(c.q, c.k_cache, c.v_cache, c.page_table, c.head_kind, c.block_mask, c.sink_tiles,
                           c.local_tiles, c.T, c.sm_scale, out=out, lse=lse)

    run()
    torch.cuda.synchronize(DEV)
    ref_o, ref_l = out.clone(), lse.clone()
    side = torch.cuda.Stream(DEV)
    side.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream(DEV).wait_stream(side)
    torch.cuda.synchronize(DEV)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize(DEV)
    for rep in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize(DEV)
        g.replay()
        torch.cuda.synchronize(DEV)
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"replay {rep} differs"
