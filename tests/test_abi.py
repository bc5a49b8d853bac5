"""C ABI checks that need no GPU: the library loads, exports every function that
include/*.h declares, and host-side validation returns the documented error codes
before any HIP call (so only fake, never-dereferenced pointers are passed)."""
import ctypes
import os
import re

import pytest

import unified_block_sparse_amd as ubs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
A = 0x10000            # a fake, 16-byte aligned "device pointer" (never dereferenced)
KIND = (ctypes.c_uint8 * 8)(0, 0, 0, 0, 1, 1, 1, 1)
NULL = None


def _declared_functions():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if not h.endswith(".h"):
            continue
        src = open(os.path.join(ROOT, "include", h)).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w ]*[\s\*]+([A-Za-z_]\w*)\s*\(", src, flags=re.M))
    return names


def test_library_exports_every_declared_symbol():
    lib = ubs.load()
    names = _declared_functions()
    assert {"sparse_prefill", "build_page_bounds", "select_pages", "sparse_decode"} <= names
    for n in names:
        assert hasattr(lib, n), f"libubs.so does not export {n}"
    assert set(ubs.EXPORTED) == names
    assert lib.ubs_version() >= 100


def _prefill(**kw):
    a = dict(q=A, k=A, v=A, pt=A, L=256, Hq=8, Hkv=8, D=128, P=64, T=128, kind=KIND, mask=A,
             sink=1, local=4, scale=0.1, out=A, lse=NULL, stream=NULL)
    a.update(kw)
    return ubs.load().sparse_prefill(a["q"], a["k"], a["v"], a["pt"], a["L"], a["Hq"], a["Hkv"], a["D"],
                                     a["P"], a["T"], a["kind"], a["mask"], a["sink"], a["local"], a["scale"],
                                     a["out"], a["lse"], a["stream"])


def _err():
    return ubs.load().ubs_last_error().decode()


@pytest.mark.parametrize("kw,code,frag", [
    (dict(D=96), -2, "D=96"),
    (dict(T=32), -2, "T=32"),
    (dict(Hq=12), -1, "multiple"),
    (dict(P=40), -2, "P=40"),
    (dict(kind=None), -1, "head_kind"),
    (dict(kind=(ctypes.c_uint8 * 8)(0, 2, 0, 0, 1, 1, 1, 1)), -1, "head_kind[1]"),
    (dict(q=None), -1, "non-NULL"),
    (dict(mask=None), -1, "block_mask"),
    (dict(L=-1), -1, "L=-1"),
    (dict(sink=-1), -1, "sink_tiles"),
    (dict(q=A + 8), -1, "aligned"),
    (dict(scale=float("nan")), -1, "sm_scale"),
    (dict(scale=0.0), -1, "sm_scale"),
    (dict(scale=-0.1), -1, "sm_scale"),
    (dict(scale=float("inf")), -1, "sm_scale"),
])
def test_prefill_validation(kw, code, frag):
    assert _prefill(**kw) == code
    assert frag in _err()


def test_prefill_empty_and_all_streaming_mask_ok():
    assert _prefill(L=0) == 0                       # nothing to launch
    assert _err() == ""
    all_stream = (ctypes.c_uint8 * 8)(*([1] * 8))
    assert _prefill(L=0, kind=all_stream, mask=None) == 0


def _bounds(**kw):
    a = dict(k=A, pt=A, sl=A, B=4, maxp=512, Hkv=8, D=128, P=64, Lp=16, kind=KIND, out=A, stream=NULL)
    a.update(kw)
    return ubs.load().build_page_bounds(a["k"], a["pt"], a["sl"], a["B"], a["maxp"], a["Hkv"], a["D"], a["P"],
                                        a["Lp"], a["kind"], a["out"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(Lp=24), -2), (dict(P=48), -2), (dict(D=32), -2), (dict(B=-1), -1), (dict(k=None), -1),
    (dict(Hkv=65), -2), (dict(out=A + 2), -1),
])
def test_bounds_validation(kw, code):
    assert _bounds(**kw) == code


def test_bounds_nothing_to_do():
    assert _bounds(B=0) == 0
    assert _bounds(kind=(ctypes.c_uint8 * 8)(*([1] * 8))) == 0   # no dense head


def _select(**kw):
    lib = ubs.load()
    a = dict(q=A, bnd=A, pt=A, sl=A, B=4, maxp=512, Hq=32, Hkv=8, D=128, P=64, Lp=64, budget=4096,
             kind=KIND, sel=A, nsel=A, ws=A, wsb=None, stream=NULL)
    a.update(kw)
    if a["wsb"] is None:
        a["wsb"] = lib.ubs_select_workspace_size(a["B"], a["maxp"], a["Hkv"])
    return lib.select_pages(a["q"], a["bnd"], a["pt"], a["sl"], a["B"], a["maxp"], a["Hq"], a["Hkv"], a["D"],
                            a["P"], a["Lp"], a["budget"], a["kind"], a["sel"], a["nsel"], a["ws"], a["wsb"],
                            a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(budget=4000), -2), (dict(budget=0), -1), (dict(Lp=2), -2), (dict(Hq=24), -2),
    (dict(maxp=20000), -2), (dict(wsb=16), -3), (dict(ws=None), -3), (dict(bnd=None), -1),
    (dict(sel=None), -1), (dict(Hq=30), -1),
])
def test_select_validation(kw, code):
    assert _select(**kw) == code


def test_select_workspace_size():
    lib = ubs.load()
    assert lib.ubs_select_workspace_size(4, 512, 8) >= 4 * 512 * 8 * 4
    assert lib.ubs_select_workspace_size(4, 512, 8) % 256 == 0


def _decode(**kw):
    lib = ubs.load()
    a = dict(q=A, k=A, v=A, pt=A, sl=A, B=4, maxp=512, Hq=32, Hkv=8, D=128, P=64, kind=KIND, sel=A, nsel=A,
             ms=64, sink=128, local=512, scale=0.088, out=A, lse=NULL, ws=A, wsb=None, stream=NULL)
    a.update(kw)
    if a["wsb"] is None:
        a["wsb"] = lib.ubs_decode_workspace_size(a["B"], a["Hq"], a["Hkv"], a["D"], a["P"], a["ms"],
                                                    a["sink"], a["local"])
    return lib.sparse_decode(a["q"], a["k"], a["v"], a["pt"], a["sl"], a["B"], a["maxp"], a["Hq"], a["Hkv"],
                             a["D"], a["P"], a["kind"], a["sel"], a["nsel"], a["ms"], a["sink"], a["local"],
                             a["scale"], a["out"], a["lse"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(P=40), -2), (dict(P=512), -2), (dict(Hq=24), -2), (dict(Hq=136, Hkv=8), -2), (dict(D=80), -2),
    (dict(sink=-1), -1), (dict(wsb=100), -3), (dict(nsel=None), -1), (dict(out=None), -1),
    (dict(k=A + 4), -1), (dict(scale=0.0), -1), (dict(scale=-1.0), -1), (dict(scale=float("nan")), -1),
])
def test_decode_validation(kw, code):
    assert _decode(**kw) == code


def test_decode_workspace_grows_with_budget():
    lib = ubs.load()
    small = lib.ubs_decode_workspace_size(4, 32, 8, 128, 64, 16, 128, 512)
    big = lib.ubs_decode_workspace_size(4, 32, 8, 128, 64, 1024, 128, 512)
    assert big > small >= 4 * 8 * 4


def _dsel(**kw):
    lib = ubs.load()
    a = dict(q=A, bnd=A, k=A, v=A, pt=A, sl=A, B=4, maxp=512, Hq=32, Hkv=8, D=128, P=64, Lp=64, budget=4096,
             kind=KIND, sink=128, local=512, scale=0.088, sel=A, nsel=A, out=A, lse=NULL, ws=A, wsb=None,
             stream=NULL)
    a.update(kw)
    if a["wsb"] is None:
        a["wsb"] = lib.ubs_decode_select_workspace_size(a["B"], a["maxp"], a["Hq"], a["Hkv"], a["D"], a["P"],
                                                        a["budget"], a["sink"], a["local"])
    return lib.sparse_decode_select(a["q"], a["bnd"], a["k"], a["v"], a["pt"], a["sl"], a["B"], a["maxp"], a["Hq"],
                                    a["Hkv"], a["D"], a["P"], a["Lp"], a["budget"], a["kind"], a["sink"],
                                    a["local"], a["scale"], a["sel"], a["nsel"], a["out"], a["lse"], a["ws"],
                                    a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    # the selection half
    (dict(budget=4000), -2), (dict(budget=0), -1), (dict(Lp=2), -2), (dict(Hq=24), -2), (dict(P=256), -2),
    (dict(maxp=20000), -2), (dict(ws=None), -3), (dict(wsb=16), -3), (dict(bnd=None), -1), (dict(sel=None), -1),
    (dict(nsel=None), -1),
    # the decode half (including a workspace that covers the scores but not the partials)
    (dict(k=None), -1), (dict(out=None), -1), (dict(k=A + 4), -1), (dict(scale=0.0), -1), (dict(sink=-1), -1),
    (dict(wsb="scores_only"), -3),
    # nothing to do
    (dict(B=0), 0),
])
def test_decode_select_validation(kw, code):
    if kw.get("wsb") == "scores_only":
        kw = dict(kw, wsb=ubs.load().ubs_select_workspace_size(4, 512, 8) + 256)
    assert _dsel(**kw) == code


def test_decode_select_workspace_is_both_workspaces():
    lib = ubs.load()
    sel = lib.ubs_select_workspace_size(4, 512, 8)
    dec = lib.ubs_decode_workspace_size(4, 32, 8, 128, 64, 64, 128, 512)
    assert lib.ubs_decode_select_workspace_size(4, 512, 32, 8, 128, 64, 4096, 128, 512) == sel + dec


def test_binding_rejects_cpu_tensors():
    import torch
    q = torch.zeros((4, 32, 128), dtype=torch.bfloat16)
    kc = torch.zeros((8, 8, 64, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        ubs.sparse_decode(q, kc, kc, torch.zeros((4, 2), dtype=torch.int32), torch.zeros(4, dtype=torch.int32),
                          [0] * 4 + [1] * 4, None, None, 128, 512, 0.1)


def _mask(**kw):
    lib = ubs.load()
    a = dict(q=A, k=A, pt=A, L=1024, Hq=32, Hkv=8, D=128, P=64, T=128, kind=KIND, num=3, den=10, mask=A,
             ws=A, wsb=None, stream=NULL)
    a.update(kw)
    if a["wsb"] is None:
        a["wsb"] = lib.ubs_mask_workspace_size(a["L"], a["Hq"], a["Hkv"], a["D"], a["T"])
    return lib.estimate_block_mask(a["q"], a["k"], a["pt"], a["L"], a["Hq"], a["Hkv"], a["D"], a["P"], a["T"],
                                   a["kind"], a["num"], a["den"], a["mask"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code,frag", [
    (dict(D=96), -2, "D=96"),
    (dict(T=32), -2, "T=32"),
    (dict(P=48), -2, "P=48"),
    (dict(Hq=12), -1, "multiple"),
    (dict(num=0), -1, "keep_num"),
    (dict(num=11), -1, "keep_num"),
    (dict(kind=None), -1, "head_kind"),
    (dict(mask=None), -1, "non-NULL"),
    (dict(q=A + 2), -1, "aligned"),
    (dict(wsb=64), -3, "workspace"),
    (dict(L=4096 * 128 + 1), -2, "tiles"),
])
def test_mask_validation(kw, code, frag):
    assert _mask(**kw) == code
    assert frag in _err()


def test_mask_nothing_to_do():
    # L = 0, and every KV head streaming: success without touching any pointer
    assert _mask(L=0, q=None, k=None, pt=None, mask=None, ws=None, wsb=0) == 0
    streaming = (ctypes.c_uint8 * 8)(1, 1, 1, 1, 1, 1, 1, 1)
    assert _mask(kind=streaming, q=None, k=None, pt=None, mask=None, ws=None, wsb=0) == 0


def test_mask_workspace_size():
    lib = ubs.load()
    assert lib.ubs_mask_workspace_size(65536, 32, 8, 128, 128) >= (32 + 8) * 512 * 128 * 4
    assert lib.ubs_mask_workspace_size(65536, 32, 8, 128, 128) % 256 == 0


def _chunk(**kw):
    a = dict(q=A, k=A, v=A, pt=A, L=1024, q0=256, Hq=8, Hkv=8, D=128, P=64, T=128, kind=KIND, mask=A,
             sink=1, local=4, scale=0.1, out=A, lse=NULL, stream=NULL)
    a.update(kw)
    return ubs.load().sparse_prefill_chunk(a["q"], a["k"], a["v"], a["pt"], a["L"], a["q0"], a["Hq"], a["Hkv"],
                                           a["D"], a["P"], a["T"], a["kind"], a["mask"], a["sink"], a["local"],
                                           a["scale"], a["out"], a["lse"], a["stream"])


@pytest.mark.parametrize("kw,code,frag", [
    (dict(q0=100), -1, "q_start=100"),
    (dict(q0=1152), -1, "q_start=1152"),
    (dict(q0=-128), -1, "q_start=-128"),
    (dict(T=32), -2, "T=32"),
    (dict(mask=None), -1, "block_mask"),
])
def test_prefill_chunk_validation(kw, code, frag):
    assert _chunk(**kw) == code
    assert frag in _err()


def test_prefill_chunk_empty_chunk_ok():
    assert _chunk(q0=1024, q=None, k=None, v=None, pt=None, mask=None, out=None) == 0


def _append(**kw):
    a = dict(kn=A, vn=A, pt=A, sl=A, B=4, maxp=64, n=1, Hkv=8, D=128, P=64, Lp=16, kind=KIND, k=A, v=A, bnd=A,
             stream=NULL)
    a.update(kw)
    return ubs.load().append_kv(a["kn"], a["vn"], a["pt"], a["sl"], a["B"], a["maxp"], a["n"], a["Hkv"], a["D"],
                                a["P"], a["Lp"], a["kind"], a["k"], a["v"], a["bnd"], a["stream"])


@pytest.mark.parametrize("kw,code,frag", [
    (dict(D=96), -2, "D=96"),
    (dict(P=48), -2, "P=48"),
    (dict(Lp=24), -2, "Lp=24"),
    (dict(n=-1), -1, "n_new=-1"),
    (dict(kind=None), -1, "head_kind"),
    (dict(k=None), -1, "non-NULL"),
    (dict(bnd=A + 2), -1, "aligned"),
])
def test_append_validation(kw, code, frag):
    assert _append(**kw) == code
    assert frag in _err()


def test_append_nothing_to_do():
    assert _append(n=0, kn=None, vn=None, pt=None, sl=None, k=None, v=None, bnd=None) == 0


def _quant(**kw):
    a = dict(k=A, v=A, pt=A, sl=A, B=4, maxp=64, Hkv=8, D=128, P=64, kc=A, vc=A, kp=A, vp=A, stream=NULL)
    a.update(kw)
    return ubs.load().quantize_kv_int4(a["k"], a["v"], a["pt"], a["sl"], a["B"], a["maxp"], a["Hkv"], a["D"],
                                       a["P"], a["kc"], a["vc"], a["kp"], a["vp"], a["stream"])


@pytest.mark.parametrize("kw,code,frag", [
    (dict(D=96), -2, "D=96"),
    (dict(P=40), -2, "P=40"),
    (dict(Hkv=0), -1, "Hkv=0"),
    (dict(B=-1), -1, "B=-1"),
    (dict(kc=None), -1, "non-NULL"),
    (dict(k=A + 8), -1, "aligned"),
    (dict(kp=A + 2), -1, "aligned"),
])
def test_quantize_int4_validation(kw, code, frag):
    assert _quant(**kw) == code
    assert frag in _err()


def test_quantize_int4_nothing_to_do():
    assert _quant(B=0, k=None, v=None, pt=None, sl=None, kc=None, vc=None, kp=None, vp=None) == 0


def _decode4(**kw):
    lib = ubs.load()
    a = dict(q=A, kc=A, vc=A, kp=A, vp=A, pt=A, sl=A, B=4, maxp=512, Hq=32, Hkv=8, D=128, P=64, kind=KIND, sel=A,
             nsel=A, ms=64, sink=128, local=512, scale=0.088, out=A, lse=NULL, ws=A, wsb=None, stream=NULL)
    a.update(kw)
    if a["wsb"] is None:
        a["wsb"] = lib.ubs_decode_workspace_size(a["B"], a["Hq"], a["Hkv"], a["D"], a["P"], a["ms"],
                                                    a["sink"], a["local"])
    return lib.sparse_decode_int4(a["q"], a["kc"], a["vc"], a["kp"], a["vp"], a["pt"], a["sl"], a["B"], a["maxp"],
                                  a["Hq"], a["Hkv"], a["D"], a["P"], a["kind"], a["sel"], a["nsel"], a["ms"],
                                  a["sink"], a["local"], a["scale"], a["out"], a["lse"], a["ws"], a["wsb"],
                                  a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(P=40), -2), (dict(Hq=24), -2), (dict(D=80), -2), (dict(sink=-1), -1), (dict(wsb=100), -3),
    (dict(nsel=None), -1), (dict(out=None), -1), (dict(kp=None), -1), (dict(kc=A + 4), -1), (dict(vp=A + 2), -1),
])
def test_decode_int4_validation(kw, code):
    assert _decode4(**kw) == code


def _varlen(**kw):
    a = dict(q=A, k=A, v=A, pt=A, maxp=16, cu=A, B=3, maxs=1000, tot=2000, Hq=8, Hkv=8, D=128, P=64, T=128,
             kind=KIND, mask=A, sink=1, local=4, scale=0.1, out=A, lse=NULL, stream=NULL)
    a.update(kw)
    return ubs.load().sparse_prefill_varlen(a["q"], a["k"], a["v"], a["pt"], a["maxp"], a["cu"], a["B"], a["maxs"],
                                            a["tot"], a["Hq"], a["Hkv"], a["D"], a["P"], a["T"], a["kind"],
                                            a["mask"], a["sink"], a["local"], a["scale"], a["out"], a["lse"],
                                            a["stream"])


@pytest.mark.parametrize("kw,code,frag", [
    (dict(T=32), -2, "T=32"),
    (dict(D=96), -2, "D=96"),
    (dict(maxp=10), -1, "cannot hold"),
    (dict(cu=None), -1, "non-NULL"),
    (dict(mask=None), -1, "block_mask"),
    (dict(B=-1), -1, "B=-1"),
    (dict(out=A + 4), -1, "aligned"),
])
def test_prefill_varlen_validation(kw, code, frag):
    assert _varlen(**kw) == code
    assert frag in _err()


def test_prefill_varlen_nothing_to_do():
    assert _varlen(B=0, q=None, k=None, v=None, pt=None, cu=None, mask=None, out=None) == 0
    assert _varlen(tot=0, q=None, k=None, v=None, pt=None, cu=None, mask=None, out=None) == 0


def test_decode_static_rejects_oversized_scratch_before_any_hip_call():
    """sparse_decode_static keeps its split partials in a 32 MiB library-owned scratch: a
    call needing more is refused with WORKSPACE_TOO_SMALL, validated on the host."""
    lib = ubs.load()
    B, Hq, Hkv, D, P, ms = 2048, 32, 8, 128, 64, 64
    need = lib.ubs_decode_workspace_size(B, Hq, Hkv, D, P, ms, 128, 512)
    assert need > 32 << 20
    rc = lib.sparse_decode_static(A, A, A, A, A, B, 512, Hq, Hkv, D, P, KIND, A, A, ms, 128, 512, 0.088, A, NULL,
                                  NULL)
    assert rc == -3 and "static scratch" in _err()
    assert lib.sparse_decode_static(A, A, A, A, A, 4, 512, Hq, Hkv, 96, P, KIND, A, A, ms, 128, 512, 0.088, A,
                                    NULL, NULL) == -2
    assert lib.sparse_decode_static(A, A, A, A, A, 0, 512, Hq, Hkv, D, P, KIND, A, A, ms, 128, 512, 0.088, A,
                                    NULL, NULL) == 0


def test_bench_helpers_validate_before_any_hip_call():
    lib = ubs.load()
    assert lib.ubs_bench_read(NULL, 1024, A, NULL) == -1
    assert lib.ubs_bench_read(A, 1024, NULL, NULL) == -1
    assert lib.ubs_bench_read(A + 4, 1024, A, NULL) == -1     # misaligned
    assert lib.ubs_bench_read(A, 8, A, NULL) == -1            # under 16 bytes
    assert lib.ubs_bench_mfma(0, A, NULL) == -1
    assert lib.ubs_bench_mfma(10, NULL, NULL) == -1

