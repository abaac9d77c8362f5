"""The C ABI without a GPU: the library loads, exports every entry point the header declares,
and rejects invalid arguments with the documented status before touching the device."""
import ctypes
import os
import re

import pytest

import compressed_hybrid_sparse_amd as chs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "chs.h")
OK, NULL, SHAPE, DTYPE, WS, UNSUP = 0, 1, 2, 3, 4, 5
P = ctypes.c_void_p
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every case below fails validation first


def declared():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(chs_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_python_exports():
    assert declared() == sorted(chs.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = chs.lib()
    for name in declared():
        assert hasattr(L, name), name
    assert chs.version() >= 100
    assert b"WORKSPACE" in L.chs_status_string(WS)


def compress(dt=1, batch=1, d=512, m=4, x=FAKE, z=FAKE, b=FAKE, cut=FAKE, cug=FAKE, maxg=10, out=FAKE):
    return chs.lib().chs_compress(dt, batch, d, m, x, z, b, cut, cug, maxg, out, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=7), DTYPE), (dict(batch=0), SHAPE), (dict(m=0), SHAPE), (dict(m=1025), SHAPE),
    (dict(d=0), SHAPE), (dict(d=12), SHAPE), (dict(dt=0, d=6), SHAPE), (dict(maxg=-1), SHAPE),
    (dict(x=None), NULL), (dict(z=None), NULL), (dict(b=None), NULL), (dict(cut=None), NULL),
    (dict(cug=None), NULL), (dict(out=None), NULL), (dict(maxg=0), OK), (dict(batch=70000), SHAPE),
])
def test_compress_validation(kw, code):
    assert compress(**kw) == code


def append(dt=1, batch=1, d=512, m=4, W=128, R=8, x=FAKE, z=FAKE, b=FAKE, n=FAKE, swa=FAKE, sl=FAKE, ring=FAKE,
           page=FAKE, pages=1, comp=FAKE, cs=FAKE, rows=100, cc=FAKE):
    return chs.lib().chs_append(dt, batch, d, m, W, R, x, z, b, n, swa, sl, ring, page, pages, comp, cs, rows, cc,
                                None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=5), DTYPE), (dict(batch=0), SHAPE), (dict(batch=65536), SHAPE), (dict(d=0), SHAPE),
    (dict(d=12), SHAPE), (dict(dt=0, d=6), SHAPE), (dict(d=4104), SHAPE), (dict(m=0), SHAPE), (dict(m=1025), SHAPE),
    (dict(W=3), SHAPE), (dict(R=3), SHAPE), (dict(m=128, W=127, R=128), SHAPE), (dict(pages=0), SHAPE),
    (dict(rows=-1), SHAPE), (dict(x=None), NULL), (dict(z=None), NULL), (dict(b=None), NULL), (dict(n=None), NULL),
    (dict(swa=None), NULL), (dict(ring=None), NULL), (dict(page=None), NULL), (dict(comp=None), NULL),
    (dict(cs=None), NULL),
])
def test_append_validation(kw, code):
    # swa_len and comp_count are optional outputs; everything else is required.
    assert append(**kw) == code


def attn_paged(dt=1, batch=1, H=64, d=512, W=128, k=512, scale=0.04, q=FAKE, swa=FAKE, sp=FAKE, nsp=4, sl=FAKE,
               pool=FAKE, npool=100, P=64, pt=FAKE, stride=8, cl=FAKE, tk=FAKE, maxc=1000, out=FAKE, lse=FAKE, ws=FAKE,
               wsb=None):
    L = chs.lib()
    if wsb is None:
        wsb = L.chs_decode_attn_workspace_size(dt, batch, H, d, W, k if tk else 0, maxc)
    return L.chs_decode_attn_paged(dt, batch, H, d, W, k, ctypes.c_float(scale), q, swa, sp, nsp, sl, pool, npool, P, pt,
                                   stride, cl, tk, maxc, out, lse, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=4), DTYPE), (dict(batch=0), SHAPE), (dict(d=96), SHAPE), (dict(scale=-1.0), SHAPE), (dict(P=0), SHAPE),
    (dict(P=48), SHAPE), (dict(P=131072), SHAPE), (dict(stride=0), SHAPE), (dict(npool=0), SHAPE), (dict(nsp=0), SHAPE),
    (dict(q=None), NULL), (dict(sl=None), NULL), (dict(cl=None), NULL), (dict(pt=None), NULL), (dict(sp=None), NULL),
    (dict(out=None), NULL), (dict(ws=None), NULL), (dict(wsb=8), WS),
])
def test_decode_attn_paged_validation(kw, code):
    assert attn_paged(**kw) == code


def append_paged(dt=1, batch=1, d=512, m=4, W=128, R=8, x=FAKE, z=FAKE, b=FAKE, n=FAKE, swa=FAKE, sp=FAKE, nsp=4,
                 sl=FAKE, ring=FAKE, pool=FAKE, npool=100, P=64, pt=FAKE, stride=8, cc=FAKE):
    return chs.lib().chs_append_paged(dt, batch, d, m, W, R, x, z, b, n, swa, sp, nsp, sl, ring, pool, npool, P, pt,
                                      stride, cc, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=4), DTYPE), (dict(batch=0), SHAPE), (dict(d=12), SHAPE), (dict(m=0), SHAPE), (dict(W=3), SHAPE),
    (dict(R=2), SHAPE), (dict(P=0), SHAPE), (dict(P=24), SHAPE), (dict(stride=0), SHAPE), (dict(nsp=0), SHAPE),
    (dict(npool=-1), SHAPE), (dict(x=None), NULL), (dict(n=None), NULL), (dict(swa=None), NULL), (dict(sp=None), NULL),
    (dict(ring=None), NULL), (dict(pool=None), NULL), (dict(pt=None), NULL),
])
def test_append_paged_validation(kw, code):
    assert append_paged(**kw) == code


def topk_paged(dt=1, batch=1, nh=4, dim=128, k=512, q=FAKE, w=FAKE, pool=FAKE, npool=100, P=64, pt=FAKE, stride=8,
               cl=FAKE, maxc=1000, s=FAKE, out=FAKE, ws=FAKE, wsb=None):
    L = chs.lib()
    if wsb is None:
        wsb = L.chs_index_topk_workspace_size(batch, maxc, k)
    return L.chs_index_topk_paged(dt, batch, nh, dim, k, q, w, pool, npool, P, pt, stride, cl, maxc, s, out, ws, wsb,
                                  None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=9), DTYPE), (dict(batch=0), SHAPE), (dict(k=0), SHAPE), (dict(nh=17), SHAPE), (dict(P=32), SHAPE),
    (dict(P=96), SHAPE), (dict(stride=0), SHAPE), (dict(npool=0), SHAPE), (dict(maxc=-1), SHAPE),
    (dict(dt=0), UNSUP), (dict(dim=96), UNSUP), (dict(dim=512), UNSUP), (dict(q=None), NULL), (dict(w=None), NULL),
    (dict(pool=None), NULL), (dict(pt=None), NULL), (dict(cl=None), NULL), (dict(out=None), NULL),
    (dict(ws=None), NULL), (dict(wsb=16), WS),
])
def test_index_topk_paged_validation(kw, code):
    assert topk_paged(**kw) == code


def gather(dt=1, batch=1, d=512, k=512, mirror=FAKE, host=0, cu=FAKE, tk=FAKE, cache=None, res=None, rows=0,
           work=FAKE, wtk=FAKE):
    return chs.lib().chs_gather_selected(dt, batch, d, k, mirror, host, cu, tk, cache, res, rows, work, wtk, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=3), DTYPE), (dict(batch=0), SHAPE), (dict(k=0), SHAPE), (dict(k=2049), SHAPE), (dict(d=0), SHAPE),
    (dict(d=12), SHAPE), (dict(rows=-1), SHAPE), (dict(mirror=None), NULL), (dict(cu=None), NULL),
    (dict(tk=None), NULL), (dict(work=None), NULL), (dict(wtk=None), NULL), (dict(res=FAKE), NULL),
])
def test_gather_selected_validation(kw, code):
    assert gather(**kw) == code


def test_gather_binding_refuses_unpinned_host_mirror():
    # The binding checks a host mirror is pinned before anything reaches the library or the GPU.
    import torch
    with pytest.raises(ValueError, match="pinned"):
        chs.gather_selected(torch.zeros(4, 8, dtype=torch.bfloat16), None, None)


def test_append_stream_struct_layout():
    # Field offsets of chs_append_stream under the C ABI (natural alignment, 8-byte pointers).
    S = chs.AppendStream
    assert S.d.offset == 0 and S.ring_size.offset == 8 and S.x_new.offset == 16
    assert S.ring_pages.offset == 80 and S.comp_count.offset == 112 and S.page_table.offset == 136
    assert S.pt_stride.offset == 144 and S.page_size.offset == 148 and S.pool_pages.offset == 152
    assert ctypes.sizeof(S) == 160


def test_append_multi_validation():
    L = chs.lib()
    arr = (chs.AppendStream * 2)()
    assert L.chs_append_multi(1, 1, 4, 0, arr, None) == SHAPE
    assert L.chs_append_multi(1, 1, 4, 5, arr, None) == SHAPE
    assert L.chs_append_multi(1, 1, 4, 1, None, None) == NULL
    assert L.chs_append_multi(1, 1, 4, 1, arr, None) == SHAPE            # d = 0
    for st in arr:
        st.d, st.window, st.ring_size = 512, 128, 8
        st.x_new = st.z_new = st.bias = st.n_tokens = st.swa_kv = st.gate_ring = st.comp_kv = 0x1000
        st.ring_page = st.comp_start = 0x1000
        st.ring_pages, st.comp_rows = 4, 100
    assert L.chs_append_multi(7, 1, 4, 2, arr, None) == DTYPE
    arr[1].x_new = None
    assert L.chs_append_multi(1, 1, 4, 2, arr, None) == NULL              # the second stream is checked too
    arr[1].x_new = 0x1000
    arr[1].page_table, arr[1].page_size, arr[1].pt_stride, arr[1].pool_pages = 0x1000, 48, 2, 10
    assert L.chs_append_multi(1, 1, 4, 2, arr, None) == SHAPE             # page size not a power of two
    arr[1].page_size = 64
    assert L.chs_append_multi(1, 1, 4, 2, arr, None) == SHAPE             # paged without window pages
    arr[1].swa_pages = 2
    assert L.chs_append_multi(1, 1, 4, 2, arr, None) == NULL              # paged without swa_page


def topk8_paged(batch=1, nh=4, dim=128, k=512, q=FAKE, w=FAKE, pool=FAKE, sc=FAKE, npool=100, P=64, pt=FAKE,
                stride=8, cl=FAKE, maxc=1000, s=FAKE, out=FAKE, ws=FAKE, wsb=None):
    L = chs.lib()
    if wsb is None:
        wsb = L.chs_index_topk_workspace_size(batch, maxc, k)
    return L.chs_index_topk_fp8_paged(batch, nh, dim, k, q, w, pool, sc, npool, P, pt, stride, cl, maxc, s, out, ws,
                                      wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), SHAPE), (dict(k=0), SHAPE), (dict(nh=17), SHAPE), (dict(P=48), SHAPE), (dict(P=32), SHAPE),
    (dict(dim=64, P=64), SHAPE), (dict(stride=0), SHAPE), (dict(npool=0), SHAPE), (dict(dim=96), UNSUP),
    (dict(dim=512), UNSUP), (dict(q=None), NULL), (dict(sc=None), NULL), (dict(pool=None), NULL),
    (dict(pt=None), NULL), (dict(cl=None), NULL), (dict(ws=None), NULL), (dict(wsb=16), WS),
    (dict(dim=256, P=32, pt=None), NULL),   # 32-row pages suffice at 256 channels: only the NULL is caught
])
def test_index_topk_fp8_paged_validation(kw, code):
    assert topk8_paged(**kw) == code


def attn8_paged(batch=1, H=64, d=512, W=128, k=512, scale=0.04, q=FAKE, swa=FAKE, ssc=FAKE, sp=FAKE, nsp=4, sl=FAKE,
                pool=FAKE, csc=FAKE, npool=100, P=64, pt=FAKE, stride=8, cl=FAKE, tk=FAKE, maxc=1000, out=FAKE,
                lse=FAKE, ws=FAKE, wsb=None):
    L = chs.lib()
    if wsb is None:
        wsb = L.chs_decode_attn_workspace_size(1, batch, H, d, W, k if tk else 0, maxc)
    return L.chs_decode_attn_fp8_paged(batch, H, d, W, k, ctypes.c_float(scale), q, swa, ssc, sp, nsp, sl, pool, csc,
                                       npool, P, pt, stride, cl, tk, maxc, out, lse, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), SHAPE), (dict(d=96), SHAPE), (dict(P=0), SHAPE), (dict(P=24), SHAPE), (dict(stride=0), SHAPE),
    (dict(npool=0), SHAPE), (dict(nsp=0), SHAPE), (dict(q=None), NULL), (dict(ssc=None), NULL), (dict(sp=None), NULL),
    (dict(csc=None), NULL), (dict(pt=None), NULL), (dict(cl=None), NULL), (dict(ws=None), NULL), (dict(wsb=8), WS),
])
def test_decode_attn_fp8_paged_validation(kw, code):
    assert attn8_paged(**kw) == code


def topk(dt=1, batch=1, nh=4, dim=128, k=512, q=FAKE, w=FAKE, kk=FAKE, cu=FAKE, maxc=1000, s=FAKE, out=FAKE,
         ws=FAKE, wsb=None):
    L = chs.lib()
    if wsb is None:
        wsb = L.chs_index_topk_workspace_size(batch, maxc, k)
    return L.chs_index_topk(dt, batch, nh, dim, k, q, w, kk, cu, maxc, s, out, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=2), DTYPE), (dict(k=0), SHAPE), (dict(k=2049), SHAPE), (dict(batch=0), SHAPE),
    (dict(maxc=-1), SHAPE), (dict(maxc=1 << 31), SHAPE), (dict(nh=0), SHAPE), (dict(nh=17), SHAPE),
    (dict(dim=4), SHAPE), (dict(dim=12), SHAPE), (dict(dim=1024), SHAPE), (dict(dt=0, dim=512), SHAPE), (dict(w=None), NULL),
    (dict(kk=None), NULL), (dict(q=None, s=None), NULL), (dict(cu=None), NULL), (dict(out=None), NULL),
    (dict(ws=None), NULL), (dict(wsb=16), WS),
])
def test_index_topk_validation(kw, code):
    assert topk(**kw) == code


def topk8(batch=1, nh=4, dim=128, k=512, q=FAKE, w=FAKE, kk=FAKE, sc=FAKE, cu=FAKE, maxc=1000, s=FAKE, out=FAKE,
          ws=FAKE, wsb=None):
    L = chs.lib()
    if wsb is None:
        wsb = L.chs_index_topk_workspace_size(batch, maxc, k)
    return L.chs_index_topk_fp8(batch, nh, dim, k, q, w, kk, sc, cu, maxc, s, out, ws, wsb, None)


def index_scores(dt=1, batch=1, nh=4, dim=128, q=FAKE, w=FAKE, kk=FAKE, cu=FAKE, maxc=1000, s=FAKE, ws=FAKE,
                 wsb=1 << 20):
    return chs.lib().chs_index_scores(dt, batch, nh, dim, q, w, kk, cu, maxc, s, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=9), DTYPE), (dict(batch=0), SHAPE), (dict(nh=0), SHAPE), (dict(nh=17), SHAPE), (dict(dim=4), SHAPE),
    (dict(dim=520), SHAPE), (dict(maxc=-1), SHAPE), (dict(maxc=(1 << 22) + 1), UNSUP), (dict(q=None), NULL),
    (dict(w=None), NULL), (dict(kk=None), NULL), (dict(cu=None), NULL), (dict(s=None), NULL), (dict(ws=None), NULL),
    (dict(wsb=16), WS), (dict(maxc=0), OK),
])
def test_index_scores_validation(kw, code):
    assert index_scores(**kw) == code


def test_index_scores_workspace_is_the_topk_workspace():
    L = chs.lib()
    assert L.chs_index_topk_workspace_size(3, 262144, 1) == L.chs_index_topk_workspace_size(3, 262144, 512)


@pytest.mark.parametrize("kw,code", [
    (dict(k=0), SHAPE), (dict(k=2049), SHAPE), (dict(batch=0), SHAPE), (dict(maxc=-1), SHAPE),
    (dict(maxc=1 << 31), SHAPE), (dict(nh=0), SHAPE), (dict(nh=17), SHAPE), (dict(dim=8), SHAPE),
    (dict(dim=24), SHAPE), (dict(dim=528), SHAPE), (dict(maxc=(1 << 22) + 1), UNSUP), (dict(q=None), NULL),
    (dict(w=None), NULL), (dict(kk=None), NULL), (dict(sc=None), NULL), (dict(cu=None), NULL),
    (dict(out=None), NULL), (dict(ws=None), NULL), (dict(wsb=16), WS),
])
def test_index_topk_fp8_validation(kw, code):
    assert topk8(**kw) == code


def attn(dt=1, batch=1, H=64, d=512, W=128, k=512, scale=0.04, q=FAKE, swa=FAKE, sl=FAKE, comp=FAKE, cu=FAKE,
         tk=FAKE, maxc=1000, out=FAKE, lse=FAKE, ws=FAKE, wsb=None):
    L = chs.lib()
    if wsb is None:
        wsb = L.chs_decode_attn_workspace_size(dt, batch, H, d, W, k if tk else 0, maxc)
    return L.chs_decode_attn(dt, batch, H, d, W, k, ctypes.c_float(scale), q, swa, sl, comp, cu, tk, maxc,
                             out, lse, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=5), DTYPE), (dict(batch=0), SHAPE), (dict(H=0), SHAPE), (dict(H=129), SHAPE),
    (dict(d=96), SHAPE), (dict(dt=0, d=1028), SHAPE), (dict(dt=0, d=6), SHAPE), (dict(W=-1), SHAPE),
    (dict(k=2049), SHAPE), (dict(scale=0.0), SHAPE), (dict(scale=float("inf")), SHAPE),
    (dict(scale=float("nan")), SHAPE), (dict(maxc=-2), SHAPE), (dict(q=None), NULL), (dict(sl=None), NULL),
    (dict(cu=None), NULL), (dict(out=None), NULL), (dict(ws=None), NULL), (dict(swa=None), NULL),
    (dict(comp=None), NULL), (dict(wsb=8), WS),
])
def test_decode_attn_validation(kw, code):
    assert attn(**kw) == code


def attn8(batch=1, H=64, d=512, W=128, k=512, scale=0.04, q=FAKE, swa=FAKE, ssc=FAKE, sl=FAKE, comp=FAKE, csc=FAKE,
          cu=FAKE, tk=FAKE, maxc=1000, out=FAKE, lse=FAKE, ws=FAKE, wsb=None):
    L = chs.lib()
    if wsb is None:
        wsb = L.chs_decode_attn_workspace_size(1, batch, H, d, W, k if tk else 0, maxc)
    return L.chs_decode_attn_fp8(batch, H, d, W, k, ctypes.c_float(scale), q, swa, ssc, sl, comp, csc, cu, tk, maxc,
                                 out, lse, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), SHAPE), (dict(H=129), SHAPE), (dict(d=96), SHAPE), (dict(W=-1), SHAPE), (dict(k=2049), SHAPE),
    (dict(scale=0.0), SHAPE), (dict(q=None), NULL), (dict(swa=None), NULL), (dict(ssc=None), NULL),
    (dict(sl=None), NULL), (dict(comp=None), NULL), (dict(csc=None), NULL), (dict(cu=None), NULL),
    (dict(out=None), NULL), (dict(ws=None), NULL), (dict(wsb=8), WS), (dict(W=0, swa=None, ssc=None, wsb=8), WS),
])
def test_decode_attn_fp8_validation(kw, code):
    assert attn8(**kw) == code


def step(batch=1, H=64, d=512, W=128, k=512, scale=0.04, nh=4, dI=128, qi=FAKE, w=FAKE, ki=FAKE, q=FAKE, swa=FAKE,
         sl=FAKE, comp=FAKE, cu=FAKE, maxc=1000, sc=FAKE, tk=FAKE, out=FAKE, lse=FAKE, ws=FAKE, wsb=None):
    L = chs.lib()
    if wsb is None:
        wsb = L.chs_decode_step_workspace_size(batch, H, d, W, k, maxc)
    return L.chs_decode_step(batch, H, d, W, k, ctypes.c_float(scale), nh, dI, qi, w, ki, q, swa, sl, comp, cu, maxc,
                             sc, tk, out, lse, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), SHAPE), (dict(H=0), SHAPE), (dict(H=129), SHAPE), (dict(d=96), SHAPE), (dict(d=1024), SHAPE),
    (dict(W=-1), SHAPE), (dict(k=0), SHAPE), (dict(k=2049), SHAPE), (dict(scale=0.0), SHAPE),
    (dict(scale=float("nan")), SHAPE), (dict(maxc=-1), SHAPE), (dict(nh=0), SHAPE), (dict(nh=17), SHAPE),
    (dict(dI=4), SHAPE), (dict(dI=1024), SHAPE), (dict(qi=None), NULL), (dict(w=None), NULL), (dict(ki=None), NULL),
    (dict(q=None), NULL), (dict(swa=None), NULL), (dict(sl=None), NULL), (dict(comp=None), NULL),
    (dict(cu=None), NULL), (dict(tk=None), NULL), (dict(out=None), NULL), (dict(ws=None), NULL), (dict(wsb=8), WS),
])
def test_decode_step_validation(kw, code):
    assert step(**kw) == code


def step8(batch=1, H=64, d=512, W=128, k=512, scale=0.04, nh=4, dI=128, qi=FAKE, w=FAKE, ki=FAKE, ks=FAKE, q=FAKE,
          swa=FAKE, ss=FAKE, sl=FAKE, comp=FAKE, cs=FAKE, cu=FAKE, maxc=1000, sc=FAKE, tk=FAKE, out=FAKE, lse=FAKE,
          ws=FAKE, wsb=None):
    L = chs.lib()
    if wsb is None:
        wsb = L.chs_decode_step_workspace_size(batch, H, d, W, k, maxc)
    return L.chs_decode_step_fp8(batch, H, d, W, k, ctypes.c_float(scale), nh, dI, qi, w, ki, ks, q, swa, ss, sl, comp,
                                 cs, cu, maxc, sc, tk, out, lse, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), SHAPE), (dict(H=0), SHAPE), (dict(d=96), SHAPE), (dict(k=0), SHAPE), (dict(k=2049), SHAPE),
    (dict(scale=0.0), SHAPE), (dict(nh=17), SHAPE), (dict(dI=24), SHAPE), (dict(dI=1024), SHAPE),
    (dict(qi=None), NULL), (dict(ki=None), NULL), (dict(ks=None), NULL), (dict(ss=None), NULL), (dict(cs=None), NULL),
    (dict(q=None), NULL), (dict(comp=None), NULL), (dict(tk=None), NULL), (dict(ws=None), NULL), (dict(wsb=8), WS),
])
def test_decode_step_fp8_validation(kw, code):
    assert step8(**kw) == code


def stepp(batch=1, H=64, d=512, W=128, k=512, scale=0.04, nh=4, dI=128, qi=FAKE, w=FAKE, kp=FAKE, q=FAKE, swa=FAKE,
          sp=FAKE, swa_pages=4, sl=FAKE, comp=FAKE, pool_pages=16, P=64, pt=FAKE, pts=16, cl=FAKE, maxc=1000,
          sc=FAKE, tk=FAKE, out=FAKE, lse=FAKE, ws=FAKE, wsb=None):
    L = chs.lib()
    if wsb is None:
        wsb = L.chs_decode_step_workspace_size(batch, H, d, W, k, maxc)
    return L.chs_decode_step_paged(batch, H, d, W, k, ctypes.c_float(scale), nh, dI, qi, w, kp, q, swa, sp, swa_pages,
                                   sl, comp, pool_pages, P, pt, pts, cl, maxc, sc, tk, out, lse, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), SHAPE), (dict(H=0), SHAPE), (dict(d=96), SHAPE), (dict(k=0), SHAPE), (dict(k=2049), SHAPE),
    (dict(scale=0.0), SHAPE), (dict(nh=17), SHAPE), (dict(P=48), SHAPE), (dict(P=32), SHAPE), (dict(pts=0), SHAPE),
    (dict(pool_pages=0), SHAPE), (dict(swa_pages=0), SHAPE), (dict(dI=96), UNSUP), (dict(qi=None), NULL),
    (dict(kp=None), NULL), (dict(sp=None), NULL), (dict(pt=None), NULL), (dict(cl=None), NULL), (dict(q=None), NULL),
    (dict(tk=None), NULL), (dict(ws=None), NULL), (dict(wsb=8), WS),
])
def test_decode_step_paged_validation(kw, code):
    assert stepp(**kw) == code


def test_decode_step_workspace_covers_both_calls():
    L = chs.lib()
    for batch, H, d, W, k, G in [(1, 64, 512, 128, 512, 262144), (64, 64, 512, 128, 512, 50000), (2, 8, 64, 128, 64, 256)]:
        need = L.chs_decode_step_workspace_size(batch, H, d, W, k, G)
        assert need >= (L.chs_index_topk_workspace_size(batch, G, k)
                        + L.chs_decode_attn_workspace_size(1, batch, H, d, W, k, G))
    assert L.chs_decode_step_workspace_size(0, 64, 512, 128, 512, 10) == 0
    assert L.chs_decode_step_workspace_size(1, 64, 512, 128, 0, 10) == 0


def test_workspace_sizes_are_monotone():
    L = chs.lib()
    a = [L.chs_index_topk_workspace_size(b, n, 512) for b, n in [(1, 1000), (1, 262144), (4, 262144)]]
    assert 0 < a[0] < a[1] < a[2]
    s = [L.chs_decode_attn_workspace_size(1, 1, 64, 512, 128, 512, 262144),
         L.chs_decode_attn_workspace_size(1, 4, 64, 512, 128, 0, 8192),
         L.chs_decode_attn_workspace_size(1, 64, 64, 512, 128, 512, 50000)]
    assert all(x > 0 for x in s)
    assert L.chs_index_topk_workspace_size(0, 10, 5) == 0


def test_workspace_clear_validation():
    L = chs.lib()
    assert L.chs_workspace_clear(None, 0, None) == OK
    assert L.chs_workspace_clear(None, 16, None) == NULL
    assert L.chs_workspace_clear(FAKE, 6, None) == SHAPE


def test_decode_step_noalloc_refuses_before_touching_the_device():
    # Checked without a GPU: a workspace beyond the scratch array and invalid shapes are refused
    # before the call looks up its device or launches anything.
    L = chs.lib()
    big = L.chs_decode_step_noalloc(64, 128, 512, 4096, 2048, ctypes.c_float(0.04), 4, 128, FAKE, FAKE, FAKE, FAKE,
                                    FAKE, FAKE, FAKE, FAKE, 1 << 22, None, FAKE, FAKE, FAKE, None)
    assert big == WS
    bad = L.chs_decode_step_noalloc(0, 64, 512, 128, 512, ctypes.c_float(0.04), 4, 128, FAKE, FAKE, FAKE, FAKE,
                                    FAKE, FAKE, FAKE, FAKE, 1000, None, FAKE, FAKE, FAKE, None)
    assert bad == SHAPE


def quantize(dt=1, n=10, d=128, x=FAKE, c=FAKE, s=FAKE):
    return chs.lib().chs_quantize_e4m3(dt, n, d, x, c, s, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=4), DTYPE), (dict(n=-1), SHAPE), (dict(d=4), SHAPE), (dict(d=12), SHAPE), (dict(d=4104), SHAPE),
    (dict(x=None), NULL), (dict(c=None), NULL), (dict(s=None), NULL), (dict(n=0, x=None), OK),
])
def test_quantize_e4m3_validation(kw, code):
    assert quantize(**kw) == code


def compress_fp8(dt=1, batch=1, d=512, m=4, x=FAKE, z=FAKE, b=FAKE, cut=FAKE, cug=FAKE, maxg=10, c=FAKE, s=FAKE):
    return chs.lib().chs_compress_fp8(dt, batch, d, m, x, z, b, cut, cug, maxg, c, s, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=7), DTYPE), (dict(batch=0), SHAPE), (dict(m=0), SHAPE), (dict(d=12), SHAPE), (dict(maxg=-1), SHAPE),
    (dict(d=1024), UNSUP), (dict(d=384), UNSUP), (dict(dt=0, d=512), UNSUP), (dict(x=None), NULL),
    (dict(c=None), NULL), (dict(s=None), NULL), (dict(maxg=0), OK), (dict(dt=0, d=256, maxg=0), OK),
])
def test_compress_fp8_validation(kw, code):
    assert compress_fp8(**kw) == code


def append_fp8(dt=1, batch=1, d=512, m=4, W=128, R=8, x=FAKE, z=FAKE, b=FAKE, n=FAKE, sc=FAKE, ss=FAKE, sl=FAKE,
               xr=FAKE, gr=FAKE, page=FAKE, pages=1, cc=FAKE, cs=FAKE, start=FAKE, rows=100, cnt=FAKE):
    return chs.lib().chs_append_fp8(dt, batch, d, m, W, R, x, z, b, n, sc, ss, sl, xr, gr, page, pages, cc, cs, start,
                                    rows, cnt, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=5), DTYPE), (dict(batch=0), SHAPE), (dict(d=12), SHAPE), (dict(m=0), SHAPE), (dict(W=3), SHAPE),
    (dict(R=3), SHAPE), (dict(pages=0), SHAPE), (dict(rows=-1), SHAPE), (dict(d=1024), UNSUP), (dict(d=520), UNSUP),
    (dict(x=None), NULL), (dict(sc=None), NULL), (dict(ss=None), NULL), (dict(xr=None), NULL), (dict(gr=None), NULL),
    (dict(page=None), NULL), (dict(cc=None), NULL), (dict(cs=None), NULL), (dict(start=None), NULL),
])
def test_append_fp8_validation(kw, code):
    assert append_fp8(**kw) == code
