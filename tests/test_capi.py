"""CPU checks of the C ABI: the library loads, exports every function the header
declares, names its status codes, and rejects bad arguments on the host before
anything is enqueued (so no GPU is needed)."""
import ctypes
import os
import re

import pytest

from sparse_attention_fp4_cache_amd import lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa2fp4.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(lib.LIB_PATH):
        import __graft_entry__

        __graft_entry__.build()
    return lib.load()


def test_header_declares_the_five_calls():
    names = declared_functions()
    for n in ("fp4_cache_write", "index_score", "topk_select", "sparse_attn_decode", "sparse_attn_prefill_chunk"):
        assert n in names
    assert set(names) == set(lib.EXPORTS)


def test_library_exports_every_declared_symbol(L):
    for n in declared_functions():
        assert hasattr(L, n), n


def test_status_strings(L):
    assert lib.status_string(0) == "ok"
    for st in (-1, -2, -3, -4, -5):
        assert lib.status_string(st) != "unknown status"
    assert lib.status_string(-99) == "unknown status"


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def _cache(page=64, slots=128, null=False):
    s = lib._CacheStruct(None if null else 0x1000, 0x1000, 0x1000, 0x1000, slots, page)
    return ctypes.byref(s)


def test_cache_write_validation(L):
    assert L.fp4_cache_write(None, FAKE, FAKE, FAKE, 1, None) == -1
    assert L.fp4_cache_write(_cache(null=True), FAKE, FAKE, FAKE, 1, None) == -1
    assert L.fp4_cache_write(_cache(page=32), FAKE, FAKE, FAKE, 1, None) == -2
    assert L.fp4_cache_write(_cache(slots=100), FAKE, FAKE, FAKE, 1, None) == -2
    assert L.fp4_cache_write(_cache(), FAKE, FAKE, FAKE, -1, None) == -2
    assert L.fp4_cache_write(_cache(), None, FAKE, FAKE, 1, None) == -1
    assert L.fp4_cache_write(_cache(), FAKE, FAKE, FAKE, 0, None) == 0  # n == 0: nothing to do


def test_index_score_validation(L):
    c = _cache()
    args = dict(q=FAKE, w=FAKE, Hi=64, soq=None, nv=FAKE, bt=FAKE, mp=2, nq=1, sc=FAKE, ld=128)

    def call(**kw):
        a = dict(args, **kw)
        return L.index_score(c, a["q"], a["w"], a["Hi"], a["soq"], a["nv"], a["bt"], a["mp"], a["nq"], a["sc"],
                             a["ld"], None)

    for hi in (0, 8, 24 + 1, 144, 256):
        assert call(Hi=hi) == -2
    assert call(nq=-1) == -2
    assert call(ld=-5) == -2
    assert call(mp=1) == -2  # block table too narrow for ld
    assert call(q=None) == -1
    assert call(nv=None) == -1
    assert call(nq=0) == 0


def test_topk_validation(L):
    ws = L.topk_select_workspace_size(2, 10000, 64)
    assert ws > 0
    assert L.topk_select(FAKE, 10000, FAKE, 2, 0, FAKE, FAKE, ws, None) == -2
    assert L.topk_select(FAKE, 10000, FAKE, 2, 4097, FAKE, FAKE, ws, None) == -2
    assert L.topk_select(FAKE, 10000, FAKE, 2, 64, None, FAKE, ws, None) == -1
    assert L.topk_select(FAKE, 10000, FAKE, 2, 64, FAKE, None, ws, None) == -4
    assert L.topk_select(FAKE, 10000, FAKE, 2, 64, FAKE, FAKE, ws - 1, None) == -4
    assert L.topk_select(FAKE, 10000, FAKE, 0, 64, FAKE, FAKE, ws, None) == 0
    # workspace grows with the number of queries
    assert L.topk_select_workspace_size(4, 10000, 64) > ws


def test_pool_build_validation(L):
    ws = L.index_pool_build_workspace_size(2, 10000, 2048)
    assert ws > 0
    assert L.index_pool_build_workspace_size(4, 10000, 2048) > ws
    call = lambda sc=FAKE, ld=10000, nv=FAKE, nq=2, npool=2048, pool=FAKE, w=FAKE, wb=ws: L.index_pool_build(
        sc, ld, nv, nq, npool, pool, w, wb, None)
    assert call(npool=0) == -2
    assert call(npool=4097) == -2
    assert call(nq=-1) == -2
    assert call(pool=None) == -1
    assert call(nv=None) == -1
    assert call(w=None) == -4
    assert call(wb=ws - 1) == -4
    assert call(nq=0) == 0


def test_index_topk_pool_validation(L):
    ws = L.index_topk_pool_workspace_size(1, 2048, 256)
    assert ws > 0
    args = lambda **kw: dict(dict(cache=_cache(), q=FAKE, w=FAKE, Hi=64, soq=None, nv=FAKE, pool=FAKE, npool=2048,
                                  bt=FAKE, mp=64, nq=1, sc=FAKE, k=256, idx=FAKE, ws=FAKE, wsb=ws), **kw)
    call = lambda a: L.index_topk_pool(a["cache"], a["q"], a["w"], a["Hi"], a["soq"], a["nv"], a["pool"], a["npool"],
                                       a["bt"], a["mp"], a["nq"], a["sc"], a["k"], a["idx"], a["ws"], a["wsb"], None)
    assert call(args(cache=_cache(null=True))) == -1
    assert call(args(Hi=40)) == -2
    assert call(args(npool=0)) == -2
    assert call(args(npool=4097)) == -2
    assert call(args(k=0)) == -2
    assert call(args(mp=0)) == -2
    assert call(args(pool=None)) == -1
    assert call(args(idx=None)) == -1
    assert call(args(ws=None)) == -4
    assert call(args(wsb=ws - 1)) == -4
    assert call(args(nq=0)) == 0


def test_index_topk_validation(L):
    ws = L.topk_select_workspace_size(1, 4096, 64)
    args = lambda **kw: dict(dict(cache=_cache(), q=FAKE, w=FAKE, Hi=64, soq=None, nv=FAKE, bt=FAKE, mp=64, nq=1,
                                  sc=FAKE, ld=4096, k=64, idx=FAKE, ws=FAKE, wsb=ws), **kw)
    call = lambda a: L.index_topk(a["cache"], a["q"], a["w"], a["Hi"], a["soq"], a["nv"], a["bt"], a["mp"], a["nq"],
                                  a["sc"], a["ld"], a["k"], a["idx"], a["ws"], a["wsb"], None)
    assert call(args(cache=_cache(null=True))) == -1
    assert call(args(Hi=40)) == -2
    assert call(args(k=0)) == -2
    assert call(args(k=4097)) == -2
    assert call(args(idx=None)) == -1
    assert call(args(ws=None)) == -4
    assert call(args(wsb=ws - 1)) == -4
    assert call(args(mp=10)) == -2
    assert call(args(nq=0)) == 0


def test_counted_pair_validation(L):
    ws = L.topk_select_workspace_size(1, 4096, 64)
    args = lambda **kw: dict(dict(cache=_cache(), q=FAKE, w=FAKE, Hi=64, soq=None, nv=FAKE, bt=FAKE, mp=64, nq=1,
                                  sc=FAKE, ld=4096, k=64, ws=FAKE, wsb=ws), **kw)
    score = lambda a: L.index_score_counted(a["cache"], a["q"], a["w"], a["Hi"], a["soq"], a["nv"], a["bt"], a["mp"],
                                            a["nq"], a["sc"], a["ld"], a["k"], a["ws"], a["wsb"], None)
    assert score(args(cache=_cache(null=True))) == -1
    assert score(args(Hi=40)) == -2
    assert score(args(k=0)) == -2
    assert score(args(k=4097)) == -2
    assert score(args(ws=None)) == -4
    assert score(args(wsb=ws - 1)) == -4
    assert score(args(mp=10)) == -2
    assert score(args(nq=0)) == 0
    sel = lambda k=64, idx=FAKE, w_=FAKE, wsb=ws, nq=1: L.topk_select_counted(FAKE, 4096, FAKE, nq, k, idx, w_, wsb,
                                                                              None)
    assert sel(k=0) == -2
    assert sel(k=4097) == -2
    assert sel(idx=None) == -1
    assert sel(w_=None) == -4
    assert sel(wsb=ws - 1) == -4
    assert sel(nq=0) == 0


def test_attention_validation(L):
    c = _cache()
    ws = L.sparse_attn_decode_workspace_size(1, 64, 2048, 128)
    assert ws >= 256

    def dec(H=64, k=2048, window=128, B=1, scale=0.04, q=FAKE, wsb=ws, ws_ptr=FAKE):
        return L.sparse_attn_decode(c, q, H, FAKE, k, FAKE, 64, FAKE, FAKE, window, scale, B, FAKE, FAKE, ws_ptr,
                                    wsb, None)

    assert dec(H=8) == -2
    assert dec(H=144) == -2
    assert dec(k=5000) == -2
    assert dec(window=129) == -2
    assert dec(B=-1) == -2
    assert dec(scale=float("nan")) == -2
    assert dec(q=None) == -1
    assert dec(B=0) == 0
    if ws > 256:
        assert dec(wsb=ws - 1) == -4
        assert dec(ws_ptr=None) == -4
    pws = L.sparse_attn_prefill_chunk_workspace_size(4096, 64, 2048, 128)
    assert L.sparse_attn_prefill_chunk(c, FAKE, 64, FAKE, 2048, FAKE, 64, -1, 16, FAKE, 0, 128, 0.04, FAKE, FAKE,
                                       FAKE, pws, None) == -2
    assert L.sparse_attn_prefill_chunk(c, FAKE, 64, FAKE, 2048, FAKE, 64, 0, -1, FAKE, 0, 128, 0.04, FAKE, FAKE,
                                       FAKE, pws, None) == -2
    assert L.sparse_attn_prefill_chunk(c, FAKE, 64, FAKE, 2048, FAKE, 64, 0, 0, FAKE, 0, 128, 0.04, FAKE, FAKE,
                                       FAKE, pws, None) == 0


def test_fp8_window_validation(L):
    assert L.swa_fp8_write(FAKE, -1, FAKE, FAKE, None) == -2
    assert L.swa_fp8_write(FAKE, 0, None, None, None) == 0
    assert L.swa_fp8_write(None, 4, FAKE, FAKE, None) == -1
    assert L.swa_fp8_write(FAKE, 4, FAKE, None, None) == -1
    c = _cache()
    ws = L.sparse_attn_decode_workspace_size(1, 64, 2048, 128)

    def dec(codes=FAKE, scales=FAKE, window=128, H=64, B=1):
        return L.sparse_attn_decode_fp8win(c, FAKE, H, FAKE, 2048, FAKE, 64, codes, scales, FAKE, window, 0.04, B,
                                           FAKE, FAKE, FAKE, ws, None)

    assert dec(codes=None) == -1
    assert dec(scales=None) == -1
    assert dec(H=8) == -2
    assert dec(window=129) == -2
    assert dec(codes=None, scales=None, window=0, B=0) == 0
    assert dec(B=0) == 0
    pws = L.sparse_attn_prefill_chunk_workspace_size(16, 64, 2048, 128)

    def pre(codes=FAKE, scales=FAKE, T=16, start=0):
        return L.sparse_attn_prefill_chunk_fp8win(c, FAKE, 64, FAKE, 2048, FAKE, 64, start, T, codes, scales, 0, 128,
                                                  0.04, FAKE, FAKE, FAKE, pws, None)

    assert pre(codes=None) == -1
    assert pre(scales=None) == -1
    assert pre(start=-1) == -2
    assert pre(T=0) == 0


def test_index_topk_noalloc_validation(L):
    c = _cache(slots=1 << 20)

    def call(nq=1, ld=128, k=16, Hi=64, q=FAKE, out=FAKE):
        return L.index_topk_noalloc(c, q, FAKE, Hi, None, FAKE, FAKE, (ld + 63) // 64, nq, FAKE, ld, k, out, None)

    assert call(Hi=24) == -2
    assert call(k=0) == -2 and call(k=4097) == -2
    assert call(q=None) == -1
    assert call(out=None) == -1
    # more than the static workspace holds: rejected before anything is enqueued
    need = lib.load().topk_select_workspace_size(4096, 1 << 20, 2048)
    assert need > lib.NOALLOC_SCRATCH_BYTES
    assert call(nq=4096, ld=1 << 20, k=2048) == -4
    assert call(nq=0) == 0
