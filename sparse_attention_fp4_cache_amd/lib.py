"""ctypes binding of libcsa2fp4.so (declared in include/csa2fp4.h).

Argument marshalling only: every function checks dtypes, shapes, contiguity and
device of torch tensors, passes raw device pointers and the current HIP stream,
and raises Csa2Error on a negative status.  All computation happens in the HIP
kernels of the library; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsa2fp4.so")

LATENT_DIM = 512
INDEX_DIM = 128
PAGE_SIZE = 64
MAX_K = 4096
MAX_WINDOW = 128

EXPORTS = (
    "csa2_status_string",
    "fp4_cache_write",
    "index_score",
    "topk_select_workspace_size",
    "topk_select",
    "index_topk",
    "index_score_counted",
    "topk_select_counted",
    "index_pool_build_workspace_size",
    "index_pool_build",
    "index_topk_pool_build_workspace_size",
    "index_topk_pool_build",
    "index_topk_pool_workspace_size",
    "index_topk_pool",
    "sparse_attn_decode_workspace_size",
    "sparse_attn_decode",
    "sparse_attn_prefill_chunk_workspace_size",
    "sparse_attn_prefill_chunk",
    "swa_fp8_write",
    "sparse_attn_decode_fp8win",
    "sparse_attn_prefill_chunk_fp8win",
    "index_topk_noalloc",
    "csa2_exact_path_count",
    "csa2_exact_path_reset",
)


class Csa2Error(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


class _CacheStruct(ctypes.Structure):
    _fields_ = [
        ("main_codes", ctypes.c_void_p),
        ("main_scales", ctypes.c_void_p),
        ("idx_codes", ctypes.c_void_p),
        ("idx_scales", ctypes.c_void_p),
        ("num_slots", ctypes.c_int64),
        ("page_size", ctypes.c_int32),
    ]


_lib = None
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t


def load() -> ctypes.CDLL:
    """Open libcsa2fp4.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        L.csa2_status_string.restype = ctypes.c_char_p
        L.csa2_status_string.argtypes = [ctypes.c_int]
        L.fp4_cache_write.argtypes = [ctypes.POINTER(_CacheStruct), _P, _P, _P, _I64, _P]
        L.index_score.argtypes = [ctypes.POINTER(_CacheStruct), _P, _P, _I32, _P, _P, _P, _I32, _I32, _P, _I64, _P]
        L.topk_select_workspace_size.argtypes = [_I32, _I64, _I32]
        L.topk_select_workspace_size.restype = _SZ
        L.topk_select.argtypes = [_P, _I64, _P, _I32, _I32, _P, _P, _SZ, _P]
        L.index_topk.argtypes = [ctypes.POINTER(_CacheStruct), _P, _P, _I32, _P, _P, _P, _I32, _I32, _P, _I64, _I32,
                                 _P, _P, _SZ, _P]
        L.index_score_counted.argtypes = [ctypes.POINTER(_CacheStruct), _P, _P, _I32, _P, _P, _P, _I32, _I32, _P,
                                          _I64, _I32, _P, _SZ, _P]
        L.topk_select_counted.argtypes = [_P, _I64, _P, _I32, _I32, _P, _P, _SZ, _P]
        L.index_pool_build_workspace_size.argtypes = [_I32, _I64, _I32]
        L.index_pool_build_workspace_size.restype = _SZ
        L.index_pool_build.argtypes = [_P, _I64, _P, _I32, _I32, _P, _P, _SZ, _P]
        L.index_topk_pool_build_workspace_size.argtypes = [_I32, _I64, _I32, _I32]
        L.index_topk_pool_build_workspace_size.restype = _SZ
        L.index_topk_pool_build.argtypes = [ctypes.POINTER(_CacheStruct), _P, _P, _I32, _P, _P, _P, _I32, _I32, _P,
                                            _I64, _I32, _P, _I32, _P, _P, _SZ, _P]
        L.index_topk_pool_workspace_size.argtypes = [_I32, _I32, _I32]
        L.index_topk_pool_workspace_size.restype = _SZ
        L.index_topk_pool.argtypes = [ctypes.POINTER(_CacheStruct), _P, _P, _I32, _P, _P, _P, _I32, _P, _I32, _I32,
                                      _P, _I32, _P, _P, _SZ, _P]
        L.sparse_attn_decode_workspace_size.argtypes = [_I32, _I32, _I32, _I32]
        L.sparse_attn_decode_workspace_size.restype = _SZ
        L.sparse_attn_decode.argtypes = [ctypes.POINTER(_CacheStruct), _P, _I32, _P, _I32, _P, _I32, _P, _P, _I32,
                                         ctypes.c_float, _I32, _P, _P, _P, _SZ, _P]
        L.sparse_attn_prefill_chunk_workspace_size.argtypes = [_I32, _I32, _I32, _I32]
        L.sparse_attn_prefill_chunk_workspace_size.restype = _SZ
        L.sparse_attn_prefill_chunk.argtypes = [ctypes.POINTER(_CacheStruct), _P, _I32, _P, _I32, _P, _I32, _I64,
                                                _I32, _P, _I32, _I32, ctypes.c_float, _P, _P, _P, _SZ, _P]
        L.swa_fp8_write.argtypes = [_P, _I64, _P, _P, _P]
        L.sparse_attn_decode_fp8win.argtypes = [ctypes.POINTER(_CacheStruct), _P, _I32, _P, _I32, _P, _I32, _P, _P,
                                                _P, _I32, ctypes.c_float, _I32, _P, _P, _P, _SZ, _P]
        L.sparse_attn_prefill_chunk_fp8win.argtypes = [ctypes.POINTER(_CacheStruct), _P, _I32, _P, _I32, _P, _I32,
                                                       _I64, _I32, _P, _P, _I32, _I32, ctypes.c_float, _P, _P, _P,
                                                       _SZ, _P]
        L.index_topk_noalloc.argtypes = [ctypes.POINTER(_CacheStruct), _P, _P, _I32, _P, _P, _P, _I32, _I32, _P,
                                         _I64, _I32, _P, _P]
        L.csa2_exact_path_count.argtypes = [ctypes.POINTER(ctypes.c_ulonglong)]
        L.csa2_exact_path_reset.argtypes = []
        for name in EXPORTS:
            if name not in ("csa2_status_string",) and not name.endswith("_size"):
                getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return load().csa2_status_string(int(status)).decode()


def _check(fn: str, st: int) -> None:
    if st != 0:
        raise Csa2Error(fn, st, status_string(st))


def _stream(stream=None) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t: torch.Tensor | None, dtype=None, name: str = "tensor", device=None):
    if t is None:
        return None
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


_U16 = torch.uint16 if hasattr(torch, "uint16") else torch.int16


def _bits16(t: torch.Tensor, name: str):
    """bf16 bit patterns: accept bfloat16, int16 or uint16 tensors (no conversion)."""
    if t.dtype not in (torch.bfloat16, torch.int16, _U16):
        raise TypeError(f"{name}: expected bf16 bit patterns, got {t.dtype}")
    return _ptr(t, None, name)


class Cache:
    """One global FP4 cache in device memory: per slot 256 + 32 + 64 + 4 bytes."""

    def __init__(self, num_slots: int, device="cuda"):
        if num_slots <= 0 or num_slots % PAGE_SIZE:
            raise ValueError("num_slots must be a positive multiple of the page size (64)")
        self.num_slots = int(num_slots)
        self.main_codes = torch.zeros((num_slots, 256), dtype=torch.uint8, device=device)
        self.main_scales = torch.zeros((num_slots, 32), dtype=torch.uint8, device=device)
        self.idx_codes = torch.zeros((num_slots, 64), dtype=torch.uint8, device=device)
        self.idx_scales = torch.zeros((num_slots, 4), dtype=torch.uint8, device=device)
        self._s = _CacheStruct(self.main_codes.data_ptr(), self.main_scales.data_ptr(), self.idx_codes.data_ptr(),
                               self.idx_scales.data_ptr(), self.num_slots, PAGE_SIZE)

    @property
    def struct(self):
        return ctypes.byref(self._s)

    def nbytes(self) -> int:
        return self.num_slots * (256 + 32 + 64 + 4)

    def clone(self) -> "Cache":
        """A second cache in fresh device memory holding the same bytes."""
        c = Cache.__new__(Cache)
        c.num_slots = self.num_slots
        for name in ("main_codes", "main_scales", "idx_codes", "idx_scales"):
            setattr(c, name, getattr(self, name).clone())
        c._s = _CacheStruct(c.main_codes.data_ptr(), c.main_scales.data_ptr(), c.idx_codes.data_ptr(),
                            c.idx_scales.data_ptr(), c.num_slots, PAGE_SIZE)
        return c


def fp4_cache_write(cache: Cache, latent: torch.Tensor, idx_key: torch.Tensor, slot: torch.Tensor, stream=None):
    n = slot.shape[0]
    if latent.shape != (n, LATENT_DIM) or idx_key.shape != (n, INDEX_DIM):
        raise ValueError("latent must be [n,512] and idx_key [n,128]")
    _check("fp4_cache_write", load().fp4_cache_write(cache.struct, _bits16(latent, "latent"),
                                                     _bits16(idx_key, "idx_key"), _ptr(slot, torch.int64, "slot"),
                                                     n, _stream(stream)))


def index_score(cache: Cache, q_idx: torch.Tensor, w: torch.Tensor, n_visible: torch.Tensor,
                block_table: torch.Tensor, scores: torch.Tensor, seq_of_query: torch.Tensor | None = None,
                stream=None):
    nq, Hi, d = q_idx.shape
    if d != INDEX_DIM or w.shape != (nq, Hi) or n_visible.shape != (nq,) or scores.dim() != 2 or scores.shape[0] != nq:
        raise ValueError("shape mismatch in index_score arguments")
    _check("index_score", load().index_score(cache.struct, _bits16(q_idx, "q_idx"), _ptr(w, torch.float32, "w"), Hi,
                                             _ptr(seq_of_query, torch.int32, "seq_of_query"),
                                             _ptr(n_visible, torch.int32, "n_visible"),
                                             _ptr(block_table, torch.int32, "block_table"), block_table.shape[1], nq,
                                             _ptr(scores, torch.float32, "scores"), scores.shape[1],
                                             _stream(stream)))


def topk_select_workspace_size(nq: int, ld: int, k: int) -> int:
    return int(load().topk_select_workspace_size(nq, ld, k))


def topk_select(scores: torch.Tensor, n_visible: torch.Tensor, k: int, topk_idx: torch.Tensor,
                ws: torch.Tensor, stream=None):
    nq, ld = scores.shape
    if topk_idx.shape != (nq, k):
        raise ValueError("topk_idx must be [nq, k]")
    _check("topk_select", load().topk_select(_ptr(scores, torch.float32, "scores"), ld,
                                             _ptr(n_visible, torch.int32, "n_visible"), nq, k,
                                             _ptr(topk_idx, torch.int32, "topk_idx"), _ptr(ws, torch.uint8, "ws"),
                                             ws.numel(), _stream(stream)))


def index_topk(cache: Cache, q_idx: torch.Tensor, w: torch.Tensor, n_visible: torch.Tensor,
               block_table: torch.Tensor, scores: torch.Tensor, k: int, topk_idx: torch.Tensor, ws: torch.Tensor,
               seq_of_query: torch.Tensor | None = None, stream=None):
    """index_score then topk_select on the same scores, as one call (same results)."""
    nq, Hi, d = q_idx.shape
    if d != INDEX_DIM or w.shape != (nq, Hi) or n_visible.shape != (nq,) or scores.dim() != 2 or scores.shape[0] != nq:
        raise ValueError("shape mismatch in index_topk arguments")
    if topk_idx.shape != (nq, k):
        raise ValueError("topk_idx must be [nq, k]")
    _check("index_topk", load().index_topk(cache.struct, _bits16(q_idx, "q_idx"), _ptr(w, torch.float32, "w"), Hi,
                                           _ptr(seq_of_query, torch.int32, "seq_of_query"),
                                           _ptr(n_visible, torch.int32, "n_visible"),
                                           _ptr(block_table, torch.int32, "block_table"), block_table.shape[1], nq,
                                           _ptr(scores, torch.float32, "scores"), scores.shape[1], k,
                                           _ptr(topk_idx, torch.int32, "topk_idx"), _ptr(ws, torch.uint8, "ws"),
                                           ws.numel(), _stream(stream)))


def index_score_counted(cache: Cache, q_idx: torch.Tensor, w: torch.Tensor, n_visible: torch.Tensor,
                        block_table: torch.Tensor, scores: torch.Tensor, k: int, ws: torch.Tensor,
                        seq_of_query: torch.Tensor | None = None, stream=None):
    """index_score that also leaves the selection's first-digit counts in ws (the first
    half of index_topk)."""
    nq, Hi, d = q_idx.shape
    if d != INDEX_DIM or w.shape != (nq, Hi) or n_visible.shape != (nq,) or scores.dim() != 2 or scores.shape[0] != nq:
        raise ValueError("shape mismatch in index_score_counted arguments")
    _check("index_score_counted",
           load().index_score_counted(cache.struct, _bits16(q_idx, "q_idx"), _ptr(w, torch.float32, "w"), Hi,
                                      _ptr(seq_of_query, torch.int32, "seq_of_query"),
                                      _ptr(n_visible, torch.int32, "n_visible"),
                                      _ptr(block_table, torch.int32, "block_table"), block_table.shape[1], nq,
                                      _ptr(scores, torch.float32, "scores"), scores.shape[1], k,
                                      _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)))


def topk_select_counted(scores: torch.Tensor, n_visible: torch.Tensor, k: int, topk_idx: torch.Tensor,
                        ws: torch.Tensor, stream=None):
    """topk_select taking its first-digit counts from ws (the second half of index_topk)."""
    nq, ld = scores.shape
    if n_visible.shape != (nq,) or topk_idx.shape != (nq, k):
        raise ValueError("shape mismatch in topk_select_counted arguments")
    _check("topk_select_counted",
           load().topk_select_counted(_ptr(scores, torch.float32, "scores"), ld, _ptr(n_visible, torch.int32, "n_visible"),
                                      nq, k, _ptr(topk_idx, torch.int32, "topk_idx"), _ptr(ws, torch.uint8, "ws"),
                                      ws.numel(), _stream(stream)))


NOALLOC_SCRATCH_BYTES = 32 << 20  # CSA2_NOALLOC_SCRATCH_BYTES


def index_topk_noalloc(cache: Cache, q_idx: torch.Tensor, w: torch.Tensor, n_visible: torch.Tensor,
                       block_table: torch.Tensor, scores: torch.Tensor, k: int, topk_idx: torch.Tensor,
                       seq_of_query: torch.Tensor | None = None, stream=None):
    """index_topk with its workspace in the library's static per-device array (the call
    allocates nothing); sizes past the array raise with CSA2_ERR_WORKSPACE."""
    nq, Hi, d = q_idx.shape
    if d != INDEX_DIM or w.shape != (nq, Hi) or n_visible.shape != (nq,) or scores.dim() != 2 or scores.shape[0] != nq:
        raise ValueError("shape mismatch in index_topk_noalloc arguments")
    if topk_idx.shape != (nq, k):
        raise ValueError("topk_idx must be [nq, k]")
    _check("index_topk_noalloc",
           load().index_topk_noalloc(cache.struct, _bits16(q_idx, "q_idx"), _ptr(w, torch.float32, "w"), Hi,
                                     _ptr(seq_of_query, torch.int32, "seq_of_query"),
                                     _ptr(n_visible, torch.int32, "n_visible"),
                                     _ptr(block_table, torch.int32, "block_table"), block_table.shape[1], nq,
                                     _ptr(scores, torch.float32, "scores"), scores.shape[1], k,
                                     _ptr(topk_idx, torch.int32, "topk_idx"), _stream(stream)))


POOL_BLOCK = 8  # entries per candidate-pool block


def index_pool_build_workspace_size(nq: int, ld: int, npool: int) -> int:
    return int(load().index_pool_build_workspace_size(nq, ld, npool))


def index_pool_build(scores: torch.Tensor, n_visible: torch.Tensor, npool: int, pool: torch.Tensor,
                     ws: torch.Tensor, stream=None):
    """The candidate pool of each query from a gatekeeper layer's scores: the npool
    blocks of 8 entries with the largest member score, ascending, -1 padded."""
    nq, ld = scores.shape
    if pool.shape != (nq, npool) or n_visible.shape != (nq,):
        raise ValueError("pool must be [nq, npool] and n_visible [nq]")
    _check("index_pool_build", load().index_pool_build(_ptr(scores, torch.float32, "scores"), ld,
                                                       _ptr(n_visible, torch.int32, "n_visible"), nq, npool,
                                                       _ptr(pool, torch.int32, "pool"), _ptr(ws, torch.uint8, "ws"),
                                                       ws.numel(), _stream(stream)))


def index_topk_pool_build_workspace_size(nq: int, ld: int, k: int, npool: int) -> int:
    return int(load().index_topk_pool_build_workspace_size(nq, ld, k, npool))


def index_topk_pool_build(cache: Cache, q_idx: torch.Tensor, w: torch.Tensor, n_visible: torch.Tensor,
                          block_table: torch.Tensor, scores: torch.Tensor, k: int, topk_idx: torch.Tensor, npool: int,
                          pool: torch.Tensor, ws: torch.Tensor, seq_of_query: torch.Tensor | None = None, stream=None):
    """index_topk then index_pool_build on the same scores, as one call (same results)."""
    nq, Hi, d = q_idx.shape
    if d != INDEX_DIM or w.shape != (nq, Hi) or n_visible.shape != (nq,) or scores.dim() != 2 or scores.shape[0] != nq:
        raise ValueError("shape mismatch in index_topk_pool_build arguments")
    if topk_idx.shape != (nq, k) or pool.shape != (nq, npool):
        raise ValueError("topk_idx must be [nq, k] and pool [nq, npool]")
    _check("index_topk_pool_build",
           load().index_topk_pool_build(cache.struct, _bits16(q_idx, "q_idx"), _ptr(w, torch.float32, "w"), Hi,
                                        _ptr(seq_of_query, torch.int32, "seq_of_query"),
                                        _ptr(n_visible, torch.int32, "n_visible"),
                                        _ptr(block_table, torch.int32, "block_table"), block_table.shape[1], nq,
                                        _ptr(scores, torch.float32, "scores"), scores.shape[1], k,
                                        _ptr(topk_idx, torch.int32, "topk_idx"), npool,
                                        _ptr(pool, torch.int32, "pool"), _ptr(ws, torch.uint8, "ws"), ws.numel(),
                                        _stream(stream)))


def index_topk_pool_workspace_size(nq: int, npool: int, k: int) -> int:
    return int(load().index_topk_pool_workspace_size(nq, npool, k))


def index_topk_pool(cache: Cache, q_idx: torch.Tensor, w: torch.Tensor, n_visible: torch.Tensor, pool: torch.Tensor,
                    block_table: torch.Tensor, scores_pool: torch.Tensor, k: int, topk_idx: torch.Tensor,
                    ws: torch.Tensor, seq_of_query: torch.Tensor | None = None, stream=None):
    """index_topk restricted to each query's candidate pool; topk_idx holds entries."""
    nq, Hi, d = q_idx.shape
    npool = pool.shape[1]
    if d != INDEX_DIM or w.shape != (nq, Hi) or n_visible.shape != (nq,) or pool.shape[0] != nq \
            or scores_pool.shape != (nq, npool * POOL_BLOCK):
        raise ValueError("shape mismatch in index_topk_pool arguments")
    if topk_idx.shape != (nq, k):
        raise ValueError("topk_idx must be [nq, k]")
    _check("index_topk_pool", load().index_topk_pool(
        cache.struct, _bits16(q_idx, "q_idx"), _ptr(w, torch.float32, "w"), Hi,
        _ptr(seq_of_query, torch.int32, "seq_of_query"), _ptr(n_visible, torch.int32, "n_visible"),
        _ptr(pool, torch.int32, "pool"), npool, _ptr(block_table, torch.int32, "block_table"), block_table.shape[1],
        nq, _ptr(scores_pool, torch.float32, "scores_pool"), k, _ptr(topk_idx, torch.int32, "topk_idx"),
        _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)))


def sparse_attn_decode_workspace_size(B: int, H: int, k: int, window: int) -> int:
    return int(load().sparse_attn_decode_workspace_size(B, H, k, window))


def sparse_attn_decode(cache: Cache, q: torch.Tensor, topk_idx: torch.Tensor, block_table: torch.Tensor,
                       swa: torch.Tensor, swa_len: torch.Tensor, softmax_scale: float, out: torch.Tensor,
                       lse: torch.Tensor, ws: torch.Tensor, stream=None):
    B, H, d = q.shape
    k = topk_idx.shape[1]
    window = swa.shape[1]
    if d != LATENT_DIM or topk_idx.shape[0] != B or swa.shape != (B, window, LATENT_DIM) or out.shape != (B, H, d) \
            or lse.shape != (B, H) or swa_len.shape != (B,):
        raise ValueError("shape mismatch in sparse_attn_decode arguments")
    _check("sparse_attn_decode", load().sparse_attn_decode(
        cache.struct, _bits16(q, "q"), H, _ptr(topk_idx, torch.int32, "topk_idx"), k,
        _ptr(block_table, torch.int32, "block_table"), block_table.shape[1], _bits16(swa, "swa"),
        _ptr(swa_len, torch.int32, "swa_len"), window, float(softmax_scale), B, _ptr(out, torch.float32, "out"),
        _ptr(lse, torch.float32, "lse"), _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)))


def sparse_attn_prefill_chunk_workspace_size(T: int, H: int, k: int, window: int) -> int:
    return int(load().sparse_attn_prefill_chunk_workspace_size(T, H, k, window))


def sparse_attn_prefill_chunk(cache: Cache, q: torch.Tensor, topk_idx: torch.Tensor, block_table: torch.Tensor,
                              chunk_start: int, swa: torch.Tensor, swa_first_valid: int, window: int,
                              softmax_scale: float, out: torch.Tensor, lse: torch.Tensor, ws: torch.Tensor,
                              stream=None):
    T, H, d = q.shape
    k = topk_idx.shape[1]
    if d != LATENT_DIM or topk_idx.shape[0] != T or swa.shape != (window - 1 + T, LATENT_DIM) \
            or out.shape != (T, H, d) or lse.shape != (T, H) or block_table.dim() != 1:
        raise ValueError("shape mismatch in sparse_attn_prefill_chunk arguments")
    _check("sparse_attn_prefill_chunk", load().sparse_attn_prefill_chunk(
        cache.struct, _bits16(q, "q"), H, _ptr(topk_idx, torch.int32, "topk_idx"), k,
        _ptr(block_table, torch.int32, "block_table"), block_table.shape[0], int(chunk_start), T,
        _bits16(swa, "swa"), int(swa_first_valid), int(window), float(softmax_scale),
        _ptr(out, torch.float32, "out"), _ptr(lse, torch.float32, "lse"), _ptr(ws, torch.uint8, "ws"),
        ws.numel(), _stream(stream)))


def swa_fp8_write(rows: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, stream=None):
    """Window rows [..., 512] bf16 -> FP8 codes [..., 512] uint8 and one E8M0 scale per
    row [...] uint8."""
    if rows.shape[-1] != LATENT_DIM or codes.shape != rows.shape or scales.shape != rows.shape[:-1]:
        raise ValueError("shape mismatch in swa_fp8_write arguments")
    n = rows.numel() // LATENT_DIM
    _check("swa_fp8_write", load().swa_fp8_write(_bits16(rows, "rows"), n, _ptr(codes, torch.uint8, "codes"),
                                                 _ptr(scales, torch.uint8, "scales"), _stream(stream)))


def sparse_attn_decode_fp8win(cache: Cache, q: torch.Tensor, topk_idx: torch.Tensor, block_table: torch.Tensor,
                              swa_codes: torch.Tensor, swa_scales: torch.Tensor, swa_len: torch.Tensor,
                              softmax_scale: float, out: torch.Tensor, lse: torch.Tensor, ws: torch.Tensor,
                              stream=None):
    B, H, d = q.shape
    k = topk_idx.shape[1]
    window = swa_codes.shape[1]
    if d != LATENT_DIM or topk_idx.shape[0] != B or swa_codes.shape != (B, window, LATENT_DIM) \
            or swa_scales.shape != (B, window) or out.shape != (B, H, d) or lse.shape != (B, H) \
            or swa_len.shape != (B,):
        raise ValueError("shape mismatch in sparse_attn_decode_fp8win arguments")
    _check("sparse_attn_decode_fp8win", load().sparse_attn_decode_fp8win(
        cache.struct, _bits16(q, "q"), H, _ptr(topk_idx, torch.int32, "topk_idx"), k,
        _ptr(block_table, torch.int32, "block_table"), block_table.shape[1], _ptr(swa_codes, torch.uint8, "swa_codes"),
        _ptr(swa_scales, torch.uint8, "swa_scales"), _ptr(swa_len, torch.int32, "swa_len"), window,
        float(softmax_scale), B, _ptr(out, torch.float32, "out"), _ptr(lse, torch.float32, "lse"),
        _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)))


def sparse_attn_prefill_chunk_fp8win(cache: Cache, q: torch.Tensor, topk_idx: torch.Tensor,
                                     block_table: torch.Tensor, chunk_start: int, swa_codes: torch.Tensor,
                                     swa_scales: torch.Tensor, swa_first_valid: int, window: int,
                                     softmax_scale: float, out: torch.Tensor, lse: torch.Tensor, ws: torch.Tensor,
                                     stream=None):
    T, H, d = q.shape
    k = topk_idx.shape[1]
    if d != LATENT_DIM or topk_idx.shape[0] != T or swa_codes.shape != (window - 1 + T, LATENT_DIM) \
            or swa_scales.shape != (window - 1 + T,) or out.shape != (T, H, d) or lse.shape != (T, H) \
            or block_table.dim() != 1:
        raise ValueError("shape mismatch in sparse_attn_prefill_chunk_fp8win arguments")
    _check("sparse_attn_prefill_chunk_fp8win", load().sparse_attn_prefill_chunk_fp8win(
        cache.struct, _bits16(q, "q"), H, _ptr(topk_idx, torch.int32, "topk_idx"), k,
        _ptr(block_table, torch.int32, "block_table"), block_table.shape[0], int(chunk_start), T,
        _ptr(swa_codes, torch.uint8, "swa_codes"), _ptr(swa_scales, torch.uint8, "swa_scales"),
        int(swa_first_valid), int(window), float(softmax_scale), _ptr(out, torch.float32, "out"),
        _ptr(lse, torch.float32, "lse"), _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)))


def exact_path_count() -> int:
    """Index scores recomputed on the exact integer path since the last reset (current
    device; synchronous)."""
    n = ctypes.c_ulonglong(0)
    _check("csa2_exact_path_count", load().csa2_exact_path_count(ctypes.byref(n)))
    return int(n.value)


def exact_path_reset() -> None:
    _check("csa2_exact_path_reset", load().csa2_exact_path_reset())


def default_softmax_scale() -> float:
    return 1.0 / math.sqrt(LATENT_DIM)
