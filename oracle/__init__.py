"""CPU oracle for the CSA2 FP4-cache hot path -- TEST INFRASTRUCTURE.

A plain, slow, obviously-correct model written from the pages describing
DeepSeek-V4.1-Flash ("DeepSeek-V4.1-Flash, expliqué pas à pas": CSA2 and FP4 KV
cache sections; "Résumé exécutif": CSA2 mode table and FP4 formats).  The
arithmetic lives in ``oracle.c``; this module only marshals numpy arrays.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  It shares no code with the GPU library.

Functions whose parity is not pinned by a value printed on the pages (they are
pinned by invariants, special cases and brute force in the tests instead):
the NV16/MX32 rounding rules, the index-score formula, the softmax scale, and the
candidate-pool rule (block ranking by the largest member score: the pages give the
pool's size and shape, 2048 blocks of 8, but not the rule).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None

LATENT_DIM = 512
INDEX_DIM = 128
PAGE_SIZE = 64

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64


def build() -> str:
    """Compile liboracle.so with gcc (see Makefile); returns its path."""
    subprocess.run(["make", "-s", "-C", _HERE], check=True)
    return _SO


def lib():
    global _lib
    if _lib is None:
        # CSA2_ORACLE_LIB names another build of oracle.c (the mutation tests load
        # copies with planted mistakes to show that the pins catch them)
        path = os.environ.get("CSA2_ORACLE_LIB")
        if path is None:
            path = _SO
            src = os.path.join(_HERE, "oracle.c")
            if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(src):
                build()
        L = ctypes.CDLL(path)
        for name in ("oracle_bf16_value", "oracle_e2m1_value", "oracle_e4m3_value", "oracle_e8m0_value"):
            getattr(L, name).restype = ctypes.c_double
        L.oracle_bf16_value.argtypes = [ctypes.c_uint16]
        L.oracle_e2m1_value.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        L.oracle_e8m0_value.argtypes = [ctypes.c_uint8]
        L.oracle_quant_nv16.argtypes = [_P, _I64, _P, _P]
        L.oracle_quant_mx32.argtypes = [_P, _I64, _P, _P]
        L.oracle_fp4_cache_write.argtypes = [_P, _P, _P, _P, _I64, _P, _P, _P, _I64]
        L.oracle_fp4_cache_write.restype = ctypes.c_int
        L.oracle_index_score.argtypes = [_P, _P, _P, _P, _I32, _P, _P, _P, _I32, _I32, _I32, _P, _I64, _P]
        L.oracle_index_score.restype = _I64
        L.oracle_topk_select.argtypes = [_P, _I64, _P, _I32, _I32, _P]
        L.oracle_pool_build.argtypes = [_P, _I64, _P, _I32, _I32, _P]
        L.oracle_index_score_pool.argtypes = [_P, _P, _P, _P, _I32, _P, _P, _P, _I32, _P, _I32, _I32, _I32, _P,
                                              _P]
        L.oracle_index_score_pool.restype = _I64
        L.oracle_topk_pool.argtypes = [_P, _P, _I32, _P, _I32, _I32, _P]
        L.oracle_sparse_attn_decode.argtypes = [_P, _P, _P, _I32, _P, _I32, _P, _I32, _I32, _P, _P, _I32,
                                                ctypes.c_float, _I32, _P, _P]
        L.oracle_sparse_attn_prefill_chunk.argtypes = [_P, _P, _P, _I32, _P, _I32, _P, _I32, _I32, _I32, _P,
                                                       _I32, _I32, ctypes.c_float, _P, _I32, _P, _P]
        L.oracle_swa_fp8_quant.argtypes = [_P, _I64, _P, _P]
        L.oracle_swa_fp8_dequant.argtypes = [_P, _P, _I64, _P]
        L.oracle_swa_fp8_dequant.restype = _I64
        L.oracle_entry_bytes.argtypes = [_I64, _I64]
        L.oracle_entry_bytes.restype = _I64
        L.oracle_bits_per_channel.argtypes = [_I64]
        L.oracle_bits_per_channel.restype = ctypes.c_double
        L.oracle_global_bytes_per_token.argtypes = [_P, _P, _I32]
        L.oracle_global_bytes_per_token.restype = ctypes.c_double
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_set_num_threads.argtypes = [_I32]
        L.oracle_causal_n_visible.argtypes = [_P, _I64, _I32, _P]
        _lib = L
    return _lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _arr(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=dtype))


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the oracle's parallel loops from now on (n <= 0: the OpenMP default)."""
    lib().oracle_set_num_threads(int(n))


# ---------------------------------------------------------------- formats --
def bf16_value(b: int) -> float:
    return lib().oracle_bf16_value(int(b))


def e2m1_value(code: int) -> float:
    return lib().oracle_e2m1_value(int(code))


def e4m3_value(b: int) -> float:
    return lib().oracle_e4m3_value(int(b))


def e8m0_value(u: int) -> float:
    return lib().oracle_e8m0_value(int(u))


def quant_nv16(x_bf16: np.ndarray):
    """Blocks of 16 bf16 (uint16 bits, last dim 16) -> (codes uint8 [..,16], scale bytes [..])."""
    x = _arr(x_bf16, np.uint16)
    nblk = x.size // 16
    codes = np.zeros(x.shape, np.uint8)
    scales = np.zeros(x.shape[:-1], np.uint8)
    lib().oracle_quant_nv16(_ptr(x), nblk, _ptr(codes), _ptr(scales))
    return codes, scales


def quant_mx32(x_bf16: np.ndarray):
    """Blocks of 32 bf16 (uint16 bits, last dim 32) -> (codes uint8 [..,32], E8M0 bytes [..])."""
    x = _arr(x_bf16, np.uint16)
    nblk = x.size // 32
    codes = np.zeros(x.shape, np.uint8)
    scales = np.zeros(x.shape[:-1], np.uint8)
    lib().oracle_quant_mx32(_ptr(x), nblk, _ptr(codes), _ptr(scales))
    return codes, scales


# ------------------------------------------------------- causal visibility --
def causal_n_visible(tokens, m: int) -> np.ndarray:
    """Entries visible to a query at each token position: entry j (tokens m*j ..
    m*j+m-1) is visible once its last token is at or before the query's."""
    tok = _arr(tokens, np.int64).reshape(-1)
    out = np.zeros(tok.shape[0], np.int32)
    lib().oracle_causal_n_visible(_ptr(tok), tok.shape[0], int(m), _ptr(out))
    return out


def decode_n_visible(ctx, m: int) -> np.ndarray:
    """A decode query is the last token of its context (token ctx - 1)."""
    return causal_n_visible(np.asarray(ctx, np.int64) - 1, m)


def prefill_n_visible(prefix_tokens: int, T: int, m: int) -> np.ndarray:
    """Query i of a chunk after `prefix_tokens` tokens sits at token prefix_tokens + i."""
    return causal_n_visible(int(prefix_tokens) + np.arange(T, dtype=np.int64), m)


# ------------------------------------------------------------------ cache --
class Cache:
    """Host copy of one global FP4 cache: per slot 256 + 32 + 64 + 4 bytes."""

    def __init__(self, num_slots: int):
        self.num_slots = int(num_slots)
        self.main_codes = np.zeros((num_slots, 256), np.uint8)
        self.main_scales = np.zeros((num_slots, 32), np.uint8)
        self.idx_codes = np.zeros((num_slots, 64), np.uint8)
        self.idx_scales = np.zeros((num_slots, 4), np.uint8)


def fp4_cache_write(cache: Cache, latent: np.ndarray, idx_key: np.ndarray, slot: np.ndarray) -> None:
    latent = _arr(latent, np.uint16)
    idx_key = _arr(idx_key, np.uint16)
    slot = _arr(slot, np.int64)
    n = slot.shape[0]
    assert latent.shape == (n, LATENT_DIM) and idx_key.shape == (n, INDEX_DIM)
    rc = lib().oracle_fp4_cache_write(_ptr(cache.main_codes), _ptr(cache.main_scales), _ptr(cache.idx_codes),
                                      _ptr(cache.idx_scales), cache.num_slots, _ptr(latent), _ptr(idx_key),
                                      _ptr(slot), n)
    if rc != 0:
        raise ValueError("slot out of range")


def index_score(cache: Cache, q_idx: np.ndarray, w: np.ndarray, n_visible: np.ndarray, block_table: np.ndarray,
                seq_of_query: np.ndarray | None = None, ld: int | None = None, page_size: int = PAGE_SIZE):
    """Returns (scores float32 [nq, ld] (unwritten positions are NaN), count of dots
    not representable in fp32, count of dots not exact in double)."""
    q_idx = _arr(q_idx, np.uint16)
    nq, Hi, d = q_idx.shape
    assert d == INDEX_DIM
    w = _arr(w, np.float32).reshape(nq, Hi)
    n_visible = _arr(n_visible, np.int32)
    block_table = _arr(block_table, np.int32)
    if ld is None:
        ld = int(n_visible.max()) if nq else 0
    scores = np.full((nq, max(ld, 1)), np.nan, np.float32)
    soq = None if seq_of_query is None else _arr(seq_of_query, np.int32)
    inexact = ctypes.c_int64(0)
    bad = lib().oracle_index_score(_ptr(cache.idx_codes), _ptr(cache.idx_scales), _ptr(q_idx), _ptr(w), Hi,
                                   _ptr(soq), _ptr(n_visible), _ptr(block_table), block_table.shape[1], page_size,
                                   nq, _ptr(scores), scores.shape[1], ctypes.byref(inexact))
    return scores[:, :ld], int(bad), int(inexact.value)


def topk_select(scores: np.ndarray, n_visible: np.ndarray, k: int) -> np.ndarray:
    scores = _arr(scores, np.float32)
    nq = scores.shape[0]
    n_visible = _arr(n_visible, np.int32)
    out = np.zeros((nq, k), np.int32)
    lib().oracle_topk_select(_ptr(scores), scores.shape[1], _ptr(n_visible), nq, k, _ptr(out))
    return out


POOL_BLOCK = 8


def pool_build(scores: np.ndarray, n_visible: np.ndarray, npool: int) -> np.ndarray:
    """Hierarchical candidate pool from a gatekeeper layer's scores: the npool blocks
    of 8 entries with the largest member score (ties to the lower block), ascending,
    -1 padded.  int32 [nq, npool]."""
    scores = _arr(scores, np.float32)
    nq, ld = scores.shape
    n_visible = _arr(n_visible, np.int32)
    pool = np.zeros((nq, npool), np.int32)
    lib().oracle_pool_build(_ptr(scores), ld, _ptr(n_visible), nq, npool, _ptr(pool))
    return pool


def index_score_pool(cache: Cache, q_idx: np.ndarray, w: np.ndarray, n_visible: np.ndarray, pool: np.ndarray,
                     block_table: np.ndarray, seq_of_query: np.ndarray | None = None, page_size: int = PAGE_SIZE):
    """Scores of the pool's members at pool positions 8r + i (NaN where a position holds
    no visible entry).  Returns (scores float32 [nq, 8 npool], dots not representable
    in fp32, dots not exact in double)."""
    q_idx = _arr(q_idx, np.uint16)
    nq, Hi, d = q_idx.shape
    assert d == INDEX_DIM
    w = _arr(w, np.float32).reshape(nq, Hi)
    n_visible = _arr(n_visible, np.int32)
    pool = _arr(pool, np.int32)
    npool = pool.shape[1]
    block_table = _arr(block_table, np.int32)
    scores = np.full((nq, npool * POOL_BLOCK), np.nan, np.float32)
    soq = None if seq_of_query is None else _arr(seq_of_query, np.int32)
    inexact = ctypes.c_int64(0)
    bad = lib().oracle_index_score_pool(_ptr(cache.idx_codes), _ptr(cache.idx_scales), _ptr(q_idx), _ptr(w), Hi,
                                        _ptr(soq), _ptr(n_visible), _ptr(pool), npool, _ptr(block_table),
                                        block_table.shape[1], page_size, nq, _ptr(scores), ctypes.byref(inexact))
    return scores, int(bad), int(inexact.value)


def topk_pool(scores_pool: np.ndarray, pool: np.ndarray, n_visible: np.ndarray, k: int) -> np.ndarray:
    """The k best visible pool members (entry indices, ascending, -1 padded)."""
    scores_pool = _arr(scores_pool, np.float32)
    pool = _arr(pool, np.int32)
    nq, npool = pool.shape
    assert scores_pool.shape == (nq, npool * POOL_BLOCK)
    n_visible = _arr(n_visible, np.int32)
    out = np.zeros((nq, k), np.int32)
    lib().oracle_topk_pool(_ptr(scores_pool), _ptr(pool), npool, _ptr(n_visible), nq, k, _ptr(out))
    return out


def sparse_attn_decode(cache: Cache, q: np.ndarray, topk_idx: np.ndarray, block_table: np.ndarray,
                       swa: np.ndarray, swa_len: np.ndarray, softmax_scale: float, page_size: int = PAGE_SIZE):
    q = _arr(q, np.uint16)
    B, H, d = q.shape
    assert d == LATENT_DIM
    topk_idx = _arr(topk_idx, np.int32)
    k = topk_idx.shape[1]
    block_table = _arr(block_table, np.int32)
    swa = _arr(swa, np.uint16)
    window = swa.shape[1]
    swa_len = _arr(swa_len, np.int32)
    out = np.zeros((B, H, LATENT_DIM), np.float32)
    lse = np.zeros((B, H), np.float32)
    lib().oracle_sparse_attn_decode(_ptr(cache.main_codes), _ptr(cache.main_scales), _ptr(q), H, _ptr(topk_idx),
                                    k, _ptr(block_table), block_table.shape[1], page_size, _ptr(swa),
                                    _ptr(swa_len), window, float(softmax_scale), B, _ptr(out), _ptr(lse))
    return out, lse


def sparse_attn_prefill_chunk(cache: Cache, q: np.ndarray, topk_idx: np.ndarray, block_table: np.ndarray,
                              swa: np.ndarray, swa_first_valid: int, window: int, softmax_scale: float,
                              which: np.ndarray | None = None, page_size: int = PAGE_SIZE):
    """Outputs for the queries in `which` (default: all); other rows are left zero."""
    q = _arr(q, np.uint16)
    T, H, d = q.shape
    topk_idx = _arr(topk_idx, np.int32)
    k = topk_idx.shape[1]
    block_table = _arr(block_table, np.int32).reshape(1, -1)
    swa = _arr(swa, np.uint16)
    assert swa.shape == (window - 1 + T, LATENT_DIM)
    out = np.zeros((T, H, LATENT_DIM), np.float32)
    lse = np.zeros((T, H), np.float32)
    wh = None if which is None else _arr(which, np.int32)
    lib().oracle_sparse_attn_prefill_chunk(_ptr(cache.main_codes), _ptr(cache.main_scales), _ptr(q), H,
                                           _ptr(topk_idx), k, _ptr(block_table), block_table.shape[1], page_size,
                                           T, _ptr(swa), int(swa_first_valid), int(window),
                                           float(softmax_scale), _ptr(wh), 0 if wh is None else wh.shape[0],
                                           _ptr(out), _ptr(lse))
    return out, lse


# -------------------------------------------------------------- footprint --
def swa_fp8_quant(x_bf16: np.ndarray):
    """Window rows [..., 512] bf16 bits -> (E4M3FN codes [..., 512], E8M0 scales [...])."""
    x = _arr(x_bf16, np.uint16)
    assert x.shape[-1] == LATENT_DIM
    rows = x.size // LATENT_DIM
    codes = np.zeros(x.shape, np.uint8)
    scales = np.zeros(x.shape[:-1], np.uint8)
    lib().oracle_swa_fp8_quant(_ptr(x), rows, _ptr(codes), _ptr(scales))
    return codes, scales


def swa_fp8_dequant(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """FP8 window rows -> bf16 bits of their exact values (raises if bf16 cannot hold
    one exactly)."""
    codes = _arr(codes, np.uint8)
    scales = _arr(scales, np.uint8)
    assert codes.shape[-1] == LATENT_DIM and codes.shape[:-1] == scales.shape
    out = np.zeros(codes.shape, np.uint16)
    bad = lib().oracle_swa_fp8_dequant(_ptr(codes), _ptr(scales), scales.size, _ptr(out))
    if bad:
        raise ValueError(f"{bad} FP8 window values are not exact in bf16")
    return out


def sparse_attn_decode_fp8win(cache: Cache, q: np.ndarray, topk_idx: np.ndarray, block_table: np.ndarray,
                              swa_codes: np.ndarray, swa_scales: np.ndarray, swa_len: np.ndarray,
                              softmax_scale: float):
    """Decode attention with an FP8 window: the window rows' exact values, then the
    same attention as sparse_attn_decode."""
    return sparse_attn_decode(cache, q, topk_idx, block_table, swa_fp8_dequant(swa_codes, swa_scales), swa_len,
                              softmax_scale)


def sparse_attn_prefill_chunk_fp8win(cache: Cache, q: np.ndarray, topk_idx: np.ndarray, block_table: np.ndarray,
                                     swa_codes: np.ndarray, swa_scales: np.ndarray, swa_first_valid: int,
                                     window: int, softmax_scale: float, which: np.ndarray | None = None):
    return sparse_attn_prefill_chunk(cache, q, topk_idx, block_table, swa_fp8_dequant(swa_codes, swa_scales),
                                     swa_first_valid, window, softmax_scale, which=which)


def entry_bytes(dim: int, block: int) -> int:
    return int(lib().oracle_entry_bytes(dim, block))


def bits_per_channel(block: int) -> float:
    return float(lib().oracle_bits_per_channel(block))


MODE_CODE = {"swa": 0, "full": 1, "reindex": 2, "reuse": 3}


def global_bytes_per_token(modes, ms) -> float:
    mode = _arr([MODE_CODE[m] for m in modes], np.int32)
    m = _arr(ms, np.int32)
    return float(lib().oracle_global_bytes_per_token(_ptr(mode), _ptr(m), len(modes)))
