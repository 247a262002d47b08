"""Seeded random shapes through the indexer stage and the attention, against the oracle.

Each case draws a batch of sequences of random lengths on randomly permuted pages, a
random number of index and attention heads, a top-k size, a window length and head
weights of either sign, then runs the scores and the selection through one of the
library's routes (index_topk, the counted pair, index_score then topk_select), a
candidate pool when the rows allow one (index_topk_pool_build, then index_topk_pool
on it), and sparse_attn_decode over the selected entries.  Scores, pools and indices
must be bit-exact; attention within the usual tolerance.  The cases reach the
selection's launch forms (chunks and one finishing workgroup, the split form, one
workgroup per short row, the paired launch) at shapes the targeted tests do not use.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_fp4_cache_amd import lib
from _helpers import attn_close, bits, dev, dev_bits, same_bits_f32, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    lib.load()


def _draw(seed):
    rng = np.random.default_rng(7100 + seed)
    B = int(rng.integers(1, 10))
    lengths = rng.integers(1, 40_000, B).astype(np.int64)
    if seed == 0:  # rows at and around the top-k size and the chunk size
        lengths = np.array([256, 255, 257, 4096, 4097, 1], np.int64)
        B = len(lengths)
    if seed == 1:  # enough rows that the gatekeeper's paired selection takes its split form
        B = 30
        lengths = rng.integers(30_000, 40_000, B).astype(np.int64)
    Hi = int(rng.choice([16, 32, 48, 64, 128]))
    H = int(rng.choice([16, 64]))
    k = int(rng.choice([1, 17, 256, 2048, 4096])) if seed > 1 else 256
    W = int(rng.choice([1, 5, 128]))
    return rng, B, lengths, Hi, H, k, W


def _run(seed):
    rng, B, lengths, Hi, H, k, W = _draw(seed)
    route = ("index_topk", "counted", "separate")[seed % 3]
    say(f"case {seed}: B={B} lengths {int(lengths.min())}..{int(lengths.max())} Hi={Hi} H={H} k={k} W={W} "
        f"route={route}")
    pages = [(int(n) + 63) // 64 for n in lengths]
    phys = rng.permutation(sum(pages)).astype(np.int32)
    bt = np.zeros((B, max(pages)), np.int32)
    off, slots = 0, []
    for b, n in enumerate(lengths):
        bt[b, :pages[b]] = phys[off:off + pages[b]]
        off += pages[b]
        j = np.arange(int(n))
        slots.append(bt[b, j // 64].astype(np.int64) * 64 + j % 64)
    slots = np.concatenate(slots)
    total = int(lengths.sum())
    lat = bits(rng.standard_normal((total, 512), dtype=np.float32))
    key = bits(rng.standard_normal((total, 128), dtype=np.float32))
    num_slots = sum(pages) * 64
    g = lib.Cache(num_slots)
    lib.fp4_cache_write(g, dev_bits(lat), dev_bits(key), dev(slots))
    o = oracle.Cache(num_slots)
    oracle.fp4_cache_write(o, lat, key, slots)

    nv = lengths.astype(np.int32)
    ld = ((int(nv.max()) + 63) // 64) * 64
    q_idx = bits(rng.standard_normal((B, Hi, 128)).astype(np.float32))
    w = (rng.standard_normal((B, Hi)) if seed % 2 else rng.random((B, Hi))).astype(np.float32)
    dq, dw, dnv, dbt = dev_bits(q_idx), dev(w), dev(nv), dev(bt)
    scores = torch.full((B, ld), float("nan"), device="cuda")
    topk = torch.full((B, k), -7, dtype=torch.int32, device="cuda")
    ws = torch.zeros(lib.topk_select_workspace_size(B, ld, k), dtype=torch.uint8, device="cuda")
    if route == "index_topk":
        lib.index_topk(g, dq, dw, dnv, dbt, scores, k, topk, ws)
    elif route == "counted":
        lib.index_score_counted(g, dq, dw, dnv, dbt, scores, k, ws)
        lib.topk_select_counted(scores, dnv, k, topk, ws)
    else:
        lib.index_score(g, dq, dw, dnv, dbt, scores)
        lib.topk_select(scores, dnv, k, topk, ws)
    torch.cuda.synchronize()
    ref_s, _, _ = oracle.index_score(o, q_idx, w, nv, bt, ld=ld)
    ref_k = oracle.topk_select(ref_s, nv, k)
    got_s = scores.cpu().numpy()
    for b in range(B):
        assert same_bits_f32(got_s[b, :nv[b]], ref_s[b, :nv[b]]), f"case {seed} row {b}: scores differ"
    assert np.array_equal(topk.cpu().numpy(), ref_k), f"case {seed}: top-k differs"

    # a candidate pool from these scores, then a second query's top-k inside it
    if int(nv.max()) > 8 * 64 and k <= 2048:
        npool = int(rng.choice([64, 512, 2048]))
        pool = torch.full((B, npool), -7, dtype=torch.int32, device="cuda")
        s2 = torch.full((B, ld), float("nan"), device="cuda")
        t2 = torch.full((B, k), -7, dtype=torch.int32, device="cuda")
        ws_g = torch.zeros(lib.index_topk_pool_build_workspace_size(B, ld, k, npool), dtype=torch.uint8,
                           device="cuda")
        lib.index_topk_pool_build(g, dq, dw, dnv, dbt, s2, k, t2, npool, pool, ws_g)
        torch.cuda.synchronize()
        ref_pool = oracle.pool_build(ref_s, nv, npool)
        assert np.array_equal(pool.cpu().numpy(), ref_pool), f"case {seed}: pool differs"
        assert torch.equal(t2, topk), f"case {seed}: gatekeeper top-k differs"
        q2 = bits(rng.standard_normal((B, Hi, 128)).astype(np.float32))
        sp = torch.full((B, 8 * npool), float("nan"), device="cuda")
        tp = torch.full((B, k), -7, dtype=torch.int32, device="cuda")
        ws_p = torch.zeros(lib.index_topk_pool_workspace_size(B, npool, k), dtype=torch.uint8, device="cuda")
        lib.index_topk_pool(g, dev_bits(q2), dw, dnv, pool, dbt, sp, k, tp, ws_p)
        torch.cuda.synchronize()
        ref_sp, _, _ = oracle.index_score_pool(o, q2, w, nv, ref_pool, bt)
        ref_tp = oracle.topk_pool(ref_sp, ref_pool, nv, k)
        got_sp = sp.cpu().numpy()
        filled = ~np.isnan(ref_sp)
        assert same_bits_f32(got_sp[filled], ref_sp[filled]), f"case {seed}: pooled scores differ"
        assert np.array_equal(tp.cpu().numpy(), ref_tp), f"case {seed}: pooled top-k differs"

    q = bits(rng.standard_normal((B, H, 512)).astype(np.float32))
    swa = bits(rng.standard_normal((B, W, 512)).astype(np.float32))
    swa_len = rng.integers(0, W + 1, B).astype(np.int32)
    scale = 1 / math.sqrt(512)
    out = torch.zeros((B, H, 512), device="cuda")
    lse = torch.zeros((B, H), device="cuda")
    ws_a = torch.zeros(max(256, lib.sparse_attn_decode_workspace_size(B, H, k, W)), dtype=torch.uint8,
                       device="cuda")
    lib.sparse_attn_decode(g, dev_bits(q), topk, dbt, dev_bits(swa), dev(swa_len), scale, out, lse, ws_a)
    ro, rl = oracle.sparse_attn_decode(o, q, ref_k, bt, swa, swa_len, scale)
    attn_close(out.cpu().numpy(), ro, lse.cpu().numpy(), rl, f"case {seed} attention")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("seed", range(10))
def test_random_shapes_against_oracle(seed):
    _run(seed)
