"""The index score is the exact dot rounded once, on every scan variant, at the edge
of the window where the FP4 matrix unit is used.

A block of 32 products is an integer S_b (|S_b| <= 4608, in units of 2^E_b).  Keys
and queries are built here so that three blocks are saturated (every element 6 X)
and one block holds a single odd product, with the block exponents spread by
s = 0 .. 12: the exact dot 1 + 3 * 4608 * 2^s (quarter units) needs every one of
fp32's 24 bits at s = 10 and is not representable in fp32 for s >= 11.  Entries
with s <= 10 must come from the matrix unit (the library's exact-path counter stays
unchanged) and equal the oracle bit for bit; entries with s >= 11 must take the
exact path (counted) and equal the oracle's single rounding.  One-hot head weights
make each score the dot of one head, so no fma chain can hide a low bit.
("DeepSeek-V4.1-Flash, expliqué pas à pas", FP4 KV cache section: indexer queries
and keys are MXFP4.)
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_attention_fp4_cache_amd import lib
from _helpers import bits, dev, dev_bits, say

pytestmark = pytest.mark.gpu

N_ENTRIES = 256
MAX_SPAN = 10  # the window the library documents (every partial sum exact in fp32)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    lib.load()


def _block(kind, e, rng):
    """32 values of one MX32 block with scale X = 2^e: 'sat' = all 6X (the largest
    block sum, 4608 quarter units); 'lowq' / 'lowk' = the max 6X at position 0 / 1
    (so X = 2^e, and the query's max meets the key's 0) and 0.5X at position 2 (one
    odd product, a block sum of 1 quarter unit)."""
    v = np.zeros(32, np.float64)
    if kind == "sat":
        v[:] = 6.0
    elif kind == "lowq":
        v[0], v[2] = 6.0, 0.5
    else:  # lowk: the max sits where the query's block is 0
        v[1], v[2] = 6.0, 0.5
    return v * 2.0 ** e


def _entries(rng):
    """Key rows and the span (of the four block exponent sums) each one produces with
    the query patterns below."""
    keys, spans, low_pos = [], [], []
    for s in range(13):
        for p in range(4):  # position of the low block
            for split in sorted({0, s // 2, s}):  # how the span divides between q and k
                k_e = s - split  # key's high blocks sit 2^(s - split) above its low block
                row = np.concatenate([_block("lowk" if b == p else "sat", k_e if b != p else 0, rng)
                                      for b in range(4)])
                keys.append(row)
                spans.append(s)
                low_pos.append((p, split))
    keys = np.array(keys)
    n = len(keys)
    assert n <= N_ENTRIES
    pad = np.tile(keys[-1], (N_ENTRIES - n, 1))
    return np.concatenate([keys, pad]), np.array(spans + [spans[-1]] * (N_ENTRIES - n)), \
        low_pos + [low_pos[-1]] * (N_ENTRIES - n)


def _query_heads(Hi, split, p):
    """Every head: query blocks with exponent `split` on the three high blocks and 0 on
    block p, so q's exponent span is `split` for every head."""
    q = np.concatenate([_block("lowq" if b == p else "sat", split if b != p else 0, None) for b in range(4)])
    return np.tile(q, (Hi, 1))


def _run_case(Hi, p, split, call, label, nq):
    rng = np.random.default_rng(7)
    keys, spans, low_pos = _entries(rng)
    # only the entries built for this (low position, split) follow the exponent
    # arithmetic below; the others are scored and compared too
    key_bits = bits(keys.astype(np.float32))
    lat = bits(np.zeros((N_ENTRIES, 512), np.float32))
    g = lib.Cache(N_ENTRIES)
    lib.fp4_cache_write(g, dev_bits(lat), dev_bits(key_bits), dev(np.arange(N_ENTRIES, dtype=np.int64)))
    o = oracle.Cache(N_ENTRIES)
    oracle.fp4_cache_write(o, lat, key_bits, np.arange(N_ENTRIES, dtype=np.int64))
    q1 = bits(_query_heads(Hi, split, p).astype(np.float32))
    q = np.repeat(q1[None], nq, axis=0)  # query i reads head i % Hi only (one-hot weights)
    w = np.tile(np.eye(Hi, dtype=np.float32), (nq // Hi, 1))
    nvis = np.full(nq, N_ENTRIES, np.int32)
    torch.cuda.synchronize()
    lib.exact_path_reset()
    got = call(g, q, w, nvis)
    torch.cuda.synchronize()
    counted = lib.exact_path_count()
    ref, not_fp32, _ = oracle.index_score(o, q, w, nvis, np.zeros((nq, 4), np.int32) + np.arange(4, dtype=np.int32),
                                          ld=N_ENTRIES)
    bad = np.argwhere(got.view(np.int32) != ref.view(np.int32))
    assert len(bad) == 0, (f"{label}: {len(bad)} scores differ, first (query, entry) {bad[0].tolist()}: "
                           f"{got[tuple(bad[0])]!r} vs {ref[tuple(bad[0])]!r}")
    # the exactness test the kernels apply: key span + the query's largest head span
    qk = _mx_exponents(q1)  # [Hi, 4]
    kk = _mx_exponents(key_bits)  # [N, 4]
    q_span = int((qk.max(1) - qk.min(1)).max())
    k_span = kk.max(1) - kk.min(1)
    want_exact = int(np.count_nonzero(k_span + q_span > MAX_SPAN)) * nq
    say(f"  {label}: {N_ENTRIES * nq} scores bit-exact; exact path {counted} (expected {want_exact}); "
        f"dots not representable in fp32 per the oracle: {not_fp32}")
    assert counted == want_exact, f"{label}: exact path taken {counted} times, expected {want_exact}"
    # the worst cases really are at the edge: s = 10 needs 24 bits, s >= 11 more
    return not_fp32


def _mx_exponents(b):
    c, u = oracle.quant_mx32(np.ascontiguousarray(b).reshape(b.shape[0], 4, 32))
    return u.astype(np.int64)


def _score_call(Hi, shared, topk=False):
    def call(g, q, w, nvis):
        nq = q.shape[0]
        scores = torch.full((nq, N_ENTRIES), float("nan"), device="cuda")
        soq = dev(np.zeros(nq, np.int32)) if shared else None
        bt = dev(np.arange(4, dtype=np.int32)[None, :].repeat(1 if shared else nq, 0))
        if topk:
            k = 16
            ws = torch.zeros(lib.topk_select_workspace_size(nq, N_ENTRIES, k), dtype=torch.uint8, device="cuda")
            idx = torch.empty((nq, k), dtype=torch.int32, device="cuda")
            lib.index_topk(g, dev_bits(q), dev(w), dev(nvis), bt, scores, k, idx, ws, seq_of_query=soq)
        else:
            lib.index_score(g, dev_bits(q), dev(w), dev(nvis), bt, scores, seq_of_query=soq)
        return scores.cpu().numpy()
    return call


# (Hi, queries share one sequence, through index_topk): each row reaches one variant
VARIANTS = [
    (16, False, False),   # one query per workgroup, 16x16x128 MFMA
    (48, False, False),   # one query per workgroup, 16x16x128, three M-tiles
    (64, False, False),   # one query per workgroup, two chained 32x32x64 MFMAs
    (64, False, True),    # the same inside index_topk (digit-1 histogram counted)
    (16, True, False),    # two queries per wavefront (prefill form), one M-tile
    (64, True, False),    # two queries per wavefront, four M-tiles
    (96, True, False),    # four queries per workgroup sharing pages
    (128, True, False),   # 128 heads of queries that share a sequence
]


@pytest.mark.parametrize("Hi,shared,topk", VARIANTS, ids=[f"Hi{v[0]}{'-shared' if v[1] else ''}"
                                                           f"{'-topk' if v[2] else ''}" for v in VARIANTS])
def test_mfma_window_worst_case_mantissas(Hi, shared, topk):
    say(f"case: exactness window, Hi={Hi}, shared={shared}, index_topk={topk}")
    seen_unrepresentable = 0
    for p in (0, 1, 3):
        for split in (0, 1):
            # queries that share a sequence take the tiled variants from 64 queries on
            nq = max(Hi, 64) if shared else Hi
            seen_unrepresentable += _run_case(Hi, p, split, _score_call(Hi, shared, topk),
                                              f"low block {p}, q span {split}", nq)
    assert seen_unrepresentable > 0  # the cases past the window do need a rounding


def test_many_single_query_workgroups_against_oracle():
    """More single-query workgroups than compute units: the standalone scan then runs
    its counting kernel with the counts switched off (160 queries x 8192 entries at 64
    heads is 640 workgroups)."""
    rng = np.random.default_rng(31)
    n, nq, Hi = 8192, 160, 64
    lat = bits(np.zeros((n, 512), np.float32))
    key = bits(rng.standard_normal((n, 128)).astype(np.float32))
    g = lib.Cache(n)
    lib.fp4_cache_write(g, dev_bits(lat), dev_bits(key), dev(np.arange(n, dtype=np.int64)))
    o = oracle.Cache(n)
    oracle.fp4_cache_write(o, lat, key, np.arange(n, dtype=np.int64))
    q = bits(rng.standard_normal((nq, Hi, 128)).astype(np.float32))
    w = rng.random((nq, Hi), dtype=np.float32)
    nvis = rng.integers(1, n + 1, nq).astype(np.int32)
    nvis[:4] = [n, 1, 64, 8191]
    bt = np.tile(np.arange(n // 64, dtype=np.int32), (nq, 1))
    scores = torch.full((nq, n), float("nan"), device="cuda")
    say(f"case: index_score {nq} single-query rows over {n} entries, Hi={Hi}")
    lib.index_score(g, dev_bits(q), dev(w), dev(nvis), dev(bt), scores)
    got = scores.cpu().numpy()
    ref, not_fp32, _ = oracle.index_score(o, q, w, nvis, bt, ld=n)
    assert not_fp32 == 0
    for r in range(nq):
        m = int(nvis[r])
        assert np.array_equal(got[r, :m].view(np.int32), ref[r, :m].view(np.int32)), f"row {r}"
        assert np.all(np.isnan(got[r, m:])), f"row {r}: wrote past n_visible"


def test_index_score_128_heads_causal_queries_of_one_sequence():
    """64 causal queries of one sequence at 128 index heads (four staged queries would
    not fit in 64 KB of LDS, so each workgroup stages one)."""
    rng = np.random.default_rng(32)
    n, nq, Hi = 3000, 64, 128
    pages = (n + 63) // 64
    lat = bits(np.zeros((n, 512), np.float32))
    key = bits(rng.standard_normal((n, 128)).astype(np.float32))
    phys = rng.permutation(pages).astype(np.int32)
    slots = phys[np.arange(n) // 64].astype(np.int64) * 64 + np.arange(n) % 64
    g = lib.Cache(pages * 64)
    lib.fp4_cache_write(g, dev_bits(lat), dev_bits(key), dev(slots))
    o = oracle.Cache(pages * 64)
    oracle.fp4_cache_write(o, lat, key, slots)
    q = bits(rng.standard_normal((nq, Hi, 128)).astype(np.float32))
    w = rng.random((nq, Hi), dtype=np.float32)
    nvis = oracle.prefill_n_visible(2 * n - 2 * nq, nq, 2)
    bt = phys[None, :]
    ld = pages * 64
    scores = torch.full((nq, ld), float("nan"), device="cuda")
    soq = np.zeros(nq, np.int32)
    say(f"case: index_score {nq} causal queries of one sequence, Hi={Hi}")
    lib.index_score(g, dev_bits(q), dev(w), dev(nvis), dev(bt), scores, seq_of_query=dev(soq))
    got = scores.cpu().numpy()
    ref, not_fp32, _ = oracle.index_score(o, q, w, nvis, bt, seq_of_query=soq, ld=ld)
    assert not_fp32 == 0
    for r in range(nq):
        m = int(nvis[r])
        assert np.array_equal(got[r, :m].view(np.int32), ref[r, :m].view(np.int32)), f"row {r}"


def _exhaustive_query_heads():
    """Query heads (4 MX32 blocks of 32) in which every finite bf16 pattern appears as
    an element: a block whose largest exponent field is F holds 2^(F-127) at element 0
    (so its shared exponent is F - 2), up to 30 patterns with exponent fields F-5 .. F
    at elements 1..30 (every E2M1 region and midpoint relative to the block scale), and
    0 at element 31.  The four blocks of a head share F."""
    heads, fields_of_head = [], []
    for F in range(1, 255):
        pats = [(s << 15) | (f << 7) | m for f in range(max(0, F - 5), F + 1) for m in range(128) for s in (0, 1)]
        blocks = []
        for i in range(0, len(pats), 30):
            chunk = pats[i:i + 30]
            chunk += [0] * (30 - len(chunk))
            blocks.append([F << 7] + chunk + [0])
        while len(blocks) % 4:
            blocks.append(blocks[0])
        for i in range(0, len(blocks), 4):
            heads.append(np.array(blocks[i:i + 4], np.uint16).reshape(128))
            fields_of_head.append(F)
    return np.stack(heads), np.array(fields_of_head)


@pytest.mark.parametrize("shared", [False, True], ids=["one-query-per-workgroup", "queries-sharing-a-sequence"])
def test_query_quantisation_every_bf16_pattern(shared):
    """Every finite bf16 pattern through the MXFP4 query quantisation (on the hardware
    convert where the block exponent allows it), read back exactly: keys are +-1 at one
    channel c of block b and 1.0 at channel 31 of the other blocks (where every query is
    0), so every key block has the same scale and, with one-hot head weights, the score
    is ReLU(+-qhat[h][32b + c]).  The dequantised values come from the oracle's MX32
    quantisation of the same blocks."""
    Hi = 16
    heads, fields = _exhaustive_query_heads()
    ngroups = (len(heads) + Hi - 1) // Hi
    pad = ngroups * Hi - len(heads)
    heads = np.concatenate([heads, np.repeat(heads[:1], pad, axis=0)])
    fields = np.concatenate([fields, np.repeat(fields[:1], pad)])
    allpat = set(int(x) for x in heads.reshape(-1))
    finite = [p for p in range(65536) if ((p >> 7) & 0xFF) != 0xFF]
    assert set(finite) <= allpat  # every finite pattern is an element somewhere
    q_groups = heads.reshape(ngroups, Hi, 128)
    q = np.repeat(q_groups, Hi, axis=0)  # query g*Hi + h reads head h of group g
    w = np.tile(np.eye(Hi, dtype=np.float32), (ngroups, 1))
    nq = q.shape[0]
    keys = []
    for b in range(4):
        for c in range(31):
            for s in (1.0, -1.0):
                k = np.zeros(128, np.float32)
                k[[32 * bb + 31 for bb in range(4) if bb != b]] = 1.0
                k[32 * b + c] = s
                k[32 * b + 31] = 1.0
                keys.append(k)
    n = 256
    keys = np.array(keys + [keys[0]] * (n - len(keys)), np.float32)
    g = lib.Cache(n)
    lib.fp4_cache_write(g, dev_bits(np.zeros((n, 512), np.uint16)), dev_bits(bits(keys)),
                        dev(np.arange(n, dtype=np.int64)))
    nvis = np.full(nq, n, np.int32)
    scores = torch.full((nq, n), float("nan"), device="cuda")
    soq = dev(np.zeros(nq, np.int32)) if shared else None
    bt = dev(np.arange(4, dtype=np.int32)[None, :].repeat(1 if shared else nq, 0))
    say(f"case: every finite bf16 pattern in {len(heads)} query heads ({nq} queries), shared={shared}")
    torch.cuda.synchronize()
    lib.exact_path_reset()
    lib.index_score(g, dev_bits(q), dev(w), dev(nvis), bt, scores, seq_of_query=soq)
    torch.cuda.synchronize()
    counted = lib.exact_path_count()
    got = scores.cpu().numpy()
    # the oracle's dequantised query values
    codes, u = oracle.quant_mx32(q_groups.reshape(-1, 32))
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)
    deq = (np.where(codes & 8, -1.0, 1.0) * mags[codes & 7] * np.exp2(u.astype(np.float64) - 127)[:, None])
    deq = deq.reshape(ngroups, Hi, 128)
    want = np.zeros((nq, n), np.float32)
    kinfo = [(b, c, s) for b in range(4) for c in range(31) for s in (1.0, -1.0)]
    kinfo += [kinfo[0]] * (n - len(kinfo))
    cols_ch = np.array([32 * b + c for b, c, _ in kinfo])
    cols_s = np.array([s for _, _, s in kinfo])
    for qi in range(nq):
        gq, h = divmod(qi, Hi)
        v = cols_s * deq[gq, h, cols_ch]
        want[qi] = np.maximum(v, 0.0).astype(np.float32)
    bad = np.argwhere(got.view(np.int32) != want.view(np.int32))
    assert len(bad) == 0, (f"{len(bad)} differ, first (query, key) {bad[0].tolist()}: {got[tuple(bad[0])]!r} vs "
                           f"{want[tuple(bad[0])]!r}")
    # entries on the MFMA path: key blocks all at u = 125, every head's blocks share u,
    # so a query takes the matrix unit unless its exponent sums leave fp32's range
    uq = u.reshape(ngroups, Hi, 4).astype(np.int64)
    lo = uq.min(axis=(1, 2)) + 125
    hi = uq.max(axis=(1, 2)) + 125
    exact_queries = int(np.count_nonzero((lo < 130) | (hi > 360))) * Hi
    say(f"  all {nq * n} scores equal the oracle's quantisation; exact path {counted} "
        f"(expected {exact_queries * n}), MFMA path for {nq - exact_queries} queries")
    assert counted == exact_queries * n
    assert nq - exact_queries > 2900
