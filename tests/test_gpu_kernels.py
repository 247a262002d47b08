"""Per-kernel GPU parity against the CPU oracle on small and adversarial inputs.
Packing, scores and indices must be bit-exact; attention within 2e-3 absolute and
1e-2 of the largest reference magnitude.  Every case feeds the same host arrays to
both sides; the oracle never sees a GPU result."""
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


def both_caches(lat, key, slots, num_slots):
    g = lib.Cache(num_slots)
    lib.fp4_cache_write(g, dev_bits(lat), dev_bits(key), dev(slots))
    o = oracle.Cache(num_slots)
    oracle.fp4_cache_write(o, lat, key, slots)
    torch.cuda.synchronize()
    return g, o


def assert_cache_equal(g, o, label, lat=None, key=None, slots=None):
    msgs = []
    for name in ("main_scales", "idx_scales", "main_codes", "idx_codes"):
        a = getattr(g, name).cpu().numpy()
        b = getattr(o, name)
        bad = np.argwhere(a != b)
        if len(bad):
            msgs.append(f"{name} differs in {len(bad)} bytes")
            if lat is not None:
                inv = {int(s): i for i, s in enumerate(slots)}
                for sl, byte in bad[:6]:
                    r = inv.get(int(sl))
                    if name.startswith("main"):
                        ch = slice(16 * byte, 16 * byte + 16) if name == "main_scales" else slice(2 * byte, 2 * byte + 2)
                        blk = slice(16 * (ch.start // 16), 16 * (ch.start // 16) + 16)
                        src = lat
                    else:
                        ch = slice(32 * byte, 32 * byte + 32) if name == "idx_scales" else slice(2 * byte, 2 * byte + 2)
                        blk = slice(32 * (ch.start // 32), 32 * (ch.start // 32) + 32)
                        src = key
                    vals = ((src[r, ch].astype(np.uint32) << 16).view(np.float32)) if r is not None else None
                    amax = float(np.abs((src[r, blk].astype(np.uint32) << 16).view(np.float32)).max()) if r is not None else None
                    msgs.append(f"  slot {sl} byte {byte}: gpu {a[sl, byte]:#04x} oracle {b[sl, byte]:#04x} "
                                f"vals {vals} block amax {amax}")
    assert not msgs, label + ": " + "; ".join(msgs)


def adversarial_rows(rng, n):
    x = rng.standard_normal((n, 512)).astype(np.float32)
    k = rng.standard_normal((n, 128)).astype(np.float32)
    kinds = rng.integers(0, 10, n)
    for i in range(n):
        t = kinds[i]
        if t == 0:
            x[i] = 0.0
            k[i] = 0.0
        elif t == 1:
            x[i] = -0.0
            k[i] *= 0.0
            k[i] = -k[i]
        elif t == 2:  # exact E2M1 midpoints at scale 1
            mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, -0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5.0,
                             -6.0], np.float32)
            x[i] = np.tile(mids, 32)
            k[i] = np.tile(mids, 8)
        elif t == 3:  # saturating
            x[i] *= 3000.0
            k[i] *= 1e30
        elif t == 4:  # E4M3-subnormal scales and tiny values
            x[i] *= 6 * 2.0 ** -9 * rng.integers(1, 9)
            k[i] *= 1e-39
        elif t == 5:  # per-block magnitudes spread wide
            x[i] *= np.repeat(np.exp2(rng.integers(-20, 12, 32)), 16).astype(np.float32)
            k[i] *= np.repeat(np.exp2(rng.integers(-60, 60, 4)), 32).astype(np.float32)
        elif t == 6:  # channel outliers
            x[i, rng.integers(0, 512, 5)] *= 8.0
            k[i, rng.integers(0, 128, 1)] *= 8.0
    return bits(x), bits(k)


def test_cache_write_random_and_adversarial():
    rng = np.random.default_rng(100)
    n = 3000
    lat, key = adversarial_rows(rng, n)
    num_slots = 64 * 64
    slots = rng.permutation(num_slots)[:n].astype(np.int64)  # scattered, unique
    say(f"case: cache_write adversarial n={n}")
    g, o = both_caches(lat, key, slots, num_slots)
    assert_cache_equal(g, o, "adversarial", lat, key, slots)


def test_cache_write_exhaustive_block_maxima():
    # every finite bf16 value as the largest magnitude of an NV16 block and an MX32 block
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = (allb.astype(np.uint32) << 16).view(np.float32)
    vals = f[np.isfinite(f)]
    rng = np.random.default_rng(101)
    n = 2048
    lat = np.zeros((n, 512), np.float32)
    key = np.zeros((n, 128), np.float32)
    nv_blocks = lat.reshape(n * 32, 16)
    mx_blocks = key.reshape(n * 4, 32)
    for blocks in (nv_blocks, mx_blocks):
        m = blocks.shape[0]
        v = np.resize(vals, m)
        blocks[:] = (np.abs(v)[:, None] * rng.uniform(-1, 1, blocks.shape)).astype(np.float32)
        blocks[:, 0] = v
    say(f"case: cache_write exhaustive block maxima ({vals.size} values)")
    lb, kb = bits(lat), bits(key)
    g, o = both_caches(lb, kb, np.arange(n, dtype=np.int64), n)
    assert_cache_equal(g, o, "exhaustive", lb, kb, np.arange(n))


def _index_case(rng, n_per_seq, Hi, nq_per_seq=1, paged=False, key_fn=None, q_fn=None, causal=False, soq=None):
    B = len(n_per_seq)
    pages = [(n + 63) // 64 for n in n_per_seq]
    total_pages = sum(pages)
    phys = rng.permutation(total_pages) if paged else np.arange(total_pages)
    max_pages = max(pages)
    bt = np.zeros((B, max_pages), np.int32)
    off = 0
    slots_all, lat_all, key_all = [], [], []
    for b, n in enumerate(n_per_seq):
        bt[b, :pages[b]] = phys[off:off + pages[b]]
        off += pages[b]
        j = np.arange(n)
        slots_all.append(bt[b, j // 64].astype(np.int64) * 64 + j % 64)
        x = rng.standard_normal((n, 512)).astype(np.float32)
        k = rng.standard_normal((n, 128)).astype(np.float32)
        if key_fn is not None:
            k = key_fn(k)
        lat_all.append(bits(x))
        key_all.append(bits(k))
    num_slots = total_pages * 64
    g, o = both_caches(np.concatenate(lat_all), np.concatenate(key_all), np.concatenate(slots_all), num_slots)
    nq = B * nq_per_seq if soq is None else len(soq)
    q = rng.standard_normal((nq, Hi, 128)).astype(np.float32)
    if q_fn is not None:
        q = q_fn(q)
    q = bits(q)
    w = rng.random((nq, Hi), dtype=np.float32)
    soq = np.repeat(np.arange(B, dtype=np.int32), nq_per_seq) if soq is None else np.asarray(soq, np.int32)
    nvis = np.array([n_per_seq[s] for s in soq], np.int32)
    if causal:  # query i of a sequence sees 3 entries more than the one before it
        rank = np.zeros(nq, np.int64)
        for b in range(B):
            idx = np.nonzero(soq == b)[0]
            rank[idx] = len(idx) - 1 - np.arange(len(idx))
        nvis = np.maximum(1, nvis - 3 * rank).astype(np.int32)
    ld = ((max(n_per_seq) + 63) // 64) * 64
    scores = torch.full((nq, ld), float("nan"), device="cuda")
    lib.index_score(g, dev_bits(q), dev(w), dev(nvis), dev(bt), scores, seq_of_query=dev(soq))
    ref, bad, inexact = oracle.index_score(o, q, w, nvis, bt, seq_of_query=soq, ld=ld)
    got = scores.cpu().numpy()
    for i in range(nq):
        n = nvis[i]
        assert same_bits_f32(got[i, :n], ref[i, :n]), f"query {i}: {int((got[i, :n] != ref[i, :n]).sum())} differ"
        assert np.all(np.isnan(got[i, n:])), "positions beyond n_visible were written"
    return bad


@pytest.mark.parametrize("Hi", [16, 64])
def test_index_score_ragged_tail(Hi):
    say(f"case: index_score ragged Hi={Hi}")
    _index_case(np.random.default_rng(200 + Hi), [1000, 77], Hi)


def test_index_score_paged_three_sequences():
    say("case: index_score paged 3 seqs Hi=32")
    _index_case(np.random.default_rng(210), [300, 1500, 64], 32, paged=True)


def test_index_score_query_tile_shared_row():
    say("case: index_score 70 causal queries on one sequence Hi=64")
    _index_case(np.random.default_rng(220), [2000], 64, nq_per_seq=70, causal=True)


@pytest.mark.parametrize("Hi", [16, 32, 48, 64])
def test_index_score_shared_sequence_tiles(Hi):
    # queries sharing a sequence: 32 per workgroup, one page range each; 1098 entries
    # are 18 pages, so the last range of 8 pages holds only two
    say(f"case: index_score 100 causal queries on one sequence Hi={Hi}, paged")
    _index_case(np.random.default_rng(260 + Hi), [1098], Hi, nq_per_seq=100, causal=True, paged=True)


def test_index_score_shared_sequence_mixed_rows():
    # workgroups whose 32 queries read two, three or (interleaved) every sequence:
    # one pass over the pages per distinct sequence
    rng = np.random.default_rng(270)
    say("case: index_score 3 sequences x 40 queries in order (workgroups straddle sequences)")
    _index_case(rng, [700, 1300, 129], 64, nq_per_seq=40, causal=True, paged=True)
    say("case: index_score 90 queries interleaved over 3 sequences")
    _index_case(rng, [900, 65, 1500], 32, soq=[i % 3 for i in range(90)], causal=True, paged=True)


def test_index_score_shared_sequence_exact_path():
    def keys(k):
        k[:, 0:32] *= 2.0 ** -12
        k[:, 64:96] *= 2.0 ** 6
        k[200:230] *= 2.0 ** -70  # with the small queries below: dots under 2^-126
        return k

    def qs(q):
        q[:, :, 32:64] *= 2.0 ** 5
        q[1, 3, :] = 0.0  # an all-zero head
        q[7, 5, 96:] = 0.0  # a head with one zero block
        q[40:44] *= 2.0 ** -70
        q[44:48] *= 2.0 ** 104  # exponent sums above the window
        return q

    for Hi in (16, 64):
        say(f"case: index_score shared-sequence tiles, exact path, Hi={Hi}")
        bad = _index_case(np.random.default_rng(280 + Hi), [600], Hi, nq_per_seq=70, key_fn=keys, q_fn=qs)
        say(f"  dots not representable in fp32: {bad}")


def test_index_score_heads_128():
    say("case: index_score Hi=128")
    _index_case(np.random.default_rng(230), [700], 128)


def test_index_score_exact_path_wide_spread():
    # block magnitudes far apart push the exponent span past the MFMA-exact range
    def keys(k):
        k[:, 0:32] *= 2.0 ** -12
        k[:, 64:96] *= 2.0 ** 6
        return k

    def qs(q):
        q[:, :, 32:64] *= 2.0 ** 5
        q[0, 3, :] = 0.0  # an all-zero head
        q[0, 5, 96:] = 0.0  # a head with one zero block
        return q

    say("case: index_score exact path (wide exponent spread, zero blocks)")
    bad = _index_case(np.random.default_rng(240), [500], 16, key_fn=keys, q_fn=qs)
    say(f"  dots not representable in fp32: {bad}")


def test_index_score_tiny_values():
    def keys(k):
        return k * 2.0 ** -70

    def qs(q):
        return q * 2.0 ** -70

    say("case: index_score tiny values (fp32-subnormal dots)")
    _index_case(np.random.default_rng(250), [300], 16, key_fn=keys, q_fn=qs)


# ------------------------------------------------------------------- top-K --
def _topk_case(scores, nvis, k, label, runs=2):
    nq, ld = scores.shape
    ws = torch.zeros(lib.topk_select_workspace_size(nq, ld, k), dtype=torch.uint8, device="cuda")
    ds = dev(scores)
    dn = dev(nvis)
    ref = oracle.topk_select(scores, nvis, k)
    for r in range(runs):  # the second run checks the workspace was left clean
        out = torch.full((nq, k), -7, dtype=torch.int32, device="cuda")
        lib.topk_select(ds, dn, k, out, ws)
        got = out.cpu().numpy()
        for q in range(nq):
            assert np.array_equal(got[q], ref[q]), f"{label} run {r} query {q}"
    say(f"  {label}: ok")


def test_topk_ties_and_padding():
    rng = np.random.default_rng(300)
    nq, ld = 6, 50_000
    s = rng.integers(0, 3000, (nq, ld)).astype(np.float32)  # many ties
    s[1] = rng.standard_normal(ld).astype(np.float32)
    s[2] = -np.abs(rng.standard_normal(ld)).astype(np.float32)  # all negative
    s[3, ::2] = 0.0
    s[3, 1::2] = -0.0  # +0 and -0 compare equal
    nvis = np.array([50_000, 49_999, 33_333, 40_000, 2048, 100], np.int32)
    say("case: top-k ties / negatives / zeros / n_visible <= k")
    _topk_case(s, nvis, 2048, "k=2048")
    _topk_case(s, nvis, 1, "k=1")
    _topk_case(s, nvis, 256, "k=256")


def test_topk_all_equal_overflows_candidate_list():
    s = np.full((2, 30_000), 1.5, np.float32)
    s[1, 7] = 2.0
    nvis = np.array([30_000, 29_000], np.int32)
    say("case: top-k all-equal scores (candidate overflow path)")
    _topk_case(s, nvis, 2048, "all-equal")


def test_topk_empty_and_short_rows():
    s = np.random.default_rng(310).standard_normal((3, 64)).astype(np.float32)
    nvis = np.array([0, 1, 64], np.int32)
    say("case: top-k empty and short rows")
    _topk_case(s, nvis, 100, "short")


@pytest.mark.timeout(600)
def test_topk_many_rows_one_workgroup_per_row():
    """At least 128 rows take the one-workgroup-per-row kernel: ragged rows, ties,
    rows with n_visible <= k, an all-equal row (its per-wavefront lists overflow and it
    takes the slow path) and rows where the selected entries cluster in one segment."""
    rng = np.random.default_rng(330)
    nq, ld = 136, 40_000
    s = rng.standard_normal((nq, ld)).astype(np.float32)
    nvis = rng.integers(1, ld + 1, nq).astype(np.int32)
    nvis[:4] = [ld, 2048, 100, 0]
    s[4] = rng.integers(0, 500, ld).astype(np.float32)   # many ties
    s[5] = 1.25                                           # all equal: overflow path
    s[6, :5000] += 50.0                                   # winners packed into the first segment
    s[7, -3000:] += 50.0                                  # ... into the last
    nvis[4:8] = ld
    say("case: top-k 136 rows (one workgroup per row)")
    _topk_case(s, nvis, 2048, "rows k=2048")
    _topk_case(s, nvis, 300, "rows k=300")


def test_topk_many_long_rows_one_workgroup_per_row():
    """260 rows of 70,000 scores (enough rows for one workgroup per row, rows longer
    than a workgroup's lists): rows whose best entries come first, last or in a few
    huge values, all-equal, tied and short rows."""
    rng = np.random.default_rng(332)
    nq, ld = 260, 70_000
    s = rng.standard_normal((nq, ld)).astype(np.float32)
    nvis = rng.integers(60_000, ld + 1, nq).astype(np.int32)
    nvis[:3] = [2048, 100, 0]
    s[3, -5000:] += 50.0                    # the best entries last
    s[4, :1100] = 1000.0 + rng.standard_normal(1100).astype(np.float32) * 1e-3  # a few huge values first
    s[5] = 2.5                              # all equal
    s[6] = rng.integers(0, 300, ld).astype(np.float32)  # many ties
    s[7, :8192] += 50.0                     # the first 8192 far above the rest
    nvis[3:8] = ld
    say("case: top-k 260 rows of 70,000 (one workgroup per row)")
    _topk_case(s, nvis, 2048, "long rows k=2048")
    _topk_case(s, nvis, 64, "long rows k=64")


def test_topk_rows_sampled_gate_and_its_fallbacks():
    """Rows of at least 32,768 scores with k <= 2048 and no counts given take the
    sampled gate: 2048 evenly spread scores set a gate, one pass lists the entries at
    or above it, and the selection is resolved from the lists.  Every branch is
    reached, each compared with the oracle:
    * the gate holds (N(0,1) rows, all lengths from 32,768 up);
    * the samples hold the row's largest scores, so fewer than k entries pass the
      gate and the row is counted after all;
    * a score that grows (or falls) along the row packs the passing entries into one
      wavefront's segment, whose list overflows: the row is listed again from the now
      known first digit (k = 512), or that listing overflows too and the row itself
      is scanned (k = 2048);
    * all-equal, tied and all-negative rows;
    * rows just under 32,768 scores beside them, which count their digits as before."""
    rng = np.random.default_rng(333)
    nq, ld = 136, 40_000
    s = rng.standard_normal((nq, ld)).astype(np.float32)
    nvis = np.full(nq, ld, np.int32)
    nvis[:3] = [32_768, 32_767, 20_000]
    for q in (3, 4):  # the gate's sample positions hold the row's largest scores
        pos = (np.arange(2048, dtype=np.int64) * int(nvis[q])) // 2048
        s[q, pos] = 100.0 + rng.random(2048).astype(np.float32)
    ramp = np.exp2(np.arange(ld) / 1000.0).astype(np.float32)
    s[5] = ramp              # grows along the row: the best entries in the last segment
    s[6] = ramp[::-1]        # falls: the best entries in the first segment
    s[7] = 3.0               # all equal
    s[8] = rng.integers(0, 200, ld).astype(np.float32)  # many ties
    s[9] = -np.abs(s[9])     # all negative
    say("case: top-k 136 rows of up to 40,000 (sampled gate and its fallbacks)")
    for k in (2048, 512, 17):
        _topk_case(s, nvis, k, f"gated rows k={k}")


def test_topk_few_long_rows_take_chunks():
    """130 rows of 70,000 scores (too few rows to fill the chip with one workgroup
    each): the chunked path with many rows, ragged, tied and short rows included.
    Its 2,340 chunk workgroups take the split form (chunk launch, then one finishing
    workgroup per row), and the all-equal row its slow path."""
    rng = np.random.default_rng(331)
    nq, ld = 130, 70_000
    s = rng.standard_normal((nq, ld)).astype(np.float32)
    nvis = rng.integers(1, ld + 1, nq).astype(np.int32)
    nvis[:4] = [ld, 2048, 100, 0]
    s[4] = rng.integers(0, 500, ld).astype(np.float32)   # many ties
    s[5] = -0.5                                           # all equal
    nvis[4:6] = ld
    say("case: top-k 130 rows of 70,000 (chunked)")
    _topk_case(s, nvis, 2048, "long rows k=2048")


def test_topk_large_row_many_chunks():
    rng = np.random.default_rng(320)
    s = (rng.standard_normal((1, 600_000)) * 3 + 20).astype(np.float32)
    say("case: top-k 600k-entry row")
    _topk_case(s, np.array([600_000], np.int32), 2048, "600k")


def test_topk_largest_k():
    """k = 4096, the largest supported: rows longer than k, equal to it, one short of
    it and empty, with ties (chunked path and one workgroup per row)."""
    rng = np.random.default_rng(333)
    nq, ld = 6, 70_000
    s = rng.standard_normal((nq, ld)).astype(np.float32)
    s[1] = rng.integers(0, 200, ld).astype(np.float32)  # many ties around the boundary
    nvis = np.array([ld, ld, 5000, 4096, 4095, 0], np.int32)
    say("case: top-k with k = 4096 (chunked)")
    _topk_case(s, nvis, 4096, "k=4096 chunked")
    s2 = rng.standard_normal((3, 12_000)).astype(np.float32)
    say("case: top-k with k = 4096 (rows of 12,000: one workgroup per row)")
    _topk_case(s2, np.array([12_000, 4097, 4096], np.int32), 4096, "k=4096 by row")


# --------------------------------------------------------------- attention --
def _attn_cache(rng, n, outliers=False):
    x = rng.standard_normal((n, 512)).astype(np.float32)
    if outliers:
        x[:, [3, 100, 200, 333, 511]] *= 8.0
    k = rng.standard_normal((n, 128)).astype(np.float32)
    num_slots = ((n + 63) // 64) * 64
    return both_caches(bits(x), bits(k), np.arange(n, dtype=np.int64), num_slots)


@pytest.mark.parametrize("H", [16, 64])
def test_attention_decode(H):
    rng = np.random.default_rng(400 + H)
    n, B, k, W = 3000, 3, 300, 128
    g, o = _attn_cache(rng, n, outliers=(H == 64))
    bt = np.tile(np.arange((n + 63) // 64, dtype=np.int32), (B, 1))
    idx = np.stack([np.sort(rng.choice(n, k, replace=False)) for _ in range(B)]).astype(np.int32)
    idx[1, 250:] = -1
    q = bits(rng.standard_normal((B, H, 512)))
    swa_f = rng.standard_normal((B, W, 512)).astype(np.float32)
    swa = bits(swa_f)
    swa_len = np.array([128, 5, 0], np.int32)
    scale = 1 / math.sqrt(512)
    out = torch.zeros((B, H, 512), device="cuda")
    lse = torch.zeros((B, H), device="cuda")
    ws = torch.zeros(lib.sparse_attn_decode_workspace_size(B, H, k, W), dtype=torch.uint8, device="cuda")
    say(f"case: attention decode H={H}")
    lib.sparse_attn_decode(g, dev_bits(q), dev(idx), dev(bt), dev_bits(swa), dev(swa_len), scale, out, lse, ws)
    ro, rl = oracle.sparse_attn_decode(o, q, idx, bt, swa, swa_len, scale)
    attn_close(out.cpu().numpy(), ro, lse.cpu().numpy(), rl, f"decode H={H}")


def test_attention_decode_empty_and_sharp():
    rng = np.random.default_rng(410)
    n, B, H, k, W = 256, 2, 16, 64, 16
    g, o = _attn_cache(rng, n)
    bt = np.tile(np.arange(4, dtype=np.int32), (B, 1))
    idx = np.full((B, k), -1, np.int32)
    idx[1, :3] = [5, 6, 7]
    q = rng.standard_normal((B, H, 512)).astype(np.float32)
    q[1] *= 40.0  # sharp softmax, one row dominates
    q = bits(q)
    swa = bits(rng.standard_normal((B, W, 512)))
    swa_len = np.array([0, 16], np.int32)
    out = torch.full((B, H, 512), 7.0, device="cuda")
    lse = torch.zeros((B, H), device="cuda")
    ws = torch.zeros(lib.sparse_attn_decode_workspace_size(B, H, k, W), dtype=torch.uint8, device="cuda")
    say("case: attention decode empty row set and sharp softmax")
    lib.sparse_attn_decode(g, dev_bits(q), dev(idx), dev(bt), dev_bits(swa), dev(swa_len), 0.05, out, lse, ws)
    ro, rl = oracle.sparse_attn_decode(o, q, idx, bt, swa, swa_len, 0.05)
    go, gl = out.cpu().numpy(), lse.cpu().numpy()
    assert np.all(go[0] == 0.0) and np.all(np.isneginf(gl[0]))
    attn_close(go, ro, gl, rl, "empty/sharp")


def test_attention_prefill_truncated_windows():
    rng = np.random.default_rng(420)
    n, T, H, k, W = 2500, 40, 64, 200, 128
    g, o = _attn_cache(rng, n)
    bt = np.arange((n + 63) // 64, dtype=np.int32)
    idx = np.stack([np.sort(rng.choice(n, k, replace=False)) for _ in range(T)]).astype(np.int32)
    idx[5, 150:] = -1
    q = bits(rng.standard_normal((T, H, 512)))
    swa = bits(rng.standard_normal((W - 1 + T, 512)))
    first_valid = 100
    scale = 1 / math.sqrt(512)
    out = torch.zeros((T, H, 512), device="cuda")
    lse = torch.zeros((T, H), device="cuda")
    ws = torch.zeros(max(256, lib.sparse_attn_prefill_chunk_workspace_size(T, H, k, W)), dtype=torch.uint8,
                     device="cuda")
    say("case: attention prefill chunk with truncated windows")
    lib.sparse_attn_prefill_chunk(g, dev_bits(q), dev(idx), dev(bt), 5000, dev_bits(swa), first_valid, W, scale,
                                  out, lse, ws)
    ro, rl = oracle.sparse_attn_prefill_chunk(o, q, idx, bt, swa, first_valid, W, scale)
    attn_close(out.cpu().numpy(), ro, lse.cpu().numpy(), rl, "prefill")


@pytest.mark.timeout(600)
def test_attention_prefill_one_workgroup_per_query():
    """Enough queries for one row range per query: the kernel that takes 64 heads per
    workgroup (two groups of 64 here).  k = 200 leaves a tile holding both selected
    entries and window rows; -1 indices and windows cut by the first valid row."""
    rng = np.random.default_rng(430)
    n, T, H, k, W = 2500, 64, 128, 200, 128
    g, o = _attn_cache(rng, n, outliers=True)
    bt = np.arange((n + 63) // 64, dtype=np.int32)
    idx = np.stack([np.sort(rng.choice(n, k, replace=False)) for _ in range(T)]).astype(np.int32)
    idx[5, 150:] = -1
    idx[9, :] = -1
    q = bits(rng.standard_normal((T, H, 512)))
    swa = bits(rng.standard_normal((W - 1 + T, 512)))
    first_valid = 100
    scale = 1 / math.sqrt(512)
    out = torch.zeros((T, H, 512), device="cuda")
    lse = torch.zeros((T, H), device="cuda")
    ws = torch.zeros(max(256, lib.sparse_attn_prefill_chunk_workspace_size(T, H, k, W)), dtype=torch.uint8,
                     device="cuda")
    say("case: attention prefill, one workgroup per (query, 64 heads)")
    lib.sparse_attn_prefill_chunk(g, dev_bits(q), dev(idx), dev(bt), 5000, dev_bits(swa), first_valid, W, scale,
                                  out, lse, ws)
    ro, rl = oracle.sparse_attn_prefill_chunk(o, q, idx, bt, swa, first_valid, W, scale)
    attn_close(out.cpu().numpy(), ro, lse.cpu().numpy(), rl, "prefill wide")


@pytest.mark.timeout(600)
def test_attention_decode_many_sequences():
    """64 sequences x 64 heads: one row range per query, 64 heads per workgroup, ragged
    window lengths and a row with no selected entries."""
    rng = np.random.default_rng(440)
    n, B, H, k, W = 2000, 64, 64, 160, 128
    g, o = _attn_cache(rng, n)
    bt = np.tile(np.arange((n + 63) // 64, dtype=np.int32), (B, 1))
    idx = np.stack([np.sort(rng.choice(n, k, replace=False)) for _ in range(B)]).astype(np.int32)
    idx[3, :] = -1
    q = bits(rng.standard_normal((B, H, 512)))
    swa = bits(rng.standard_normal((B, W, 512)))
    swa_len = rng.integers(0, W + 1, B).astype(np.int32)
    swa_len[3] = 0
    scale = 1 / math.sqrt(512)
    out = torch.zeros((B, H, 512), device="cuda")
    lse = torch.zeros((B, H), device="cuda")
    ws = torch.zeros(lib.sparse_attn_decode_workspace_size(B, H, k, W), dtype=torch.uint8, device="cuda")
    say("case: attention decode, 64 sequences")
    lib.sparse_attn_decode(g, dev_bits(q), dev(idx), dev(bt), dev_bits(swa), dev(swa_len), scale, out, lse, ws)
    ro, rl = oracle.sparse_attn_decode(o, q, idx, bt, swa, swa_len, scale)
    attn_close(out.cpu().numpy(), ro, lse.cpu().numpy(), rl, "decode 64 sequences")


@pytest.mark.timeout(600)
def test_attention_largest_k_and_window():
    """k = 4096 selected entries plus a 128-row window (4,224 rows, the most a query
    attends to): decode (row ranges and the merge) and a prefill chunk of 64 queries
    (one workgroup per query over all 4,224 rows)."""
    rng = np.random.default_rng(450)
    n, H, k, W = 9000, 64, 4096, 128
    g, o = _attn_cache(rng, n)
    scale = 1 / math.sqrt(512)
    B = 2
    bt = np.tile(np.arange((n + 63) // 64, dtype=np.int32), (B, 1))
    idx = np.stack([np.sort(rng.choice(n, k, replace=False)) for _ in range(B)]).astype(np.int32)
    idx[1, 4000:] = -1
    q = bits(rng.standard_normal((B, H, 512)))
    swa = bits(rng.standard_normal((B, W, 512)))
    swa_len = np.array([128, 77], np.int32)
    out = torch.zeros((B, H, 512), device="cuda")
    lse = torch.zeros((B, H), device="cuda")
    ws = torch.zeros(lib.sparse_attn_decode_workspace_size(B, H, k, W), dtype=torch.uint8, device="cuda")
    say("case: attention decode, k = 4096 and a full window")
    lib.sparse_attn_decode(g, dev_bits(q), dev(idx), dev(bt), dev_bits(swa), dev(swa_len), scale, out, lse, ws)
    ro, rl = oracle.sparse_attn_decode(o, q, idx, bt, swa, swa_len, scale)
    attn_close(out.cpu().numpy(), ro, lse.cpu().numpy(), rl, "decode k=4096")
    T = 64
    bt1 = np.arange((n + 63) // 64, dtype=np.int32)
    idx = np.stack([np.sort(rng.choice(n, k, replace=False)) for _ in range(T)]).astype(np.int32)
    idx[7, 3000:] = -1
    q = bits(rng.standard_normal((T, H, 512)))
    swa = bits(rng.standard_normal((W - 1 + T, 512)))
    out = torch.zeros((T, H, 512), device="cuda")
    lse = torch.zeros((T, H), device="cuda")
    ws = torch.zeros(max(256, lib.sparse_attn_prefill_chunk_workspace_size(T, H, k, W)), dtype=torch.uint8,
                     device="cuda")
    say("case: attention prefill, k = 4096 and a full window, 64 queries")
    lib.sparse_attn_prefill_chunk(g, dev_bits(q), dev(idx), dev(bt1), 20000, dev_bits(swa), 0, W, scale, out, lse,
                                  ws)
    ro, rl = oracle.sparse_attn_prefill_chunk(o, q, idx, bt1, swa, 0, W, scale)
    attn_close(out.cpu().numpy(), ro, lse.cpu().numpy(), rl, "prefill k=4096")


def test_index_topk_largest_k():
    rng = np.random.default_rng(304)
    say("case: index_topk with k = 4096 (rows longer, equal and shorter than k)")
    _fused_vs_separate(rng, [70000, 4096, 3000, 20000], 64, 4096)


def test_index_score_reveals_query_quantisation():
    # keys +-1 at one channel each and one-hot head weights make every score equal
    # max(+-qhat[h][c], 0), so the dequantised query is compared value by value;
    # random bf16 bit patterns put block exponents across the whole range (both the
    # hardware-convert and the compare-based quantisation paths run)
    rng = np.random.default_rng(260)
    n, Hi, groups = 256, 16, 4
    key = np.zeros((n, 128), np.float32)
    for c in range(128):
        key[2 * c, c] = 1.0
        key[2 * c + 1, c] = -1.0
    lat = np.zeros((n, 512), np.float32)
    g, o = both_caches(bits(lat), bits(key), np.arange(n, dtype=np.int64), n)
    raw = rng.integers(0, 65536, (groups, Hi, 128)).astype(np.uint16)
    f = (raw.astype(np.uint32) << 16).view(np.float32)
    raw[~np.isfinite(f)] = 0x3F80
    raw[1] = bits(rng.standard_normal((Hi, 128)) * 3.0)  # a typical group as well
    q = np.repeat(raw, Hi, axis=0)  # [groups*Hi, Hi, 128]
    w = np.tile(np.eye(Hi, dtype=np.float32), (groups, 1))
    nq = groups * Hi
    nvis = np.full(nq, n, np.int32)
    bt = np.tile(np.arange(4, dtype=np.int32), (nq, 1))
    scores = torch.full((nq, n), float("nan"), device="cuda")
    say("case: index_score query quantisation revealed by one-hot keys")
    lib.index_score(g, dev_bits(q), dev(w), dev(nvis), dev(bt), scores, seq_of_query=dev(np.zeros(nq, np.int32)))
    ref, _, _ = oracle.index_score(o, q, w, nvis, bt, seq_of_query=np.zeros(nq, np.int32), ld=n)
    got = scores.cpu().numpy()
    bad = np.argwhere(got.view(np.int32) != ref.view(np.int32))
    assert len(bad) == 0, f"{len(bad)} differ, first {bad[:5].tolist()}: {got[tuple(bad[0])]} vs {ref[tuple(bad[0])]}"


def _fused_vs_separate(rng, n_per_seq, Hi, k, key_fn=None, seq_of_query=None, reps=2, counted=False):
    """index_topk (or, with counted, index_score_counted then topk_select_counted)
    against index_score followed by topk_select (bit for bit), on a paged cache;
    called `reps` times on one workspace (it must be left clean)."""
    B = len(n_per_seq)
    pages = [(n + 63) // 64 for n in n_per_seq]
    phys = rng.permutation(sum(pages))
    bt = np.zeros((B, max(pages)), np.int32)
    off, lat, key, slots = 0, [], [], []
    for b, n in enumerate(n_per_seq):
        bt[b, :pages[b]] = phys[off:off + pages[b]]
        off += pages[b]
        j = np.arange(n)
        slots.append(bt[b, j // 64].astype(np.int64) * 64 + j % 64)
        kk = rng.standard_normal((n, 128)).astype(np.float32)
        key.append(bits(key_fn(kk) if key_fn else kk))
        lat.append(bits(np.zeros((n, 512), np.float32)))
    g = lib.Cache(sum(pages) * 64)
    lib.fp4_cache_write(g, dev_bits(np.concatenate(lat)), dev_bits(np.concatenate(key)), dev(np.concatenate(slots)))
    if seq_of_query is None:
        nq, soq, nvis = B, None, np.array(n_per_seq, np.int32)
    else:
        soq = np.asarray(seq_of_query, np.int32)
        nq = len(soq)
        nvis = np.array([max(1, n_per_seq[s] - 7 * i % 50) for i, s in enumerate(soq)], np.int32)
    ld = ((int(nvis.max()) + 63) // 64) * 64
    q = bits(rng.standard_normal((nq, Hi, 128)).astype(np.float32))
    w = rng.random((nq, Hi), dtype=np.float32)
    dq, dw, dnv, dbt = dev_bits(q), dev(w), dev(nvis), dev(bt)
    dsoq = None if soq is None else dev(soq)
    ws = torch.zeros(lib.topk_select_workspace_size(nq, ld, k), dtype=torch.uint8, device="cuda")
    s_sep = torch.full((nq, ld), float("nan"), device="cuda")
    i_sep = torch.full((nq, k), -7, dtype=torch.int32, device="cuda")
    lib.index_score(g, dq, dw, dnv, dbt, s_sep, seq_of_query=dsoq)
    lib.topk_select(s_sep, dnv, k, i_sep, ws)
    for rep in range(reps):
        s_f = torch.full((nq, ld), float("nan"), device="cuda")
        i_f = torch.full((nq, k), -7, dtype=torch.int32, device="cuda")
        if counted:
            lib.index_score_counted(g, dq, dw, dnv, dbt, s_f, k, ws, seq_of_query=dsoq)
            lib.topk_select_counted(s_f, dnv, k, i_f, ws)
        else:
            lib.index_topk(g, dq, dw, dnv, dbt, s_f, k, i_f, ws, seq_of_query=dsoq)
        torch.cuda.synchronize()
        a, b = s_f.cpu().numpy(), s_sep.cpu().numpy()
        for r in range(nq):
            assert same_bits_f32(a[r, :nvis[r]], b[r, :nvis[r]]), f"rep {rep} row {r}: scores differ"
        assert torch.equal(i_f, i_sep), f"rep {rep}: top-k differs"
    # the workspace needs no clearing between calls: a separate selection after the
    # fused calls still matches
    i_again = torch.full((nq, k), -7, dtype=torch.int32, device="cuda")
    lib.topk_select(s_sep, dnv, k, i_again, ws)
    torch.cuda.synchronize()
    assert torch.equal(i_again, i_sep), "selection after fused calls differs"


def test_index_topk_fused_equals_separate_calls():
    rng = np.random.default_rng(300)
    say("case: index_topk fused (3 ragged sequences, one with n <= k), twice on one workspace")
    _fused_vs_separate(rng, [20000, 200, 9000], 64, 256)
    say("case: index_topk fused, one long row (many chunks)")
    _fused_vs_separate(rng, [70000], 64, 2048)


def test_index_score_counted_then_topk_select_counted_equal_separate_calls():
    rng = np.random.default_rng(303)
    say("case: counted pair (3 ragged sequences, one with n <= k), twice on one workspace")
    _fused_vs_separate(rng, [20000, 200, 9000], 64, 256, counted=True)
    say("case: counted pair, one long row (many chunks)")
    _fused_vs_separate(rng, [300003], 64, 2048, counted=True)
    say("case: counted pair, queries sharing sequences (a counting pass after the scan)")
    _fused_vs_separate(rng, [5000, 3000], 32, 128, seq_of_query=[0] * 40 + [1] * 30, counted=True)
    say("case: counted pair, 16 index heads, one chunk per row")
    _fused_vs_separate(rng, [3000, 4096, 50], 16, 64, counted=True)


def test_index_topk_fused_exact_path_entries():
    def keys(k):
        k[:, 0:32] *= 2.0 ** -12
        k[:, 64:96] *= 2.0 ** 6
        return k

    say("case: index_topk fused with exact-path entries (wide exponent spread)")
    _fused_vs_separate(np.random.default_rng(301), [6000], 16, 512, key_fn=keys)


def test_index_topk_best_entries_crowd_one_range():
    """The best 3000 entries first, then last, in a row of 300,000: one range of the
    row holds the whole top k (every other chunk of the selection lists nothing)."""
    def first(k):
        k[:3000] *= 3.0
        return k

    def last(k):
        k[-3000:] *= 3.0
        return k

    say("case: index_topk, best entries crowded at the start of a 300K row")
    _fused_vs_separate(np.random.default_rng(303), [300000], 64, 2048, key_fn=first, reps=1)
    say("case: index_topk, best entries crowded at the end of a 300K row")
    _fused_vs_separate(np.random.default_rng(304), [300000], 64, 2048, key_fn=last, reps=1)


def test_index_topk_all_scores_tied():
    """Every key equal, so every score ties: the threshold bin holds every entry and
    overflows the candidate lists; ties go to the lower index."""
    def same(k):
        k[:] = k[0]
        return k

    say("case: index_topk, all scores tied in a 100K row and a 5K row")
    _fused_vs_separate(np.random.default_rng(305), [100000, 5000], 64, 2048, key_fn=same, reps=1)


def test_index_topk_long_rows_of_different_lengths():
    """Rows of up to 1.1M entries (538 scan workgroups and 269 selection chunks per
    query), eight queries of different lengths (two at or below k); keys drawn on the
    device.  index_topk against index_score then topk_select, bit for bit."""
    n_max, Hi, k = 1_100_000, 64, 2048
    n = [n_max, 900_000, 524_288, 70_000, 2048, 1000, 300_001, 4097]
    pages = (n_max + 63) // 64
    g = lib.Cache(pages * 64)
    gen = torch.Generator(device="cuda").manual_seed(306)
    key = torch.randn((pages * 64, 128), device="cuda", generator=gen).to(torch.bfloat16).view(torch.int16)
    lat = torch.zeros((pages * 64, 512), dtype=torch.int16, device="cuda")
    lib.fp4_cache_write(g, lat, key, torch.arange(pages * 64, dtype=torch.int64, device="cuda"))
    del lat, key
    nq = len(n)
    q = torch.randn((nq, Hi, 128), device="cuda", generator=gen).to(torch.bfloat16).view(torch.int16)
    w = torch.rand((nq, Hi), device="cuda", generator=gen)
    nvis = torch.tensor(n, dtype=torch.int32, device="cuda")
    bt = torch.arange(pages, dtype=torch.int32, device="cuda").repeat(nq, 1)
    ld = pages * 64
    ws = torch.zeros(lib.topk_select_workspace_size(nq, ld, k), dtype=torch.uint8, device="cuda")
    s_sep = torch.full((nq, ld), float("nan"), device="cuda")
    i_sep = torch.full((nq, k), -7, dtype=torch.int32, device="cuda")
    say(f"case: index_topk over rows of up to {n_max} entries ({nq} queries)")
    lib.index_score(g, q, w, nvis, bt, s_sep)
    lib.topk_select(s_sep, nvis, k, i_sep, ws)
    s_f = torch.full((nq, ld), float("nan"), device="cuda")
    i_f = torch.full((nq, k), -7, dtype=torch.int32, device="cuda")
    lib.index_topk(g, q, w, nvis, bt, s_f, k, i_f, ws)
    torch.cuda.synchronize()
    for r in range(nq):
        assert torch.equal(s_f[r, :n[r]].view(torch.int32), s_sep[r, :n[r]].view(torch.int32)), f"row {r} scores"
    assert torch.equal(i_f, i_sep), "top-k differs"


def _gate_vs_separate(rng, n_per_seq, Hi, k, npool, key_fn=None, seq_of_query=None, reps=2):
    """index_topk_pool_build against index_topk then index_pool_build (scores, top-k
    and pool bit for bit), `reps` times on one workspace."""
    B = len(n_per_seq)
    pages = [(n + 63) // 64 for n in n_per_seq]
    phys = rng.permutation(sum(pages))
    bt = np.zeros((B, max(pages)), np.int32)
    off, key, slots = 0, [], []
    for b, n in enumerate(n_per_seq):
        bt[b, :pages[b]] = phys[off:off + pages[b]]
        off += pages[b]
        j = np.arange(n)
        slots.append(bt[b, j // 64].astype(np.int64) * 64 + j % 64)
        kk = rng.standard_normal((n, 128)).astype(np.float32)
        key.append(bits(key_fn(kk) if key_fn else kk))
    g = lib.Cache(sum(pages) * 64)
    nall = sum(n_per_seq)
    lib.fp4_cache_write(g, dev_bits(np.zeros((nall, 512), np.uint16)), dev_bits(np.concatenate(key)),
                        dev(np.concatenate(slots)))
    if seq_of_query is None:
        nq, soq, nvis = B, None, np.array(n_per_seq, np.int32)
    else:
        soq = np.asarray(seq_of_query, np.int32)
        nq = len(soq)
        nvis = np.array([max(1, n_per_seq[s] - 7 * i % 50) for i, s in enumerate(soq)], np.int32)
    ld = ((int(nvis.max()) + 63) // 64) * 64
    q = bits(rng.standard_normal((nq, Hi, 128)).astype(np.float32))
    w = rng.random((nq, Hi), dtype=np.float32)
    dq, dw, dnv, dbt = dev_bits(q), dev(w), dev(nvis), dev(bt)
    dsoq = None if soq is None else dev(soq)
    ws_t = torch.zeros(lib.topk_select_workspace_size(nq, ld, k), dtype=torch.uint8, device="cuda")
    ws_p = torch.zeros(lib.index_pool_build_workspace_size(nq, ld, npool), dtype=torch.uint8, device="cuda")
    s_sep = torch.full((nq, ld), float("nan"), device="cuda")
    i_sep = torch.full((nq, k), -7, dtype=torch.int32, device="cuda")
    p_sep = torch.full((nq, npool), -7, dtype=torch.int32, device="cuda")
    lib.index_topk(g, dq, dw, dnv, dbt, s_sep, k, i_sep, ws_t, seq_of_query=dsoq)
    lib.index_pool_build(s_sep, dnv, npool, p_sep, ws_p)
    ws_g = torch.zeros(lib.index_topk_pool_build_workspace_size(nq, ld, k, npool), dtype=torch.uint8, device="cuda")
    for rep in range(reps):
        s_g = torch.full((nq, ld), float("nan"), device="cuda")
        i_g = torch.full((nq, k), -7, dtype=torch.int32, device="cuda")
        p_g = torch.full((nq, npool), -7, dtype=torch.int32, device="cuda")
        lib.index_topk_pool_build(g, dq, dw, dnv, dbt, s_g, k, i_g, npool, p_g, ws_g, seq_of_query=dsoq)
        torch.cuda.synchronize()
        a, b = s_g.cpu().numpy(), s_sep.cpu().numpy()
        for r in range(nq):
            assert same_bits_f32(a[r, :nvis[r]], b[r, :nvis[r]]), f"rep {rep} row {r}: scores differ"
        assert torch.equal(i_g, i_sep), f"rep {rep}: top-k differs"
        assert torch.equal(p_g, p_sep), f"rep {rep}: pool differs"


def test_index_topk_pool_build_equals_separate_calls():
    def spread(kk):
        kk[:, 0:32] *= 2.0 ** -12
        kk[:, 64:96] *= 2.0 ** 6
        return kk

    say("case: index_topk_pool_build, one 300,003-entry row, pool 2048")
    _gate_vs_separate(np.random.default_rng(320), [300003], 64, 2048, 2048)
    say("case: index_topk_pool_build, ragged rows (some keep every block), pool 1024")
    _gate_vs_separate(np.random.default_rng(321), [70000, 9001, 100, 8200], 64, 256, 1024)
    say("case: index_topk_pool_build with exact-path entries, 16 heads")
    _gate_vs_separate(np.random.default_rng(322), [40001], 16, 512, 300, key_fn=spread)
    say("case: index_topk_pool_build, three rows in one paired selection launch (one keeps every block)")
    _gate_vs_separate(np.random.default_rng(324), [300003, 140001, 5000], 64, 2048, 2048)
    say("case: index_topk_pool_build, six 200,003-entry rows (the paired launch in its split form)")
    _gate_vs_separate(np.random.default_rng(325), [200003] * 6, 64, 2048, 2048, reps=1)
    say("case: index_topk_pool_build, queries sharing sequences (the two calls in turn)")
    _gate_vs_separate(np.random.default_rng(323), [5000, 3000], 32, 128, 64, seq_of_query=[0] * 40 + [1] * 30)


def test_index_topk_query_tiles_fall_back():
    say("case: index_topk with a sequence map and 70 queries (tiles of queries, separate counting pass)")
    _fused_vs_separate(np.random.default_rng(302), [5000, 3000], 32, 128, seq_of_query=[0] * 40 + [1] * 30)


# -------------------------------------------------- candidate pool --------
def _pool_case(rng, n_per_seq, Hi, npool, k, key_fn=None, reps=2):
    """Full scan -> pool (index_pool_build) -> scan and top-K inside the pool
    (index_topk_pool), against the oracle on the same inputs; twice on the same
    workspaces (they must be left clean)."""
    B = len(n_per_seq)
    pages = [(n + 63) // 64 for n in n_per_seq]
    phys = rng.permutation(sum(pages))
    bt = np.zeros((B, max(pages)), np.int32)
    off, lat, key, slots = 0, [], [], []
    for b, n in enumerate(n_per_seq):
        bt[b, :pages[b]] = phys[off:off + pages[b]]
        off += pages[b]
        j = np.arange(n)
        slots.append(bt[b, j // 64].astype(np.int64) * 64 + j % 64)
        kk = rng.standard_normal((n, 128)).astype(np.float32)
        key.append(bits(key_fn(kk) if key_fn else kk))
        lat.append(bits(np.zeros((n, 512), np.float32)))
    lat, key, slots = np.concatenate(lat), np.concatenate(key), np.concatenate(slots)
    g, o = both_caches(lat, key, slots, sum(pages) * 64)
    nvis = np.array(n_per_seq, np.int32)
    ld = ((int(nvis.max()) + 63) // 64) * 64
    q0 = bits(rng.standard_normal((B, Hi, 128)).astype(np.float32))   # gatekeeper layer
    q1 = bits(rng.standard_normal((B, Hi, 128)).astype(np.float32))   # pooled layer
    w0 = rng.random((B, Hi), dtype=np.float32)
    w1 = rng.random((B, Hi), dtype=np.float32)
    dnv, dbt = dev(nvis), dev(bt)
    # gatekeeper scan (GPU), the same scores from the oracle
    s_full = torch.full((B, ld), float("nan"), device="cuda")
    lib.index_score(g, dev_bits(q0), dev(w0), dnv, dbt, s_full)
    ref_full, _, _ = oracle.index_score(o, q0, w0, nvis, bt, ld=ld)
    got_full = s_full.cpu().numpy()
    for r in range(B):
        assert same_bits_f32(got_full[r, :nvis[r]], ref_full[r, :nvis[r]])
    ref_pool = oracle.pool_build(ref_full, nvis, npool)
    ref_ps, _, _ = oracle.index_score_pool(o, q1, w1, nvis, ref_pool, bt)
    ref_top = oracle.topk_pool(ref_ps, ref_pool, nvis, k)
    ws_b = torch.zeros(lib.index_pool_build_workspace_size(B, ld, npool), dtype=torch.uint8, device="cuda")
    ws_t = torch.zeros(lib.index_topk_pool_workspace_size(B, npool, k), dtype=torch.uint8, device="cuda")
    for rep in range(reps):
        pool = torch.full((B, npool), -7, dtype=torch.int32, device="cuda")
        lib.index_pool_build(s_full, dnv, npool, pool, ws_b)
        ps = torch.full((B, npool * 8), float("nan"), device="cuda")
        top = torch.full((B, k), -7, dtype=torch.int32, device="cuda")
        lib.index_topk_pool(g, dev_bits(q1), dev(w1), dnv, pool, dbt, ps, k, top, ws_t)
        torch.cuda.synchronize()
        assert np.array_equal(pool.cpu().numpy(), ref_pool), f"rep {rep}: pool differs"
        got_ps = ps.cpu().numpy()
        for r in range(B):
            vis = ~np.isnan(ref_ps[r])
            npv = int(vis.sum())
            assert vis[:npv].all(), "visible pool positions are a prefix"
            assert same_bits_f32(got_ps[r, :npv], ref_ps[r, :npv]), f"rep {rep} row {r}: pool scores differ"
            assert np.all(np.isnan(got_ps[r, npv:])), "positions without an entry were written"
        assert np.array_equal(top.cpu().numpy(), ref_top), f"rep {rep}: pool top-k differs"
    return ref_pool


def test_pool_build_and_topk_inside_pool():
    rng = np.random.default_rng(400)
    say("case: pool of 256 blocks over 3 paged sequences (partial last blocks), k = 300, Hi = 64")
    _pool_case(rng, [20001, 3005, 777], 64, 256, 300)
    say("case: pool of 2048 blocks over one 70,000-entry sequence, k = 2048, Hi = 16")
    _pool_case(rng, [70000], 16, 2048, 2048)
    say("case: pool of 300 blocks over 2 sequences, k = 500, Hi = 128")
    _pool_case(rng, [5003, 2999], 128, 300, 500)


def test_pool_covering_every_block_and_short_pools():
    rng = np.random.default_rng(401)
    say("case: pools larger than the sequences (every block), k above the visible members")
    pool = _pool_case(rng, [500, 61, 8, 0], 16, 128, 700)
    assert list(pool[0, :63]) == list(range(63)) and np.all(pool[0, 63:] == -1)
    assert np.all(pool[3] == -1), "a query with no visible entry has an empty pool"


def test_pool_queries_sharing_sequences():
    """Pools for several queries per sequence (a prefill chunk's causal rows): the
    full scan, the pools and the pooled scan address each sequence's pages through
    seq_of_query."""
    rng = np.random.default_rng(403)
    n_per_seq = [9000, 3000]
    pages = [(n + 63) // 64 for n in n_per_seq]
    phys = rng.permutation(sum(pages))
    bt = np.zeros((2, max(pages)), np.int32)
    bt[0, :pages[0]] = phys[:pages[0]]
    bt[1, :pages[1]] = phys[pages[0]:]
    lat, key, slots = [], [], []
    for b, n in enumerate(n_per_seq):
        j = np.arange(n)
        slots.append(bt[b, j // 64].astype(np.int64) * 64 + j % 64)
        key.append(bits(rng.standard_normal((n, 128)).astype(np.float32)))
        lat.append(bits(np.zeros((n, 512), np.float32)))
    g, o = both_caches(np.concatenate(lat), np.concatenate(key), np.concatenate(slots), sum(pages) * 64)
    soq = np.array([0, 0, 0, 1, 1, 1, 1], np.int32)
    nvis = np.array([9000, 8999, 4321, 3000, 2999, 17, 0], np.int32)
    nq, Hi, npool, k = len(soq), 16, 200, 300
    ld = ((int(nvis.max()) + 63) // 64) * 64
    q0 = bits(rng.standard_normal((nq, Hi, 128)).astype(np.float32))
    q1 = bits(rng.standard_normal((nq, Hi, 128)).astype(np.float32))
    w0 = rng.random((nq, Hi), dtype=np.float32)
    w1 = rng.random((nq, Hi), dtype=np.float32)
    say("case: pools for 7 queries on 2 sequences (seq_of_query)")
    dnv, dbt, dsoq = dev(nvis), dev(bt), dev(soq)
    s_full = torch.full((nq, ld), float("nan"), device="cuda")
    lib.index_score(g, dev_bits(q0), dev(w0), dnv, dbt, s_full, seq_of_query=dsoq)
    ref_full, _, _ = oracle.index_score(o, q0, w0, nvis, bt, seq_of_query=soq, ld=ld)
    ref_pool = oracle.pool_build(ref_full, nvis, npool)
    ref_ps, _, _ = oracle.index_score_pool(o, q1, w1, nvis, ref_pool, bt, seq_of_query=soq)
    ref_top = oracle.topk_pool(ref_ps, ref_pool, nvis, k)
    pool = torch.full((nq, npool), -7, dtype=torch.int32, device="cuda")
    ws_b = torch.zeros(lib.index_pool_build_workspace_size(nq, ld, npool), dtype=torch.uint8, device="cuda")
    lib.index_pool_build(s_full, dnv, npool, pool, ws_b)
    ps = torch.full((nq, npool * 8), float("nan"), device="cuda")
    top = torch.full((nq, k), -7, dtype=torch.int32, device="cuda")
    ws_t = torch.zeros(lib.index_topk_pool_workspace_size(nq, npool, k), dtype=torch.uint8, device="cuda")
    lib.index_topk_pool(g, dev_bits(q1), dev(w1), dnv, pool, dbt, ps, k, top, ws_t, seq_of_query=dsoq)
    torch.cuda.synchronize()
    assert np.array_equal(pool.cpu().numpy(), ref_pool), "pool differs"
    got_ps = ps.cpu().numpy()
    for r in range(nq):
        npv = int((~np.isnan(ref_ps[r])).sum())
        assert same_bits_f32(got_ps[r, :npv], ref_ps[r, :npv]), f"row {r}: pool scores differ"
    assert np.array_equal(top.cpu().numpy(), ref_top), "pool top-k differs"


def test_pool_with_tied_keys():
    def keys(k):
        k[1000:3000] = k[1000]  # 2000 entries with one key: tied scores across many blocks
        return k

    say("case: pool with 2000 tied entries (ties to the lower block and entry)")
    _pool_case(np.random.default_rng(402), [6000], 16, 300, 500, key_fn=keys)


# -------------------------------------------------------------- FP8 window --------
def _fp8_rows(rng, n):
    """Window rows with the cases the FP8 format has: ties between E4M3 neighbours,
    zero and -0 rows, bf16 subnormal and huge rows, outlier channels."""
    x = (rng.standard_normal((n, 512)) * np.exp(rng.uniform(-20, 20, (n, 1)))).astype(np.float32)
    x[:, 7] *= 8.0
    x[1] = 0.0
    x[2] = -0.0
    x[3] = rng.standard_normal(512).astype(np.float32) * np.float32(1e-39)  # bf16 subnormals
    x[4] = rng.standard_normal(512).astype(np.float32) * np.float32(1e37)
    # row 5: scale 2^0 (amax 448) and E4M3 midpoints
    e4 = np.array([oracle.e4m3_value(b) for b in range(0x7F)])
    mids = (e4[8:-1] + e4[9:]) / 2
    x[5] = 0.0
    x[5, 0] = 448.0
    x[5, 1:1 + len(mids)] = mids * np.where(np.arange(len(mids)) % 2, -1, 1)
    return bits(x)


def test_swa_fp8_write_bit_exact():
    rng = np.random.default_rng(500)
    rows = _fp8_rows(rng, 3001)
    say("case: FP8 window rows, 3001 rows with ties, zero, subnormal and huge rows")
    codes = torch.full((3001, 512), 0x55, dtype=torch.uint8, device="cuda")
    scales = torch.full((3001,), 0x55, dtype=torch.uint8, device="cuda")
    lib.swa_fp8_write(dev_bits(rows), codes, scales)
    rc, rs = oracle.swa_fp8_quant(rows)
    assert np.array_equal(scales.cpu().numpy(), rs), "FP8 window scales differ"
    got = codes.cpu().numpy()
    bad = np.argwhere(got != rc)
    assert len(bad) == 0, f"{len(bad)} FP8 codes differ, first {bad[:4].tolist()}"


def _fp8_window(rng, shape):
    x = rng.standard_normal(shape).astype(np.float32)
    x[..., [3, 200]] *= 8.0
    return bits(x)


@pytest.mark.parametrize("H", [16, 64])
def test_attention_decode_fp8_window(H):
    rng = np.random.default_rng(510 + H)
    n, B, k, W = 3000, 3, 300, 128
    g, o = _attn_cache(rng, n)
    bt = np.tile(np.arange((n + 63) // 64, dtype=np.int32), (B, 1))
    idx = np.stack([np.sort(rng.choice(n, k, replace=False)) for _ in range(B)]).astype(np.int32)
    idx[1, 250:] = -1
    q = bits(rng.standard_normal((B, H, 512)))
    rows = _fp8_window(rng, (B, W, 512))
    codes = torch.zeros((B, W, 512), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((B, W), dtype=torch.uint8, device="cuda")
    lib.swa_fp8_write(dev_bits(rows), codes, scales)
    swa_len = np.array([128, 5, 0], np.int32)
    scale = 1 / math.sqrt(512)
    ws = torch.zeros(lib.sparse_attn_decode_workspace_size(B, H, k, W), dtype=torch.uint8, device="cuda")
    say(f"case: attention decode, FP8 window, H={H}")
    out = torch.zeros((B, H, 512), device="cuda")
    lse = torch.zeros((B, H), device="cuda")
    lib.sparse_attn_decode_fp8win(g, dev_bits(q), dev(idx), dev(bt), codes, scales, dev(swa_len), scale, out, lse, ws)
    rc, rs = oracle.swa_fp8_quant(rows)
    ro, rl = oracle.sparse_attn_decode_fp8win(o, q, idx, bt, rc, rs, swa_len, scale)
    attn_close(out.cpu().numpy(), ro, lse.cpu().numpy(), rl, f"decode FP8 window H={H}")
    # the same kernel fed the bf16 rows of the window's exact values: identical bits
    out2 = torch.zeros_like(out)
    lse2 = torch.zeros_like(lse)
    lib.sparse_attn_decode(g, dev_bits(q), dev(idx), dev(bt), dev_bits(oracle.swa_fp8_dequant(rc, rs)), dev(swa_len),
                           scale, out2, lse2, ws)
    assert torch.equal(out.view(torch.int32), out2.view(torch.int32))
    assert torch.equal(lse.view(torch.int32), lse2.view(torch.int32))


@pytest.mark.parametrize("T", [40, 160])
def test_attention_prefill_fp8_window(T):
    # T = 40: several row ranges per query; T = 160: one workgroup per query (64 heads)
    rng = np.random.default_rng(520 + T)
    n, H, k, W = 2500, 64, 200, 128
    g, o = _attn_cache(rng, n)
    bt = np.arange((n + 63) // 64, dtype=np.int32)
    idx = np.stack([np.sort(rng.choice(n, k, replace=False)) for _ in range(T)]).astype(np.int32)
    idx[5, 150:] = -1
    q = bits(rng.standard_normal((T, H, 512)))
    rows = _fp8_window(rng, (W - 1 + T, 512))
    codes = torch.zeros((W - 1 + T, 512), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((W - 1 + T,), dtype=torch.uint8, device="cuda")
    lib.swa_fp8_write(dev_bits(rows), codes, scales)
    first_valid = 100
    scale = 1 / math.sqrt(512)
    ws = torch.zeros(max(256, lib.sparse_attn_prefill_chunk_workspace_size(T, H, k, W)), dtype=torch.uint8,
                     device="cuda")
    say(f"case: attention prefill, FP8 window, T={T}")
    out = torch.zeros((T, H, 512), device="cuda")
    lse = torch.zeros((T, H), device="cuda")
    lib.sparse_attn_prefill_chunk_fp8win(g, dev_bits(q), dev(idx), dev(bt), 5000, codes, scales, first_valid, W, scale,
                                         out, lse, ws)
    rc, rs = oracle.swa_fp8_quant(rows)
    ro, rl = oracle.sparse_attn_prefill_chunk_fp8win(o, q, idx, bt, rc, rs, first_valid, W, scale)
    attn_close(out.cpu().numpy(), ro, lse.cpu().numpy(), rl, f"prefill FP8 window T={T}")
    out2 = torch.zeros_like(out)
    lse2 = torch.zeros_like(lse)
    lib.sparse_attn_prefill_chunk(g, dev_bits(q), dev(idx), dev(bt), 5000, dev_bits(oracle.swa_fp8_dequant(rc, rs)),
                                  first_valid, W, scale, out2, lse2, ws)
    assert torch.equal(out.view(torch.int32), out2.view(torch.int32))
    assert torch.equal(lse.view(torch.int32), lse2.view(torch.int32))
