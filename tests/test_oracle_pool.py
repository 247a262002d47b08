"""Pins of the oracle's hierarchical candidate pool (CPU only).

The pages give the pool's size and shape (about 16,000 positions as 2048 blocks of 8,
assembled by the first decoder layer from its scan of the whole cache; later layers
may not search outside it) but not the rule that picks the blocks.  The reading
pinned here ranks blocks by their largest visible member score, ties to the lower
block.  Pins: brute force on small inputs, the tie rule, partial last blocks, and the
special case of a pool that covers every block, where scoring and selecting inside the
pool must equal the full scan and the full top-K (both pinned elsewhere).
"""
import numpy as np

import oracle
from sparse_attention_fp4_cache_amd.workloads import to_bf16_bits

B = oracle.POOL_BLOCK


def _brute_pool(s_row, n, npool):
    nb = (n + B - 1) // B
    bmax = [max(float(x) for x in s_row[B * b:min(B * b + B, n)]) for b in range(nb)]
    ranked = sorted(range(nb), key=lambda b: (-bmax[b], b))  # best first, ties to the lower block
    keep = sorted(ranked[:min(npool, nb)])
    return keep + [-1] * (npool - len(keep))


def test_pool_build_brute_force_ties_and_partial_blocks():
    rng = np.random.default_rng(11)
    nq, L = 6, 203
    s = rng.standard_normal((nq, L)).astype(np.float32)
    s[1] = rng.integers(0, 5, L).astype(np.float32)  # many tied block maxima
    s[2, :] = 3.0                                   # every block tied
    s[3, 100:] = 1e30                               # beyond n_visible: must not count
    nv = np.array([203, 203, 203, 100, 8, 0], np.int32)
    npool = 7
    pool = oracle.pool_build(s, nv, npool)
    for q in range(nq):
        assert list(pool[q]) == _brute_pool(s[q], int(nv[q]), npool), q
    assert list(pool[2]) == list(range(npool))      # all tied: the first blocks
    assert list(pool[4]) == [0] + [-1] * (npool - 1)
    assert np.all(pool[5] == -1)


def test_pool_covering_every_block_is_every_block():
    rng = np.random.default_rng(12)
    s = rng.standard_normal((2, 70)).astype(np.float32)
    nv = np.array([70, 33], np.int32)
    pool = oracle.pool_build(s, nv, 16)
    assert list(pool[0]) == list(range(9)) + [-1] * 7
    assert list(pool[1]) == list(range(5)) + [-1] * 11


def _cache(rng, n):
    lat = to_bf16_bits(rng.standard_normal((n, 512)).astype(np.float32))
    key = to_bf16_bits(rng.standard_normal((n, 128)).astype(np.float32))
    c = oracle.Cache(((n + 63) // 64) * 64)
    oracle.fp4_cache_write(c, lat, key, np.arange(n))
    return c


def test_pool_scores_are_the_full_scores_of_the_pool_members():
    rng = np.random.default_rng(13)
    n = 300
    c = _cache(rng, 320)
    q = to_bf16_bits(rng.standard_normal((2, 16, 128)).astype(np.float32))
    w = rng.random((2, 16), dtype=np.float32)
    # sequence 1 reads the physical pages in reverse order
    bt = np.array([[0, 1, 2, 3, 4], [4, 3, 2, 1, 0]], np.int32)
    nv = np.array([n, 250], np.int32)
    soq = np.array([0, 1], np.int32)
    full, bad, _ = oracle.index_score(c, q, w, nv, bt, seq_of_query=soq, ld=320)
    assert bad == 0
    pool = np.array([[1, 5, 17, 36, 37, -1], [0, 2, 30, 31, -1, -1]], np.int32)  # 37 and 31: partial last blocks
    ps, bad, _ = oracle.index_score_pool(c, q, w, nv, pool, bt, seq_of_query=soq)
    assert bad == 0
    for qq in range(2):
        for p in range(pool.shape[1] * B):
            blk = pool[qq, p // B]
            j = blk * B + p % B
            if blk < 0 or j >= nv[qq]:
                assert np.isnan(ps[qq, p])
            else:
                assert ps[qq, p].tobytes() == full[qq, j].tobytes()


def test_topk_pool_brute_force_and_covering_pool_equals_full_topk():
    rng = np.random.default_rng(14)
    n = 260
    c = _cache(rng, 320)
    q = to_bf16_bits(rng.standard_normal((3, 16, 128)).astype(np.float32))
    w = rng.random((3, 16), dtype=np.float32)
    bt = np.array([[0, 1, 2, 3, 4]] * 3, np.int32)
    nv = np.array([n, 200, 9], np.int32)
    full, _, _ = oracle.index_score(c, q, w, nv, bt, ld=320)
    k = 40
    want_full = oracle.topk_select(full, nv, k)
    # a pool that covers every block: the same selection as the full top-K
    cover = oracle.pool_build(full, nv, 64)
    ps, _, _ = oracle.index_score_pool(c, q, w, nv, cover, bt)
    assert np.array_equal(oracle.topk_pool(ps, cover, nv, k), want_full)
    # a pool of 6 blocks: brute force over its members
    pool = oracle.pool_build(full, nv, 6)
    ps, _, _ = oracle.index_score_pool(c, q, w, nv, pool, bt)
    got = oracle.topk_pool(ps, pool, nv, k)
    for qq in range(3):
        members = [int(b) * B + i for b in pool[qq] if b >= 0 for i in range(B) if int(b) * B + i < nv[qq]]
        ranked = sorted(members, key=lambda j: (-float(full[qq, j]), j))
        want = sorted(ranked[:k])
        assert list(got[qq]) == want + [-1] * (k - len(want)), qq
