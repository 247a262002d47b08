"""index_topk_noalloc (workspace in the library's static device array, for callers
that cannot allocate) against index_topk with a caller workspace: scores and indices
bit for bit, on two calls in a row, the second smaller (the array keeps the first
call's bytes).  Also a call past the array's size is refused."""
import numpy as np
import pytest
import torch

from sparse_attention_fp4_cache_amd import lib
from _helpers import bits, dev, dev_bits, say

pytestmark = pytest.mark.gpu


def _case(rng, g, n_rows, Hi, k, pages):
    nq = len(n_rows)
    q = dev_bits(bits(rng.standard_normal((nq, Hi, 128)).astype(np.float32)))
    w = dev(rng.random((nq, Hi), dtype=np.float32))
    nvis = dev(np.array(n_rows, np.int32))
    bt = dev(np.tile(rng.permutation(pages).astype(np.int32), (nq, 1)))
    ld = ((max(n_rows) + 63) // 64) * 64
    ws = torch.zeros(lib.topk_select_workspace_size(nq, ld, k), dtype=torch.uint8, device="cuda")
    s_ref = torch.full((nq, ld), float("nan"), device="cuda")
    i_ref = torch.full((nq, k), -7, dtype=torch.int32, device="cuda")
    lib.index_topk(g, q, w, nvis, bt, s_ref, k, i_ref, ws)
    s_na = torch.full((nq, ld), float("nan"), device="cuda")
    i_na = torch.full((nq, k), -7, dtype=torch.int32, device="cuda")
    lib.index_topk_noalloc(g, q, w, nvis, bt, s_na, k, i_na)
    torch.cuda.synchronize()
    for r in range(nq):
        n = n_rows[r]
        assert torch.equal(s_na[r, :n].view(torch.int32), s_ref[r, :n].view(torch.int32)), f"row {r}: scores"
    assert torch.equal(i_na, i_ref), "top-k differs"


def test_index_topk_noalloc_matches_index_topk_twice():
    lib.load()
    rng = np.random.default_rng(700)
    pages = 2048  # 131,072 slots
    n = pages * 64
    g = lib.Cache(n)
    lat = dev_bits(np.zeros((n, 512), np.uint16))
    key = dev_bits(bits(rng.standard_normal((n, 128)).astype(np.float32)))
    lib.fp4_cache_write(g, lat, key, dev(np.arange(n, dtype=np.int64)))
    say("case: index_topk_noalloc, 6 rows up to 131,072 entries, k = 2048, then 3 rows up to 20,000, k = 256")
    _case(rng, g, [n, 100_000, 70_000, 2048, 1500, 131_000], 64, 2048, pages)
    _case(rng, g, [20_000, 5000, 300], 64, 256, pages)
    say("  both calls bit-identical to index_topk with a caller workspace")
    with pytest.raises(lib.Csa2Error) as e:
        lib.index_topk_noalloc(g, torch.zeros((512, 64, 128), dtype=torch.int16, device="cuda"),
                               torch.zeros((512, 64), device="cuda"), torch.full((512,), n, dtype=torch.int32,
                                                                                 device="cuda"),
                               torch.zeros((512, pages), dtype=torch.int32, device="cuda"),
                               torch.zeros((512, n), device="cuda"), 2048,
                               torch.zeros((512, 2048), dtype=torch.int32, device="cuda"))
    assert e.value.status == -4
