"""Mode invariants and persist-and-reload of the cache, on the GPU path.

* Reuse with the source layer's query and window reproduces the source layer's
  output bit for bit, and Reindex with the Full layer's indexer query and weights
  reproduces its scores and indices ("Résumé exécutif", CSA2 mode table: Reindex
  recomputes indices on the shared cache, Reuse takes them as they are).
* The cache is plain bytes: written once, copied to host memory and to disk, and
  loaded into a fresh allocation, it gives the very same decode outputs ("DeepSeek-
  V4.1-Flash, expliqué pas à pas", on-disk cache passage: the global KV is stored
  whole and reused on a prefix hit).
Both sides are also compared with the oracle.
"""
import dataclasses
import os

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_fp4_cache_amd import lib
from sparse_attention_fp4_cache_amd.step import DecodeStep
from sparse_attention_fp4_cache_amd.workloads import WORKLOADS, small_variant
from _helpers import attn_close, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    lib.load()


def _ints(t):
    return t.view(torch.int32).cpu().numpy()


def _mode_workload():
    base = WORKLOADS["decode_131k"]
    return dataclasses.replace(small_variant(base, ctx=[20000, 9000]), name="modes",
                               layers=("full", "reuse", "reindex", "reuse"))


def test_reuse_with_source_query_and_reindex_with_full_indexer_inputs():
    wl = _mode_workload()
    say(f"case: mode invariants ({wl.B} sequences, contexts {wl.ctx}, layers {wl.layers})")
    st = DecodeStep(wl, "cuda")
    st.build_cache()
    F, U1, X, U2 = st.layers
    # layer 1 (Reuse) gets the Full layer's query and window; layer 2 (Reindex) its
    # indexer query and weights; layer 3 (Reuse) reuses layer 2's indices
    U1["q"], U1["swa"], U1["swa_len"] = F["q"].clone(), F["swa"].clone(), F["swa_len"].clone()
    X["q_idx"], X["w"] = F["q_idx"].clone(), F["w"].clone()
    U2["q"], U2["swa"], U2["swa_len"] = X["q"].clone(), X["swa"].clone(), X["swa_len"].clone()
    st.run(keep_scores=True)
    torch.cuda.synchronize()
    assert np.array_equal(_ints(U1["out"]), _ints(F["out"])) and np.array_equal(_ints(U1["lse"]), _ints(F["lse"]))
    say("  Reuse with the Full layer's query and window: output bit-identical")
    assert torch.equal(X["topk"], F["topk"])
    assert np.array_equal(_ints(X["scores"]), _ints(F["scores"]))
    say("  Reindex with the Full layer's indexer query and weights: scores and indices bit-identical")
    assert np.array_equal(_ints(U2["out"]), _ints(X["out"])) and np.array_equal(_ints(U2["lse"]), _ints(X["lse"]))
    # and the source layer against the oracle
    o = oracle.Cache(wl.num_slots)
    for b in range(wl.B):
        n = int(wl.n_entries[b])
        lat, key = wl.cache_rows(b, 0, n)
        oracle.fp4_cache_write(o, lat, key, wl.slots(b, 0, n))
    d = wl.layer_inputs(0)
    bt = wl.block_table()
    nv = oracle.decode_n_visible(wl.ctx, wl.m)
    assert np.array_equal(nv, wl.n_visible())
    ref_s, not_fp32, _ = oracle.index_score(o, d["q_idx"], d["w"], nv, bt, ld=st.ld)
    assert not_fp32 == 0
    ref_k = oracle.topk_select(ref_s, nv, wl.K)
    assert np.array_equal(F["topk"].cpu().numpy(), ref_k)
    ro, rl = oracle.sparse_attn_decode(o, d["q"], ref_k, bt, d["swa"], d["swa_len"], st.scale)
    attn_close(F["out"].cpu().numpy(), ro, F["lse"].cpu().numpy(), rl, "source layer against the oracle")


def test_cache_persisted_and_reloaded_gives_identical_outputs(tmp_path):
    wl = dataclasses.replace(_mode_workload(), layers=("full", "reuse", "reindex"))
    say(f"case: cache persisted to disk and reloaded ({wl.num_slots} slots, {wl.num_slots * 356} bytes)")
    st = DecodeStep(wl, "cuda")
    st.build_cache()
    st.run()
    torch.cuda.synchronize()
    ref = [(L["out"].clone(), L["lse"].clone()) for L in st.layers]
    # the four planes, as bytes, to disk
    path = os.path.join(str(tmp_path), "cache.npz")
    planes = {name: getattr(st.cache, name).cpu().numpy() for name in
              ("main_codes", "main_scales", "idx_codes", "idx_scales")}
    np.savez(path, **planes)
    assert sum(p.nbytes for p in planes.values()) == 356 * wl.num_slots
    # a fresh allocation, loaded from the file (no pickled objects)
    with np.load(path, allow_pickle=False) as f:
        fresh = lib.Cache(wl.num_slots, "cuda")
        for name in planes:
            getattr(fresh, name).copy_(torch.from_numpy(f[name]).cuda())
    old = st.cache
    del st.cache
    old.main_codes.fill_(0xFF)  # the first copy is gone for good
    st.cache = fresh
    for L in st.layers:
        L["out"].zero_()
        L["lse"].zero_()
    st.run()
    torch.cuda.synchronize()
    for li, (L, (o, l)) in enumerate(zip(st.layers, ref)):
        assert torch.equal(L["out"].view(torch.int32), o.view(torch.int32)), f"layer {li} out"
        assert torch.equal(L["lse"].view(torch.int32), l.view(torch.int32)), f"layer {li} lse"
    say("  every layer's output bit-identical after the reload")
    # the reloaded bytes are the oracle's cache
    oc = oracle.Cache(wl.num_slots)
    for b in range(wl.B):
        n = int(wl.n_entries[b])
        lat, key = wl.cache_rows(b, 0, n)
        oracle.fp4_cache_write(oc, lat, key, wl.slots(b, 0, n))
    for name in planes:
        assert np.array_equal(getattr(fresh, name).cpu().numpy(), getattr(oc, name)), name
