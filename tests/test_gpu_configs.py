"""Whole-step GPU parity at the five workload configurations, at their full sizes.

Each case builds the seeded synthetic inputs once, runs the step through the C ABI
(the same calls and launch configurations the benchmark times), and compares with
the CPU oracle run on the very same host arrays:
  * cache bytes, indexer scores and top-k indices bit-exact;
  * attention within 2e-3 absolute and 1e-2 of the largest reference magnitude.
Where the oracle would take too long (the 4096-query prefill chunk), sampled
queries are checked one by one and every query is checked for properties that
hold at any size.  The oracle never sees a GPU result.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_fp4_cache_amd import lib
from sparse_attention_fp4_cache_amd.step import DecodeStep, PrefillStep, ScheduleDecodeStep
from sparse_attention_fp4_cache_amd.workloads import WORKLOADS
from _helpers import attn_close, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    lib.load()


def oracle_cache(wl):
    """The oracle's own cache, written from the same seeded rows as the GPU cache."""
    o = oracle.Cache(wl.num_slots)
    for b in range(wl.B):
        n = int(wl.n_entries[b]) + (wl.n_chunk_entries if wl.kind == "prefill" else 0)
        lat, key = wl.cache_rows(b, 0, n)
        oracle.fp4_cache_write(o, lat, key, wl.slots(b, 0, n))
    return o


def cache_equal(st, o, label):
    for name in ("main_codes", "main_scales", "idx_codes", "idx_scales"):
        a = getattr(st.cache, name).cpu().numpy()
        b = getattr(o, name)
        nbad = int(np.count_nonzero(a != b))
        assert nbad == 0, f"{label}: {name} differs in {nbad} bytes"


def scores_equal(got, ref, nvis, label):
    for r in range(ref.shape[0]):
        n = int(nvis[r])
        g = np.ascontiguousarray(got[r, :n]).view(np.int32)
        e = np.ascontiguousarray(ref[r, :n]).view(np.int32)
        bad = np.flatnonzero(g != e)
        assert len(bad) == 0, (f"{label}: row {r}: {len(bad)} scores differ, first entry {bad[0]}: "
                               f"{got[r, bad[0]]!r} vs {ref[r, bad[0]]!r}")


def topk_equal(got, ref, label):
    bad = np.argwhere(got != ref)
    assert len(bad) == 0, f"{label}: {len(bad)} top-k slots differ, first {bad[:4].tolist()}"


def run_decode_case(name, attn_rows=None, wl=None):
    wl = WORKLOADS[name] if wl is None else wl
    say(f"case: {name} (B={wl.B}, entries {int(wl.n_entries.min())}..{int(wl.n_entries.max())}, "
        f"H={wl.H}, K={wl.K}, layers {','.join(wl.layers)})")
    st = DecodeStep(wl, "cuda")
    st.build_cache()
    st.run(keep_scores=True)
    torch.cuda.synchronize()
    o = oracle_cache(wl)
    cache_equal(st, o, name)
    say("  cache bytes equal")
    bt = wl.block_table()
    # visibility from the oracle's own causal rule; the GPU step was given the
    # workload's array, which must be the same
    nv = oracle.decode_n_visible(wl.ctx, wl.m)
    assert np.array_equal(nv, wl.n_visible()), "visible entries differ from the oracle's causal rule"
    latest = ref_pool = None
    for li, L in enumerate(st.layers):
        d = wl.layer_inputs(li)
        if L["mode"] == "reindex" and wl.npool > 0:
            # scores and selection inside the Full layer's candidate pool
            ref_ps, not_fp32, _ = oracle.index_score_pool(o, d["q_idx"], d["w"], nv, ref_pool, bt)
            assert not_fp32 == 0
            npv = np.count_nonzero(~np.isnan(ref_ps), axis=1)
            scores_equal(L["scores"].cpu().numpy(), ref_ps, npv, f"{name} layer {li} pool scores")
            latest = oracle.topk_pool(ref_ps, ref_pool, nv, wl.K)
            topk_equal(L["topk"].cpu().numpy(), latest, f"{name} layer {li} pool top-k")
            say(f"  layer {li} (reindex over the pool): scores and top-k bit-exact")
        elif L["mode"] in ("full", "reindex"):
            ref_s, not_fp32, _ = oracle.index_score(o, d["q_idx"], d["w"], nv, bt, ld=st.ld)
            assert not_fp32 == 0
            scores_equal(L["scores"].cpu().numpy(), ref_s, nv, f"{name} layer {li} scores")
            latest = oracle.topk_select(ref_s, nv, wl.K)
            topk_equal(L["topk"].cpu().numpy(), latest, f"{name} layer {li} top-k")
            say(f"  layer {li} ({L['mode']}): scores and top-k bit-exact")
            if L["mode"] == "full" and wl.npool > 0:
                ref_pool = oracle.pool_build(ref_s, nv, wl.npool)
                topk_equal(L["pool"].cpu().numpy(), ref_pool, f"{name} layer {li} candidate pool")
                say(f"  layer {li}: candidate pool of {wl.npool} blocks bit-exact")
        rows = np.arange(wl.B) if attn_rows is None else np.asarray(attn_rows)
        if wl.fp8_window:
            codes, scales = oracle.swa_fp8_quant(d["swa"][rows])
            assert np.array_equal(L["swa8"].cpu().numpy()[rows], codes), f"layer {li}: FP8 window codes differ"
            assert np.array_equal(L["swa8_scale"].cpu().numpy()[rows], scales), f"layer {li}: FP8 scales differ"
            ro, rl = oracle.sparse_attn_decode_fp8win(o, d["q"][rows], latest[rows], bt[rows], codes, scales,
                                                      d["swa_len"][rows], st.scale)
        else:
            ro, rl = oracle.sparse_attn_decode(o, d["q"][rows], latest[rows], bt[rows], d["swa"][rows],
                                               d["swa_len"][rows], st.scale)
        attn_close(L["out"].cpu().numpy()[rows], ro, L["lse"].cpu().numpy()[rows], rl,
                   f"{name} layer {li} ({L['mode']}) attention")
    return st


def test_config_tiny_decode():
    run_decode_case("tiny_decode")


@pytest.mark.timeout(600)
def test_config_decode_131k_outliers():
    run_decode_case("decode_131k")


@pytest.mark.timeout(900)
def test_config_ragged_decode_32_paged():
    # scores, top-k and attention for all 32 sequences
    run_decode_case("ragged_decode_32")


@pytest.mark.timeout(1200)
def test_config_decode_1m_10layer_and_graph_replay():
    st = run_decode_case("decode_1m_10layer")
    graph_replays_equal_eager(st)


@pytest.mark.timeout(1200)
def test_config_decode_1m_10layer_fp8_window():
    # every layer's window in FP8: codes and scales bit-exact, attention within tolerance
    st = run_decode_case("decode_1m_10layer_fp8win")
    graph_replays_equal_eager(st)


@pytest.mark.timeout(900)
def test_config_ragged_decode_32_candidate_pool():
    # a Full layer, a Reindex layer inside pools of 1024 blocks (rows with fewer
    # than 8192 entries keep every block), and a Reuse layer
    wl = dataclasses.replace(WORKLOADS["ragged_decode_32"], name="ragged_decode_32_pool",
                             layers=("full", "reindex", "reuse"), npool=1024)
    run_decode_case(wl.name, attn_rows=np.arange(0, 32, 4), wl=wl)


@pytest.mark.timeout(1200)
def test_config_decode_1m_10layer_pool_and_graph_replay():
    st = run_decode_case("decode_1m_10layer_pool")
    graph_replays_equal_eager(st)


@pytest.mark.timeout(1500)
def test_config_decode_1m_whole_schedule():
    """One token through all 40 layers: three m = 2 encoder caches, the m = 1 decoder
    cache (1,048,576 entries), window-only layers, pooled decoder Reindex layers."""
    sw = WORKLOADS["decode_1m_schedule"]
    say(f"case: {sw.name} ({len(sw.modes)} layers, writers {sw.writers()}, pool {sw.npool} blocks)")
    st = ScheduleDecodeStep(sw, "cuda")
    st.build_cache()
    st.run(keep_scores=True)
    torch.cuda.synchronize()
    qw = sw.query_workload()
    refs = {}
    for w in sw.writers():
        cw = sw.cache_workload(w)
        o = oracle_cache(cw)
        C = st.caches[w]
        for name in ("main_codes", "main_scales", "idx_codes", "idx_scales"):
            nbad = int(np.count_nonzero(getattr(C["cache"], name).cpu().numpy() != getattr(o, name)))
            assert nbad == 0, f"cache of layer {w}: {name} differs in {nbad} bytes"
        nv_o = oracle.decode_n_visible(cw.ctx, cw.m)
        assert np.array_equal(nv_o, cw.n_visible()), "visible entries differ from the oracle's causal rule"
        refs[w] = (o, cw.block_table(), nv_o)
        say(f"  cache of layer {w} (m = {cw.m}, {int(cw.n_entries[0])} entries): bytes equal")
    latest, pools = {}, {}
    for li, L in enumerate(st.layers):
        d = qw.layer_inputs(li)
        mode, src = L["mode"], L["src"]
        if mode == "swa":
            o, bt, nv = next(iter(refs.values()))
            ro, rl = oracle.sparse_attn_decode(o, d["q"], np.zeros((1, 0), np.int32), bt, d["swa"], d["swa_len"],
                                               st.scale)
            attn_close(L["out"].cpu().numpy(), ro, L["lse"].cpu().numpy(), rl, f"layer {li} (window only)")
            continue
        o, bt, nv = refs[src]
        if mode == "reindex" and sw.npool > 0:
            ref_ps, not_fp32, _ = oracle.index_score_pool(o, d["q_idx"], d["w"], nv, pools[src], bt)
            assert not_fp32 == 0
            npv = np.count_nonzero(~np.isnan(ref_ps), axis=1)
            scores_equal(L["scores"].cpu().numpy(), ref_ps, npv, f"layer {li} pool scores")
            latest[src] = oracle.topk_pool(ref_ps, pools[src], nv, sw.K)
            topk_equal(L["topk"].cpu().numpy(), latest[src], f"layer {li} pool top-k")
            say(f"  layer {li} (reindex over the pool): scores and top-k bit-exact")
        elif mode in ("full", "reindex"):
            ref_s, not_fp32, _ = oracle.index_score(o, d["q_idx"], d["w"], nv, bt, ld=st.caches[src]["ld"])
            assert not_fp32 == 0
            scores_equal(L["scores"].cpu().numpy(), ref_s, nv, f"layer {li} scores")
            latest[src] = oracle.topk_select(ref_s, nv, sw.K)
            topk_equal(L["topk"].cpu().numpy(), latest[src], f"layer {li} top-k")
            say(f"  layer {li} ({mode}): scores and top-k bit-exact")
            if mode == "full" and st.caches[src]["pooled"]:
                pools[src] = oracle.pool_build(ref_s, nv, sw.npool)
                topk_equal(L["pool"].cpu().numpy(), pools[src], f"layer {li} candidate pool")
        ro, rl = oracle.sparse_attn_decode(o, d["q"], latest[src], bt, d["swa"], d["swa_len"], st.scale)
        attn_close(L["out"].cpu().numpy(), ro, L["lse"].cpu().numpy(), rl, f"layer {li} ({mode}) attention")
    say("  all 40 layers' attention within tolerance")
    graph_replays_equal_eager(st)


def graph_replays_equal_eager(st):
    # the benchmark replays the step as one HIP graph: every replay must equal the
    # eager step bit for bit, with eager work and synchronisations in between
    ref = [(L["out"].clone(), L["lse"].clone(), None if "topk" not in L else L["topk"].clone()) for L in st.layers]
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        st.run()
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        st.run()
    torch.cuda.synchronize()
    for rep in range(3):
        for L in st.layers:  # clear every output the graph must rewrite
            L["out"].zero_()
            L["lse"].zero_()
            if "topk" in L:
                L["topk"].fill_(-7)
        for P in ([st.pool] if getattr(st, "npool", 0) > 0 else
                  [C["pool"] for C in getattr(st, "caches", {}).values() if C.get("pooled")]):
            P.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for li, (L, (o, l, t)) in enumerate(zip(st.layers, ref)):
            assert torch.equal(L["out"].view(torch.int32), o.view(torch.int32)), f"replay {rep} layer {li} out"
            assert torch.equal(L["lse"].view(torch.int32), l.view(torch.int32)), f"replay {rep} layer {li} lse"
            if t is not None:
                assert torch.equal(L["topk"], t), f"replay {rep} layer {li} top-k"
        st.run()  # eager work between replays
        torch.cuda.synchronize()
    say("  graph replays equal the eager step")


def run_prefill_case(name, which):
    wl = WORKLOADS[name]
    T, K = wl.chunk, wl.K
    d = wl.layer_inputs(0)
    say(f"case: {name} (prefix {int(wl.n_entries[0])} entries + {wl.n_chunk_entries} in-chunk, T={T}, K={K}, "
        f"window rows from {d['swa_first_valid']})")
    st = PrefillStep(wl, "cuda")
    st.build_cache()
    st.run()
    torch.cuda.synchronize()
    o = oracle_cache(wl)
    cache_equal(st, o, name)
    say("  cache bytes equal (prefix + chunk entries)")
    nv = oracle.prefill_n_visible(int(wl.ctx[0]), T, wl.m)
    assert np.array_equal(nv, wl.n_visible()), "visible entries differ from the oracle's causal rule"
    topk = st.topk.cpu().numpy()
    # properties over every query: K distinct indices below n_visible, ascending
    assert topk.shape == (T, K)
    assert np.all(topk >= 0) and np.all(topk < nv[:, None]), "index out of the causal range"
    assert np.all(np.diff(topk, axis=1) > 0), "indices not strictly ascending"
    lse = st.lse.cpu().numpy()
    assert np.all(np.isfinite(lse)), "non-finite lse"
    say("  all queries: top-k causal, distinct, ascending; lse finite")
    # sampled queries, one by one
    which = np.asarray(which, np.int32)
    bt = wl.block_table()
    ref_s, not_fp32, _ = oracle.index_score(o, d["q_idx"][which], d["w"][which], nv[which], bt,
                                            seq_of_query=np.zeros(len(which), np.int32), ld=st.ld)
    assert not_fp32 == 0
    got_s = st.scores[torch.from_numpy(which.astype(np.int64)).cuda()].cpu().numpy()
    scores_equal(got_s, ref_s, nv[which], f"{name} sampled scores")
    ref_k = oracle.topk_select(ref_s, nv[which], K)
    topk_equal(topk[which], ref_k, f"{name} sampled top-k")
    say(f"  queries {which.tolist()}: scores and top-k bit-exact")
    idx_full = np.full((T, K), -1, np.int32)
    idx_full[which] = ref_k
    ro, rl = oracle.sparse_attn_prefill_chunk(o, d["q"], idx_full, bt[0], d["swa"], d["swa_first_valid"], wl.W,
                                              st.scale, which=which)
    attn_close(st.out.cpu().numpy()[which], ro[which], lse[which], rl[which], f"{name} sampled attention")
    say(f"  queries {which.tolist()}: attention within tolerance")


# The prefill scan serves 16 queries per workgroup (two per wavefront), so a tile
# covers queries 16t .. 16t+15; the samples below take every position of whole tiles.
def _tiles(*starts):
    return sorted({q for s in starts for q in range(s, s + 16)})


@pytest.mark.timeout(1200)
def test_config_prefill_chunk_4096():
    # the first tile, the 16 queries around 2047/2048 (halves of two tiles), the last tile
    run_prefill_case("prefill_chunk_4096", _tiles(0, 2040, 4080))


@pytest.mark.timeout(1200)
def test_config_bounded_replay_128_at_1m():
    # the window restarts at the replay: query 0 sees one window row, query 127 all
    # 128; the first and last tiles
    run_prefill_case("replay_128_1m", _tiles(0, 112))
