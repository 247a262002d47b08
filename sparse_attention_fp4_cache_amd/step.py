"""Layer-mode composition of the CSA2 step from the five library calls.

Source: "Résumé exécutif", CSA2 mode table, and "DeepSeek V4.1 Flash et le cerveau
divisé", memory section:
  Full    -- computes its cache (here: rewrites the newest entry), its indexer
             scores and its own top-k indices, then attends;
  Reindex -- reuses the source layer's cache and indexer keys, recomputes indices
             from its own indexer query, then attends;
  Reuse   -- reuses the cache and the most recent indices, only attends.
Every layer has its own main query and its own sliding window.

With a candidate pool (workload npool > 0; "DeepSeek V4.1 Flash et le cerveau
divisé", memory section) only the Full layer scans the whole cache: its scores
give each query a pool of npool blocks of 8 consecutive entries, and the Reindex
layers score and select inside that pool.

This module only allocates device buffers and sequences calls; all arithmetic is
in the HIP kernels behind ``lib``.
"""
from __future__ import annotations

import copy

import numpy as np
import torch

from . import lib
from .workloads import PAGE_SIZE, ScheduleWorkload, Workload


def to_device_bits(a: np.ndarray, device) -> torch.Tensor:
    """uint16 bf16 bit patterns -> device int16 tensor (same bits)."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)


class DecodeStep:
    """Device state for a decode workload and one step over its layer schedule.

    The cache holds every sequence's entries before the step.  A Full layer
    rewrites the newest entry of each sequence (same bytes), then scores, selects
    and attends; Reindex layers score with their own indexer query; Reuse layers
    attend with the latest indices.
    """

    def __init__(self, wl: Workload, device="cuda", softmax_scale: float | None = None, fused_index: bool = True):
        """fused_index: run each indexer stage as one index_topk call (same results
        as index_score followed by topk_select, one launch fewer)."""
        assert wl.kind == "decode"
        self.wl = wl
        self.fused_index = fused_index
        self.device = device
        self.scale = lib.default_softmax_scale() if softmax_scale is None else softmax_scale
        B, K, W = wl.B, wl.K, wl.W
        self.cache = lib.Cache(wl.num_slots, device)
        self.block_table = torch.from_numpy(wl.block_table()).to(device)
        nv = wl.n_visible()
        self.n_visible = torch.from_numpy(nv).to(device)
        self.ld = int(((int(nv.max()) + PAGE_SIZE - 1) // PAGE_SIZE) * PAGE_SIZE)
        self.scores = torch.zeros((B, self.ld), dtype=torch.float32, device=device)
        self.topk = torch.full((B, K), -1, dtype=torch.int32, device=device)
        self.ws_topk = torch.zeros(lib.topk_select_workspace_size(B, self.ld, K), dtype=torch.uint8, device=device)
        self.ws_attn = torch.zeros(lib.sparse_attn_decode_workspace_size(B, wl.H, K, W), dtype=torch.uint8,
                                   device=device)
        self.npool = wl.npool
        if self.npool > 0:
            P = self.npool
            self.pool = torch.full((B, P), -1, dtype=torch.int32, device=device)
            self.ws_pool = torch.zeros(lib.index_pool_build_workspace_size(B, self.ld, P), dtype=torch.uint8,
                                       device=device)
            self.scores_pool = torch.zeros((B, lib.POOL_BLOCK * P), dtype=torch.float32, device=device)
            self.ws_topk_pool = torch.zeros(lib.index_topk_pool_workspace_size(B, P, K), dtype=torch.uint8,
                                            device=device)
            # the Full layer's top-k and pool as one call
            self.ws_gate = torch.zeros(lib.index_topk_pool_build_workspace_size(B, self.ld, K, P), dtype=torch.uint8,
                                       device=device)
        self.layers = []
        for li, mode in enumerate(wl.layers):
            d = wl.layer_inputs(li)
            L = {"mode": mode, "q": to_device_bits(d["q"], device), "swa": to_device_bits(d["swa"], device),
                 "swa_len": torch.from_numpy(d["swa_len"]).to(device),
                 "out": torch.zeros((B, wl.H, 512), dtype=torch.float32, device=device),
                 "lse": torch.zeros((B, wl.H), dtype=torch.float32, device=device)}
            if mode in ("full", "reindex"):
                L["q_idx"] = to_device_bits(d["q_idx"], device)
                L["w"] = torch.from_numpy(d["w"]).to(device)
                L["topk"] = torch.full((B, K), -1, dtype=torch.int32, device=device)
                L["scores"] = None
            if wl.fp8_window:  # the window rows in FP8, quantised once on the device
                L["swa8"] = torch.zeros((B, W, 512), dtype=torch.uint8, device=device)
                L["swa8_scale"] = torch.zeros((B, W), dtype=torch.uint8, device=device)
                lib.swa_fp8_write(L["swa"], L["swa8"], L["swa8_scale"])
            self.layers.append(L)
        self.new_latent = None

    # ------------------------------------------------------------- cache --
    def build_cache(self, rows_per_call: int = 1 << 16):
        """Write every sequence's entries (host-generated bf16 rows) into the cache."""
        self.new_latent, self.new_key, self.new_slot = _write_decode_cache(self.cache, self.wl, self.device,
                                                                           rows_per_call)

    def cache_bytes(self) -> int:
        return self.cache.nbytes()

    def replica(self) -> "DecodeStep":
        """The same step over a copy of the cache in other device memory (query
        inputs, outputs and workspaces are shared; run replicas one at a time)."""
        r = copy.copy(self)
        r.cache = self.cache.clone()
        return r

    # -------------------------------------------------------------- step --
    def run(self, keep_scores: bool = False, hook=None):
        """One decode step over the layer schedule (enqueued on the current stream).
        hook(phase, name), if given, is called with "start"/"end" around each call."""
        call = _caller(hook)
        latest = None
        for L in self.layers:
            mode = L["mode"]
            if mode == "full":
                call("fp4_cache_write", lib.fp4_cache_write, self.cache, self.new_latent, self.new_key,
                     self.new_slot)
            if mode == "reindex" and self.npool > 0:
                call("index_topk_pool", lib.index_topk_pool, self.cache, L["q_idx"], L["w"], self.n_visible,
                     self.pool, self.block_table, self.scores_pool, self.wl.K, L["topk"], self.ws_topk_pool)
                if keep_scores:
                    L["scores"] = self.scores_pool.clone()
                latest = L["topk"]
            elif mode in ("full", "reindex"):
                if mode == "full" and self.npool > 0 and self.fused_index:
                    # the gatekeeper layer: top-k and candidate pool from one scan
                    call("index_topk_pool_build", lib.index_topk_pool_build, self.cache, L["q_idx"], L["w"],
                         self.n_visible, self.block_table, self.scores, self.wl.K, L["topk"], self.npool, self.pool,
                         self.ws_gate)
                    if keep_scores:
                        L["scores"] = self.scores.clone()
                        L["pool"] = self.pool.clone()
                elif self.fused_index:
                    call("index_topk", lib.index_topk, self.cache, L["q_idx"], L["w"], self.n_visible,
                         self.block_table, self.scores, self.wl.K, L["topk"], self.ws_topk)
                    if keep_scores:
                        L["scores"] = self.scores.clone()
                else:
                    call("index_score", lib.index_score, self.cache, L["q_idx"], L["w"], self.n_visible,
                         self.block_table, self.scores)
                    if keep_scores:
                        L["scores"] = self.scores.clone()
                    call("topk_select", lib.topk_select, self.scores, self.n_visible, self.wl.K, L["topk"],
                         self.ws_topk)
                latest = L["topk"]
                if mode == "full" and self.npool > 0 and not self.fused_index:
                    call("index_pool_build", lib.index_pool_build, self.scores, self.n_visible, self.npool,
                         self.pool, self.ws_pool)
                    if keep_scores:
                        L["pool"] = self.pool.clone()
            if latest is None:
                raise ValueError("a reuse layer needs an earlier full or reindex layer")
            if self.wl.fp8_window:
                call("sparse_attn_decode_fp8win", lib.sparse_attn_decode_fp8win, self.cache, L["q"], latest,
                     self.block_table, L["swa8"], L["swa8_scale"], L["swa_len"], self.scale, L["out"], L["lse"],
                     self.ws_attn)
            else:
                call("sparse_attn_decode", lib.sparse_attn_decode, self.cache, L["q"], latest, self.block_table,
                     L["swa"], L["swa_len"], self.scale, L["out"], L["lse"], self.ws_attn)


def _write_decode_cache(cache, wl: Workload, device, rows_per_call: int):
    """Write every sequence's entries of a decode workload into `cache`; returns the
    newest entry of every sequence (latent, key, slot), which a Full layer rewrites
    each step."""
    last_lat, last_key, last_slot = [], [], []
    for b in range(wl.B):
        n = int(wl.n_entries[b])
        lat, key = wl.cache_rows(b, 0, n)
        slots = wl.slots(b, 0, n)
        for s in range(0, n, rows_per_call):
            e = min(n, s + rows_per_call)
            lib.fp4_cache_write(cache, to_device_bits(lat[s:e], device), to_device_bits(key[s:e], device),
                                torch.from_numpy(slots[s:e]).to(device))
        last_lat.append(lat[n - 1])
        last_key.append(key[n - 1])
        last_slot.append(slots[n - 1])
        del lat, key
    return (to_device_bits(np.stack(last_lat), device), to_device_bits(np.stack(last_key), device),
            torch.from_numpy(np.array(last_slot, np.int64)).to(device))


class ScheduleDecodeStep:
    """Device state for one decode token through a whole layer schedule with one
    cache per Full layer ("Résumé exécutif", CSA2 section: of 40 layers only four
    write a cache and the other 36 read their source's; every layer keeps its own
    query and window).  Window-only layers attend their window alone (k = 0)."""

    def __init__(self, sw: ScheduleWorkload, device="cuda", softmax_scale: float | None = None):
        self.wl = sw
        self.device = device
        self.scale = lib.default_softmax_scale() if softmax_scale is None else softmax_scale
        K, W, H = sw.K, sw.W, sw.H
        pooled = {sw.source(l) for l, md in enumerate(sw.modes) if md == "reindex"} if sw.npool > 0 else set()
        self.caches = {}
        for w in sw.writers():
            cw = sw.cache_workload(w)
            nv = cw.n_visible()
            ld = int(((int(nv.max()) + PAGE_SIZE - 1) // PAGE_SIZE) * PAGE_SIZE)
            C = {"wl": cw, "cache": lib.Cache(cw.num_slots, device),
                 "block_table": torch.from_numpy(cw.block_table()).to(device),
                 "n_visible": torch.from_numpy(nv).to(device), "ld": ld,
                 "scores": torch.zeros((1, ld), dtype=torch.float32, device=device),
                 "ws_topk": torch.zeros(lib.topk_select_workspace_size(1, ld, K), dtype=torch.uint8, device=device),
                 "pooled": w in pooled}
            if C["pooled"]:
                P = sw.npool
                C["pool"] = torch.full((1, P), -1, dtype=torch.int32, device=device)
                C["ws_pool"] = torch.zeros(lib.index_pool_build_workspace_size(1, ld, P), dtype=torch.uint8,
                                           device=device)
                C["scores_pool"] = torch.zeros((1, lib.POOL_BLOCK * P), dtype=torch.float32, device=device)
                C["ws_topk_pool"] = torch.zeros(lib.index_topk_pool_workspace_size(1, P, K), dtype=torch.uint8,
                                                device=device)
                C["ws_gate"] = torch.zeros(lib.index_topk_pool_build_workspace_size(1, ld, K, P), dtype=torch.uint8,
                                           device=device)
            self.caches[w] = C
        self.ws_attn = torch.zeros(max(lib.sparse_attn_decode_workspace_size(1, H, K, W),
                                       lib.sparse_attn_decode_workspace_size(1, H, 0, W)), dtype=torch.uint8,
                                   device=device)
        self.no_topk = torch.zeros((1, 0), dtype=torch.int32, device=device)
        qw = sw.query_workload()
        self.layers = []
        for li, mode in enumerate(sw.modes):
            d = qw.layer_inputs(li)
            L = {"mode": mode, "src": sw.source(li), "q": to_device_bits(d["q"], device),
                 "swa": to_device_bits(d["swa"], device), "swa_len": torch.from_numpy(d["swa_len"]).to(device),
                 "out": torch.zeros((1, H, 512), dtype=torch.float32, device=device),
                 "lse": torch.zeros((1, H), dtype=torch.float32, device=device)}
            if mode in ("full", "reindex"):
                L["q_idx"] = to_device_bits(d["q_idx"], device)
                L["w"] = torch.from_numpy(d["w"]).to(device)
                L["topk"] = torch.full((1, K), -1, dtype=torch.int32, device=device)
                L["scores"] = None
            self.layers.append(L)

    def build_cache(self, rows_per_call: int = 1 << 16):
        for C in self.caches.values():
            C["new"] = _write_decode_cache(C["cache"], C["wl"], self.device, rows_per_call)

    def cache_bytes(self) -> int:
        return sum(C["cache"].nbytes() for C in self.caches.values())

    def replica(self) -> "ScheduleDecodeStep":
        """The same step over copies of every cache (other buffers shared)."""
        r = copy.copy(self)
        r.caches = {w: dict(C, cache=C["cache"].clone()) for w, C in self.caches.items()}
        return r

    def run(self, keep_scores: bool = False, hook=None):
        """One decode token through every layer (enqueued on the current stream)."""
        call = _caller(hook)
        latest = {}
        any_cache = next(iter(self.caches.values()))
        K = self.wl.K
        for L in self.layers:
            mode = L["mode"]
            if mode == "swa":
                call("sparse_attn_decode", lib.sparse_attn_decode, any_cache["cache"], L["q"], self.no_topk,
                     any_cache["block_table"], L["swa"], L["swa_len"], self.scale, L["out"], L["lse"], self.ws_attn)
                continue
            C = self.caches[L["src"]]
            if mode == "full":
                lat, key, slot = C["new"]
                call("fp4_cache_write", lib.fp4_cache_write, C["cache"], lat, key, slot)
            if mode == "reindex" and C["pooled"]:
                call("index_topk_pool", lib.index_topk_pool, C["cache"], L["q_idx"], L["w"], C["n_visible"],
                     C["pool"], C["block_table"], C["scores_pool"], K, L["topk"], C["ws_topk_pool"])
                if keep_scores:
                    L["scores"] = C["scores_pool"].clone()
                latest[L["src"]] = L["topk"]
            elif mode == "full" and C["pooled"]:
                # the gatekeeper layer of a pooled cache: top-k and pool from one scan
                call("index_topk_pool_build", lib.index_topk_pool_build, C["cache"], L["q_idx"], L["w"],
                     C["n_visible"], C["block_table"], C["scores"], K, L["topk"], self.wl.npool, C["pool"],
                     C["ws_gate"])
                if keep_scores:
                    L["scores"] = C["scores"].clone()
                    L["pool"] = C["pool"].clone()
                latest[L["src"]] = L["topk"]
            elif mode in ("full", "reindex"):
                call("index_topk", lib.index_topk, C["cache"], L["q_idx"], L["w"], C["n_visible"],
                     C["block_table"], C["scores"], K, L["topk"], C["ws_topk"])
                if keep_scores:
                    L["scores"] = C["scores"].clone()
                latest[L["src"]] = L["topk"]
            if L["src"] not in latest:
                raise ValueError("a reuse layer needs an earlier full or reindex layer on its cache")
            call("sparse_attn_decode", lib.sparse_attn_decode, C["cache"], L["q"], latest[L["src"]],
                 C["block_table"], L["swa"], L["swa_len"], self.scale, L["out"], L["lse"], self.ws_attn)


class PrefillStep:
    """Device state for a prefill chunk: a cached prefix, then one chunk step that
    writes the chunk's entries, scores every query over its causally visible
    entries, selects per-query top-k and attends with per-query windows."""

    def __init__(self, wl: Workload, device="cuda", softmax_scale: float | None = None):
        assert wl.kind == "prefill"
        self.wl = wl
        self.device = device
        self.scale = lib.default_softmax_scale() if softmax_scale is None else softmax_scale
        T, K, W = wl.chunk, wl.K, wl.W
        self.cache = lib.Cache(wl.num_slots, device)
        bt = wl.block_table()
        self.block_table2d = torch.from_numpy(bt).to(device)
        self.block_table = self.block_table2d[0].contiguous()
        nv = wl.n_visible()
        self.n_visible = torch.from_numpy(nv).to(device)
        self.seq_of_query = torch.zeros(T, dtype=torch.int32, device=device)
        self.ld = int(((int(nv.max()) + PAGE_SIZE - 1) // PAGE_SIZE) * PAGE_SIZE)
        self.scores = torch.zeros((T, self.ld), dtype=torch.float32, device=device)
        self.topk = torch.full((T, K), -1, dtype=torch.int32, device=device)
        self.ws_topk = torch.zeros(lib.topk_select_workspace_size(T, self.ld, K), dtype=torch.uint8, device=device)
        self.ws_attn = torch.zeros(max(256, lib.sparse_attn_prefill_chunk_workspace_size(T, wl.H, K, W)),
                                   dtype=torch.uint8, device=device)
        d = wl.layer_inputs(0)
        self.q = to_device_bits(d["q"], device)
        self.q_idx = to_device_bits(d["q_idx"], device)
        self.w = torch.from_numpy(d["w"]).to(device)
        self.swa = to_device_bits(d["swa"], device)
        self.swa_first_valid = int(d["swa_first_valid"])
        self.out = torch.zeros((T, wl.H, 512), dtype=torch.float32, device=device)
        self.lse = torch.zeros((T, wl.H), dtype=torch.float32, device=device)

    def build_cache(self, rows_per_call: int = 1 << 16):
        wl = self.wl
        n = int(wl.n_entries[0])
        nc = wl.n_chunk_entries
        lat, key = wl.cache_rows(0, 0, n + nc)
        slots = wl.slots(0, 0, n + nc)
        for s in range(0, n, rows_per_call):
            e = min(n, s + rows_per_call)
            lib.fp4_cache_write(self.cache, to_device_bits(lat[s:e], self.device),
                                to_device_bits(key[s:e], self.device), torch.from_numpy(slots[s:e]).to(self.device))
        self.chunk_latent = to_device_bits(lat[n:n + nc], self.device)
        self.chunk_key = to_device_bits(key[n:n + nc], self.device)
        self.chunk_slot = torch.from_numpy(slots[n:n + nc]).to(self.device)

    def cache_bytes(self) -> int:
        return self.cache.nbytes()

    def replica(self) -> "PrefillStep":
        """The same chunk step over a copy of the cache (other buffers shared)."""
        r = copy.copy(self)
        r.cache = self.cache.clone()
        return r

    def run(self, hook=None):
        wl = self.wl
        call = _caller(hook)
        call("fp4_cache_write", lib.fp4_cache_write, self.cache, self.chunk_latent, self.chunk_key, self.chunk_slot)
        call("index_score", lib.index_score, self.cache, self.q_idx, self.w, self.n_visible, self.block_table2d,
             self.scores, seq_of_query=self.seq_of_query)
        call("topk_select", lib.topk_select, self.scores, self.n_visible, wl.K, self.topk, self.ws_topk)
        call("sparse_attn_prefill_chunk", lib.sparse_attn_prefill_chunk, self.cache, self.q, self.topk,
             self.block_table, int(wl.ctx[0]), self.swa, self.swa_first_valid, wl.W, self.scale, self.out, self.lse,
             self.ws_attn)


def _caller(hook):
    def call(name, fn, *a, **kw):
        if hook is not None:
            hook("start", name)
        fn(*a, **kw)
        if hook is not None:
            hook("end", name)

    return call
