"""Seeded synthetic workloads for the CSA2 FP4-cache step.

This module only draws random inputs and lays out page tables; it holds none of
the method's arithmetic (no quantisation, scoring, selection or attention), so
both the GPU path and the CPU oracle can consume the very same arrays.

Every tensor comes from its own PCG64 stream keyed by (config, layer, tensor), so
an array never depends on the order in which others were generated.  Normals are
drawn in float32 and rounded to bf16 (round-to-nearest-even) by torch; indexer
head weights are U[0, 1) float32.

The shapes stand in for the 1M-token agent sessions the pages describe
("DeepSeek-V4.1-Flash, expliqué pas à pas": intro on agent workloads and the
1,048,576-token context; "Résumé exécutif": result table).  No trace, dataset or
trained weight is used.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Sequence

import numpy as np

LATENT_DIM = 512
INDEX_DIM = 128
PAGE_SIZE = 64

# tensor ids for the per-tensor random streams
_T_LATENT, _T_IDXKEY, _T_Q, _T_QIDX, _T_W, _T_SWA, _T_CTX, _T_PAGES, _T_OUTL_LAT, _T_OUTL_IDX = range(10)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One configuration of the step.

    kind      "decode" (one query token per sequence) or "prefill" (a chunk of T
              query tokens of one sequence).
    ctx       context tokens per sequence (decode) / prefix tokens (prefill).
    m         tokens per compressed entry (disjoint groups).
    layers    layer modes of one step, e.g. ("full",) or ("full", "reuse", ...).
    npool     0: Reindex layers rescan the whole cache.  > 0: the step's Full layer
              turns its scores into a candidate pool of npool blocks of 8
              consecutive entries, and the Reindex layers score and select inside
              it ("DeepSeek V4.1 Flash et le cerveau divisé", memory section: about
              16,000 positions at 1M entries, i.e. 2048 blocks).
    swa_replay prefill only: the chunk is a bounded replay of the prompt's last
              tokens, and its sliding window starts at the replay's first token s,
              so query t sees window tokens max(s, t - W + 1) .. t ("DeepSeek-V4.1-
              Flash, expliqué pas à pas", bounded SWA replay in the on-disk cache
              chapter; the interval's formula is lost there, this is its plain
              reading).
    fp8_window decode only: every layer's window rows are stored in FP8 ("DeepSeek-
              V4.1-Flash, expliqué pas à pas", FP4 KV cache section) and attended
              from there; the rows are the same seeded bf16 rows, quantised once.
    """

    name: str
    cfg_id: int
    kind: str
    B: int
    ctx: tuple
    H: int
    Hi: int
    K: int
    W: int = 128
    m: int = 2
    layers: tuple = ("full",)
    outliers: bool = False
    paged_random: bool = False
    chunk: int = 0  # prefill: new query tokens
    seed: int = 0
    npool: int = 0  # decode: >0 -> Reindex layers scan a candidate pool of npool blocks of 8 entries
    swa_replay: bool = False  # prefill: the window starts at the chunk's first token (bounded replay)
    fp8_window: bool = False  # decode: window rows kept in FP8 (E4M3FN, one E8M0 scale per row)

    # ------------------------------------------------------------ geometry --
    @property
    def n_entries(self) -> np.ndarray:
        """Compressed entries per sequence in the cache before the step."""
        return np.array([c // self.m for c in self.ctx], np.int64)

    @property
    def n_chunk_entries(self) -> int:
        return self.chunk // self.m

    def pages_per_seq(self) -> np.ndarray:
        total = self.n_entries + (self.n_chunk_entries if self.kind == "prefill" else 0)
        return np.array([math.ceil(int(n) / PAGE_SIZE) for n in total], np.int64)

    @property
    def max_pages(self) -> int:
        return int(self.pages_per_seq().max())

    @property
    def num_slots(self) -> int:
        return int(self.pages_per_seq().sum()) * PAGE_SIZE

    def rng(self, layer: int, tensor: int) -> np.random.Generator:
        return np.random.Generator(np.random.PCG64(np.random.SeedSequence(self.seed,
                                                                         spawn_key=(self.cfg_id, layer, tensor))))

    # -------------------------------------------------------- page tables --
    def block_table(self) -> np.ndarray:
        """int32 [B, max_pages]: logical page -> physical page.  Identity packing
        (sequence after sequence) unless paged_random, where the physical pages
        are a seeded permutation.  Unused tail entries hold page 0."""
        pps = self.pages_per_seq()
        total = int(pps.sum())
        phys = np.arange(total, dtype=np.int64)
        if self.paged_random:
            phys = self.rng(0, _T_PAGES).permutation(total)
        bt = np.zeros((self.B, self.max_pages), np.int32)
        off = 0
        for b in range(self.B):
            bt[b, :pps[b]] = phys[off:off + pps[b]]
            off += int(pps[b])
        return bt

    def slots(self, b: int, first: int, count: int) -> np.ndarray:
        """Physical slots of logical entries first .. first+count-1 of sequence b."""
        bt = self.block_table()
        j = np.arange(first, first + count, dtype=np.int64)
        return bt[b, j // PAGE_SIZE].astype(np.int64) * PAGE_SIZE + j % PAGE_SIZE

    # ------------------------------------------------------------ tensors --
    def _normal_bf16(self, layer: int, tensor: int, shape, outlier_channels=None) -> np.ndarray:
        x = self.rng(layer, tensor).standard_normal(shape, dtype=np.float32)
        if outlier_channels is not None:
            x[..., outlier_channels] *= np.float32(8.0)
        return to_bf16_bits(x)

    def outlier_channels(self):
        """1% of channels scaled x8 (a fixed set per family, drawn once from the seed)."""
        if not self.outliers:
            return None, None
        lat = np.sort(self.rng(0, _T_OUTL_LAT).choice(LATENT_DIM, round(0.01 * LATENT_DIM), replace=False))
        idx = np.sort(self.rng(0, _T_OUTL_IDX).choice(INDEX_DIM, round(0.01 * INDEX_DIM), replace=False))
        return lat, idx

    def cache_rows(self, b: int, first: int, count: int):
        """bf16 latent [count, 512] and indexer key [count, 128] for logical entries
        first .. first+count-1 of sequence b (streams keyed by sequence, drawn whole
        and sliced so any sub-range is consistent)."""
        total = int(self.n_entries[b]) + (self.n_chunk_entries if self.kind == "prefill" else 0)
        lat_ch, idx_ch = self.outlier_channels()
        lat = self._normal_bf16(1000 + b, _T_LATENT, (total, LATENT_DIM), lat_ch)
        key = self._normal_bf16(1000 + b, _T_IDXKEY, (total, INDEX_DIM), idx_ch)
        return lat[first:first + count], key[first:first + count]

    def n_queries(self) -> int:
        return self.B if self.kind == "decode" else self.chunk

    def layer_inputs(self, layer: int) -> dict:
        """Per-layer query-side inputs: q [nq, H, 512], q_idx [nq, Hi, 128],
        w [nq, Hi] (float32 U[0,1)), window rows."""
        nq = self.n_queries()
        lat_ch, _ = self.outlier_channels()
        d = {
            "q": self._normal_bf16(layer, _T_Q, (nq, self.H, LATENT_DIM)),
            "q_idx": self._normal_bf16(layer, _T_QIDX, (nq, self.Hi, INDEX_DIM)),
            "w": self.rng(layer, _T_W).random((nq, self.Hi), dtype=np.float32),
        }
        if self.kind == "decode":
            d["swa"] = self._normal_bf16(layer, _T_SWA, (self.B, self.W, LATENT_DIM), lat_ch)
            d["swa_len"] = np.full(self.B, self.W, np.int32)
        else:
            d["swa"] = self._normal_bf16(layer, _T_SWA, (self.W - 1 + self.chunk, LATENT_DIM), lat_ch)
            # window row r holds token ctx - (W - 1) + r; rows below swa_first_valid
            # do not exist (before the prompt, or before a replay's first token)
            d["swa_first_valid"] = self.W - 1 if self.swa_replay else max(0, self.W - 1 - int(self.ctx[0]))
        return d

    def n_visible(self) -> np.ndarray:
        """Entries visible to each query.  Decode: all entries of its sequence.
        Prefill: query i at token t = P + i sees entry j iff its m tokens are all
        at or before t, i.e. j < (t + 1) // m."""
        if self.kind == "decode":
            return self.n_entries.astype(np.int32)
        t = int(self.ctx[0]) + np.arange(self.chunk, dtype=np.int64)
        return ((t + 1) // self.m).astype(np.int32)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even (torch)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def ragged_contexts(cfg_id: int, B: int, lo: int, hi: int, seed: int = 0) -> tuple:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(cfg_id, 0, _T_CTX))))
    return tuple(int(c) for c in rng.integers(lo, hi + 1, size=B))


@dataclasses.dataclass(frozen=True)
class ScheduleWorkload:
    """One decode token through a whole layer schedule with several caches.

    modes[l] is "swa" (attention over the layer's own window only), "full" (writes
    its own cache, scores and selects), "reindex" (scores and selects on the cache
    of the latest Full layer) or "reuse" (attends with the latest indices on that
    cache).  m[l] is the tokens per entry of the cache layer l reads.  Each Full
    layer's cache has its own seeded rows (cache_workload); the query-side inputs of
    every layer come from query_workload().layer_inputs(l).  npool > 0: Reindex
    layers score and select inside the candidate pool built from their Full
    layer's scores.
    """

    name: str
    cfg_id: int
    ctx: int
    H: int
    Hi: int
    K: int
    W: int = 128
    modes: tuple = ()
    m: tuple = ()
    npool: int = 0
    seed: int = 0
    kind: str = "schedule"
    B: int = 1

    @property
    def layers(self) -> tuple:
        return self.modes

    def writers(self) -> list:
        return [i for i, md in enumerate(self.modes) if md == "full"]

    def source(self, layer: int):
        """The Full layer whose cache `layer` reads (None for a window-only layer)."""
        if self.modes[layer] == "swa":
            return None
        w = [i for i in self.writers() if i <= layer]
        if not w:
            raise ValueError(f"layer {layer} reads a cache before any Full layer")
        return w[-1]

    def cache_workload(self, writer: int) -> Workload:
        """The single-cache workload that lays out and seeds the cache of Full layer
        `writer` (config id 100 * cfg_id + writer)."""
        return Workload(f"{self.name}_cache{writer}", 100 * self.cfg_id + writer, "decode", B=1, ctx=(self.ctx,),
                        H=self.H, Hi=self.Hi, K=self.K, W=self.W, m=self.m[writer], layers=("full",), seed=self.seed)

    def query_workload(self) -> Workload:
        """Per-layer query-side inputs (q, q_idx, w, window), keyed by layer."""
        return Workload(self.name, self.cfg_id, "decode", B=1, ctx=(self.ctx,), H=self.H, Hi=self.Hi, K=self.K,
                        W=self.W, m=2, layers=self.modes, seed=self.seed)


def published_schedule():
    """The published 40-layer allocation ("DeepSeek-V4.1-Flash, expliqué pas à pas",
    CSA2 mode table; "Résumé exécutif", CSA2 section): encoder layers 0-1 window
    only, then 3 groups of [Full + 5 Reuse] with m = 2 (writers 2, 8, 14); decoder 5
    groups of 4 with m = 1: [Full + 3 Reuse] (writer 20), then 4 x [Reindex + 3 Reuse].
    Returns (modes, m) per layer."""
    modes = ["swa", "swa"] + ["full"] + ["reuse"] * 5 + ["full"] + ["reuse"] * 5 + ["full"] + ["reuse"] * 5
    m = [0, 0] + [2] * 18
    modes += ["full"] + ["reuse"] * 3
    for _ in range(4):
        modes += ["reindex"] + ["reuse"] * 3
    m += [1] * 20
    return tuple(modes), tuple(m)


C4_LAYERS = ("full", "reuse", "reindex", "reuse", "reindex", "reuse", "reindex", "reuse", "reindex", "reuse")

WORKLOADS = {
    "tiny_decode": Workload("tiny_decode", 1, "decode", B=1, ctx=(4096,), H=16, Hi=16, K=256),
    "decode_131k": Workload("decode_131k", 2, "decode", B=1, ctx=(131072,), H=64, Hi=64, K=2048, outliers=True),
    "ragged_decode_32": Workload("ragged_decode_32", 3, "decode", B=32, ctx=ragged_contexts(3, 32, 8192, 65536),
                                 H=64, Hi=64, K=2048, paged_random=True),
    "decode_1m_10layer": Workload("decode_1m_10layer", 4, "decode", B=1, ctx=(1048576,), H=64, Hi=64, K=2048,
                                  layers=C4_LAYERS),
    # eight 1M-token sessions decoding together: the 10-layer step at batch 8
    "decode_1m_10layer_b8": Workload("decode_1m_10layer_b8", 8, "decode", B=8, ctx=(1048576,) * 8, H=64, Hi=64,
                                     K=2048, layers=C4_LAYERS),
    # the same inputs as decode_1m_10layer; the four Reindex layers use the pool
    "decode_1m_10layer_pool": Workload("decode_1m_10layer_pool", 4, "decode", B=1, ctx=(1048576,), H=64, Hi=64,
                                       K=2048, layers=C4_LAYERS, npool=2048),
    "prefill_chunk_4096": Workload("prefill_chunk_4096", 5, "prefill", B=1, ctx=(262144,), H=64, Hi=64, K=2048,
                                   chunk=4096),
    # bounded replay of the last 128 tokens of a 1,048,576-token prompt: every query
    # has its causal top-K over the whole cache; the window restarts at the replay
    # the same inputs as decode_1m_10layer with every layer's window in FP8
    "decode_1m_10layer_fp8win": Workload("decode_1m_10layer_fp8win", 4, "decode", B=1, ctx=(1048576,), H=64,
                                         Hi=64, K=2048, layers=C4_LAYERS, fp8_window=True),
    # one token through all 40 layers at 1,048,576 tokens: three m = 2 encoder
    # caches (524,288 entries each) and the m = 1 decoder cache (1,048,576 entries),
    # 0.87 GiB in all; the decoder's Reindex layers select inside 2048-block pools
    "decode_1m_schedule": ScheduleWorkload("decode_1m_schedule", 7, 1048576, H=64, Hi=64, K=2048,
                                           modes=published_schedule()[0], m=published_schedule()[1], npool=2048),
    "replay_128_1m": Workload("replay_128_1m", 6, "prefill", B=1, ctx=(1048576 - 128,), H=64, Hi=64, K=2048,
                              chunk=128, swa_replay=True),
}


def small_variant(wl: Workload, ctx: Sequence[int], chunk: int | None = None, name: str | None = None,
                  **kw) -> Workload:
    """Same recipe at a reduced size (parity cases the oracle finishes quickly)."""
    return dataclasses.replace(wl, name=name or (wl.name + "_small"), ctx=tuple(int(c) for c in ctx),
                               B=len(ctx) if wl.kind == "decode" else 1,
                               chunk=wl.chunk if chunk is None else chunk, **kw)
