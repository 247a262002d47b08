// topk_select.hip -- per-query top-k over fp32 scores, ties to the lower index,
// output in ascending index order.
//
// Source: "DeepSeek-V4.1-Flash, expliqué pas à pas", attention forms and CSA2 section:
// the indexer keeps only the best-scoring entries (top-k).
//
// Scores become order-preserving 32-bit keys; the selection is the set of the k
// largest 64-bit composites (key << 32) | (0xFFFFFFFF - index), which are all
// distinct, so the answer is unique.  Two launches over a grid of
// (chunks of 4096 consecutive scores) x (queries):
//   1. hist   : 4096-bin histogram of the top 12 key bits, added to a per-query
//               global histogram.
//   2. select : every workgroup finds the threshold bin b* (where the running count
//               from the top reaches k) and appends the composites of its entries in
//               bins >= b* -- the fewer than k entries above b* plus the b*
//               candidates -- in index order to a per-query list, recording
//               (offset, count) for its chunk.  The last workgroup of a query
//               (arrival counter) gathers the chunks' lists in chunk order,
//               radix-selects the boundary composite among the b* candidates and
//               keeps the listed entries at or above it with an ordered compaction,
//               so the k indices come out ascending without a sort.  It then clears
//               the histogram and counters, leaving the workspace zero for the next
//               call.  If the list overflows, the last workgroup selects from the
//               score row itself.
// Cross-workgroup data goes through device-coherent (sc1) stores and loads; a
// workgroup waits for its stores to complete before it announces them with the
// arrival atomic, so no cache-wide write-back or invalidate is needed.
#include "common.hpp"
#include "host_common.hpp"

namespace csa2 {

constexpr int kBins = 4096;  // top 12 key bits
constexpr int kBinShift = 20;
constexpr int kThreads = 512;
constexpr int kPer = 8;  // consecutive scores per thread
constexpr int kChunk = kThreads * kPer;
constexpr int kListCap = 8192;   // listed entries per query resolved in LDS
constexpr int kMaxChunksFast = 2048;  // chunk bookkeeping in LDS (rows up to 8M entries)

struct TopkCtl {
  uint32_t listed;  // entries appended to the list so far
  uint32_t arrive;
  uint32_t pad[14];
};
static_assert(sizeof(TopkCtl) == 64, "TopkCtl is 64 bytes");

struct TopkWs {
  TopkCtl* ctl;              // [nq]
  uint32_t* hist;            // [nq][kBins]
  unsigned long long* info;  // [nq][nchunk]: (list offset << 32) | count of the chunk
  unsigned long long* list;  // [nq][kListCap]: composites of the entries in bins >= b*
};

__host__ __device__ inline size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

__host__ __device__ inline size_t ws_bytes_for(int nq, long long nchunk) {
  return align_up(sizeof(TopkCtl) * (size_t)nq) + align_up(sizeof(uint32_t) * kBins * (size_t)nq) +
         align_up(sizeof(unsigned long long) * (size_t)nchunk * (size_t)nq) +
         align_up(sizeof(unsigned long long) * kListCap * (size_t)nq);
}

__host__ __device__ inline TopkWs carve(void* base, int nq, long long nchunk) {
  unsigned char* p = (unsigned char*)base;
  TopkWs w;
  w.ctl = (TopkCtl*)p;
  p += align_up(sizeof(TopkCtl) * (size_t)nq);
  w.hist = (uint32_t*)p;
  p += align_up(sizeof(uint32_t) * kBins * (size_t)nq);
  w.info = (unsigned long long*)p;
  p += align_up(sizeof(unsigned long long) * (size_t)nchunk * (size_t)nq);
  w.list = (unsigned long long*)p;
  return w;
}

CSA2_DEV unsigned long long composite(uint32_t key, uint32_t idx) {
  return ((unsigned long long)key << 32) | (unsigned long long)(0xFFFFFFFFu - idx);
}
CSA2_DEV uint32_t index_of(unsigned long long c) { return 0xFFFFFFFFu - (uint32_t)(c & 0xFFFFFFFFull); }

// Device-coherent (agent-scope) accesses: on gfx950 these are plain loads/stores
// with the sc1 bit.
template <typename T>
CSA2_DEV void st_agent(T* p, T v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
template <typename T>
CSA2_DEV T ld_agent(T* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
CSA2_DEV void wait_all_memory() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// This thread's kPer consecutive keys of a chunk, all loads in flight together.
CSA2_DEV void load_keys(const float* __restrict__ row, int64_t base, int64_t n, uint32_t (&key)[kPer]) {
  float v[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int64_t j = base + (int64_t)threadIdx.x * kPer + i;
    v[i] = (j < n) ? row[j] : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) key[i] = score_key(v[i]);
}

// Block-wide inclusive scan (kThreads threads) of one value per thread: wave scans
// and one LDS exchange.  wsum: kThreads/64 u32 of LDS.
CSA2_DEV uint32_t block_inclusive_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  constexpr int nw = kThreads / 64;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  if (lane == 63) wsum[wid] = v;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < nw; ++w) {
    const uint32_t s = wsum[w];
    before += (w < wid) ? s : 0u;
    all += s;
  }
  __syncthreads();
  *total = all;
  return v + before;
}

// Histogram h[0..kBins) in LDS: digit D with count(digit > D) < need <= count(digit >= D).
// Returns D; *above = count(digit > D).  Requires 1 <= need <= total count.
CSA2_DEV int find_digit(const uint32_t* h, uint32_t need, uint32_t* wsum, int* dig_s, uint32_t* above_s,
                        uint32_t* above) {
  constexpr int per = kBins / kThreads;
  const int t = threadIdx.x;
  // thread t owns bins [kBins - per*(t+1), kBins - per*t): threads in order walk the
  // bins from the top down
  const int hi = kBins - per * t;
  uint32_t s = 0;
#pragma unroll
  for (int i = 1; i <= per; ++i) s += h[hi - i];
  uint32_t total;
  const uint32_t incl = block_inclusive_scan(s, wsum, &total);  // count in bins >= hi - per
  const uint32_t excl = incl - s;                                // count in bins >= hi
  if (excl < need && need <= incl) {
    uint32_t acc = excl;
    for (int i = 1; i <= per; ++i) {
      const uint32_t c = h[hi - i];
      if (acc + c >= need) {
        *dig_s = hi - i;
        *above_s = acc;
        break;
      }
      acc += c;
    }
  }
  __syncthreads();
  const int D = *dig_s;
  *above = *above_s;
  __syncthreads();
  return D;
}

// ---------------------------------------------------------------- kernel 1 --
__global__ __launch_bounds__(kThreads) void topk_hist_kernel(const float* __restrict__ scores, int64_t ld,
                                                             const int32_t* __restrict__ n_visible, int k,
                                                             TopkWs ws) {
  __shared__ uint32_t lh[kBins];
  const int q = blockIdx.y, tid = threadIdx.x;
  const int64_t n = n_visible[q];
  const int64_t base = (int64_t)blockIdx.x * kChunk;
  if (n <= k || base >= n) return;
  for (int b = tid; b < kBins; b += kThreads) lh[b] = 0;
  uint32_t key[kPer];
  load_keys(scores + (int64_t)q * ld, base, n, key);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    if (base + (int64_t)tid * kPer + i < n) atomicAdd(&lh[key[i] >> kBinShift], 1u);
  __syncthreads();
  uint32_t* gh = ws.hist + (size_t)q * kBins;
  for (int b = tid; b < kBins; b += kThreads) {
    const uint32_t c = lh[b];
    if (c) atomicAdd(&gh[b], c);
  }
}

struct SelectSmem {
  uint32_t h[kBins];
  unsigned long long list[kListCap];
  uint32_t cpos[kMaxChunksFast];  // chunk -> first position in the ordered list
  uint32_t wsum[kThreads / 64];
  uint32_t above_s, base_s;
  int dig_s, is_last;
  unsigned long long min_s;
};

// Candidates of bin b*: the listed entries in LDS, or (slow path) the score row.
struct LdsCands {
  const unsigned long long* c;
  int n;
  uint32_t bstar;
  template <typename F>
  CSA2_DEV void each(F&& f) const {
    for (int i = threadIdx.x; i < n; i += kThreads) {
      const unsigned long long x = c[i];
      if ((uint32_t)(x >> (32 + kBinShift)) == bstar) f(x);
    }
  }
};
struct RowCands {
  const float* row;
  int64_t n;
  uint32_t bstar;
  template <typename F>
  CSA2_DEV void each(F&& f) const {
    for (int64_t i = threadIdx.x; i < n; i += kThreads) {
      const uint32_t key = score_key(row[i]);
      if ((key >> kBinShift) == bstar) f(composite(key, (uint32_t)i));
    }
  }
};

// need-th largest composite among the candidates (all share the top 12 key bits):
// 12-bit digits of composite bits 51..0, stopping as soon as every candidate left
// under the chosen prefix is selected.
template <typename Src>
CSA2_DEV unsigned long long select_boundary(const Src& src, uint32_t need, uint32_t bstar, SelectSmem& sm) {
  const int tid = threadIdx.x;
  unsigned long long prefix = bstar;  // composite >> hi
  int hi = 52;
  while (true) {
    const int width = hi >= 12 ? 12 : hi;
    const int lo = hi - width;
    for (int b = tid; b < kBins; b += kThreads) sm.h[b] = 0;
    __syncthreads();
    src.each([&](unsigned long long x) {
      if ((x >> hi) == prefix) atomicAdd(&sm.h[(int)((x >> lo) & ((1ull << width) - 1))], 1u);
    });
    __syncthreads();
    uint32_t above;
    const int D = find_digit(sm.h, need, sm.wsum, &sm.dig_s, &sm.above_s, &above);
    const uint32_t cnt = sm.h[D];
    __syncthreads();
    need -= above;
    prefix = (prefix << width) | (unsigned long long)D;
    hi = lo;
    if (hi == 0) return prefix;
    if (cnt == need) {  // all of them are in: the boundary is their minimum
      if (tid == 0) sm.min_s = ~0ull;
      __syncthreads();
      src.each([&](unsigned long long x) {
        if ((x >> hi) == prefix) atomicMin(&sm.min_s, x);
      });
      __syncthreads();
      const unsigned long long m = sm.min_s;
      __syncthreads();
      return m;
    }
  }
}

// ---------------------------------------------------------------- kernel 2 --
__global__ __launch_bounds__(kThreads) void topk_select_kernel(const float* __restrict__ scores, int64_t ld,
                                                               const int32_t* __restrict__ n_visible, int k,
                                                               int32_t* __restrict__ topk_idx, TopkWs ws,
                                                               int nchunk) {
  __shared__ SelectSmem sm;
  const int q = blockIdx.y, tid = threadIdx.x;
  const int64_t n = n_visible[q];
  const int64_t base = (int64_t)blockIdx.x * kChunk;
  int32_t* out = topk_idx + (int64_t)q * k;
  if (n <= k) {  // everything visible is selected, then -1 padding
    for (int64_t i = base + tid; i < min(base + (int64_t)kChunk, n); i += kThreads) out[i] = (int32_t)i;
    if (blockIdx.x == 0)
      for (int64_t i = n + tid; i < k; i += kThreads) out[i] = -1;
    return;
  }
  if (base >= n) return;
  const int nch = (int)((n + kChunk - 1) / kChunk);
  TopkCtl* ctl = ws.ctl + q;
  uint32_t* gh = ws.hist + (size_t)q * kBins;
  unsigned long long* info = ws.info + (size_t)q * nchunk;
  unsigned long long* glist = ws.list + (size_t)q * kListCap;
  const float* row = scores + (int64_t)q * ld;

  uint32_t key[kPer];
  load_keys(row, base, n, key);
  for (int b = tid; b < kBins; b += kThreads) sm.h[b] = gh[b];
  if (tid == 0) sm.dig_s = 0;
  __syncthreads();
  uint32_t above_b;
  const uint32_t bstar = (uint32_t)find_digit(sm.h, (uint32_t)k, sm.wsum, &sm.dig_s, &sm.above_s, &above_b);

  // list this chunk's entries in bins >= b*, in index order
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    if (base + (int64_t)tid * kPer + i < n && (key[i] >> kBinShift) >= bstar) m |= 1u << i;
  uint32_t tot;
  const uint32_t off = block_inclusive_scan((uint32_t)__popc(m), sm.wsum, &tot) - (uint32_t)__popc(m);
  if (tid == 0) {
    const uint32_t r = tot ? atomicAdd(&ctl->listed, tot) : 0u;
    sm.base_s = r;
    st_agent(info + blockIdx.x, ((unsigned long long)r << 32) | tot);
  }
  __syncthreads();
  uint32_t p = sm.base_s + off;
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    if (m & (1u << i)) {
      if (p < (uint32_t)kListCap)
        st_agent(glist + p, composite(key[i], (uint32_t)(base + (int64_t)tid * kPer + i)));
      ++p;
    }
  wait_all_memory();  // this workgroup's list entries are visible device-wide
  __syncthreads();
  if (tid == 0) sm.is_last = (atomicAdd(&ctl->arrive, 1u) == (uint32_t)(nch - 1));
  __syncthreads();
  if (!sm.is_last) return;

  // ---- last workgroup of this query: every list entry is in place
  const uint32_t listed = ld_agent(&ctl->listed);
  const uint32_t need = (uint32_t)k - above_b;  // 1 <= need <= entries in b*
  if (listed <= (uint32_t)kListCap && nch <= kMaxChunksFast) {
    // chunk c's entries go to positions cpos[c] .. of the chunk-ordered list
    uint32_t carry = 0;
    for (int c0 = 0; c0 < nch; c0 += kThreads) {
      const int c = c0 + tid;
      const uint32_t cnt = (c < nch) ? (uint32_t)ld_agent(info + c) : 0u;
      uint32_t t2;
      const uint32_t incl = block_inclusive_scan(cnt, sm.wsum, &t2);
      if (c < nch) sm.cpos[c] = carry + incl - cnt;
      carry += t2;
    }
    __syncthreads();
    for (int c = tid; c < nch; c += kThreads) {
      const unsigned long long inf = ld_agent(info + c);
      const uint32_t src0 = (uint32_t)(inf >> 32), cn = (uint32_t)inf, dst0 = sm.cpos[c];
      uint32_t i = 0;
      for (; i + 4 <= cn; i += 4) {  // four loads in flight at a time
        const unsigned long long a0 = ld_agent(glist + src0 + i), a1 = ld_agent(glist + src0 + i + 1);
        const unsigned long long a2 = ld_agent(glist + src0 + i + 2), a3 = ld_agent(glist + src0 + i + 3);
        sm.list[dst0 + i] = a0;
        sm.list[dst0 + i + 1] = a1;
        sm.list[dst0 + i + 2] = a2;
        sm.list[dst0 + i + 3] = a3;
      }
      for (; i < cn; ++i) sm.list[dst0 + i] = ld_agent(glist + src0 + i);
    }
    __syncthreads();
    const LdsCands src{sm.list, (int)listed, bstar};
    const unsigned long long boundary = select_boundary(src, need, bstar, sm);
    // ordered compaction of the listed entries at or above the boundary
    constexpr int per = kListCap / kThreads;
    uint32_t keep = 0;
#pragma unroll
    for (int i = 0; i < per; ++i) {
      const int e = tid * per + i;
      if (e < (int)listed && sm.list[e] >= boundary) keep |= 1u << i;
    }
    uint32_t total;
    uint32_t o = block_inclusive_scan((uint32_t)__popc(keep), sm.wsum, &total) - (uint32_t)__popc(keep);
#pragma unroll
    for (int i = 0; i < per; ++i)
      if (keep & (1u << i)) {
        if (o < (uint32_t)k) out[o] = (int32_t)index_of(sm.list[tid * per + i]);
        ++o;
      }
  } else {
    // slow path (list overflow or very long rows): boundary from the score row, then
    // an ordered scan of the row, kThreads entries per round
    const RowCands src{row, n, bstar};
    const unsigned long long boundary = select_boundary(src, need, bstar, sm);
    uint32_t written = 0;
    for (int64_t r0 = 0; r0 < n; r0 += kThreads) {
      const int64_t i = r0 + tid;
      bool keep = false;
      if (i < n) {
        const uint32_t key = score_key(row[i]);
        const uint32_t bin = key >> kBinShift;
        keep = bin > bstar || (bin == bstar && composite(key, (uint32_t)i) >= boundary);
      }
      uint32_t t2;
      const uint32_t incl = block_inclusive_scan(keep ? 1u : 0u, sm.wsum, &t2);
      if (keep && written + incl - 1 < (uint32_t)k) out[written + incl - 1] = (int32_t)i;
      written += t2;
    }
  }
  // leave the workspace clean for the next call
  for (int b = tid; b < kBins; b += kThreads) gh[b] = 0u;
  if (tid == 0) {
    ctl->listed = 0u;
    ctl->arrive = 0u;
  }
}

}  // namespace csa2

using namespace csa2;

extern "C" size_t topk_select_workspace_size(int32_t nq, int64_t ld, int32_t k) {
  (void)k;
  if (nq <= 0) return 256;
  const long long nchunk = ld > 0 ? (ld + kChunk - 1) / kChunk : 1;
  return ws_bytes_for(nq, nchunk);
}

extern "C" int topk_select(const float* scores, int64_t ld, const int32_t* n_visible, int32_t nq, int32_t k,
                           int32_t* topk_idx, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (nq < 0 || ld < 0 || k < 1 || k > CSA2_MAX_K) return CSA2_ERR_SHAPE;
  if (ld >= ((int64_t)1 << 31)) return CSA2_ERR_SHAPE;
  if (nq == 0) return CSA2_OK;
  if (!n_visible || !topk_idx || (ld > 0 && !scores)) return CSA2_ERR_NULL;
  if (!ws || ws_bytes < topk_select_workspace_size(nq, ld, k)) return CSA2_ERR_WORKSPACE;
  const long long nchunk = ld > 0 ? (ld + kChunk - 1) / kChunk : 1;
  const long long kchunk = (k + kChunk - 1) / kChunk;  // the n <= k path writes k outputs
  const long long grid_x = nchunk > kchunk ? nchunk : kchunk;
  const TopkWs w = carve(ws, nq, nchunk);
  const dim3 grid((unsigned)grid_x, (unsigned)nq);
  if (ld > 0) hipLaunchKernelGGL(topk_hist_kernel, grid, dim3(kThreads), 0, stream, scores, ld, n_visible, k, w);
  hipLaunchKernelGGL(topk_select_kernel, grid, dim3(kThreads), 0, stream, scores, ld, n_visible, k, topk_idx, w,
                     (int)nchunk);
  return launch_status();
}
