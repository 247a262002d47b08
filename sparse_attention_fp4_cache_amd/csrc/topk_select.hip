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
//   1. hist   : 4096-bin histogram of the top 12 key bits (digit 1), added to a
//               per-query global histogram (index_topk folds this pass into the
//               scoring pass).
//   2. select : every workgroup finds the threshold bin b* of digit 1 (where the
//               running count from the top reaches k), writes the composites of its
//               entries in bins >= b* -- in index order -- to its own fixed region
//               of a per-query list, records their count, and adds its b* entries to
//               a second 4096-bin histogram of the next 12 key bits (digit 2).  The
//               last workgroup of a query (arrival counter) reads the digit-2
//               histogram to fix the boundary's top 24 key bits, resolves the rest
//               (rarely more than a few candidates) by radix steps over the list,
//               then copies the regions in chunk order and keeps the entries at or
//               above the boundary with a ballot-based ordered compaction, so the k
//               indices come out ascending without a sort.  It clears both
//               histograms and the counter, leaving the workspace zero for the next
//               call.  If a chunk's candidates overflow its region, the last
//               workgroup selects from the score row itself.
// Cross-workgroup data goes through device-coherent (sc1) stores and loads; a
// workgroup waits for its stores and atomics to complete before it announces them
// with the arrival atomic, so no cache-wide write-back or invalidate is needed.
#include "common.hpp"
#include "host_common.hpp"
#include "topk_internal.hpp"

namespace csa2 {

constexpr int kBins = kTopkBins;  // 12-bit digits
constexpr int kBinShift = kTopkBinShift;
constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kPer = 8;  // consecutive scores per thread
constexpr int kChunk = kThreads * kPer;
constexpr int kListCap = 8192;        // listed entries per query (fixed regions per chunk)
constexpr int kMaxChunksFast = 2048;  // chunk bookkeeping in LDS (rows up to 8M entries)

struct TopkCtl {
  uint32_t arrive;
  uint32_t pad[15];
};
static_assert(sizeof(TopkCtl) == 64, "TopkCtl is 64 bytes");

struct TopkWs {
  TopkCtl* ctl;              // [nq]
  uint32_t* hist;            // [nq][kBins]: digit 1 (key bits 31..20)
  uint32_t* hist2;           // [nq][kBins]: digit 2 (key bits 19..8) of the b* entries
  uint32_t* count;           // [nq][nchunk]: entries of the chunk in bins >= b*
  unsigned long long* list;  // [nq][kListCap]: chunk c's entries at c * (kListCap / nch)
};

__host__ __device__ inline size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

__host__ __device__ inline size_t ws_bytes_for(int nq, long long nchunk) {
  return align_up(sizeof(TopkCtl) * (size_t)nq) + 2 * align_up(sizeof(uint32_t) * kBins * (size_t)nq) +
         align_up(sizeof(uint32_t) * (size_t)nchunk * (size_t)nq) +
         align_up(sizeof(unsigned long long) * kListCap * (size_t)nq);
}

__host__ __device__ inline TopkWs carve(void* base, int nq, long long nchunk) {
  unsigned char* p = (unsigned char*)base;
  TopkWs w;
  w.ctl = (TopkCtl*)p;
  p += align_up(sizeof(TopkCtl) * (size_t)nq);
  w.hist = (uint32_t*)p;
  p += align_up(sizeof(uint32_t) * kBins * (size_t)nq);
  w.hist2 = (uint32_t*)p;
  p += align_up(sizeof(uint32_t) * kBins * (size_t)nq);
  w.count = (uint32_t*)p;
  p += align_up(sizeof(uint32_t) * (size_t)nchunk * (size_t)nq);
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
// and one LDS exchange.  wsum: kWaves u32 of LDS.
CSA2_DEV uint32_t block_inclusive_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  if (lane == 63) wsum[wid] = v;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t s = wsum[w];
    before += (w < wid) ? s : 0u;
    all += s;
  }
  __syncthreads();
  *total = all;
  return v + before;
}

// Copy kBins counters into LDS with every load in flight before the first store
// (a strided loop would wait for each load in turn).
template <bool kCoherent>
CSA2_DEV void load_bins(uint32_t* dst, uint32_t* src) {
  constexpr int per = kBins / kThreads;
  uint32_t v[per];
#pragma unroll
  for (int i = 0; i < per; ++i) {
    uint32_t* p = src + threadIdx.x + i * kThreads;
    v[i] = kCoherent ? ld_agent(p) : *p;
  }
#pragma unroll
  for (int i = 0; i < per; ++i) dst[threadIdx.x + i * kThreads] = v[i];
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
  uint32_t cpos[kMaxChunksFast + 1];  // chunk -> first position in the ordered list
  uint32_t wsum[kWaves];
  uint32_t above_s, ovf, more;
  int dig_s, is_last;
  unsigned long long min_s;
};

// Candidates of the boundary: the listed entries in LDS, or (slow path) the score row.
struct LdsCands {
  const unsigned long long* c;
  int n;
  template <typename F>
  CSA2_DEV void each(F&& f) const {
    for (int i = threadIdx.x; i < n; i += kThreads) f(c[i]);
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

// need-th largest composite among the candidates whose top (64 - hi) bits equal
// `prefix`: 12-bit digits of the composite below bit hi, stopping as soon as every
// candidate left under the chosen prefix is selected.  `cnt` is the number of
// candidates under `prefix` (they are all selected when cnt == need).
template <typename Src>
CSA2_DEV unsigned long long select_boundary(const Src& src, uint32_t need, unsigned long long prefix, int hi,
                                            uint32_t cnt, SelectSmem& sm) {
  const int tid = threadIdx.x;
  while (true) {
    if (cnt == need || hi == 0) {  // all of them are in: the boundary is their minimum
      if (hi == 0) return prefix;
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
    cnt = sm.h[D];
    __syncthreads();
    need -= above;
    prefix = (prefix << width) | (unsigned long long)D;
    hi = lo;
  }
}

// Ordered compaction of the list entries >= boundary into out[0..k): every
// wavefront owns a contiguous segment of the list (at most 16 x 64 entries, read
// into registers at once), counts its kept entries with ballots, and after one
// exchange of the counts writes them at their positions.
CSA2_DEV void compact_list(const unsigned long long* list, int total, unsigned long long boundary, int k,
                           int32_t* __restrict__ out, uint32_t* wsum) {
  constexpr int kIt = kListCap / (64 * kWaves);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int per_w = (((total + kWaves - 1) / kWaves) + 63) & ~63;
  const int s0 = wid * per_w, s1 = min(s0 + per_w, total);
  unsigned long long x[kIt];
#pragma unroll
  for (int j = 0; j < kIt; ++j) {
    const int e = s0 + 64 * j + lane;
    x[j] = e < s1 ? list[e] : 0ull;  // 0 is below every boundary
  }
  uint32_t cnt = 0;
#pragma unroll
  for (int j = 0; j < kIt; ++j) cnt += (uint32_t)__popcll(__builtin_amdgcn_ballot_w64(x[j] >= boundary));
  if (lane == 0) wsum[wid] = cnt;
  __syncthreads();
  uint32_t pos = 0;
  for (int w = 0; w < wid; ++w) pos += wsum[w];
#pragma unroll
  for (int j = 0; j < kIt; ++j) {
    const bool keep = x[j] >= boundary;
    const unsigned long long m = __builtin_amdgcn_ballot_w64(keep);
    const uint32_t o = pos + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    if (keep && o < (uint32_t)k) out[o] = (int32_t)index_of(x[j]);
    pos += (uint32_t)__popcll(m);
  }
  __syncthreads();  // wsum is reused by the caller
}

// ---------------------------------------------------------------- kernel 2 --
__global__ __launch_bounds__(kThreads) void topk_select_kernel(const float* __restrict__ scores, int64_t ld,
                                                               const int32_t* __restrict__ n_visible, int k,
                                                               int32_t* __restrict__ topk_idx, TopkWs ws,
                                                               int nchunk) {
  __shared__ SelectSmem sm;
  const int q = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
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
  const int cap = kListCap / nch;  // region of each chunk in the list (0: always the slow path)
  TopkCtl* ctl = ws.ctl + q;
  uint32_t* gh = ws.hist + (size_t)q * kBins;
  uint32_t* gh2 = ws.hist2 + (size_t)q * kBins;
  uint32_t* gcount = ws.count + (size_t)q * nchunk;
  unsigned long long* glist = ws.list + (size_t)q * kListCap;
  const float* row = scores + (int64_t)q * ld;

  uint32_t key[kPer];
  load_keys(row, base, n, key);
  load_bins<false>(sm.h, gh);
  if (tid == 0) sm.dig_s = 0;
  __syncthreads();
  uint32_t above_b;
  const uint32_t bstar = (uint32_t)find_digit(sm.h, (uint32_t)k, sm.wsum, &sm.dig_s, &sm.above_s, &above_b);

  // this chunk's entries in bins >= b*, in index order, into its region; its b*
  // entries also go into the digit-2 histogram
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const bool vis = base + (int64_t)tid * kPer + i < n;
    const uint32_t bin = key[i] >> kBinShift;
    if (vis && bin >= bstar) m |= 1u << i;
    if (vis && bin == bstar) atomicAdd(&gh2[(key[i] >> 8) & (kBins - 1)], 1u);
  }
  uint32_t tot;
  const uint32_t off = block_inclusive_scan((uint32_t)__popc(m), sm.wsum, &tot) - (uint32_t)__popc(m);
  uint32_t p = off;
  unsigned long long* region = glist + (size_t)blockIdx.x * cap;
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    if (m & (1u << i)) {
      if (p < (uint32_t)cap) st_agent(region + p, composite(key[i], (uint32_t)(base + (int64_t)tid * kPer + i)));
      ++p;
    }
  if (tid == 0) st_agent(gcount + blockIdx.x, tot);
  wait_all_memory();  // this workgroup's list entries, count and histogram adds are done
  __syncthreads();
  if (tid == 0) sm.is_last = (atomicAdd(&ctl->arrive, 1u) == (uint32_t)(nch - 1));
  __syncthreads();
  if (!sm.is_last) return;

  // ---- last workgroup of this query: every region, count and histogram is in place
  const uint32_t need = (uint32_t)k - above_b;  // 1 <= need <= entries in b*
  // one round of device-coherent loads: the chunk counts, the digit-2 histogram and
  // the first 64 slots of the regions of up to 16 chunks per wavefront (read before
  // the counts say how many are filled; only the filled ones are kept)
  constexpr int kG = 16;
  const bool one_pass = nch <= kThreads;  // rows up to 2M entries
  const uint32_t my_cnt = (one_pass && tid < nch) ? ld_agent(gcount + tid) : 0u;
  uint32_t h2[kBins / kThreads];
#pragma unroll
  for (int i = 0; i < kBins / kThreads; ++i) h2[i] = ld_agent(gh2 + tid + i * kThreads);
  unsigned long long spec[kG];
#pragma unroll
  for (int u = 0; u < kG; ++u) {
    const int c = wid + u * kWaves;
    spec[u] = (c < nch && lane < cap) ? ld_agent(glist + (size_t)c * cap + lane) : 0ull;
  }
  if (tid == 0) {
    sm.ovf = one_pass ? 0u : 1u;
    sm.more = nch > kG * kWaves ? 1u : 0u;
  }
#pragma unroll
  for (int i = 0; i < kBins / kThreads; ++i) sm.h[tid + i * kThreads] = h2[i];
  uint32_t total = 0;
  if (one_pass) {
    uint32_t t2;
    const uint32_t incl = block_inclusive_scan(my_cnt, sm.wsum, &t2);
    if (tid < nch) sm.cpos[tid] = incl - my_cnt;
    if (my_cnt > (uint32_t)cap) sm.ovf = 1u;
    if (my_cnt > 64u) sm.more = 1u;
    total = t2;
    if (tid == 0) sm.cpos[nch] = total;
  }
  __syncthreads();
  if (sm.ovf == 0u) {
    // the regions, in chunk order, into LDS: one wavefront per chunk, lanes across
    // the chunk's entries
#pragma unroll
    for (int u = 0; u < kG; ++u) {
      const int c = min(wid + u * kWaves, nch);  // clamped: chunks past the end are empty
      const uint32_t pos = sm.cpos[c], cn = sm.cpos[min(c + 1, nch)] - pos;
      if ((uint32_t)lane < cn) sm.list[pos + lane] = spec[u];
    }
    if (sm.more) {  // rare: more than 16 chunks per wavefront, or more than 64 entries in a region
      for (int c = wid; c < nch; c += kWaves) {
        const uint32_t pos = sm.cpos[c], cn = sm.cpos[c + 1] - pos;
        const uint32_t from = c < kG * kWaves ? 64u : 0u;
        for (uint32_t j = from + lane; j < cn; j += 64) sm.list[pos + j] = ld_agent(glist + (size_t)c * cap + j);
      }
    }
    __syncthreads();
    // digit 2 of the boundary from the histogram the workgroups built
    uint32_t above2;
    const int D2 = find_digit(sm.h, need, sm.wsum, &sm.dig_s, &sm.above_s, &above2);
    const uint32_t cnt2 = sm.h[D2];
    __syncthreads();
    const unsigned long long prefix = ((unsigned long long)bstar << 12) | (unsigned long long)D2;  // key bits 31..8
    const LdsCands src{sm.list, (int)total};
    const unsigned long long boundary = select_boundary(src, need - above2, prefix, 40, cnt2, sm);
    compact_list(sm.list, (int)total, boundary, k, out, sm.wsum);
  } else {
    // slow path (a region overflowed, or very long rows): boundary from the score
    // row, then an ordered scan of the row, kThreads entries per round
    const RowCands src{row, n, bstar};
    const unsigned long long boundary = select_boundary(src, need, (unsigned long long)bstar, 52, 0xFFFFFFFFu, sm);
    uint32_t written = 0;
    for (int64_t r0 = 0; r0 < n; r0 += kThreads) {
      const int64_t i = r0 + tid;
      bool keep = false;
      if (i < n) {
        const uint32_t kk = score_key(row[i]);
        const uint32_t bin = kk >> kBinShift;
        keep = bin > bstar || (bin == bstar && composite(kk, (uint32_t)i) >= boundary);
      }
      uint32_t t2;
      const uint32_t incl = block_inclusive_scan(keep ? 1u : 0u, sm.wsum, &t2);
      if (keep && written + incl - 1 < (uint32_t)k) out[written + incl - 1] = (int32_t)i;
      written += t2;
    }
  }
  // leave the workspace clean for the next call
  for (int b = tid; b < kBins; b += kThreads) {
    gh[b] = 0u;
    gh2[b] = 0u;
  }
  if (tid == 0) ctl->arrive = 0u;
}

}  // namespace csa2

using namespace csa2;

extern "C" size_t topk_select_workspace_size(int32_t nq, int64_t ld, int32_t k) {
  (void)k;
  if (nq <= 0) return 256;
  const long long nchunk = ld > 0 ? (ld + kChunk - 1) / kChunk : 1;
  return ws_bytes_for(nq, nchunk);
}

namespace csa2 {

uint32_t* topk_digit1_hist(void* ws, int32_t nq, int64_t ld) {
  const long long nchunk = ld > 0 ? (ld + kChunk - 1) / kChunk : 1;
  return carve(ws, nq, nchunk).hist;
}

int topk_enqueue(const float* scores, int64_t ld, const int32_t* n_visible, int32_t nq, int32_t k,
                 int32_t* topk_idx, void* ws, hipStream_t stream, bool hist_done) {
  const long long nchunk = ld > 0 ? (ld + kChunk - 1) / kChunk : 1;
  const long long kchunk = (k + kChunk - 1) / kChunk;  // the n <= k path writes k outputs
  const long long grid_x = nchunk > kchunk ? nchunk : kchunk;
  const TopkWs w = carve(ws, nq, nchunk);
  const dim3 grid((unsigned)grid_x, (unsigned)nq);
  if (ld > 0 && !hist_done)
    hipLaunchKernelGGL(topk_hist_kernel, grid, dim3(kThreads), 0, stream, scores, ld, n_visible, k, w);
  hipLaunchKernelGGL(topk_select_kernel, grid, dim3(kThreads), 0, stream, scores, ld, n_visible, k, topk_idx, w,
                     (int)nchunk);
  return launch_status();
}

}  // namespace csa2

extern "C" int topk_select(const float* scores, int64_t ld, const int32_t* n_visible, int32_t nq, int32_t k,
                           int32_t* topk_idx, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (nq < 0 || ld < 0 || k < 1 || k > CSA2_MAX_K) return CSA2_ERR_SHAPE;
  if (ld >= ((int64_t)1 << 31)) return CSA2_ERR_SHAPE;
  if (nq == 0) return CSA2_OK;
  if (!n_visible || !topk_idx || (ld > 0 && !scores)) return CSA2_ERR_NULL;
  if (!ws || ws_bytes < topk_select_workspace_size(nq, ld, k)) return CSA2_ERR_WORKSPACE;
  return topk_enqueue(scores, ld, n_visible, nq, k, topk_idx, ws, stream, false);
}
