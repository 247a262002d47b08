// topk_select.hip -- per-query top-k over fp32 scores, ties to the lower index,
// output in ascending index order.
//
// Source: "DeepSeek-V4.1-Flash, expliqué pas à pas", attention forms and CSA2 section:
// the indexer keeps only the best-scoring entries (top-k).
//
// Scores become order-preserving 32-bit keys; the selection is the set of the k
// largest 64-bit composites (key << 32) | (0xFFFFFFFF - index), which are all
// distinct, so the answer is unique.  Three launches, each a grid of
// (chunks of 8192 scores) x (queries):
//   1. hist   : 4096-bin histogram of the top 12 key bits -> global histogram.
//   2. filter : every workgroup finds the threshold bin b* (the bin where the running
//               count from the top reaches k), counts its chunk's entries above b*
//               and appends the entries of bin b* to a candidate list.  The last
//               workgroup of a query (arrival counter) radix-selects the exact
//               boundary composite inside bin b* from the candidates (or, if they
//               overflow the list, from the score row itself), turns the per-chunk
//               counts into output offsets, and clears the histogram, counters and
//               flags so the workspace is zero again for the next call.
//   3. write  : every workgroup re-reads its chunk in index order and writes the
//               selected indices at its offset (ordered compaction, deterministic).
#include "common.hpp"
#include "host_common.hpp"

namespace csa2 {

constexpr int kBins = 4096;  // top 12 key bits
constexpr int kBinShift = 20;
constexpr int kChunk = 8192;  // scores per workgroup
constexpr int kPerThread = kChunk / 256;
constexpr int kCap = 4096;  // bin candidates resolved from LDS
constexpr int kMaxChunks = 4096;

struct TopkCtl {
  uint32_t cand_count;
  uint32_t arrive;
  uint32_t overflow;
  uint32_t bstar;
  unsigned long long boundary;
  uint32_t pad[10];
};
static_assert(sizeof(TopkCtl) == 64, "TopkCtl is 64 bytes");

struct TopkWs {
  TopkCtl* ctl;                 // [nq]
  uint32_t* hist;               // [nq][kBins]
  uint32_t* sure;               // [nq][nchunk]
  uint32_t* offs;               // [nq][nchunk]
  unsigned long long* cand;     // [nq][kCap]
};

__host__ __device__ inline size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

__host__ __device__ inline size_t ws_bytes_for(int nq, long long nchunk) {
  return align_up(sizeof(TopkCtl) * (size_t)nq) + align_up(sizeof(uint32_t) * kBins * (size_t)nq) +
         2 * align_up(sizeof(uint32_t) * (size_t)nq * (size_t)nchunk) +
         align_up(sizeof(unsigned long long) * kCap * (size_t)nq);
}

__host__ __device__ inline TopkWs carve(void* base, int nq, long long nchunk) {
  unsigned char* p = (unsigned char*)base;
  TopkWs w;
  w.ctl = (TopkCtl*)p;
  p += align_up(sizeof(TopkCtl) * (size_t)nq);
  w.hist = (uint32_t*)p;
  p += align_up(sizeof(uint32_t) * kBins * (size_t)nq);
  w.sure = (uint32_t*)p;
  p += align_up(sizeof(uint32_t) * (size_t)nq * (size_t)nchunk);
  w.offs = (uint32_t*)p;
  p += align_up(sizeof(uint32_t) * (size_t)nq * (size_t)nchunk);
  w.cand = (unsigned long long*)p;
  return w;
}

CSA2_DEV unsigned long long composite(uint32_t key, uint32_t idx) {
  return ((unsigned long long)key << 32) | (unsigned long long)(0xFFFFFFFFu - idx);
}

template <typename T>
CSA2_DEV T ld_agent(const T* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Block-wide (256 threads) exclusive scan of one value per thread; returns the
// exclusive prefix and writes the total to *total.  red: 256 u32 of LDS.
CSA2_DEV uint32_t block_exclusive_scan(uint32_t v, uint32_t* red, uint32_t* total) {
  const int tid = threadIdx.x;
  red[tid] = v;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    uint32_t t = (tid >= o) ? red[tid - o] : 0u;
    __syncthreads();
    red[tid] += t;
    __syncthreads();
  }
  const uint32_t incl = red[tid];
  *total = red[255];
  __syncthreads();
  return incl - v;
}

// In a histogram h[0..nb) (LDS), find the digit D such that the count of entries
// with digit > D is < need and with digit >= D is >= need (need >= 1).  Returns D
// and writes the count strictly above it.  Uses 256 threads; nb multiple of 256.
CSA2_DEV int find_digit(const uint32_t* h, int nb, uint32_t need, uint32_t* red, uint32_t* above_out, int* dig) {
  const int tid = threadIdx.x;
  const int per = nb / 256;
  uint32_t s = 0;
  for (int i = 0; i < per; ++i) s += h[tid * per + i];
  // exclusive suffix sum over threads: counts in digits above this thread's range
  red[255 - tid] = s;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    uint32_t t = (tid >= o) ? red[tid - o] : 0u;
    __syncthreads();
    red[tid] += t;
    __syncthreads();
  }
  const uint32_t incl_rev = red[255 - tid];  // sum over threads >= tid
  const uint32_t above_thread = incl_rev - s;  // sum over threads > tid
  if (above_thread < need && need <= incl_rev) {
    uint32_t acc = above_thread;
    for (int i = per - 1; i >= 0; --i) {
      const uint32_t c = h[tid * per + i];
      if (acc + c >= need) {
        *dig = tid * per + i;
        *above_out = acc;
        break;
      }
      acc += c;
    }
  }
  __syncthreads();
  const int D = *dig;
  __syncthreads();
  return D;
}

// ---------------------------------------------------------------- kernel 1 --
__global__ __launch_bounds__(256) void topk_hist_kernel(const float* __restrict__ scores, int64_t ld,
                                                        const int32_t* __restrict__ n_visible, int k, TopkWs ws) {
  __shared__ uint32_t lh[kBins];
  const int q = blockIdx.y, tid = threadIdx.x;
  const int64_t n = n_visible[q];
  const int64_t base = (int64_t)blockIdx.x * kChunk;
  if (n <= k || base >= n) return;
  for (int b = tid; b < kBins; b += 256) lh[b] = 0;
  __syncthreads();
  const float* row = scores + (int64_t)q * ld;
  const int64_t end = min(base + (int64_t)kChunk, n);
  for (int64_t i = base + tid; i < end; i += 256) atomicAdd(&lh[score_key(row[i]) >> kBinShift], 1u);
  __syncthreads();
  uint32_t* gh = ws.hist + (size_t)q * kBins;
  for (int b = tid; b < kBins; b += 256)
    if (lh[b]) atomicAdd(&gh[b], lh[b]);
}

// Candidate sources for the boundary selection inside bin b*.
struct LdsCands {
  const unsigned long long* c;
  int n;
  template <typename F>
  CSA2_DEV void each(F&& f) const {
    for (int i = threadIdx.x; i < n; i += 256) f(c[i]);
  }
};
struct RowCands {
  const float* row;
  int64_t n;
  uint32_t bstar;
  template <typename F>
  CSA2_DEV void each(F&& f) const {
    for (int64_t i = threadIdx.x; i < n; i += 256) {
      const uint32_t key = score_key(row[i]);
      if ((key >> kBinShift) == bstar) f(composite(key, (uint32_t)i));
    }
  }
};

// Radix-select the need-th largest composite among the candidates (all share the
// top 12 key bits = b*): 12-bit digits over composite bits 51..0, stopping early
// once every candidate left under the chosen prefix is selected.
template <typename Src>
CSA2_DEV unsigned long long select_boundary(const Src& src, uint32_t need, uint32_t bstar, uint32_t* h,
                                            uint32_t* red, uint32_t* above_s, int* dig_s,
                                            unsigned long long* min_s) {
  const int tid = threadIdx.x;
  unsigned long long prefix = bstar;  // value of composite >> hi
  int hi = 52;
  while (hi > 0) {
    const int width = hi >= 12 ? 12 : hi;
    const int lo = hi - width;
    const int nb = 1 << width;
    for (int b = tid; b < kBins; b += 256) h[b] = 0;
    __syncthreads();
    src.each([&](unsigned long long x) {
      if ((x >> hi) == prefix) atomicAdd(&h[(int)((x >> lo) & (unsigned long long)(nb - 1))], 1u);
    });
    __syncthreads();
    uint32_t above = 0;
    const int D = find_digit(h, kBins, need, red, above_s, dig_s);
    above = *above_s;
    const uint32_t cnt = h[D];
    __syncthreads();
    need -= above;
    prefix = (prefix << width) | (unsigned long long)D;
    hi = lo;
    if (cnt == need || hi == 0) {
      if (hi == 0) return prefix;
      // all candidates under this prefix are selected: the boundary is their minimum
      if (tid == 0) *min_s = ~0ull;
      __syncthreads();
      src.each([&](unsigned long long x) {
        if ((x >> hi) == prefix) atomicMin(min_s, x);
      });
      __syncthreads();
      const unsigned long long m = *min_s;
      __syncthreads();
      return m;
    }
  }
  return prefix;
}

// ---------------------------------------------------------------- kernel 2 --
__global__ __launch_bounds__(256) void topk_filter_kernel(const float* __restrict__ scores, int64_t ld,
                                                          const int32_t* __restrict__ n_visible, int k, TopkWs ws,
                                                          int nchunk) {
  __shared__ uint32_t h[kBins];
  __shared__ unsigned long long cands[kCap];
  __shared__ uint32_t red[256];
  __shared__ uint32_t above_s;
  __shared__ int dig_s;
  __shared__ unsigned long long min_s;
  __shared__ int is_last;
  const int q = blockIdx.y, tid = threadIdx.x;
  const int64_t n = n_visible[q];
  const int64_t base = (int64_t)blockIdx.x * kChunk;
  if (n <= k || base >= n) return;
  const int nch = (int)((n + kChunk - 1) / kChunk);
  TopkCtl* ctl = ws.ctl + q;
  uint32_t* gh = ws.hist + (size_t)q * kBins;

  // threshold bin from the global histogram
  for (int b = tid; b < kBins; b += 256) h[b] = ld_agent(gh + b);
  __syncthreads();
  if (tid == 0) dig_s = 0;
  __syncthreads();
  const uint32_t bstar = (uint32_t)find_digit(h, kBins, (uint32_t)k, red, &above_s, &dig_s);
  const uint32_t above_b = above_s;

  // this chunk: count entries above b*, append entries of b*
  const float* row = scores + (int64_t)q * ld;
  const int64_t end = min(base + (int64_t)kChunk, n);
  uint32_t sure = 0;
  unsigned long long* cand = ws.cand + (size_t)q * kCap;
  for (int64_t i = base + tid; i < end; i += 256) {
    const uint32_t key = score_key(row[i]);
    const uint32_t bin = key >> kBinShift;
    if (bin > bstar) ++sure;
    else if (bin == bstar) {
      const uint32_t pos = atomicAdd(&ctl->cand_count, 1u);
      if (pos < (uint32_t)kCap) cand[pos] = composite(key, (uint32_t)i);
      else atomicOr(&ctl->overflow, 1u);
    }
  }
  uint32_t total;
  block_exclusive_scan(sure, red, &total);
  if (tid == 0) ws.sure[(size_t)q * nchunk + blockIdx.x] = total;
  __threadfence();
  __syncthreads();
  if (tid == 0) is_last = (atomicAdd(&ctl->arrive, 1u) == (uint32_t)(nch - 1));
  __syncthreads();
  if (!is_last) return;
  __threadfence();

  // ---- last workgroup of this query: exact boundary inside bin b*
  const uint32_t need = (uint32_t)k - above_b;
  const uint32_t ccount = ld_agent(&ctl->cand_count);
  const bool overflow = ld_agent(&ctl->overflow) != 0u;
  unsigned long long boundary;
  if (!overflow) {
    for (uint32_t i = tid; i < ccount; i += 256) cands[i] = ld_agent(cand + i);
    __syncthreads();
    LdsCands src{cands, (int)ccount};
    boundary = select_boundary(src, need, bstar, h, red, &above_s, &dig_s, &min_s);
  } else {
    RowCands src{row, n, bstar};
    boundary = select_boundary(src, need, bstar, h, red, &above_s, &dig_s, &min_s);
  }

  // per-chunk selected counts -> exclusive offsets (h reused as the count array)
  uint32_t* cnt = h;
  for (int c = tid; c < kMaxChunks; c += 256) cnt[c] = (c < nch) ? ld_agent(ws.sure + (size_t)q * nchunk + c) : 0u;
  __syncthreads();
  auto add_selected = [&](unsigned long long x) {
    if (x >= boundary) atomicAdd(&cnt[(0xFFFFFFFFu - (uint32_t)(x & 0xFFFFFFFFull)) / kChunk], 1u);
  };
  if (!overflow) {
    LdsCands src{cands, (int)ccount};
    src.each(add_selected);
  } else {
    RowCands src{row, n, bstar};
    src.each(add_selected);
  }
  __syncthreads();
  // exclusive scan of cnt[0..nch): 16 chunk counts per thread
  const int per = kMaxChunks / 256;
  uint32_t s = 0;
  for (int i = 0; i < per; ++i) s += cnt[tid * per + i];
  const uint32_t pre = block_exclusive_scan(s, red, &total);
  uint32_t acc = pre;
  for (int i = 0; i < per; ++i) {
    const int c = tid * per + i;
    if (c < nch) ws.offs[(size_t)q * nchunk + c] = acc;
    acc += cnt[c];
  }
  // leave the workspace clean for the next call
  for (int b = tid; b < kBins; b += 256) gh[b] = 0u;
  if (tid == 0) {
    ctl->bstar = bstar;
    ctl->boundary = boundary;
    ctl->cand_count = 0u;
    ctl->overflow = 0u;
    ctl->arrive = 0u;
  }
}

// ---------------------------------------------------------------- kernel 3 --
__global__ __launch_bounds__(256) void topk_write_kernel(const float* __restrict__ scores, int64_t ld,
                                                         const int32_t* __restrict__ n_visible, int k,
                                                         int32_t* __restrict__ topk_idx, TopkWs ws, int nchunk) {
  __shared__ uint32_t red[256];
  const int q = blockIdx.y, tid = threadIdx.x;
  const int64_t n = n_visible[q];
  const int64_t base = (int64_t)blockIdx.x * kChunk;
  int32_t* out = topk_idx + (int64_t)q * k;
  if (n <= k) {  // everything visible is selected, then -1 padding
    for (int64_t i = base + tid; i < min(base + (int64_t)kChunk, n); i += 256) out[i] = (int32_t)i;
    if (blockIdx.x == 0)
      for (int64_t i = n + tid; i < k; i += 256) out[i] = -1;
    return;
  }
  if (base >= n) return;
  const uint32_t bstar = ws.ctl[q].bstar;
  const unsigned long long boundary = ws.ctl[q].boundary;
  const float* row = scores + (int64_t)q * ld;
  const int64_t t0 = base + (int64_t)tid * kPerThread;
  uint32_t mask = 0;  // bit i: entry t0 + i selected
#pragma unroll 4
  for (int i = 0; i < kPerThread; ++i) {
    const int64_t j = t0 + i;
    if (j < n) {
      const uint32_t key = score_key(row[j]);
      const uint32_t bin = key >> kBinShift;
      if (bin > bstar || (bin == bstar && composite(key, (uint32_t)j) >= boundary)) mask |= 1u << i;
    }
  }
  uint32_t total;
  uint32_t pos = ws.offs[(size_t)q * nchunk + blockIdx.x] + block_exclusive_scan(__popc(mask), red, &total);
  while (mask) {
    const int i = __ffs(mask) - 1;
    mask &= mask - 1;
    if (pos < (uint32_t)k) out[pos] = (int32_t)(t0 + i);  // always true when the counts are consistent
    ++pos;
  }
}

}  // namespace csa2

using namespace csa2;

extern "C" size_t topk_select_workspace_size(int32_t nq, int64_t ld, int32_t k) {
  (void)k;
  if (nq <= 0 || ld <= 0) return 256;
  return ws_bytes_for(nq, (ld + kChunk - 1) / kChunk);
}

extern "C" int topk_select(const float* scores, int64_t ld, const int32_t* n_visible, int32_t nq, int32_t k,
                           int32_t* topk_idx, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (nq < 0 || ld < 0 || k < 1 || k > CSA2_MAX_K) return CSA2_ERR_SHAPE;
  if (ld > (int64_t)kChunk * kMaxChunks) return CSA2_ERR_SHAPE;
  if (nq == 0) return CSA2_OK;
  if (!n_visible || !topk_idx || (ld > 0 && !scores)) return CSA2_ERR_NULL;
  if (!ws || ws_bytes < topk_select_workspace_size(nq, ld, k)) return CSA2_ERR_WORKSPACE;
  const long long nchunk = ld > 0 ? (ld + kChunk - 1) / kChunk : 1;
  const TopkWs w = carve(ws, nq, nchunk);
  const dim3 grid((unsigned)nchunk, (unsigned)nq);
  if (ld > 0) {
    hipLaunchKernelGGL(topk_hist_kernel, grid, dim3(256), 0, stream, scores, ld, n_visible, k, w);
    hipLaunchKernelGGL(topk_filter_kernel, grid, dim3(256), 0, stream, scores, ld, n_visible, k, w, (int)nchunk);
  }
  hipLaunchKernelGGL(topk_write_kernel, grid, dim3(256), 0, stream, scores, ld, n_visible, k, topk_idx, w,
                     (int)nchunk);
  return launch_status();
}
