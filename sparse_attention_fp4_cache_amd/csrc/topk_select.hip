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
//   1. hist   : 4096-bin histogram of the top 12 key bits (digit 1), added to one
//               of four copies of a per-query global histogram (by workgroup
//               index; the select pass sums them).  index_topk folds this pass into
//               the scoring pass.
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

#include <algorithm>
#include <type_traits>

namespace csa2 {

constexpr int kBins = kTopkBins;  // 12-bit digits
constexpr int kBinShift = kTopkBinShift;
constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kPer = 8;  // consecutive scores per thread
constexpr int kChunk = kThreads * kPer;
constexpr int kListCap = 12288;       // listed entries of a query that the last workgroup holds in LDS
constexpr int kMinRegion = 128;       // least list slots per chunk (the top-K's share of a chunk, with margin)
constexpr int kMaxChunksFast = 2048;  // chunk bookkeeping in LDS (rows up to 8M entries)

struct TopkCtl {
  uint32_t arrive;
  uint32_t pad[15];
};
static_assert(sizeof(TopkCtl) == 64, "TopkCtl is 64 bytes");

struct TopkWs {
  TopkCtl* ctl;              // [nq]
  uint32_t* hist;            // [nq][kTopkHistCopies][kBins]: digit 1 (key bits 31..20)
  uint32_t* hist2;           // [nq][kBins]: digit 2 (key bits 19..8) of the b* entries
  uint32_t* count;           // [nq][nchunk]: entries of the chunk in bins >= b*
  unsigned long long* list;  // [nq][list_slots(nchunk)]: chunk c's entries at c * region_slots(nch)
};

__host__ __device__ inline size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

// List slots of each chunk of a row of nch chunks.  A chunk lists its entries at or
// above the threshold bin: about (k + the bin's population) / nch of them, and the
// 12-bit bin of a narrow score distribution can hold more entries than k, so every
// region keeps at least kMinRegion slots.
__host__ __device__ inline long long region_slots(long long nch) {
  const long long even = (kListCap / nch) & ~1LL;
  return even > kMinRegion ? even : kMinRegion;
}
// List slots per query for rows of up to nchunk chunks (nch * region_slots(nch) is
// largest at nch = nchunk or where kListCap / nch still exceeds kMinRegion).
__host__ __device__ inline long long list_slots(long long nchunk) {
  return nchunk * kMinRegion > kListCap ? nchunk * kMinRegion : kListCap;
}

__host__ __device__ inline size_t ws_bytes_for(int nq, long long nchunk) {
  return align_up(sizeof(TopkCtl) * (size_t)nq) + align_up(sizeof(uint32_t) * kBins * kTopkHistCopies * (size_t)nq) +
         align_up(sizeof(uint32_t) * kBins * (size_t)nq) +
         align_up(sizeof(uint32_t) * (size_t)nchunk * (size_t)nq) +
         align_up(sizeof(unsigned long long) * (size_t)list_slots(nchunk) * (size_t)nq);
}

__host__ __device__ inline TopkWs carve(void* base, int nq, long long nchunk) {
  unsigned char* p = (unsigned char*)base;
  TopkWs w;
  w.ctl = (TopkCtl*)p;
  p += align_up(sizeof(TopkCtl) * (size_t)nq);
  w.hist = (uint32_t*)p;
  p += align_up(sizeof(uint32_t) * kBins * kTopkHistCopies * (size_t)nq);
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
// 16 bytes at byte offset `off` of a buffer of `num_bytes` bytes, read with the sc1
// cache policy (the coherence of the agent-scope accesses above).  A raw buffer
// descriptor: dword 3 = 0x00020000 is the gfx9 format word for plain 32-bit data;
// offsets at or past num_bytes read zeros instead of faulting.
typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));
constexpr int kCpolSc1 = 16;
CSA2_DEV uint4 ld_agent16(const void* base, uint32_t num_bytes, uint32_t off) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)num_bytes, 0x00020000);
  const v4u32 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCpolSc1);
  return make_uint4(v.x, v.y, v.z, v.w);
}

CSA2_DEV void wait_all_memory() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// This thread's kPer consecutive keys of a chunk, all loads in flight together:
// two 16-byte loads when the row is 16-byte aligned and the chunk is whole.
CSA2_DEV void load_keys(const float* __restrict__ row, int64_t base, int64_t n, uint32_t (&key)[kPer]) {
  float v[kPer];
  const int64_t j0 = base + (int64_t)threadIdx.x * kPer;
  if (((reinterpret_cast<uintptr_t>(row) & 15u) == 0) && base + kChunk <= n) {
    const float4 a = reinterpret_cast<const float4*>(row + j0)[0], b = reinterpret_cast<const float4*>(row + j0)[1];
    v[0] = a.x, v[1] = a.y, v[2] = a.z, v[3] = a.w, v[4] = b.x, v[5] = b.y, v[6] = b.z, v[7] = b.w;
  } else {
#pragma unroll
    for (int i = 0; i < kPer; ++i) v[i] = (j0 + i < n) ? row[j0 + i] : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) key[i] = score_key(v[i]);
}

// Block-wide inclusive scan (kThreads threads) of one value per thread: DPP wave
// scans and one LDS exchange behind one LDS-only barrier (loads, stores and atomics
// in flight stay in flight).  wsum: kWaves u32 of LDS that no
// thread may write again before every thread has passed the next barrier (callers
// alternate between two such areas).
CSA2_DEV uint32_t block_inclusive_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  v = wave_incl_scan(v);
  if (lane == 63) wsum[wid] = v;
  lds_barrier();
  const uint4 w0 = reinterpret_cast<const uint4*>(wsum)[0], w1 = reinterpret_cast<const uint4*>(wsum)[1];
  const uint32_t w[kWaves] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    before += (i < wid) ? w[i] : 0u;
    all += w[i];
  }
  *total = all;
  return v + before;
}
static_assert(kWaves == 8, "block_inclusive_scan reads 8 wave sums");

constexpr int kPerBins = kBins / kThreads;  // bins per thread in a digit search

// Thread t's bins of a digit search: [kBins - 8(t+1), kBins - 8t), so that threads in
// order walk the bins from the top down.
CSA2_DEV int bins_lo() { return kBins - kPerBins * ((int)threadIdx.x + 1); }

struct Digit {
  int d;           // the digit
  uint32_t above;  // count in digits above it
  uint32_t cnt;    // count in it
};

// Digit D with count(digit > D) < need <= count(digit >= D) of a histogram whose
// bins [bins_lo(), bins_lo() + 8) this thread holds in h (ascending).  Requires
// 1 <= need <= total count.  res: LDS slot written by one thread before the barrier
// and read by all after it; wsum as for block_inclusive_scan.
CSA2_DEV Digit find_digit(const uint32_t (&h)[kPerBins], uint32_t need, uint32_t* wsum, Digit* res) {
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < kPerBins; ++i) s += h[i];
  uint32_t total;
  const uint32_t incl = block_inclusive_scan(s, wsum, &total);  // count in bins >= bins_lo()
  const uint32_t excl = incl - s;                                // count in bins above them
  if (excl < need && need <= incl) {
    uint32_t acc = excl;
    bool found = false;
#pragma unroll
    for (int i = kPerBins - 1; i >= 0; --i) {
      if (!found && acc + h[i] >= need) {
        *res = Digit{bins_lo() + i, acc, h[i]};
        found = true;
      }
      acc += h[i];
    }
  }
  lds_barrier();
  return *res;
}

// This thread's bins of an LDS histogram, for find_digit.
CSA2_DEV void bins_from_lds(const uint32_t* h, uint32_t (&v)[kPerBins]) {
  const uint4 a = reinterpret_cast<const uint4*>(h + bins_lo())[0], b = reinterpret_cast<const uint4*>(h + bins_lo())[1];
  v[0] = a.x, v[1] = a.y, v[2] = a.z, v[3] = a.w, v[4] = b.x, v[5] = b.y, v[6] = b.z, v[7] = b.w;
}
static_assert(kPerBins == 8, "digit searches hold 8 bins per thread");

// ---------------------------------------------------------------- kernel 1 --
__global__ __launch_bounds__(kThreads) void topk_hist_kernel(const float* __restrict__ scores, int64_t ld,
                                                             const int32_t* __restrict__ n_visible, int k,
                                                             TopkWs ws, int ncopies) {
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
  uint32_t* gh = ws.hist + ((size_t)q * kTopkHistCopies + blockIdx.x % ncopies) * kBins;
  for (int b = tid; b < kBins; b += kThreads) {
    const uint32_t c = lh[b];
    if (c) atomicAdd(&gh[b], c);
  }
}

struct SelectSmem {
  uint32_t h[kBins];                  // LDS histogram of the radix rounds (rare)
  unsigned long long list[kListCap];  // the listed entries of a query, in index order
  uint32_t cpos[kMaxChunksFast + 1];  // chunk -> first position in the ordered list
  uint32_t wsum[4][kWaves];           // wave sums of block scans (used in rotation)
  Digit dig[4];                       // digit-search results (used in rotation)
  unsigned long long cand[64];        // the few candidates under the boundary prefix
  uint32_t ncand, ovf, more;
  int is_last;
  unsigned long long min_s, bnd_s;
};

// LDS of a chunk workgroup that leaves the final pass to topk_select_kernel<2>.
struct ChunkSmem {
  uint32_t wsum[4][kWaves];
  Digit dig[4];
  int is_last;
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
template <typename Src, typename Smem>
CSA2_DEV unsigned long long select_boundary(const Src& src, uint32_t need, unsigned long long prefix, int hi,
                                            uint32_t cnt, Smem& sm) {
  const int tid = threadIdx.x;
  int parity = 0;
  while (true) {
    if (cnt == need || hi == 0) {  // all of them are in: the boundary is their minimum
      if (hi == 0) return prefix;
      if (tid == 0) sm.min_s = ~0ull;
      lds_barrier();
      src.each([&](unsigned long long x) {
        if ((x >> hi) == prefix) atomicMin(&sm.min_s, x);
      });
      lds_barrier();
      const unsigned long long m = sm.min_s;
      lds_barrier();
      return m;
    }
    const int width = hi >= 12 ? 12 : hi;
    const int lo = hi - width;
    for (int b = tid; b < kBins; b += kThreads) sm.h[b] = 0;
    lds_barrier();
    src.each([&](unsigned long long x) {
      if ((x >> hi) == prefix) atomicAdd(&sm.h[(int)((x >> lo) & ((1ull << width) - 1))], 1u);
    });
    lds_barrier();
    uint32_t hv[kPerBins];
    bins_from_lds(sm.h, hv);
    const Digit D = find_digit(hv, need, sm.wsum[2 + parity], &sm.dig[2 + parity]);
    parity ^= 1;
    cnt = D.cnt;
    need -= D.above;
    prefix = (prefix << width) | (unsigned long long)D.d;
    hi = lo;
  }
}

// The need-th largest of the (at most 64) listed entries under a 24-bit key prefix:
// they are gathered into LDS, and one wavefront ranks every one against the others.
template <typename Src, typename Smem>
CSA2_DEV unsigned long long small_boundary(const Src& src, unsigned long long prefix, uint32_t need, Smem& sm) {
  src.each([&](unsigned long long x) {
    if ((x >> 40) == prefix) sm.cand[atomicAdd(&sm.ncand, 1u)] = x;
  });
  lds_barrier();
  if (threadIdx.x < 64) {
    const int nc = (int)sm.ncand, lane = threadIdx.x;
    const unsigned long long mine = lane < nc ? sm.cand[lane] : 0ull;
    uint32_t rank = 0;  // candidates above this one
    for (int j = 0; j < nc; ++j) rank += sm.cand[j] > mine ? 1u : 0u;
    if (lane < nc && rank == need - 1) sm.bnd_s = mine;
  }
  lds_barrier();
  return sm.bnd_s;
}

// Ordered compaction of the list entries >= boundary into out[0..k): every
// wavefront owns a contiguous segment of the list (at most 16 x 64 entries, read
// into registers at once), counts its kept entries with ballots, and after one
// exchange of the counts writes them at their positions.
CSA2_DEV int32_t out_index(const int32_t* __restrict__ pool_row, int64_t i);
CSA2_DEV void compact_list(const unsigned long long* list, int total, unsigned long long boundary, int k,
                           int32_t* __restrict__ out, uint32_t* wsum, const int32_t* __restrict__ pool_row) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int per_w = (((total + kWaves - 1) / kWaves) + 63) & ~63;
  const int s0 = wid * per_w, s1 = min(s0 + per_w, total);
  auto entry = [&](int e) { return e < s1 ? list[e] : 0ull; };  // 0 is below every boundary
  uint32_t cnt = 0;
  for (int e0 = s0; e0 < s1; e0 += 64) cnt += (uint32_t)__popcll(__builtin_amdgcn_ballot_w64(entry(e0 + lane) >= boundary));
  if (lane == 0) wsum[wid] = cnt;
  lds_barrier();
  uint32_t pos = 0;
  for (int w = 0; w < wid; ++w) pos += wsum[w];
  for (int e0 = s0; e0 < s1; e0 += 64) {  // the segment again, from LDS
    const unsigned long long x = entry(e0 + lane);
    const bool keep = x >= boundary;
    const unsigned long long m = __builtin_amdgcn_ballot_w64(keep);
    const uint32_t o = pos + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    if (keep && o < (uint32_t)k) out[o] = out_index(pool_row, index_of(x));
    pos += (uint32_t)__popcll(m);
  }
  lds_barrier();  // wsum is reused by the caller
}

// Selected position i of a row -> the index written out: i itself, or, when the row
// is a candidate pool (blocks of 8 entries listed in pool_row), the entry at pool
// position i.
CSA2_DEV int32_t out_index(const int32_t* __restrict__ pool_row, int64_t i) {
  return pool_row ? 8 * pool_row[i >> 3] + (int32_t)(i & 7) : (int32_t)i;
}

// One selection over nq rows: its scores, visible counts, k, output and workspace.
struct SelectJob {
  const float* scores;
  int64_t ld;
  const int32_t* n_visible;
  int k;
  int32_t* topk_idx;
  TopkWs ws;
  int nchunk, ncopies;
  const int32_t* pool;
  int npool;
  int nq;
};

// ---------------------------------------------------------------- kernel 2 --
// Rows 0 .. ja.nq-1 of the grid serve job ja, the rows after them job jb (two
// independent selections in one launch; jb.nq = 0 for one).
// MODE 0: chunk workgroups, and the last one to arrive finishes its row (one launch).
// MODE 1: chunk workgroups only; MODE 2: the finishing pass, one workgroup per row,
// launched after MODE 1.  Only the finishing pass holds the 96 KB list in LDS, so the
// chunk workgroups of MODE 1 run several to a compute unit: with thousands of chunks
// (many rows) the single-launch form runs them one per unit.
template <int MODE>
__global__ __launch_bounds__(kThreads) void topk_select_kernel(SelectJob ja, SelectJob jb) {
  __shared__ typename std::conditional<MODE == 1, ChunkSmem, SelectSmem>::type sm;
  const bool second = (int)blockIdx.y >= ja.nq;  // uniform
  const SelectJob jj = second ? jb : ja;
  const float* __restrict__ scores = jj.scores;
  const int64_t ld = jj.ld;
  const int32_t* __restrict__ n_visible = jj.n_visible;
  const int k = jj.k;
  int32_t* __restrict__ topk_idx = jj.topk_idx;
  const TopkWs ws = jj.ws;
  const int nchunk = jj.nchunk, ncopies = jj.ncopies;
  const int32_t* __restrict__ pool = jj.pool;
  const int npool = jj.npool;
  const int q = second ? (int)blockIdx.y - ja.nq : (int)blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int64_t n = n_visible[q];
  const int64_t base = (int64_t)blockIdx.x * kChunk;
  int32_t* out = topk_idx + (int64_t)q * k;
  const int32_t* pool_row = pool ? pool + (int64_t)q * npool : nullptr;
  if (n <= k) {  // everything visible is selected, then -1 padding (by the chunk workgroups)
    if (MODE != 2) {
      for (int64_t i = base + tid; i < min(base + (int64_t)kChunk, n); i += kThreads) out[i] = out_index(pool_row, i);
      if (blockIdx.x == 0)
        for (int64_t i = n + tid; i < k; i += kThreads) out[i] = -1;
    }
    return;
  }
  if (base >= n) return;
  const int nch = (int)((n + kChunk - 1) / kChunk);
  const int cap = (int)region_slots(nch);  // region of each chunk in the list
  TopkCtl* ctl = ws.ctl + q;
  uint32_t* gh = ws.hist + (size_t)q * kTopkHistCopies * kBins;  // its copies, kBins apart
  uint32_t* gh2 = ws.hist2 + (size_t)q * kBins;
  uint32_t* gcount = ws.count + (size_t)q * nchunk;
  unsigned long long* glist = ws.list + (size_t)q * (size_t)list_slots(nchunk);
  const uint32_t list_bytes = (uint32_t)(nch * cap) * 8u;  // this row's regions
  const float* row = scores + (int64_t)q * ld;

  uint32_t key[kPer];
  if (MODE != 2) load_keys(row, base, n, key);
  uint32_t hb[kPerBins];
  uint32_t nz1 = 0;  // bit r: one of this thread's bins of copy r is nonzero (cleared at the end)
  {
    uint4 h[kTopkHistCopies][2];
#pragma unroll
    for (int r = 0; r < kTopkHistCopies; ++r) {
      if (r < ncopies) {  // uniform
        h[r][0] = reinterpret_cast<const uint4*>(gh + r * kBins + bins_lo())[0];
        h[r][1] = reinterpret_cast<const uint4*>(gh + r * kBins + bins_lo())[1];
      } else {
        h[r][0] = h[r][1] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
#pragma unroll
    for (int r = 0; r < kTopkHistCopies; ++r)
      nz1 |= ((h[r][0].x | h[r][0].y | h[r][0].z | h[r][0].w | h[r][1].x | h[r][1].y | h[r][1].z | h[r][1].w) != 0u
                  ? 1u
                  : 0u)
             << r;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint4 t = h[0][j];
#pragma unroll
      for (int r = 1; r < kTopkHistCopies; ++r) t = make_uint4(t.x + h[r][j].x, t.y + h[r][j].y, t.z + h[r][j].z, t.w + h[r][j].w);
      hb[4 * j] = t.x, hb[4 * j + 1] = t.y, hb[4 * j + 2] = t.z, hb[4 * j + 3] = t.w;
    }
  }
  const Digit d1 = find_digit(hb, (uint32_t)k, sm.wsum[0], &sm.dig[0]);
  const uint32_t bstar = (uint32_t)d1.d, above_b = d1.above;

  if constexpr (MODE != 2) {
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
  const uint32_t off = block_inclusive_scan((uint32_t)__popc(m), sm.wsum[1], &tot) - (uint32_t)__popc(m);
  uint32_t p = off;
  unsigned long long* region = glist + (size_t)blockIdx.x * cap;
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    if (m & (1u << i)) {
      if (p < (uint32_t)cap) st_agent(region + p, composite(key[i], (uint32_t)(base + (int64_t)tid * kPer + i)));
      ++p;
    }
  if (tid == 0) st_agent(gcount + blockIdx.x, tot);
  if constexpr (MODE == 1) {
    return;  // the finishing pass is the next launch
  } else {
    wait_all_memory();  // this workgroup's list entries, count and histogram adds are done
    __syncthreads();
    if (tid == 0) sm.is_last = (atomicAdd(&ctl->arrive, 1u) == (uint32_t)(nch - 1));
    __syncthreads();
    if (!sm.is_last) return;
  }
  }  // MODE != 2

  if constexpr (MODE != 1) {
  // ---- last workgroup of this query: every region, count and histogram is in place
  const uint32_t need = (uint32_t)k - above_b;  // 1 <= need <= entries in b*
  // one round of device-coherent loads: the chunk counts, the digit-2 histogram and
  // the first kSpec slots of the regions of the first kSpecChunks chunks (thread t:
  // 8 slots of chunk t / 4), read before the counts say how many are filled; only
  // the filled ones are kept.  Slots past the list read zeros.
  constexpr int kSpec = 32;
  constexpr int kSpecChunks = kThreads * 8 / kSpec;
  const bool one_pass = nch <= kThreads;  // rows up to 2M entries
  const uint32_t my_cnt = (one_pass && tid < nch) ? ld_agent(gcount + tid) : 0u;
  uint32_t h2[kPerBins];
  {
    const uint4 a0 = ld_agent16(gh2, kBins * 4u, (uint32_t)bins_lo() * 4u);
    const uint4 a1 = ld_agent16(gh2, kBins * 4u, (uint32_t)bins_lo() * 4u + 16u);
    h2[0] = a0.x, h2[1] = a0.y, h2[2] = a0.z, h2[3] = a0.w, h2[4] = a1.x, h2[5] = a1.y, h2[6] = a1.z, h2[7] = a1.w;
  }
  const int spec_c = tid >> 2, spec_s0 = 8 * (tid & 3);
  unsigned long long spec[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 v = ld_agent16(glist, list_bytes, (uint32_t)(spec_c * cap + spec_s0 + 2 * i) * 8u);
    spec[2 * i] = ((unsigned long long)v.y << 32) | v.x;
    spec[2 * i + 1] = ((unsigned long long)v.w << 32) | v.z;
  }
  if (tid == 0) {
    sm.ovf = one_pass ? 0u : 1u;
    sm.more = nch > kSpecChunks ? 1u : 0u;
    sm.ncand = 0u;
  }
  uint32_t total = 0;
  if (one_pass) {  // uniform
    uint32_t t2;
    const uint32_t incl = block_inclusive_scan(my_cnt, sm.wsum[0], &t2);
    if (tid < nch) sm.cpos[tid] = incl - my_cnt;
    if (my_cnt > (uint32_t)cap) sm.ovf = 1u;
    if (my_cnt > (uint32_t)kSpec) sm.more = 1u;
    total = t2;
    if (tid == 0) {
      sm.cpos[nch] = total;
      if (total > (uint32_t)kListCap) sm.ovf = 1u;  // more than the LDS list holds
    }
  }
  lds_barrier();
  if (sm.ovf == 0u) {
    // the filled slots, in chunk order, into LDS
    if (spec_c < nch && spec_c < kSpecChunks) {
      const uint32_t pos = sm.cpos[spec_c], cn = sm.cpos[spec_c + 1] - pos;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if ((uint32_t)(spec_s0 + j) < cn) sm.list[pos + spec_s0 + j] = spec[j];
    }
    if (sm.more) {  // rare: chunks past kSpecChunks, or more than kSpec entries in a region
      for (int c = wid; c < nch; c += kWaves) {
        const uint32_t pos = sm.cpos[c], cn = sm.cpos[c + 1] - pos;
        const uint32_t from = c < kSpecChunks ? (uint32_t)kSpec : 0u;
        for (uint32_t j = from + lane; j < cn; j += 64) sm.list[pos + j] = ld_agent(glist + (size_t)c * cap + j);
      }
    }
    // digit 2 of the boundary from the histogram the workgroups built
    const Digit d2 = find_digit(h2, need, sm.wsum[1], &sm.dig[1]);  // its barriers also publish the list
    const unsigned long long prefix = ((unsigned long long)bstar << 12) | (unsigned long long)d2.d;  // key bits 31..8
    const uint32_t need2 = need - d2.above;
    unsigned long long boundary;
    if (d2.cnt <= 64u) {
      boundary = small_boundary(LdsCands{sm.list, (int)total}, prefix, need2, sm);
    } else {
      const LdsCands src{sm.list, (int)total};
      boundary = select_boundary(src, need2, prefix, 40, d2.cnt, sm);
    }
    compact_list(sm.list, (int)total, boundary, k, out, sm.wsum[0], pool_row);
  } else {
    // slow path (a region overflowed, or very long rows): boundary from the score
    // row, then an ordered scan of the row, kThreads entries per round
    const RowCands src{row, n, bstar};
    const unsigned long long boundary = select_boundary(src, need, (unsigned long long)bstar, 52, 0xFFFFFFFFu, sm);
    uint32_t written = 0;
    int parity = 0;
    for (int64_t r0 = 0; r0 < n; r0 += kThreads) {
      const int64_t i = r0 + tid;
      bool keep = false;
      if (i < n) {
        const uint32_t kk = score_key(row[i]);
        const uint32_t bin = kk >> kBinShift;
        keep = bin > bstar || (bin == bstar && composite(kk, (uint32_t)i) >= boundary);
      }
      uint32_t t2;
      const uint32_t incl = block_inclusive_scan(keep ? 1u : 0u, sm.wsum[parity], &t2);
      parity ^= 1;
      if (keep && written + incl - 1 < (uint32_t)k) out[written + incl - 1] = out_index(pool_row, i);
      written += t2;
    }
  }
  // leave the workspace clean for the next call: only the runs of 8 bins seen nonzero
  const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
  for (int r = 0; r < kTopkHistCopies; ++r)
    if (nz1 & (1u << r)) {
      reinterpret_cast<uint4*>(gh + r * kBins + bins_lo())[0] = z4;
      reinterpret_cast<uint4*>(gh + r * kBins + bins_lo())[1] = z4;
    }
  if ((h2[0] | h2[1] | h2[2] | h2[3] | h2[4] | h2[5] | h2[6] | h2[7]) != 0u) {
    reinterpret_cast<uint4*>(gh2 + bins_lo())[0] = z4;
    reinterpret_cast<uint4*>(gh2 + bins_lo())[1] = z4;
  }
  if (tid == 0) ctl->arrive = 0u;
  }  // MODE != 1
}

// ------------------------------------------------------- one row per workgroup --
// For many query rows (a prefill chunk): one workgroup selects one row.  The digit-1
// histogram comes from the counting pass; each wavefront then walks its own
// contiguous eighth of the row once, appending the entries in bins >= b* -- in index
// order -- to its own LDS list (ballot-free: a DPP prefix sum of per-lane counts), and
// counting the b* entries' next 12 key bits into an LDS digit-2 histogram.  The
// eight lists, taken in wavefront order, are the row's candidates in index order;
// the boundary and the ordered compaction follow as in the last workgroup above.
// Two workgroups share a compute unit (LDS <= 80 KB and <= 128 VGPRs each), so each
// unit keeps twice the row bytes in flight: 0.81 against 1.27 ms for 4096 rows of
// 132K scores, where a deeper counting round with one workgroup per unit gained
// nothing.  The listing walks 4 x 256 entries per step (70 VGPRs, no scratch): 8 x 256
// needed spills at 128 VGPRs and was no faster.
constexpr int kRowCap = 1008;           // listed entries per wavefront segment
constexpr int kRowSelectQueries = 128;  // rows from which this kernel is used ...
// ... when they fill the chip or are short: a few long rows (a 128-token replay over
// a 1M-token cache) would leave most compute units idle while one workgroup per row
// streams megabytes, so they take the chunked path.  Rows of more than one chunk and
// at most kRowShort scores (a Reindex layer's candidate pool of 2048 blocks) take this
// kernel at any count: one workgroup reads the 64 KB in about the time the chunked
// path spends on its cross-workgroup hand-over (21.9 against 25.0 us per pooled
// index_topk at 1M), while at 65,536 scores the chunked path is faster (43 against
// 55 us for the gatekeeper layer's call).  A row of one chunk has no hand-over.
constexpr int64_t kRowShort = 16384;
inline bool select_by_row(int32_t nq, int64_t ld) {
  return (nq >= kRowSelectQueries && (nq >= 256 || ld <= 65536)) || (ld > kChunk && ld <= kRowShort);
}
struct RowSmem {
  unsigned long long list[kWaves][kRowCap];
  uint32_t h[kBins];  // digit-1 or digit-2 counts, then radix-round scratch
  uint32_t cnt[kWaves];
  uint32_t wtot[kWaves];  // entries each wavefront selected, past kRowCap too
  uint32_t wsum[4][kWaves];
  Digit dig[4];
  unsigned long long cand[64];
  uint32_t ncand, ovf;
  unsigned long long min_s, bnd_s;
};
static_assert(sizeof(RowSmem) <= 80 * 1024, "two row workgroups per compute unit");
struct RowLists {
  const unsigned long long (*list)[kRowCap];
  const uint32_t* cnt;
  template <typename F>
  CSA2_DEV void each(F&& f) const {
    for (int w = 0; w < kWaves; ++w)
      for (int i = threadIdx.x; i < (int)cnt[w]; i += kThreads) f(list[w][i]);
  }
};

// One walk of a wavefront's segment [s0, s1) of the row, U x 256 entries per step
// (thread: 4 consecutive entries per 256; order within a step: u, then lane, then the
// 4 entries): the entries whose keys `sel` accepts go, in index order, to the
// wavefront's LDS list (its first kRowCap of them), and `tally` sees every key.
// Returns how many entries were accepted (uniform).  On a 16-byte aligned row the
// whole steps take unguarded 16-byte loads, each step's issued before the step ahead
// of it is listed, so two steps of the row are in flight per wavefront; a partial
// last step (and an unaligned row) takes loads guarded per element.
constexpr int kListU = 4;
// FULL: the whole step lies inside the segment, so no entry needs its bound checked.
template <bool FULL, typename Sel, typename Tally>
CSA2_DEV void row_list_step(const uint32_t (&key)[kListU][4], int64_t e0, int64_t s1, unsigned long long* __restrict__ list,
                            int lane, uint32_t& wcount, Sel& sel, Tally& tally) {
  constexpr int U = kListU;
  uint32_t keep = 0;  // bit 4u + i
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (FULL || e0 + 256 * u + 4 * lane + i < s1) {
        if (sel(key[u][i])) keep |= 1u << (4 * u + i);
        tally(key[u][i]);
      }
    }
  // positions: a DPP prefix sum over the lanes of each u's counts, two u per scan
  // (16-bit halves: at most 256 per half)
  uint32_t before = wcount;
#pragma unroll
  for (int u = 0; u < U; u += 2) {
    const uint32_t c0 = (uint32_t)__popc((keep >> (4 * u)) & 15u), c1 = (uint32_t)__popc((keep >> (4 * u + 4)) & 15u);
    const uint32_t incl = wave_incl_scan(c0 | (c1 << 16));
    const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
    const uint32_t ex0 = (incl & 0xFFFFu) - c0, ex1 = (incl >> 16) - c1;
    uint32_t p0 = before + ex0, p1 = before + (tot & 0xFFFFu) + ex1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (keep & (1u << (4 * u + i))) {
        if (p0 < (uint32_t)kRowCap) list[p0] = composite(key[u][i], (uint32_t)(e0 + 256 * u + 4 * lane + i));
        ++p0;
      }
      if (keep & (1u << (4 * u + 4 + i))) {
        if (p1 < (uint32_t)kRowCap) list[p1] = composite(key[u + 1][i], (uint32_t)(e0 + 256 * (u + 1) + 4 * lane + i));
        ++p1;
      }
    }
    before += (tot & 0xFFFFu) + (tot >> 16);
  }
  wcount = before;
}

template <typename Sel, typename Tally>
CSA2_DEV uint32_t row_list_pass(const float* __restrict__ row, int64_t s0, int64_t s1, bool aligned,
                                unsigned long long* __restrict__ list, int lane, Sel sel, Tally tally) {
  constexpr int U = kListU;
  uint32_t wcount = 0;
  uint32_t key[U][4];
  int64_t e0 = s0;
  if (aligned) {
    const int64_t whole = s0 + (s1 - s0) / (256 * U) * (256 * U);  // end of the whole steps
    // two register sets in turn: the next step's loads go out before this step is listed
    float4 a[U], b[U];
    auto load = [&](float4 (&v)[U], int64_t at) {
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = *reinterpret_cast<const float4*>(row + at + 256 * u + 4 * lane);
    };
    auto list_step = [&](const float4 (&v)[U]) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        key[u][0] = score_key(v[u].x), key[u][1] = score_key(v[u].y);
        key[u][2] = score_key(v[u].z), key[u][3] = score_key(v[u].w);
      }
      row_list_step<true>(key, e0, s1, list, lane, wcount, sel, tally);
      e0 += 256 * U;
    };
    // Every step loads the next one unconditionally (the last whole step re-reads
    // itself, unused): with no load under a condition, each wait counts exactly the
    // loads issued after the ones it waits for.
    if (e0 < whole) {  // uniform branches throughout
      const int64_t last = whole - 256 * U;
      load(a, e0);
      while (true) {
        load(b, min(e0 + 256 * U, last));
        list_step(a);
        if (e0 >= whole) break;
        load(a, min(e0 + 256 * U, last));
        list_step(b);
        if (e0 >= whole) break;
      }
    }
  }
  for (; e0 < s1; e0 += 256 * U) {  // a partial step, or an unaligned row
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = e0 + 256 * u + 4 * lane;
#pragma unroll
      for (int i = 0; i < 4; ++i) key[u][i] = score_key(j + i < s1 ? row[j + i] : 0.0f);
    }
    row_list_step<false>(key, e0, s1, list, lane, wcount, sel, tally);
  }
  return wcount;
}

CSA2_DEV void zero_bins(uint32_t* h) {
#pragma unroll
  for (int i = 0; i < kBins / kThreads; ++i) h[threadIdx.x + i * kThreads] = 0u;
}

// Sampled gate for long rows with no counts given.  The row's own first-digit count
// would cost a whole read of the row before the listing pass; instead the workgroup
// reads kGateSamples scores spread evenly over the row and takes as gate G the
// sample's r-th largest key, cut to its top 24 bits, with r about twice the share
// k / n of the sample.  One pass then lists every entry with key >= G and counts
// their first digits.  When at least k entries pass, the k-th largest of the row is
// among them, the counts give its first digit exactly, and the boundary and the
// output come from the lists alone.  Otherwise the exact path runs: a gate above the
// k-th largest (rare: the sample holds twice the expected number) costs the counting
// pass after all, and a list that overflowed its kRowCap slots costs a second
// listing pass from the now known first digit.  Either way the selection is the
// exact one; the gate only decides how many passes over the row it takes.
constexpr int64_t kGateMinRow = 32768;  // rows from which the gate is tried
constexpr int kGateMaxK = 2048;         // k up to which twice its share fits the lists
constexpr int kGateSamples = 4 * kThreads;

// ncopies == 0: no counting pass ran.  Long rows try the sampled gate above; the
// others (and rows where the gate falls short) count their first digits themselves,
// in a read of the row that leaves it in the caches for the listing pass.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void topk_row_kernel(const float* __restrict__ scores, int64_t ld,
                                                            const int32_t* __restrict__ n_visible, int k,
                                                            int32_t* __restrict__ topk_idx, uint32_t* __restrict__ hist,
                                                            int ncopies, const int32_t* __restrict__ pool, int npool) {
  __shared__ RowSmem sm;
  const int q = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform across the wavefront
  const int64_t n = n_visible[q];
  int32_t* out = topk_idx + (int64_t)q * k;
  const int32_t* pool_row = pool ? pool + (int64_t)q * npool : nullptr;
  if (n <= k) {  // everything visible is selected, then -1 padding
    for (int i = tid; i < k; i += kThreads) out[i] = i < n ? out_index(pool_row, i) : -1;
    return;
  }
  const float* row = scores + (int64_t)q * ld;
  uint32_t* gh = hist + (size_t)q * kTopkHistCopies * kBins;
  const bool aligned = (reinterpret_cast<uintptr_t>(row) & 15u) == 0;
  // this wavefront's segment [s0, s1) of the listing passes
  const int64_t seg = (((n + kWaves - 1) / kWaves) + 255) & ~(int64_t)255;
  const int64_t s0 = min(n, (int64_t)wid * seg), s1 = min(n, s0 + seg);
  uint32_t bstar = 0, above_b = 0;
  bool known = false;   // bstar / above_b hold the row's first digit of the boundary
  bool listed = false;  // the lists hold every entry of digit >= bstar, sm.h its b* digit-2 counts

  if (ncopies == 0 && n >= kGateMinRow && k <= kGateMaxK) {
    // the gate: two radix rounds over the samples (first digit, then the next 12 bits)
    uint32_t sk[kGateSamples / kThreads];
#pragma unroll
    for (int i = 0; i < kGateSamples / kThreads; ++i)
      sk[i] = score_key(row[((int64_t)(tid + kThreads * i) * n) / kGateSamples]);
    const uint32_t r = (uint32_t)min<int64_t>(kGateSamples, (2 * (int64_t)kGateSamples * k + n - 1) / n + 4);
    zero_bins(sm.h);
    lds_barrier();
#pragma unroll
    for (int i = 0; i < kGateSamples / kThreads; ++i) atomicAdd(&sm.h[sk[i] >> kBinShift], 1u);
    lds_barrier();
    uint32_t hs[kPerBins];
    bins_from_lds(sm.h, hs);
    const Digit g1 = find_digit(hs, r, sm.wsum[0], &sm.dig[0]);  // its barriers: every thread has read its bins
    zero_bins(sm.h);
    lds_barrier();
#pragma unroll
    for (int i = 0; i < kGateSamples / kThreads; ++i)
      if ((sk[i] >> kBinShift) == (uint32_t)g1.d) atomicAdd(&sm.h[(sk[i] >> 8) & (kBins - 1)], 1u);
    lds_barrier();
    bins_from_lds(sm.h, hs);
    const Digit g2 = find_digit(hs, r - g1.above, sm.wsum[1], &sm.dig[1]);
    const uint32_t gate = ((uint32_t)g1.d << kBinShift) | ((uint32_t)g2.d << 8);
    zero_bins(sm.h);
    lds_barrier();
    // one pass: every entry with key >= gate listed, its first digit counted
    const uint32_t wc = row_list_pass(
        row, s0, s1, aligned, sm.list[wid], lane, [&](uint32_t key) { return key >= gate; },
        [&](uint32_t key) {
          if (key >= gate) atomicAdd(&sm.h[key >> kBinShift], 1u);
        });
    if (lane == 0) {
      sm.cnt[wid] = min(wc, (uint32_t)kRowCap);
      sm.wtot[wid] = wc;
    }
    lds_barrier();
    uint32_t passed = 0;
    bool ovf = false;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      passed += sm.wtot[w];
      ovf |= sm.wtot[w] > (uint32_t)kRowCap;
    }
    if (passed >= (uint32_t)k) {  // uniform: the boundary's first digit, exactly
      uint32_t hv[kPerBins];
      bins_from_lds(sm.h, hv);
      const Digit d1 = find_digit(hv, (uint32_t)k, sm.wsum[2], &sm.dig[2]);  // its barriers: the counts are read
      bstar = (uint32_t)d1.d;
      above_b = d1.above;
      known = true;
      zero_bins(sm.h);
      if (tid == 0) {
        sm.ovf = 0u;
        sm.ncand = 0u;
      }
      lds_barrier();
      if (!ovf) {  // the lists hold every entry >= gate: the b* entries' digit-2 counts from them
        const RowLists src{sm.list, sm.cnt};
        src.each([&](unsigned long long x) {
          if ((uint32_t)(x >> 52) == bstar) atomicAdd(&sm.h[(uint32_t)(x >> 40) & (kBins - 1)], 1u);
        });
        listed = true;
      }
    }
  }

  if (!known) {
    uint32_t hb[kPerBins] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
    if (ncopies == 0) {
      zero_bins(sm.h);
      lds_barrier();
      // four 16-byte loads in flight per thread per round (8192 entries per round)
      for (int64_t r0 = 0; r0 < n; r0 += 4 * 4 * kThreads) {
        float v[4][4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int64_t j = r0 + 4 * (tid + u * kThreads);
          if (aligned && j + 4 <= n) {
            const float4 f = *reinterpret_cast<const float4*>(row + j);
            v[u][0] = f.x, v[u][1] = f.y, v[u][2] = f.z, v[u][3] = f.w;
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) v[u][i] = j + i < n ? row[j + i] : 0.0f;
          }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (r0 + 4 * (tid + u * kThreads) + i < n) atomicAdd(&sm.h[score_key(v[u][i]) >> kBinShift], 1u);
      }
      lds_barrier();
      bins_from_lds(sm.h, hb);
      lds_barrier();  // every thread has its bins before the digit-2 histogram is cleared below
    }
    uint4 hc[kTopkHistCopies][2];
#pragma unroll
    for (int r = 0; r < kTopkHistCopies; ++r)
      if (r < ncopies) {  // uniform
        hc[r][0] = reinterpret_cast<const uint4*>(gh + r * kBins + bins_lo())[0];
        hc[r][1] = reinterpret_cast<const uint4*>(gh + r * kBins + bins_lo())[1];
      }
#pragma unroll
    for (int r = 0; r < kTopkHistCopies; ++r)
      if (r < ncopies) {
        const uint4 a0 = hc[r][0], a1 = hc[r][1];
        hb[0] += a0.x, hb[1] += a0.y, hb[2] += a0.z, hb[3] += a0.w;
        hb[4] += a1.x, hb[5] += a1.y, hb[6] += a1.z, hb[7] += a1.w;
        // only this workgroup reads the row's histogram: return it to zero
        if ((a0.x | a0.y | a0.z | a0.w | a1.x | a1.y | a1.z | a1.w) != 0u) {
          reinterpret_cast<uint4*>(gh + r * kBins + bins_lo())[0] = make_uint4(0u, 0u, 0u, 0u);
          reinterpret_cast<uint4*>(gh + r * kBins + bins_lo())[1] = make_uint4(0u, 0u, 0u, 0u);
        }
      }
    zero_bins(sm.h);
    if (tid == 0) {
      sm.ovf = 0u;
      sm.ncand = 0u;
    }
    const Digit d1 = find_digit(hb, (uint32_t)k, sm.wsum[0], &sm.dig[0]);  // its barriers publish the zeroing
    bstar = (uint32_t)d1.d;
    above_b = d1.above;
  }

  if (!listed) {
    // this wavefront's entries in bins >= b*, in index order, into its list; the b*
    // entries' next 12 key bits into the digit-2 histogram
    const uint32_t wc = row_list_pass(
        row, s0, s1, aligned, sm.list[wid], lane, [&](uint32_t key) { return (key >> kBinShift) >= bstar; },
        [&](uint32_t key) {
          if ((key >> kBinShift) == bstar) atomicAdd(&sm.h[(key >> 8) & (kBins - 1)], 1u);
        });
    if (lane == 0) {
      sm.cnt[wid] = min(wc, (uint32_t)kRowCap);
      if (wc > (uint32_t)kRowCap) sm.ovf = 1u;
    }
  }
  lds_barrier();
  const uint32_t need = (uint32_t)k - above_b;  // 1 <= need <= entries in b*
  if (sm.ovf == 0u) {
    uint32_t hv[kPerBins];
    bins_from_lds(sm.h, hv);
    const Digit d2 = find_digit(hv, need, sm.wsum[1], &sm.dig[1]);
    const unsigned long long prefix = ((unsigned long long)bstar << 12) | (unsigned long long)d2.d;  // key bits 31..8
    const uint32_t need2 = need - d2.above;
    const RowLists src{sm.list, sm.cnt};
    const unsigned long long boundary = d2.cnt <= 64u ? small_boundary(src, prefix, need2, sm)
                                                      : select_boundary(src, need2, prefix, 40, d2.cnt, sm);
    // ordered compaction: wavefront wid's list after the kept entries of the lists before it
    const int cn = (int)sm.cnt[wid];
    uint32_t kept = 0;
    for (int i0 = 0; i0 < cn; i0 += 64) {
      const unsigned long long x = i0 + lane < cn ? sm.list[wid][i0 + lane] : 0ull;  // 0 is below every boundary
      kept += (uint32_t)__popcll(__builtin_amdgcn_ballot_w64(x >= boundary));
    }
    if (lane == 0) sm.wsum[0][wid] = kept;
    lds_barrier();
    uint32_t pos = 0;
    for (int w = 0; w < wid; ++w) pos += sm.wsum[0][w];
    for (int i0 = 0; i0 < cn; i0 += 64) {
      const unsigned long long x = i0 + lane < cn ? sm.list[wid][i0 + lane] : 0ull;
      const bool kp = x >= boundary;
      const unsigned long long m = __builtin_amdgcn_ballot_w64(kp);
      const uint32_t o = pos + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      if (kp && o < (uint32_t)k) out[o] = out_index(pool_row, index_of(x));
      pos += (uint32_t)__popcll(m);
    }
  } else {
    // a segment listed more than kRowCap entries: boundary from the row, then an
    // ordered scan of the row, kThreads entries per round
    const RowCands src{row, n, bstar};
    const unsigned long long boundary = select_boundary(src, need, (unsigned long long)bstar, 52, 0xFFFFFFFFu, sm);
    uint32_t written = 0;
    int parity = 0;
    for (int64_t r0 = 0; r0 < n; r0 += kThreads) {
      const int64_t i = r0 + tid;
      bool kp = false;
      if (i < n) {
        const uint32_t kk = score_key(row[i]);
        const uint32_t bin = kk >> kBinShift;
        kp = bin > bstar || (bin == bstar && composite(kk, (uint32_t)i) >= boundary);
      }
      uint32_t t2;
      const uint32_t incl = block_inclusive_scan(kp ? 1u : 0u, sm.wsum[parity], &t2);
      parity ^= 1;
      if (kp && written + incl - 1 < (uint32_t)k) out[written + incl - 1] = out_index(pool_row, i);
      written += t2;
    }
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

namespace csa2 {

size_t topk_zero_bytes(int32_t nq, int64_t ld) {
  (void)ld;  // the zeroed part (control words, digit-1 and digit-2 histograms) comes first in carve()
  return align_up(sizeof(TopkCtl) * (size_t)nq) + align_up(sizeof(uint32_t) * kBins * kTopkHistCopies * (size_t)nq) +
         align_up(sizeof(uint32_t) * kBins * (size_t)nq);
}

// Zero n16 16-byte words (a kernel, not a memset: it may be captured into a graph).
__global__ __launch_bounds__(256) void zero_fill_kernel(uint4* __restrict__ p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

int zero_fill(void* p, size_t bytes, hipStream_t stream) {
  const size_t n16 = bytes / 16;  // callers pass multiples of 256 bytes
  if (n16 == 0) return CSA2_OK;
  const unsigned blocks = (unsigned)std::min<size_t>((n16 + 255) / 256, 1024);
  hipLaunchKernelGGL(zero_fill_kernel, dim3(blocks), dim3(256), 0, stream, static_cast<uint4*>(p), n16);
  return launch_status();
}

uint32_t* topk_digit1_hist(void* ws, int32_t nq, int64_t ld) {
  const long long nchunk = ld > 0 ? (ld + kChunk - 1) / kChunk : 1;
  return carve(ws, nq, nchunk).hist;
}

static long long select_grid_x(int64_t ld, int32_t k) {
  const long long nchunk = ld > 0 ? (ld + kChunk - 1) / kChunk : 1;
  const long long kchunk = (k + kChunk - 1) / kChunk;  // the n <= k path writes k outputs
  return nchunk > kchunk ? nchunk : kchunk;
}

// Chunk workgroups in one launch with their finishing pass while they fit the chip
// about twice; beyond that the chunks run as their own launch (several workgroups per
// compute unit) and one workgroup per row finishes: topk_select over 128 rows of 524K
// scores (16,384 chunks) takes 215 against 544 us, the 8-sequence 1M decode step 674
// against 735 us.
constexpr long long kSplitChunks = 512;
static void launch_select(dim3 grid, const SelectJob& ja, const SelectJob& jb, hipStream_t stream) {
  if ((long long)grid.x * grid.y <= kSplitChunks) {
    hipLaunchKernelGGL(topk_select_kernel<0>, grid, dim3(kThreads), 0, stream, ja, jb);
    return;
  }
  hipLaunchKernelGGL(topk_select_kernel<1>, grid, dim3(kThreads), 0, stream, ja, jb);
  hipLaunchKernelGGL(topk_select_kernel<2>, dim3(1u, grid.y), dim3(kThreads), 0, stream, ja, jb);
}

static SelectJob select_job(const float* scores, int64_t ld, const int32_t* n_visible, int32_t nq, int32_t k,
                            int32_t* topk_idx, void* ws, int ncopies, const int32_t* pool, int npool) {
  const long long nchunk = ld > 0 ? (ld + kChunk - 1) / kChunk : 1;
  return SelectJob{scores, ld, n_visible, k, topk_idx, carve(ws, nq, nchunk), (int)nchunk, ncopies, pool, npool, nq};
}

int topk_enqueue(const float* scores, int64_t ld, const int32_t* n_visible, int32_t nq, int32_t k,
                 int32_t* topk_idx, void* ws, hipStream_t stream, bool hist_done, int copies, const int32_t* pool,
                 int npool) {
  const long long nchunk = ld > 0 ? (ld + kChunk - 1) / kChunk : 1;
  const TopkWs w = carve(ws, nq, nchunk);
  const dim3 grid((unsigned)select_grid_x(ld, k), (unsigned)nq);
  const int ncopies = hist_done ? copies : topk_hist_copies(nchunk);
  const bool by_row = select_by_row(nq, ld);
  if (ld > 0 && !hist_done && !by_row)
    hipLaunchKernelGGL(topk_hist_kernel, grid, dim3(kThreads), 0, stream, scores, ld, n_visible, k, w, ncopies);
  if (by_row) {  // many rows: one workgroup per row, counting its own row
    hipLaunchKernelGGL(topk_row_kernel, dim3((unsigned)nq), dim3(kThreads), 0, stream, scores, ld, n_visible, k,
                       topk_idx, w.hist, hist_done ? ncopies : 0, pool, npool);
    return launch_status();
  }
  SelectJob none{};
  launch_select(grid, select_job(scores, ld, n_visible, nq, k, topk_idx, ws, ncopies, pool, npool), none, stream);
  return launch_status();
}

int topk_count(const float* scores, int64_t ld, const int32_t* n_visible, int32_t nq, int32_t k, void* ws,
               int copies, hipStream_t stream) {
  if (ld <= 0 || nq == 0) return CSA2_OK;
  const long long nchunk = (ld + kChunk - 1) / kChunk;
  const dim3 grid((unsigned)select_grid_x(ld, k), (unsigned)nq);
  hipLaunchKernelGGL(topk_hist_kernel, grid, dim3(kThreads), 0, stream, scores, ld, n_visible, k,
                     carve(ws, nq, nchunk), copies);
  return launch_status();
}

int topk_enqueue_pair(const float* scores_a, int64_t ld_a, const int32_t* n_visible_a, int32_t nq_a, int32_t k_a,
                      int32_t* topk_a, void* ws_a, int copies_a, const float* scores_b, int64_t ld_b,
                      const int32_t* n_visible_b, int32_t nq_b, int32_t k_b, int32_t* topk_b, void* ws_b,
                      int copies_b, hipStream_t stream) {
  if (select_by_row(nq_a, ld_a) || select_by_row(nq_b, ld_b) || ld_a <= 0 || ld_b <= 0) {
    const int st = topk_enqueue(scores_a, ld_a, n_visible_a, nq_a, k_a, topk_a, ws_a, stream, true, copies_a,
                                nullptr, 0);
    if (st != CSA2_OK) return st;
    return topk_enqueue(scores_b, ld_b, n_visible_b, nq_b, k_b, topk_b, ws_b, stream, true, copies_b, nullptr, 0);
  }
  const long long ga = select_grid_x(ld_a, k_a), gb = select_grid_x(ld_b, k_b);
  const dim3 grid((unsigned)(ga > gb ? ga : gb), (unsigned)(nq_a + nq_b));
  launch_select(grid, select_job(scores_a, ld_a, n_visible_a, nq_a, k_a, topk_a, ws_a, copies_a, nullptr, 0),
                select_job(scores_b, ld_b, n_visible_b, nq_b, k_b, topk_b, ws_b, copies_b, nullptr, 0), stream);
  return launch_status();
}

}  // namespace csa2

namespace csa2 {

// ---- candidate pool: block maxima, then the top npool blocks -------------------
// Thread b of row q: the largest of the visible members of block b (8 entries), the
// first member kept on ties, and the row's count of blocks with a visible member.
constexpr int kBmaxThreads = 256;
__global__ __launch_bounds__(kBmaxThreads) void pool_bmax_kernel(const float* __restrict__ scores, int64_t ld,
                                                                 const int32_t* __restrict__ n_visible,
                                                                 float* __restrict__ bmax, int64_t ldb,
                                                                 int32_t* __restrict__ nblocks) {
  const int q = blockIdx.y;
  const int64_t n = n_visible[q], nb = (n + 7) / 8;
  if (blockIdx.x == 0 && threadIdx.x == 0) nblocks[q] = (int32_t)nb;
  const int64_t b = (int64_t)blockIdx.x * kBmaxThreads + threadIdx.x;
  if (b >= nb) return;
  const float* r = scores + (int64_t)q * ld + 8 * b;
  float v[8];
  if (8 * b + 8 <= n && (reinterpret_cast<uintptr_t>(r) & 15u) == 0) {
    const float4 a = reinterpret_cast<const float4*>(r)[0], c = reinterpret_cast<const float4*>(r)[1];
    v[0] = a.x, v[1] = a.y, v[2] = a.z, v[3] = a.w, v[4] = c.x, v[5] = c.y, v[6] = c.z, v[7] = c.w;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 8 * b + i < n ? r[i] : -INFINITY;
  }
  float m = v[0];
#pragma unroll
  for (int i = 1; i < 8; ++i)
    if (v[i] > m) m = v[i];
  bmax[(int64_t)q * ldb + b] = m;
}

static int64_t pool_ldb(int64_t ld) { return (ld + 7) / 8; }

PoolWs pool_ws_carve(void* ws, int32_t nq, int64_t ld) {
  PoolWs p;
  p.ldb = pool_ldb(ld);
  p.bmax = reinterpret_cast<float*>(ws);
  p.nblocks = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(ws) +
                                         align_up((size_t)nq * (size_t)p.ldb * sizeof(float)));
  p.ws_topk = reinterpret_cast<char*>(p.nblocks) + align_up((size_t)nq * sizeof(int32_t));
  return p;
}

}  // namespace csa2

extern "C" size_t index_pool_build_workspace_size(int32_t nq, int64_t ld, int32_t npool) {
  if (nq <= 0 || ld < 0 || npool < 1) return 0;
  const int64_t ldb = pool_ldb(ld);
  return align_up((size_t)nq * (size_t)ldb * sizeof(float)) + align_up((size_t)nq * sizeof(int32_t)) +
         topk_select_workspace_size(nq, ldb, npool);
}

extern "C" int index_pool_build(const float* scores, int64_t ld, const int32_t* n_visible, int32_t nq,
                                int32_t npool, int32_t* pool, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (nq < 0 || ld < 0 || npool < 1 || npool > CSA2_MAX_K) return CSA2_ERR_SHAPE;
  if (ld >= ((int64_t)1 << 31)) return CSA2_ERR_SHAPE;
  if (nq == 0) return CSA2_OK;
  if (!n_visible || !pool || (ld > 0 && !scores)) return CSA2_ERR_NULL;
  if (!ws || ws_bytes < index_pool_build_workspace_size(nq, ld, npool)) return CSA2_ERR_WORKSPACE;
  const PoolWs pw = pool_ws_carve(ws, nq, ld);
  const int64_t ldb = pw.ldb;
  float* bmax = pw.bmax;
  int32_t* nb = pw.nblocks;
  void* ws_topk = pw.ws_topk;
  const dim3 grid((unsigned)std::max<int64_t>(1, (ldb + kBmaxThreads - 1) / kBmaxThreads), (unsigned)nq);
  hipLaunchKernelGGL(pool_bmax_kernel, grid, dim3(kBmaxThreads), 0, stream, scores, ld, n_visible, bmax, ldb, nb);
  if (launch_status() != CSA2_OK) return CSA2_ERR_LAUNCH;
  return topk_enqueue(bmax, ldb, nb, nq, npool, pool, ws_topk, stream, false, 1, nullptr, 0);
}

extern "C" int topk_select_counted(const float* scores, int64_t ld, const int32_t* n_visible, int32_t nq,
                                   int32_t k, int32_t* topk_idx, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (nq < 0 || ld < 0 || k < 1 || k > CSA2_MAX_K) return CSA2_ERR_SHAPE;
  if (ld >= ((int64_t)1 << 31)) return CSA2_ERR_SHAPE;
  if (nq == 0) return CSA2_OK;
  if (!n_visible || !topk_idx || (ld > 0 && !scores)) return CSA2_ERR_NULL;
  if (!ws || ws_bytes < topk_select_workspace_size(nq, ld, k)) return CSA2_ERR_WORKSPACE;
  return topk_enqueue(scores, ld, n_visible, nq, k, topk_idx, ws, stream, true, kTopkHistCopies, nullptr, 0);
}

extern "C" int topk_select(const float* scores, int64_t ld, const int32_t* n_visible, int32_t nq, int32_t k,
                           int32_t* topk_idx, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (nq < 0 || ld < 0 || k < 1 || k > CSA2_MAX_K) return CSA2_ERR_SHAPE;
  if (ld >= ((int64_t)1 << 31)) return CSA2_ERR_SHAPE;
  if (nq == 0) return CSA2_OK;
  if (!n_visible || !topk_idx || (ld > 0 && !scores)) return CSA2_ERR_NULL;
  if (!ws || ws_bytes < topk_select_workspace_size(nq, ld, k)) return CSA2_ERR_WORKSPACE;
  return topk_enqueue(scores, ld, n_visible, nq, k, topk_idx, ws, stream, false, 1, nullptr, 0);
}
