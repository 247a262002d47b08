// topk_internal.hpp -- the selection's pieces that the fused indexer stage shares
// (not part of the C ABI).
#pragma once
#include <cstddef>
#include <cstdint>
#include <hip/hip_runtime.h>

namespace csa2 {

constexpr int kTopkBins = 4096;      // digit-1 bins: the top 12 bits of the score key
constexpr int kTopkBinShift = 20;
// Copies of each query's digit-1 histogram: workgroup w adds its counts into copy
// w % copies and the selection sums the copies.  Hundreds of workgroups adding into
// one copy serialise on the same few hot bins; four copies remove that.  Rows with
// few contributing workgroups keep one copy (less for every reader to sum).
constexpr int kTopkHistCopies = 4;
inline int topk_hist_copies(long long writers_per_row) { return writers_per_row >= 64 ? kTopkHistCopies : 1; }

// Per-query digit-1 histograms ([nq][kTopkHistCopies][kTopkBins] u32) inside a
// top-k workspace.
uint32_t* topk_digit1_hist(void* ws, int32_t nq, int64_t ld);

// Enqueue the selection; with hist_done the digit-1 histograms are already filled
// (by the scoring pass, in `copies` copies) and the counting launch is skipped.
// With pool (int32 [nq][npool] blocks of 8 entries), the rows are candidate-pool
// scores and the output holds the entries at the selected pool positions.
// Arguments were validated by the caller.
int topk_enqueue(const float* scores, int64_t ld, const int32_t* n_visible, int32_t nq, int32_t k,
                 int32_t* topk_idx, void* ws, hipStream_t stream, bool hist_done, int copies, const int32_t* pool,
                 int npool);

// The counting pass alone: each row's digit-1 histogram into `copies` copies of the
// top-k workspace ws (rows with n_visible <= k are not counted).
int topk_count(const float* scores, int64_t ld, const int32_t* n_visible, int32_t nq, int32_t k, void* ws,
               int copies, hipStream_t stream);

// Two selections whose digit-1 histograms are already counted (copies_a / copies_b
// copies), in one launch when both take the chunked path, else one after the other.
int topk_enqueue_pair(const float* scores_a, int64_t ld_a, const int32_t* n_visible_a, int32_t nq_a, int32_t k_a,
                      int32_t* topk_a, void* ws_a, int copies_a, const float* scores_b, int64_t ld_b,
                      const int32_t* n_visible_b, int32_t nq_b, int32_t k_b, int32_t* topk_b, void* ws_b,
                      int copies_b, hipStream_t stream);

// The candidate-pool workspace of index_pool_build (nq rows of ld scores): the block
// maxima [nq][ldb] (ldb = ceil(ld / 8)), the blocks per row [nq], then the top-npool
// selection's workspace over the block maxima.
struct PoolWs {
  int64_t ldb = 0;
  float* bmax = nullptr;
  int32_t* nblocks = nullptr;
  void* ws_topk = nullptr;
};
PoolWs pool_ws_carve(void* ws, int32_t nq, int64_t ld);

// Bytes at the start of a top-k workspace for (nq, ld) that must be zero before a
// call (its counters and histograms; a multiple of 256); the rest is scratch that
// every call writes before reading.
size_t topk_zero_bytes(int32_t nq, int64_t ld);
// Enqueue a kernel that zeroes `bytes` (a multiple of 16) at p.
int zero_fill(void* p, size_t bytes, hipStream_t stream);

}  // namespace csa2
