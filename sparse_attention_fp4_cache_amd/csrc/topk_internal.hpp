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

}  // namespace csa2
