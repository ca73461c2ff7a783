// Recall Window of float32 heads for any window count and either layout (calib_sort.hip):
// the tails of each head collected through a histogram of their leading 16 bits
// (calib_hist.hip), sorted by a radix sort, and scanned for the first shortest window.
#pragma once

#include "calib_hist.hpp"

namespace fa3q {

struct SortPlan {
  HistPlan hp;          // parts of the counting and collecting passes (one batch at a time)
  int64_t N = 0;        // values per head
  int32_t nblk = 1;     // workgroups per head in the sorting passes and the window scan
  size_t rec_bytes = 0, cut_bytes = 0, best_bytes = 0, bcount_bytes = 0, list_bytes = 0;
  size_t bytes = 0;     // the workspace, reused by every batch of a call in turn
};

// Plan for float32 (B, H, S, D), or with bshd (B, S, H, D), batches with K = N - t + 1 windows
// per head; a row (S*D, or D values) must be a multiple of 4 values and N = B*S*D below 2^32.
int sort_plan(bool bshd, int64_t B, int64_t H, int64_t S, int64_t D, int64_t K, SortPlan& sp);

// Windows of nb batches into win_min/win_max [nb][H], one batch after the other on stream.
int sort_launch(const void* const* xs, int64_t nb, int64_t H, int64_t t, int64_t K, const SortPlan& sp,
                float* win_min, float* win_max, void* workspace, hipStream_t stream);

}  // namespace fa3q
