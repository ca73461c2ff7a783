// Recall Window of 16-bit inputs through one histogram per head (calib_hist.hip):
// the path the calibration entry points take when the window count is past what the
// streaming tail selection keeps on chip.
#pragma once

#include "fa3q_internal.hpp"

namespace fa3q {

constexpr int kHistMaxBatches = 16;

struct HistPlan {
  int vpv = 8;            // values per 16-byte vector: 8 (16-bit input) or 4 (float32)
  int64_t Lv = 0;         // 16-byte vectors per row: a (b, h) slab of S*D values, or (BSHD) D values
  int64_t nrows = 0;      // rows per head: B, or (BSHD) B*S; row j of head h starts at vector (j*H + h)*Lv
  int64_t Qv = 0;         // vectors per head
  bool rows = false;      // rows of at most one vector per thread: parts are whole rows
  int64_t part_vecs = 0;  // vectors per part (whole rows when rows is set)
  int64_t part_rows = 0;  // rows per part when rows is set
  int64_t P = 0;          // parts per head
  int64_t head_words = 0; // workspace words per head: P part records, at least 65536
  size_t bytes = 0;       // workspace per batch: H regions of head_words uint32
};

// Plan for nb batches of (B, H, S, D), or with bshd (B, S, H, D), of vpv values per 16-byte
// vector (8: 16-bit values, 4: float32); a row (S*D, or D values) must be a multiple of vpv
// values and N = B*S*D below 2^32.  Batch b uses the workspace bytes [b*bytes, (b+1)*bytes).
int hist_plan(int64_t nb, bool bshd, int vpv, int64_t B, int64_t H, int64_t S, int64_t D, HistPlan& hp);

// Windows of nb (<= kHistMaxBatches) batches into win_min/win_max [nb][H]; f16: float16
// input, else bf16; t = int(ratio*N), K = N - t + 1.
int hist_launch(const void* const* xs, int64_t nb, int64_t H, bool f16, int64_t t, int64_t K, const HistPlan& hp,
                float* win_min, float* win_max, void* workspace, hipStream_t stream);

// Per-head state of the float32 path: the leading 16-bit keys (high halves of the 32-bit
// order keys) holding ranks K - 1 and t - 1, the number of values whose leading key is at
// most a_max or at least m_min (both tails of the sorted head), and the collecting pass's
// append counter.
struct TailCut {
  uint32_t a_max;
  uint32_t m_min;
  uint32_t M;
  uint32_t fill;
};

// One float32 batch x (hp planned with vpv 4 and nb 1): counts each head's leading keys into
// records (hp.bytes), sets cut[h] and best[h] = ~0, and appends the 32-bit keys of head h's M
// collected values to lists + h*stride, in no particular order.
int hist_f32_collect(const void* x, int64_t H, int64_t t, int64_t K, const HistPlan& hp, uint32_t* records,
                     TailCut* cut, uint64_t* best, uint32_t* lists, int64_t stride, hipStream_t stream);

}  // namespace fa3q
