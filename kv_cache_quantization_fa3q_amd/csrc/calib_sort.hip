// Recall Window of float32 heads for any window count and either layout.
//
// msModelSlim page "FA3量化：Flash Attention 3激活量化算法说明", section 原理 -> 算法流程:
// head h's N values are sorted (s[0] <= ... <= s[N-1]), t = int(ratio*N), and among the
// windows [s[i], s[i+t-1]], i = 0 .. K-1 with K = N - t + 1, the one with the smallest
// length wins (here: float32 length, smallest i on ties).
//
// Per batch, on one stream:
//   calib_hist.hip  counts the leading 16 bits of every value's 32-bit order key, finds the
//                   leading keys that hold ranks K - 1 and t - 1, and appends the keys of
//                   every value at or below the first or at or above the second to a list of
//                   M values per head (M >= K; the list holds both tails of the sorted head).
//   lsd_count_kernel + lsd_scatter_kernel, four times: a stable least-significant-digit
//                   radix sort of each list, 8 bits a pass, between two buffers (back in the
//                   first after the fourth pass).  A head's list is cut into nblk blocks of
//                   whole 8192-key tiles; the count kernel gives each block's digit counts,
//                   from which every scatter workgroup derives its block's first position for
//                   each digit (digits in order, blocks in order).  A tile is ranked in LDS:
//                   each wave takes 1024 consecutive keys, 64 at a time, and ranks each key
//                   among the earlier keys of its digit from a per-wave counter and the lanes
//                   of the same digit (a per-wave LDS table of lane masks gives them), so the
//                   order within a digit is the list order (stable).  The tile is then laid out by digit in LDS and
//                   written with consecutive lanes on consecutive positions of a digit's run.
//   sort_window_kernel  the K windows [L[i], L[M-K+i]] of the sorted list L: float32 lengths,
//                   the smallest (length, i) per workgroup, combined with a 64-bit atomic min.
//   sort_finish_kernel  the winning window's ends as values.
#include <cmath>

#include "calib_sort.hpp"

namespace fa3q {
namespace {

constexpr int kSortThreads = 256;                  // counting and window workgroups
constexpr int kSortWaves = kSortThreads / kWave;   // 4
constexpr int kScatterThreads = 512;               // scatter workgroups
constexpr int kScatterWaves = kScatterThreads / kWave;  // 8
constexpr int kSlots = 16;                         // keys per thread per tile
constexpr int kTile = kScatterThreads * kSlots;    // 8192 keys: a block is whole tiles
constexpr int kCountTile = kSortThreads * kSlots;  // 4096 keys per step of the counting workgroup
constexpr int kWaveKeys = kWave * kSlots;          // 1024 consecutive keys per wave and tile
constexpr int kDigits = 256;
constexpr int kMaxBlocks = 64;
constexpr int64_t kTargetGroups = 2048;            // sorting workgroups per launch, when the lists allow
static_assert(kDigits == kSortThreads && kDigits <= kScatterThreads, "one digit per thread in the per-digit steps");
static_assert(kTile % kCountTile == 0, "counting steps tile a block");

struct SortArgs {
  const uint32_t* src;  // [H][stride] keys, M of head h in its row
  uint32_t* dst;
  int64_t stride;
  const TailCut* cut;   // M per head
  uint32_t* bcount;     // [H][kDigits][nblk] keys of each digit in each block
  int32_t nblk;
  int32_t shift;        // the digit: (key >> shift) & 255
};

struct WinArgs {
  const uint32_t* list;  // [H][stride] sorted keys
  int64_t stride;
  const TailCut* cut;
  uint64_t* best;        // [H] smallest (length bits, window) so far
  uint32_t K;
  int32_t nblk;
  int32_t H;
  float* win_min;        // [H] (this batch's slice)
  float* win_max;
};

// Keys [start, end) of a head's list of M that block blk takes: whole tiles, as evenly as
// the tile count divides.
__device__ __forceinline__ void block_range(uint32_t M, int nblk, int blk, uint64_t& start, uint64_t& end) {
  const uint64_t tiles = (static_cast<uint64_t>(M) + kTile - 1) / kTile;
  const uint64_t per = (tiles + nblk - 1) / nblk;
  start = min(static_cast<uint64_t>(blk) * per * kTile, static_cast<uint64_t>(M));
  end = min(start + per * kTile, static_cast<uint64_t>(M));
}

// Exclusive scan of one value per thread over the kWaves waves of the workgroup (scr: kWaves
// words, free on entry; the caller separates two uses by a barrier).
template <int kWaves>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* scr) {
  const int lane = lane_id(), wave = static_cast<int>(threadIdx.x) / kWave;
  uint32_t inc = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint32_t u = __shfl_up(inc, o);
    if (lane >= o) inc += u;
  }
  if (lane == kWave - 1) scr[wave] = inc;
  __syncthreads();
  uint32_t before = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) before += w < wave ? scr[w] : 0u;
  return before + inc - v;
}

// Counts go to kCountCopies copies of the histogram, lane l to copy l % kCountCopies, so lanes
// of one digit (the leading byte of a tail takes few values) meet in one counter at most
// 64 / kCountCopies at a time; a copy's row is kDigits + 1 words, so one digit's counters in
// the copies sit in different banks.
constexpr int kCountCopies = 16;

__global__ __launch_bounds__(kSortThreads) void lsd_count_kernel(SortArgs a) {
  __shared__ uint32_t cnt[kCountCopies * (kDigits + 1)];
  const int tid = static_cast<int>(threadIdx.x);
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const int h = static_cast<int>(blockIdx.x) / a.nblk, blk = static_cast<int>(blockIdx.x) % a.nblk;
  for (int i = tid; i < kCountCopies * (kDigits + 1); i += kSortThreads) cnt[i] = 0;
  uint32_t* mine = cnt + (lane % kCountCopies) * (kDigits + 1);
  __syncthreads();
  uint64_t start, end;
  block_range(a.cut[h].M, a.nblk, blk, start, end);
  const uint32_t* src = a.src + static_cast<int64_t>(h) * a.stride;
  uint32_t k[kSlots];
  {
    const uint64_t w0 = start + static_cast<uint64_t>(wave) * kWaveKeys + lane;
#pragma unroll
    for (int s = 0; s < kSlots; ++s) k[s] = w0 + s * kWave < end ? src[w0 + s * kWave] : 0u;
  }
  for (uint64_t t0 = start; t0 < end; t0 += kCountTile) {
    const uint64_t w0 = t0 + static_cast<uint64_t>(wave) * kWaveKeys + lane;
    uint32_t kn[kSlots];  // the next step's keys, loading while these are counted
#pragma unroll
    for (int s = 0; s < kSlots; ++s)
      kn[s] = w0 + kCountTile + s * kWave < end ? src[w0 + kCountTile + s * kWave] : 0u;
#pragma unroll
    for (int s = 0; s < kSlots; ++s) {
      if (w0 + s * kWave < end) atomicAdd(&mine[(k[s] >> a.shift) & 0xffu], 1u);  // counts need no order
    }
#pragma unroll
    for (int s = 0; s < kSlots; ++s) k[s] = kn[s];
  }
  __syncthreads();
  uint32_t total = 0;
#pragma unroll
  for (int c = 0; c < kCountCopies; ++c) total += cnt[c * (kDigits + 1) + tid];
  a.bcount[(static_cast<int64_t>(h) * kDigits + tid) * a.nblk + blk] = total;
}

template <bool kMatch>
__global__ __launch_bounds__(kScatterThreads) void lsd_scatter_kernel(SortArgs a) {
  __shared__ uint64_t peer[kMatch ? 8 : kScatterWaves * kDigits];  // [wave][digit]: the lanes of each digit (zero between uses)
  __shared__ uint32_t cnt[kScatterWaves * kDigits];   // [wave][digit]: keys so far, then tile positions
  __shared__ uint32_t tstart[kDigits];                // the digit's first position in the laid-out tile
  __shared__ uint32_t gbase[kDigits];                 // the digit's next list position from this block
  __shared__ uint32_t stage[kTile];
  __shared__ uint32_t scr[kScatterWaves];
  const int tid = static_cast<int>(threadIdx.x);
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const bool digit_thread = tid < kDigits;  // the per-digit steps: digit tid
  const int h = static_cast<int>(blockIdx.x) / a.nblk, blk = static_cast<int>(blockIdx.x) % a.nblk;
  uint64_t start, end;
  block_range(a.cut[h].M, a.nblk, blk, start, end);
  if (start >= end) return;
  if constexpr (!kMatch) {
#pragma unroll
    for (int i = 0; i < kScatterWaves * kDigits / kScatterThreads; ++i) peer[i * kScatterThreads + tid] = 0;
  }
  {
    // digit tid: keys of smaller digits in the head, plus its keys in earlier blocks (the scan's
    // barrier also orders the peer table's zeroing before its first use)
    uint32_t tot = 0, before = 0;
    if (digit_thread) {
      const uint32_t* bc = a.bcount + (static_cast<int64_t>(h) * kDigits + tid) * a.nblk;
      for (int b = 0; b < a.nblk; ++b) {
        const uint32_t v = bc[b];
        tot += v;
        before += b < blk ? v : 0u;
      }
    }
    const uint32_t ex = block_exclusive_scan<kScatterWaves>(tot, scr);
    if (digit_thread) gbase[tid] = ex + before;
  }
  const uint32_t* src = a.src + static_cast<int64_t>(h) * a.stride;
  uint32_t* dst = a.dst + static_cast<int64_t>(h) * a.stride;
  const uint64_t bit = uint64_t{1} << lane;
  uint32_t k[kSlots];
  {
    const uint64_t w0 = start + static_cast<uint64_t>(wave) * kWaveKeys + lane;
#pragma unroll
    for (int s = 0; s < kSlots; ++s) k[s] = w0 + s * kWave < end ? src[w0 + s * kWave] : 0u;
  }
  for (uint64_t t0 = start; t0 < end; t0 += kTile) {
    const uint64_t w0 = t0 + static_cast<uint64_t>(wave) * kWaveKeys + lane;
    uint32_t rk[kSlots];
#pragma unroll
    for (int i = 0; i < kScatterWaves * kDigits / kScatterThreads; ++i) cnt[i * kScatterThreads + tid] = 0;
    __syncthreads();
    // rank of each key among the wave's earlier keys of its digit (slots in order, lanes in
    // order), the earlier slots' count from the per-wave counter.  The lanes of one digit come
    // from the wave's peer table (each lane sets its bit, reads its digit's mask, clears it), or,
    // for the leading byte, which tails share among a handful of values (so that the table's
    // atomics queue), from one ballot per digit bit.  A wave's LDS operations complete in the
    // order it issues them.
    if constexpr (kMatch) {
  #pragma unroll
      for (int s = 0; s < kSlots; ++s) {
        const bool valid = w0 + s * kWave < end;
        const uint32_t d = (k[s] >> a.shift) & 0xffu;
        uint32_t* c = &cnt[wave * kDigits + d];
        uint64_t peers = __builtin_amdgcn_ballot_w64(valid);
  #pragma unroll
        for (int i = 0; i < 8; ++i) {
          const bool one = (d >> i) & 1u;
          const uint64_t m = __builtin_amdgcn_ballot_w64(one);
          peers &= one ? m : ~m;
        }
        const uint32_t base = valid ? *c : 0u;
        const uint32_t r = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(peers >> 32),
                                                     __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(peers), 0u));
        rk[s] = base + r;
        if (valid && r == 0) *c = base + static_cast<uint32_t>(__popcll(peers));  // the digit's first lane
      }
    } else {
  #pragma unroll
      for (int s = 0; s < kSlots; ++s) {
        const bool valid = w0 + s * kWave < end;
        const uint32_t d = (k[s] >> a.shift) & 0xffu;
        uint64_t* pt = &peer[wave * kDigits + d];
        uint32_t* c = &cnt[wave * kDigits + d];
        if (valid) atomicOr(reinterpret_cast<unsigned long long*>(pt), static_cast<unsigned long long>(bit));
        const uint64_t peers = valid ? *pt : uint64_t{0};
        const uint32_t base = valid ? *c : 0u;
        const uint32_t r = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(peers >> 32),
                                                     __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(peers), 0u));
        rk[s] = base + r;
        if (valid) {
          *pt = 0;
          if (r == 0) *c = base + static_cast<uint32_t>(__popcll(peers));  // the digit's first lane
        }
      }
    }
    __syncthreads();
    // digit tid: its tile count, its first position in the laid-out tile, each wave's first
    uint32_t tot = 0, cw[kScatterWaves];
    if (digit_thread) {
#pragma unroll
      for (int w = 0; w < kScatterWaves; ++w) {
        cw[w] = cnt[w * kDigits + tid];
        tot += cw[w];
      }
    }
    const uint32_t ts = block_exclusive_scan<kScatterWaves>(tot, scr);
    if (digit_thread) {
      tstart[tid] = ts;
      uint32_t run = ts;
#pragma unroll
      for (int w = 0; w < kScatterWaves; ++w) {
        cnt[w * kDigits + tid] = run;
        run += cw[w];
      }
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < kSlots; ++s) {
      if (w0 + s * kWave < end) {
        const uint32_t d = (k[s] >> a.shift) & 0xffu;
        stage[cnt[wave * kDigits + d] + rk[s]] = k[s];
      }
    }
    // the next tile's keys load while this one is written out
    {
      const uint64_t w1 = w0 + kTile;
#pragma unroll
      for (int s = 0; s < kSlots; ++s) k[s] = w1 + s * kWave < end ? src[w1 + s * kWave] : 0u;
    }
    __syncthreads();
    const uint32_t n = static_cast<uint32_t>(min(end - t0, static_cast<uint64_t>(kTile)));
    for (uint32_t i = static_cast<uint32_t>(tid); i < n; i += kScatterThreads) {
      const uint32_t key = stage[i];
      const uint32_t d = (key >> a.shift) & 0xffu;
      dst[gbase[d] + (i - tstart[d])] = key;
    }
    __syncthreads();
    if (digit_thread) gbase[tid] += tot;  // read again only after the next tile's barriers
  }
}

__device__ __forceinline__ float value_of(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}

__global__ __launch_bounds__(kSortThreads) void sort_window_kernel(WinArgs a) {
  __shared__ uint64_t wbest[kSortWaves];
  const int tid = static_cast<int>(threadIdx.x);
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const int h = static_cast<int>(blockIdx.x) / a.nblk, blk = static_cast<int>(blockIdx.x) % a.nblk;
  const uint32_t M = a.cut[h].M;
  if (M < a.K) return;  // never, for counts that add up (M >= K); the finish kernel then writes NaN
  const uint32_t per = (a.K + a.nblk - 1) / a.nblk;
  const uint32_t i0 = min(static_cast<uint64_t>(blk) * per, static_cast<uint64_t>(a.K));
  const uint32_t i1 = min(static_cast<uint64_t>(i0) + per, static_cast<uint64_t>(a.K));
  const uint32_t* lo = a.list + static_cast<int64_t>(h) * a.stride;
  const uint32_t* up = lo + (M - a.K);  // the K largest: s[t-1 .. N-1]
  uint64_t best = ~uint64_t{0};
  for (uint32_t i = i0 + static_cast<uint32_t>(tid); i < i1; i += kSortThreads) {
    const float len = value_of(up[i]) - value_of(lo[i]);
    // lengths are >= +0, so their bits order as unsigned: the smallest (length, i) wins
    const uint64_t cand = (static_cast<uint64_t>(__float_as_uint(len)) << 32) | i;
    best = cand < best ? cand : best;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint64_t u = __shfl_xor(best, o);
    best = u < best ? u : best;
  }
  if (lane == 0) wbest[wave] = best;
  __syncthreads();
  if (tid == 0) {
    uint64_t b = wbest[0];
#pragma unroll
    for (int w = 1; w < kSortWaves; ++w) b = wbest[w] < b ? wbest[w] : b;
    if (b != ~uint64_t{0}) atomicMin(reinterpret_cast<unsigned long long*>(&a.best[h]), static_cast<unsigned long long>(b));
  }
}

__global__ __launch_bounds__(256) void sort_finish_kernel(WinArgs a) {
  const int64_t h = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (h >= a.H) return;
  const uint64_t b = a.best[h];
  const uint32_t M = a.cut[h].M, i = static_cast<uint32_t>(b);
  if (M < a.K || b == ~uint64_t{0}) {
    a.win_min[h] = a.win_max[h] = __uint_as_float(0x7fc00000u);
    return;
  }
  const uint32_t* lo = a.list + h * a.stride;
  a.win_min[h] = value_of(lo[i]);
  a.win_max[h] = value_of(lo[M - a.K + i]);
}

}  // namespace

int sort_plan(bool bshd, int64_t B, int64_t H, int64_t S, int64_t D, int64_t K, SortPlan& sp) {
  const int st = hist_plan(1, bshd, 4, B, H, S, D, sp.hp);
  if (st != FA3Q_OK) return st;
  sp.N = B * S * D;
  if (K < 1 || K > sp.N) return FA3Q_ERR_RATIO;
  // enough workgroups to fill the chip for lists of about 2K keys (whatever M turns out to be,
  // the blocks cover it), never below four tiles each
  const int64_t m_est = std::min<int64_t>(sp.N, 2 * K);
  const int64_t by_heads = (kTargetGroups + H - 1) / H;
  const int64_t by_tiles = (m_est + 2 * kTile - 1) / (2 * kTile);
  sp.nblk = static_cast<int32_t>(std::max<int64_t>(1, std::min<int64_t>({by_heads, by_tiles, kMaxBlocks})));
  if (H * sp.nblk > (int64_t{1} << 31) - 1) return FA3Q_ERR_SHAPE;
  sp.rec_bytes = sp.hp.bytes;
  sp.cut_bytes = round_up(static_cast<size_t>(H) * sizeof(TailCut), 256);
  sp.best_bytes = round_up(static_cast<size_t>(H) * sizeof(uint64_t), 256);
  sp.bcount_bytes = round_up(static_cast<size_t>(H) * kDigits * sp.nblk * sizeof(uint32_t), 256);
  sp.list_bytes = round_up(static_cast<size_t>(H) * static_cast<size_t>(sp.N) * sizeof(uint32_t), 256);
  sp.bytes = sp.rec_bytes + sp.cut_bytes + sp.best_bytes + sp.bcount_bytes + 2 * sp.list_bytes;
  return FA3Q_OK;
}

int sort_launch(const void* const* xs, int64_t nb, int64_t H, int64_t t, int64_t K, const SortPlan& sp,
                float* win_min, float* win_max, void* workspace, hipStream_t stream) {
  unsigned char* w = static_cast<unsigned char*>(workspace);
  uint32_t* records = reinterpret_cast<uint32_t*>(w);
  TailCut* cut = reinterpret_cast<TailCut*>(w + sp.rec_bytes);
  uint64_t* best = reinterpret_cast<uint64_t*>(w + sp.rec_bytes + sp.cut_bytes);
  uint32_t* bcount = reinterpret_cast<uint32_t*>(w + sp.rec_bytes + sp.cut_bytes + sp.best_bytes);
  uint32_t* list_a = reinterpret_cast<uint32_t*>(w + sp.rec_bytes + sp.cut_bytes + sp.best_bytes + sp.bcount_bytes);
  uint32_t* list_b = reinterpret_cast<uint32_t*>(reinterpret_cast<unsigned char*>(list_a) + sp.list_bytes);
  const dim3 g_blocks(static_cast<unsigned>(H * sp.nblk)), blk(kSortThreads), blk_sc(kScatterThreads);
  for (int64_t b = 0; b < nb; ++b) {
    const int st = hist_f32_collect(xs[b], H, t, K, sp.hp, records, cut, best, list_a, sp.N, stream);
    if (st != FA3Q_OK) return st;
    SortArgs sa;
    sa.stride = sp.N;
    sa.cut = cut;
    sa.bcount = bcount;
    sa.nblk = sp.nblk;
    for (int pass = 0; pass < 4; ++pass) {
      sa.src = (pass & 1) ? list_b : list_a;
      sa.dst = (pass & 1) ? list_a : list_b;
      sa.shift = 8 * pass;
      hipLaunchKernelGGL(lsd_count_kernel, g_blocks, blk, 0, stream, sa);
      hipLaunchKernelGGL(pass == 3 ? lsd_scatter_kernel<true> : lsd_scatter_kernel<false>, g_blocks, blk_sc, 0, stream,
                         sa);
    }
    WinArgs wa;
    wa.list = list_a;  // four passes: sorted back into the first buffer
    wa.stride = sp.N;
    wa.cut = cut;
    wa.best = best;
    wa.K = static_cast<uint32_t>(K);
    wa.nblk = sp.nblk;
    wa.H = static_cast<int32_t>(H);
    wa.win_min = win_min + b * H;
    wa.win_max = win_max + b * H;
    hipLaunchKernelGGL(sort_window_kernel, g_blocks, blk, 0, stream, wa);
    hipLaunchKernelGGL(sort_finish_kernel, dim3(static_cast<unsigned>((H + 255) / 256)), dim3(256), 0, stream, wa);
  }
  return launch_status();
}

}  // namespace fa3q
