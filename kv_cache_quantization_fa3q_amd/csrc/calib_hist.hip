// Recall Window of 16-bit inputs (bf16, float16) for any window count, through one
// histogram per head.
//
// msModelSlim page "FA3量化：Flash Attention 3激活量化算法说明", section 原理 -> 算法流程:
// head h's N values are sorted (s[0] <= ... <= s[N-1]), t = int(ratio*N), and among the
// windows [s[i], s[i+t-1]], i = 0 .. N-t, the one with the smallest length wins (here:
// float32 length, smallest i on ties).
//
// A 16-bit input has at most 65536 distinct values, so the sorted head is fully described
// by the count of each value: with the keys k (order-preserving images of the values) and
// inc[k] the number of values whose key is <= k, s[r] is the value of the smallest key k
// with inc[k] > r.  The windows need no sort either.  The first shortest window starts at
// the first index of its lower value: if s[i-1] == s[i], the window at i-1 has the same
// lower end and an upper end s[i+t-2] <= s[i+t-1], so it is at most as long (float32
// subtraction is monotone), and the first minimum cannot be at i.  So only one window per
// distinct value a matters, the one at its first index f(a) = inc[a] - count[a], and
// only while f(a) <= N - t; its upper end is s[f(a) + t - 1].  Among these candidates the
// smallest (length, a) is exactly the first shortest window of the sorted head.
//
//   calib_hist_kernel         one streaming pass.  Each workgroup counts the values of one
//                             part of one head into a 65536-bin LDS histogram of packed
//                             16-bit counters (two bins per dword), one bin per raw 16-bit
//                             pattern, and writes the part's counters to the workspace.
//                             Counters wrap, exactly accounted:
//                             atomics on one dword are serialised, so each wrap of a 16-bit
//                             field is seen by exactly one increment (the one that returned
//                             0xffff in that field, or, for the upper field, a lower-field
//                             increment that returned 0xffffffff and so carried it over).
//                             That increment logs the wrap.  With W_lo lower and W_hi upper
//                             wraps of dword d, bins 2d and 2d+1 hold
//                             lower + 65536 W_lo and upper + 65536 W_hi - W_lo values (each
//                             lower wrap also carried one into the upper field).
//   calib_hist_window_kernel  one workgroup per head: sums the parts (reading the bins in
//                             key order: patterns of non-negative values ascend with their
//                             keys, those of negative values descend), scans the counts,
//                             lists the distinct values with their inc[] (in LDS while they
//                             fit, else as inc[] over all bins in the workspace), and finds
//                             each candidate's upper end by binary search over inc[].

#include <cmath>

#include "calib_hist.hpp"

namespace fa3q {
namespace {

constexpr int kHistThreads = 1024;
constexpr int kBins = 65536;
constexpr int kHistUnroll = 4;  // 16-byte vectors per thread in flight
constexpr uint32_t kMaxEvents = 2048;  // counter wraps one workgroup can log
// at most two wraps per 65536 values of a part (a lower wrap and the upper wrap its carry
// completes), so parts of this size never overflow the log
constexpr int64_t kMaxPartValues = static_cast<int64_t>(kMaxEvents) * 32768;
constexpr int kBinsPerThread = kBins / kHistThreads;  // 64
constexpr int kCtlWords = 64;  // scan and reduction scratch at the start of LDS
// one part's record in the workspace: the packed counters as they stand in LDS, a header,
// then the logged wraps (the pattern whose 16-bit field wrapped)
constexpr int64_t kPartPacked = kBins / 2;
constexpr int64_t kPartWords = kPartPacked + 64 + kMaxEvents;
enum Hdr : int { kHdrEvents = 0 };
constexpr int64_t kMinPartValues = int64_t{1} << 19;  // parts smaller than this do not pay for their record
// distinct values the window kernel keeps in LDS: a 16-bit key and a 32-bit inc[] each
constexpr int kWinCap = 24576;
constexpr size_t kWinLds = kCtlWords * 4 + std::max<size_t>(static_cast<size_t>(kWinCap) * 6, kBins * 2);

static_assert(kBinsPerThread * kHistThreads == kBins, "bins per thread");
static_assert(kWinLds <= kLdsLimit, "LDS budget");
static_assert(kWinLds >= kCtlWords * 4 + kBins * 2, "the window kernel counts wraps in its LDS");

struct HistArgs {
  const void* x[kHistMaxBatches];
  uint32_t* hist;        // [nb][H] regions of head_words: P part records each
  int64_t Lv;            // 16-byte vectors per row (row j of head h at vector (j*H + h)*Lv)
  int64_t nrows;         // rows per head
  int64_t Qv;            // vectors per head: nrows * Lv
  int64_t part_vecs;     // vectors per part (the last part may be shorter)
  int64_t part_rows;     // rows per part (kRows kernels)
  int64_t head_words;    // workspace words per head: P part records, at least 65536
  int32_t H;
  int32_t P;
  uint32_t t;            // target_num (window kernel)
  uint32_t K;            // windows: N - t + 1 (window kernel)
  float* win_min;        // [nb*H] (window kernel)
  float* win_max;
  int32_t f16;           // 1: float16 input, 0: bf16 (window kernel)
};

typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_nt16(const uint4* p) {
  const u32x4v v = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float value16(uint32_t key, bool f16) {
  const uint32_t bits = (key & 0x8000u) ? (key ^ 0x8000u) : (key ^ 0xffffu);
  return f16 ? static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)))
             : __uint_as_float(bits << 16);
}

// Counts the values of U vectors into the packed LDS histogram (with kAll false, lanes whose
// valid[u] is false skip vector u).  Pattern p lives in dword p >> 1 (byte offset (p << 1) &
// 0x1fffc), field p & 1, and is counted by adding 1 << (16 (p & 1)); both come straight
// from the dword x holding two patterns (a shift amount's low five bits: (x << 4) & 31 is
// 16 (x & 1)).  A field can only wrap once it holds 0xffff, so while no returned dword has
// bit 15 of either field set (one OR per increment) no wrap happened; otherwise each
// increment is looked at and its wraps logged (see the file header).
template <int U, bool kAll>
__device__ __forceinline__ void count_vecs(uint32_t* hist, uint32_t* ev, uint32_t* nev, const uint4 (&v)[U],
                                           const bool (&valid)[U]) {
  uint32_t o[U][8];  // returned dwords
  unsigned char* base = reinterpret_cast<unsigned char*>(hist);
  uint32_t seen = 0;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t xs[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t x = xs[d];
      const uint32_t a0 = (x << 1) & 0x1fffcu, i0 = 1u << ((x << 4) & 31u);
      const uint32_t a1 = (x >> 15) & 0x1fffcu, i1 = 1u << ((x >> 12) & 16u);
      o[u][2 * d] = 0;
      o[u][2 * d + 1] = 0;
      if (kAll || valid[u]) {
        o[u][2 * d] = atomicAdd(reinterpret_cast<uint32_t*>(base + a0), i0);
        o[u][2 * d + 1] = atomicAdd(reinterpret_cast<uint32_t*>(base + a1), i1);
      }
      seen |= o[u][2 * d] | o[u][2 * d + 1];
    }
  }
  if (seen & 0x80008000u) {  // rare: some field of a touched dword held 0x8000 or more
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t xs[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t p = (i & 1) ? (xs[i >> 1] >> 16) : (xs[i >> 1] & 0xffffu);
        const uint32_t oo = o[u][i];
        const bool counted = kAll || valid[u];
        // upper field: this increment wrapped it (odd pattern), or its carry did (even, 0xffffffff)
        const bool wrap_lo = counted && !(p & 1u) && (oo & 0xffffu) == 0xffffu;
        const bool wrap_hi = counted && ((p & 1u) ? (oo >> 16) == 0xffffu : oo == 0xffffffffu);
        if (wrap_lo || wrap_hi) {
          const uint32_t e = atomicAdd(nev, (wrap_lo && wrap_hi) ? 2u : 1u);
          if (wrap_lo) ev[e] = p;
          if (wrap_hi) ev[e + (wrap_lo ? 1u : 0u)] = p | 1u;
        }
      }
    }
  }
}

// Streams head vectors [q0, q1) of head h in batch xb into the LDS histogram, U vectors per
// thread in flight, one row segment at a time (rows longer than a round of the workgroup).
template <int U>
__device__ __forceinline__ void count_range(const HistArgs& a, const uint4* xb, int h, int64_t q, int64_t q_end,
                                            uint32_t* hist, uint32_t* ev, uint32_t* nev) {
  const int tid = static_cast<int>(threadIdx.x);
  constexpr int64_t kRound = static_cast<int64_t>(kHistThreads) * U;
  while (q < q_end) {
    const int64_t b = q / a.Lv;
    const int64_t w = q - b * a.Lv;
    const int64_t n = min(q_end - q, a.Lv - w);
    const uint4* src = xb + (b * a.H + h) * a.Lv + w;
    int64_t i0 = 0;
    for (; i0 + kRound <= n; i0 += kRound) {  // full rounds: every lane counts all U vectors
      uint4 v[U];
      bool valid[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        valid[u] = true;
        v[u] = load_nt16(src + i0 + u * kHistThreads + tid);
      }
      count_vecs<U, true>(hist, ev, nev, v, valid);
    }
    if (i0 < n) {  // the segment's last, partial round
      uint4 v[U];
      bool valid[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t i = i0 + u * kHistThreads + tid;
        valid[u] = i < n;
        v[u] = load_nt16(src + min(i, n - 1));  // in bounds; a re-read vector is not counted
      }
      count_vecs<U, false>(hist, ev, nev, v, valid);
    }
    q += n;
  }
}

// Streams rows [j0, j1) of head h in batch xb (rows of Lv <= kHistThreads vectors, as the
// (b, s) rows of D values of a (B, S, H, D) tensor) into the LDS histogram.  The workgroup
// takes G = kHistThreads / Lv rows per step, thread t vector t % Lv of row t / Lv (threads
// past G * Lv idle), so a thread's vectors lie a fixed stride apart and need no division;
// U steps in flight.
template <int U>
__device__ __forceinline__ void count_rows(const HistArgs& a, const uint4* xb, int h, int64_t j0, int64_t j1,
                                           uint32_t* hist, uint32_t* ev, uint32_t* nev) {
  const int tid = static_cast<int>(threadIdx.x);
  const int R = static_cast<int>(a.Lv);
  const int G = kHistThreads / R;
  const int rt = tid / R;
  const int wt = tid - rt * R;
  const bool on = rt < G;
  const int64_t nrows = j1 - j0;
  const int64_t stride = static_cast<int64_t>(G) * a.H * R;  // vectors from one step to the next
  const uint4* first = xb + (j0 * a.H + h) * R + wt;          // row j0: in every part
  const uint4* mine = xb + ((j0 + rt) * a.H + h) * R + wt;    // dereferenced only for rows < j1
  const int64_t full = nrows / G;                              // steps whose G rows all exist
  int64_t g = 0;
  if (G * R == kHistThreads) {
    for (; g + U <= full; g += U) {
      uint4 v[U];
      bool valid[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        valid[u] = true;
        v[u] = load_nt16(mine + (g + u) * stride);
      }
      count_vecs<U, true>(hist, ev, nev, v, valid);
    }
  }
  for (; g * G < nrows; g += U) {
    uint4 v[U];
    bool valid[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      valid[u] = on && (g + u) * G + rt < nrows;
      v[u] = load_nt16(valid[u] ? mine + (g + u) * stride : first);  // a vector not counted is re-read from row j0
    }
    count_vecs<U, false>(hist, ev, nev, v, valid);
  }
}

// Exclusive scans of two values per thread over the 1024 threads at once; tot gets the sums.
__device__ __forceinline__ uint2 block_exclusive_scan2(uint2 v, uint32_t* scratch, uint2* tot) {
  const int tid = static_cast<int>(threadIdx.x);
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  constexpr int kWaves = kHistThreads / kWave;
  uint2 inc = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint32_t ux = __shfl_up(inc.x, o), uy = __shfl_up(inc.y, o);
    if (lane >= o) {
      inc.x += ux;
      inc.y += uy;
    }
  }
  if (lane == kWave - 1) {
    scratch[wave] = inc.x;
    scratch[kWaves + wave] = inc.y;
  }
  __syncthreads();
  // every wave sums the totals of the waves before it (16 values: no second barrier)
  uint32_t bx = 0, by = 0, tx = 0, ty = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t sx = scratch[w], sy = scratch[kWaves + w];
    bx += w < wave ? sx : 0u;
    by += w < wave ? sy : 0u;
    tx += sx;
    ty += sy;
  }
  *tot = make_uint2(tx, ty);
  return make_uint2(bx + inc.x - v.x, by + inc.y - v.y);
}

__device__ __forceinline__ void zero_hist(uint32_t* hist) {
  for (int i = static_cast<int>(threadIdx.x); i < kBins / 8; i += kHistThreads)
    reinterpret_cast<uint4*>(hist)[i] = make_uint4(0, 0, 0, 0);
}

// Per-thread counts from the packed 16-bit counters of dwords dw0 .. dw0+31 (pattern order).
__device__ __forceinline__ void add_packed(uint32_t (&c)[kBinsPerThread], const uint32_t* words, int dw0) {
#pragma unroll
  for (int i = 0; i < kBinsPerThread / 8; ++i) {
    const uint4 v = reinterpret_cast<const uint4*>(words + dw0)[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      c[8 * i + 2 * k] += w[k] & 0xffffu;
      c[8 * i + 2 * k + 1] += w[k] >> 16;
    }
  }
}

// Applies logged wraps to the thread's 32 dwords (patterns 2*dw0 .. 2*dw0+63, counts cp in
// pattern order): the wraps are counted per pattern in the packed LDS histogram `cnt`
// (zeroed by the caller), then dword d gets 65536 W_lo more in its lower pattern and
// 65536 W_hi - W_lo more in its upper one.
__device__ __forceinline__ void add_wraps(uint32_t (&cp)[kBinsPerThread], uint32_t* cnt, int dw0,
                                          const uint32_t* pats, uint32_t n) {
  const int tid = static_cast<int>(threadIdx.x);
  for (uint32_t e = tid; e < n; e += kHistThreads) {
    const uint32_t p = pats[e];
    atomicAdd(&cnt[p >> 1], 1u << ((p & 1u) << 4));
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kBinsPerThread / 2; ++i) {
    const uint32_t w = cnt[dw0 + i];
    cp[2 * i] += (w & 0xffffu) << 16;
    cp[2 * i + 1] += ((w >> 16) << 16) - (w & 0xffffu);
  }
  __syncthreads();
}

// Thread t holds the 64 keys [64t, 64t+64): patterns 2*dw0 .. 2*dw0+63, ascending with the
// keys for non-negative values (key = pattern ^ 0x8000), descending for negative ones
// (key = 0xffff - pattern).
__device__ __forceinline__ int first_dword(int bin0) { return bin0 < 0x8000 ? (0xffc0 - bin0) / 2 : (bin0 - 0x8000) / 2; }

__device__ __forceinline__ void to_key_order(uint32_t (&c)[kBinsPerThread], int bin0) {
  if (bin0 < 0x8000) {  // uniform per wave
#pragma unroll
    for (int i = 0; i < kBinsPerThread / 2; ++i) {
      const uint32_t t = c[i];
      c[i] = c[kBinsPerThread - 1 - i];
      c[kBinsPerThread - 1 - i] = t;
    }
  }
}

// The Recall Window of head bh from its counts (thread t: keys [64t, 64t+64) in c, key
// order).  lds: kCtlWords of scratch, then room for kWinCap distinct values; inc_g: 65536
// words of global memory for inc[] when the distinct values do not fit in LDS (the caller
// has read whatever it held).
__device__ void window_from_counts(uint32_t (&c)[kBinsPerThread], uint32_t* lds, uint32_t* inc_g, const HistArgs& a,
                                   int64_t bh) {
  uint32_t* ctl = lds;                                  // [kCtlWords] scan and reduction scratch
  uint32_t* inc_l = lds + kCtlWords;                    // [kWinCap] inc of each distinct value
  uint16_t* key_l = reinterpret_cast<uint16_t*>(inc_l + kWinCap);  // [kWinCap] its key
  const int tid = static_cast<int>(threadIdx.x);
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const int bin0 = tid * kBinsPerThread;
  const bool f16 = a.f16 != 0;

  uint32_t sum = 0, nz = 0;
#pragma unroll
  for (int i = 0; i < kBinsPerThread; ++i) {
    sum += c[i];
    nz += c[i] ? 1u : 0u;
  }
  uint2 tot;
  const uint2 pj = block_exclusive_scan2(make_uint2(sum, nz), ctl, &tot);
  const uint32_t pre0 = pj.x, j0 = pj.y, distinct = tot.y;
  const bool in_lds = distinct <= static_cast<uint32_t>(kWinCap);

  uint64_t best = ~uint64_t{0};
  uint32_t best_hi = 0;
  if (in_lds) {
    uint32_t run = pre0, j = j0;
#pragma unroll
    for (int i = 0; i < kBinsPerThread; ++i) {
      if (c[i]) {
        run += c[i];
        inc_l[j] = run;
        key_l[j] = static_cast<uint16_t>(bin0 + i);
        ++j;
      }
    }
    __syncthreads();
    // candidates: each distinct value a whose first index f(a) is below K; the window's
    // upper end is the smallest key m with inc[m] > f(a) + t - 1
    for (uint32_t j = static_cast<uint32_t>(tid); j < distinct; j += kHistThreads) {
      const uint32_t f = j ? inc_l[j - 1] : 0u;
      if (f >= a.K) break;  // f grows with j
      const uint32_t r = f + a.t - 1;
      uint32_t lo_i = j, hi_i = distinct - 1;  // inc_l[distinct-1] = N > r
      while (lo_i < hi_i) {
        const uint32_t mid = (lo_i + hi_i) >> 1;
        if (inc_l[mid] > r) hi_i = mid; else lo_i = mid + 1;
      }
      const uint32_t kl = key_l[j], ku = key_l[lo_i];
      const float len = value16(ku, f16) - value16(kl, f16);
      const uint64_t cand = (static_cast<uint64_t>(__float_as_uint(len)) << 32) | j;
      if (cand < best) {
        best = cand;
        best_hi = (kl << 16) | ku;
      }
    }
  } else {
    // inc[] over all bins in global memory (each thread writes its own 64 bins)
    __syncthreads();
    uint32_t run = pre0;
#pragma unroll
    for (int i = 0; i < kBinsPerThread; ++i) {
      run += c[i];
      inc_g[bin0 + i] = run;
    }
    __threadfence();
    __syncthreads();
    uint32_t f = pre0;
    for (int i = 0; i < kBinsPerThread; ++i) {
      const uint32_t kl = static_cast<uint32_t>(bin0 + i);
      const uint32_t inc_k = __hip_atomic_load(inc_g + kl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (inc_k > f && f < a.K) {
        const uint32_t r = f + a.t - 1;
        uint32_t lo_i = kl, hi_i = kBins - 1;
        while (lo_i < hi_i) {
          const uint32_t mid = (lo_i + hi_i) >> 1;
          const uint32_t im = __hip_atomic_load(inc_g + mid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (im > r) hi_i = mid; else lo_i = mid + 1;
        }
        const float len = value16(lo_i, f16) - value16(kl, f16);
        const uint64_t cand = (static_cast<uint64_t>(__float_as_uint(len)) << 32) | kl;
        if (cand < best) {
          best = cand;
          best_hi = (kl << 16) | lo_i;
        }
      }
      f = inc_k;
    }
  }
  // lengths are >= +0, so their bits order as unsigned: the smallest (length, index) wins
  uint64_t m = best;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint64_t u = __shfl_xor(m, o);
    m = u < m ? u : m;
  }
  uint64_t* wbest = reinterpret_cast<uint64_t*>(ctl + 32);  // past the scan scratch
  if (lane == 0) wbest[wave] = m;
  __syncthreads();
  if (wave == 0) {  // the last wave-level step: lane w takes wave w's best
    uint64_t g = lane < kHistThreads / kWave ? wbest[lane] : ~uint64_t{0};
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) {
      const uint64_t u = __shfl_xor(g, o);
      g = u < g ? u : g;
    }
    g = __shfl(g, 0);
    if (lane < kHistThreads / kWave) wbest[lane] = g;  // hand it back to every wave
  }
  __syncthreads();
  const uint64_t g = wbest[wave];
  if (best == g && g != ~uint64_t{0}) {  // exactly one thread holds the winning candidate
    a.win_min[bh] = value16(best_hi >> 16, f16);
    a.win_max[bh] = value16(best_hi & 0xffffu, f16);
  }
}

// LDS of the counting kernel (static, so the histogram's address folds into each atomic's
// offset): the packed counters, the wrap log and its count; with kWhole the same LDS then
// serves the window search of the head.
constexpr int kHistSmemWords = std::max<int>(kBins / 2 + kMaxEvents + 16,
                                             kCtlWords + kWinCap + kWinCap / 2);
static_assert(static_cast<size_t>(kHistSmemWords) * 4 <= kLdsLimit, "LDS budget");

// kWhole: one part per head (P = 1); the workgroup holds the head's whole histogram and
// finds the window itself.  Otherwise it writes its part's record for the window kernel.
// kRows: rows of at most kHistThreads vectors, parts of whole rows (count_rows).
template <bool kWhole, bool kRows>
__global__ __launch_bounds__(kHistThreads) void calib_hist_kernel(HistArgs a) {
  __shared__ uint32_t smem[kHistSmemWords];
  uint32_t* hist = smem;               // [32768] two 16-bit counters per dword
  uint32_t* ev = smem + kBins / 2;     // [kMaxEvents] patterns whose field wrapped
  uint32_t* nev = ev + kMaxEvents;     // wrap count
  const int tid = static_cast<int>(threadIdx.x);
  zero_hist(hist);
  if (tid == 0) *nev = 0;
  __syncthreads();

  const int part = static_cast<int>(blockIdx.x) % a.P;
  const int bh = static_cast<int>(blockIdx.x) / a.P;  // batch * H + head
  const int h = bh % a.H;
  const int bi = bh / a.H;
  const uint4* xb = static_cast<const uint4*>(a.x[bi]);

  if constexpr (kRows) {
    const int64_t j0 = static_cast<int64_t>(part) * a.part_rows;
    count_rows<kHistUnroll>(a, xb, h, j0, min(j0 + a.part_rows, a.nrows), hist, ev, nev);
  } else {
    const int64_t q = static_cast<int64_t>(part) * a.part_vecs;
    count_range<kHistUnroll>(a, xb, h, q, min(q + a.part_vecs, a.Qv), hist, ev, nev);
  }
  __syncthreads();

  if constexpr (kWhole) {
    const int bin0 = tid * kBinsPerThread;
    const int dw0 = first_dword(bin0);
    uint32_t c[kBinsPerThread];
#pragma unroll
    for (int i = 0; i < kBinsPerThread; ++i) c[i] = 0;
    add_packed(c, hist, dw0);
    const uint32_t ne = *nev;
    __syncthreads();  // every thread has its counts: the LDS is free again
    if (ne) {
      zero_hist(hist);
      __syncthreads();
      add_wraps(c, hist, dw0, ev, ne);
    }
    to_key_order(c, bin0);
    window_from_counts(c, smem, a.hist + static_cast<int64_t>(bh) * a.head_words, a, bh);
  } else {
    // the part's record: the packed counters, the header and the wrap log
    uint32_t* out = a.hist + static_cast<int64_t>(bh) * a.head_words + static_cast<int64_t>(part) * kPartWords;
    for (int i = tid; i < kBins / 8; i += kHistThreads)
      reinterpret_cast<uint4*>(out)[i] = reinterpret_cast<const uint4*>(hist)[i];
    const uint32_t ne = *nev;
    if (tid == 0) out[kPartPacked + kHdrEvents] = ne;
    for (uint32_t e = tid; e < ne; e += kHistThreads) out[kPartPacked + 64 + e] = ev[e];
  }
}

// One workgroup per head after the parts' records are written: their counts summed, the
// window found from them.
__global__ __launch_bounds__(kHistThreads) void calib_hist_window_kernel(HistArgs a) {
  extern __shared__ uint32_t lds[];
  uint32_t* cnt = lds + kCtlWords;  // packed wrap counts (rare), before the window search
  const int tid = static_cast<int>(threadIdx.x);
  const int64_t bh = blockIdx.x;
  uint32_t* hs = a.hist + bh * a.head_words;
  const int bin0 = tid * kBinsPerThread;
  const int dw0 = first_dword(bin0);
  uint32_t c[kBinsPerThread];
#pragma unroll
  for (int i = 0; i < kBinsPerThread; ++i) c[i] = 0;
  uint32_t n_events = 0;
  for (int p = 0; p < a.P; ++p) {
    const uint32_t* rec = hs + static_cast<int64_t>(p) * kPartWords;
    add_packed(c, rec, dw0);
    n_events += rec[kPartPacked + kHdrEvents];
  }
  if (n_events) {
    // logged wraps (rare: a pattern past 65535 values in one part)
    for (int p = 0; p < a.P; ++p) {
      const uint32_t* rec = hs + static_cast<int64_t>(p) * kPartWords;
      zero_hist(cnt);
      __syncthreads();
      add_wraps(c, cnt, dw0, rec + kPartPacked + 64, rec[kPartPacked + kHdrEvents]);
    }
  }
  to_key_order(c, bin0);
  window_from_counts(c, lds, hs, a, bh);
}

}  // namespace

int hist_plan(int64_t nb, bool bshd, int64_t B, int64_t H, int64_t S, int64_t D, HistPlan& hp) {
  if (nb <= 0 || nb > kHistMaxBatches || B <= 0 || H <= 0 || S <= 0 || D <= 0) return FA3Q_ERR_SHAPE;
  const int64_t row = bshd ? D : S * D;
  if (row % 8 != 0) return FA3Q_ERR_SHAPE;
  const int64_t N = B * S * D;
  if (N >= (int64_t{1} << 32)) return FA3Q_ERR_SHAPE;
  hp.Lv = row / 8;
  hp.nrows = bshd ? B * S : B;
  hp.Qv = hp.nrows * hp.Lv;
  hp.rows = hp.Lv <= kHistThreads;
  // parts per head: at least one workgroup per CU over the nb batches' heads, parts not so
  // small that their records cost more than their data, and small enough for the wrap log
  int64_t P = std::max<int64_t>(1, (256 + nb * H - 1) / (nb * H));
  P = std::min<int64_t>(P, std::max<int64_t>(1, N / kMinPartValues));
  P = std::max<int64_t>(P, (N + kMaxPartValues - 1) / kMaxPartValues);
  if (hp.rows) {
    // parts of whole rows; a row holds at most 8 * kHistThreads values, so the wrap log's
    // bound is kept by adding parts
    P = std::min<int64_t>(P, hp.nrows);
    int64_t per = (hp.nrows + P - 1) / P;
    while (per > 1 && per * hp.Lv * 8 > kMaxPartValues) {
      ++P;
      per = (hp.nrows + P - 1) / P;
    }
    hp.part_rows = per;
    hp.part_vecs = per * hp.Lv;
    hp.P = (hp.nrows + per - 1) / per;
  } else {
    P = std::min<int64_t>(P, hp.Qv);
    hp.part_rows = 0;
    hp.part_vecs = (hp.Qv + P - 1) / P;
    hp.P = (hp.Qv + hp.part_vecs - 1) / hp.part_vecs;
  }
  if (hp.part_vecs * 8 > kMaxPartValues) return FA3Q_ERR_SHAPE;
  if (kHistMaxBatches * H * hp.P > (int64_t{1} << 31) - 1) return FA3Q_ERR_SHAPE;
  hp.head_words = std::max<int64_t>(hp.P * kPartWords, kBins);
  hp.bytes = static_cast<size_t>(H * hp.head_words) * sizeof(uint32_t);
  return FA3Q_OK;
}

int hist_launch(const void* const* xs, int64_t nb, int64_t H, bool f16, int64_t t, int64_t K, const HistPlan& hp,
                float* win_min, float* win_max, void* workspace, hipStream_t stream) {
  const int st = allow_dynamic_lds(reinterpret_cast<const void*>(calib_hist_window_kernel), kWinLds);
  if (st != FA3Q_OK) return st;
  HistArgs ha;
  for (int b = 0; b < kHistMaxBatches; ++b) ha.x[b] = b < nb ? xs[b] : nullptr;
  ha.hist = static_cast<uint32_t*>(workspace);
  ha.Lv = hp.Lv;
  ha.nrows = hp.nrows;
  ha.Qv = hp.Qv;
  ha.part_vecs = hp.part_vecs;
  ha.part_rows = hp.part_rows;
  ha.head_words = hp.head_words;
  ha.H = static_cast<int32_t>(H);
  ha.P = static_cast<int32_t>(hp.P);
  ha.t = static_cast<uint32_t>(t);
  ha.K = static_cast<uint32_t>(K);
  ha.win_min = win_min;
  ha.win_max = win_max;
  ha.f16 = f16 ? 1 : 0;
  const dim3 blk(kHistThreads);
  if (hp.P == 1) {  // each head counted by one workgroup, which also finds its window
    const dim3 g(static_cast<unsigned>(nb * H));
    if (hp.rows)
      hipLaunchKernelGGL((calib_hist_kernel<true, true>), g, blk, 0, stream, ha);
    else
      hipLaunchKernelGGL((calib_hist_kernel<true, false>), g, blk, 0, stream, ha);
  } else {
    const dim3 g(static_cast<unsigned>(nb * H * hp.P));
    if (hp.rows)
      hipLaunchKernelGGL((calib_hist_kernel<false, true>), g, blk, 0, stream, ha);
    else
      hipLaunchKernelGGL((calib_hist_kernel<false, false>), g, blk, 0, stream, ha);
    hipLaunchKernelGGL(calib_hist_window_kernel, dim3(static_cast<unsigned>(nb * H)), blk, kWinLds, stream, ha);
  }
  return launch_status();
}

}  // namespace fa3q
