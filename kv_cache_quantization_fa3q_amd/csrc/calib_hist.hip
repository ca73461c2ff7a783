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
// scratch at the start of LDS: scan totals [0, 32), per-wave best candidates [32, 64), the
// keys holding ranks K - 1 and t - 1 at kCtlRanks
constexpr int kCtlWords = 72;
constexpr int kCtlRanks = 64;
// one part's record in the workspace: the packed counters as they stand in LDS, a header,
// then the logged wraps (the pattern whose 16-bit field wrapped)
constexpr int64_t kPartPacked = kBins / 2;
constexpr int64_t kPartWords = kPartPacked + 64 + kMaxEvents;
enum Hdr : int { kHdrEvents = 0 };
constexpr int64_t kMinPartValues = int64_t{1} << 19;  // parts smaller than this do not pay for their record
// heads of at least this many parts have their records summed by calib_hist_sum_kernel (many
// workgroups per head) into 65536 counts after the records, which the head's window or cut
// workgroup then reads instead of the records
constexpr int kSumMinParts = 5;
constexpr int kSumThreads = 256;
constexpr int kSumDwords = kSumThreads;                // packed dwords (2 bins each) per summing workgroup
constexpr int kSumSlices = kBins / 2 / kSumDwords;     // summing workgroups per head (128)
constexpr int kSumUnroll = 8;                          // records in flight per thread
// distinct values the window kernel keeps in LDS: a 16-bit key and a 32-bit inc[] each
constexpr int kWinCap = 24576;
constexpr size_t kWinLds = kCtlWords * 4 + std::max<size_t>(static_cast<size_t>(kWinCap) * 6, kBins * 2 + kBins / 4 + 4);

static_assert(kBinsPerThread * kHistThreads == kBins, "bins per thread");
static_assert(kSumSlices * kSumDwords * 2 == kBins, "summing slices cover the bins");
static_assert(kBins / 8 % kHistThreads == 0 && kBinsPerThread == 64, "a record is 8 chunks of 16 bytes per thread");
static_assert(kWinLds <= kLdsLimit, "LDS budget");
static_assert(kWinLds >= kCtlWords * 4 + kBins * 2, "the window kernel counts wraps in its LDS");
// the merge-path search: a 16-bit prefix of every key and a prefix per 16 keys (and N) after the
// control words
constexpr int kMergeWords = kCtlWords + kBins / 2 + kBins / 16 + 1;
static_assert(kWinLds >= static_cast<size_t>(kMergeWords) * 4, "merge-path search in the window kernel's LDS");

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

// The 16-bit patterns a 16-byte vector holds, two per dword: its own eight (16-bit input),
// or (kF32) the high halves of its four float32 values.  The high half of a float32 value's
// order-preserving 32-bit key is the 16-bit key of its high-half pattern, so their histogram
// orders float32 values by their leading 16 bits.
template <bool kF32>
__device__ __forceinline__ void pattern_dwords(const uint4& v, uint32_t (&xs)[kF32 ? 2 : 4]) {
  if constexpr (kF32) {
    xs[0] = (v.x >> 16) | (v.y & 0xffff0000u);
    xs[1] = (v.z >> 16) | (v.w & 0xffff0000u);
  } else {
    xs[0] = v.x;
    xs[1] = v.y;
    xs[2] = v.z;
    xs[3] = v.w;
  }
}

// Counts the patterns of U vectors into the packed LDS histogram (with kAll false, lanes whose
// valid[u] is false skip vector u).  Pattern p lives in dword p >> 1 (byte offset (p << 1) &
// 0x1fffc), field p & 1, and is counted by adding 1 << (16 (p & 1)); both come straight
// from the dword x holding two patterns (a shift amount's low five bits: (x << 4) & 31 is
// 16 (x & 1)).  A field can only wrap once it holds 0xffff, so while no returned dword has
// bit 15 of either field set (one OR per increment) no wrap happened; otherwise each
// increment is looked at and its wraps logged (see the file header).
template <int U, bool kAll, bool kF32>
__device__ __forceinline__ void count_vecs(uint32_t* hist, uint32_t* ev, uint32_t* nev, const uint4 (&v)[U],
                                           const bool (&valid)[U]) {
  constexpr int W = kF32 ? 2 : 4;  // dwords of patterns per vector
  uint32_t o[U][2 * W];  // returned dwords
  unsigned char* base = reinterpret_cast<unsigned char*>(hist);
  uint32_t seen = 0;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    uint32_t xs[W];
    pattern_dwords<kF32>(v[u], xs);
#pragma unroll
    for (int d = 0; d < W; ++d) {
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
      uint32_t xs[W];
      pattern_dwords<kF32>(v[u], xs);
#pragma unroll
      for (int i = 0; i < 2 * W; ++i) {
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

// Streams head vectors [q0, q1) of head h in batch xb through f (f.run<kAll>(v, valid) on U
// vectors per thread in flight), one row segment at a time (rows longer than a round of the
// workgroup).  Every thread makes the same calls, so f may hold workgroup barriers.
template <int U, class F>
__device__ __forceinline__ void stream_range(const HistArgs& a, const uint4* xb, int h, int64_t q, int64_t q_end,
                                             F& f) {
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
      f.template run<true>(v, valid);
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
      f.template run<false>(v, valid);
    }
    q += n;
  }
}

// Streams rows [j0, j1) of head h in batch xb (rows of Lv <= kHistThreads vectors, as the
// (b, s) rows of D values of a (B, S, H, D) tensor) through f, as stream_range.  The workgroup
// takes G = kHistThreads / Lv rows per step, thread t vector t % Lv of row t / Lv (threads
// past G * Lv idle), so a thread's vectors lie a fixed stride apart and need no division;
// U steps in flight.
template <int U, class F>
__device__ __forceinline__ void stream_rows(const HistArgs& a, const uint4* xb, int h, int64_t j0, int64_t j1, F& f) {
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
      f.template run<true>(v, valid);
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
    f.template run<false>(v, valid);
  }
}

// The counting pass's visitor: the vectors' patterns into the packed LDS histogram.
template <int U, bool kF32>
struct CountVisit {
  uint32_t* hist;
  uint32_t* ev;
  uint32_t* nev;
  template <bool kAll>
  __device__ __forceinline__ void run(const uint4 (&v)[U], const bool (&valid)[U]) {
    count_vecs<U, kAll, kF32>(hist, ev, nev, v, valid);
  }
};

// v, as a value the compiler cannot see through: running sums over the counts built from it
// cannot be shared between loops, which would keep 64 partial sums live across them
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
  __asm__ volatile("" : "+v"(v));
  return v;
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

// Thread t holds the 64 keys [64t, 64t+64) = bin0 .. bin0+63, in key order.  Their patterns
// fill dwords dw0 .. dw0+31 of the packed counters, ascending with the keys for non-negative
// values (key = pattern ^ 0x8000), descending for negative ones (key = 0xffff - pattern).
// So key pair m (keys bin0 + 2m, bin0 + 2m + 1) is dword dw0 + m (lower field first) or,
// with rev (bin0 < 0x8000, uniform per wave), dword dw0 + 31 - m with the upper field
// first.  The helpers below read in key order with selects, not branches: a branch would
// keep the counts live in both orders.
__device__ __forceinline__ int first_dword(int bin0) { return bin0 < 0x8000 ? (0xffc0 - bin0) / 2 : (bin0 - 0x8000) / 2; }

// Adds the packed 16-bit counters of the thread's keys (dwords dw0 .. dw0+31 of words).
__device__ __forceinline__ void add_packed(uint32_t (&c)[kBinsPerThread], const uint32_t* words, int dw0, bool rev) {
#pragma unroll
  for (int q = 0; q < kBinsPerThread / 8; ++q) {  // key pairs 4q .. 4q+3
    const uint4 v = reinterpret_cast<const uint4*>(words + dw0)[rev ? 7 - q : q];
    const uint32_t w[4] = {rev ? v.w : v.x, rev ? v.z : v.y, rev ? v.y : v.z, rev ? v.x : v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = w[e] & 0xffffu, hi = w[e] >> 16;
      c[8 * q + 2 * e] += rev ? hi : lo;
      c[8 * q + 2 * e + 1] += rev ? lo : hi;
    }
  }
}

// Applies logged wraps to the thread's keys: the wraps are counted per pattern in the packed
// LDS histogram `cnt` (zeroed by the caller), then dword d gives its lower pattern 65536 W_lo
// more values and its upper one 65536 W_hi - W_lo more.
__device__ __forceinline__ void add_wraps(uint32_t (&c)[kBinsPerThread], uint32_t* cnt, int dw0, bool rev,
                                          const uint32_t* pats, uint32_t n) {
  const int tid = static_cast<int>(threadIdx.x);
  for (uint32_t e = tid; e < n; e += kHistThreads) {
    const uint32_t p = pats[e];
    atomicAdd(&cnt[p >> 1], 1u << ((p & 1u) << 4));
  }
  __syncthreads();
#pragma unroll
  for (int m = 0; m < kBinsPerThread / 2; ++m) {
    const uint32_t w = cnt[dw0 + (rev ? kBinsPerThread / 2 - 1 - m : m)];
    const uint32_t lo_add = (w & 0xffffu) << 16;
    const uint32_t hi_add = ((w >> 16) << 16) - (w & 0xffffu);
    c[2 * m] += rev ? hi_add : lo_add;
    c[2 * m + 1] += rev ? lo_add : hi_add;
  }
  __syncthreads();
}

// The Recall Window of head bh from its counts (thread t: keys [64t, 64t+64) in c, key
// order).  lds: kCtlWords of scratch, then room for kWinCap distinct values or for the
// merge search's prefixes; inc_g: 65536 words of global memory for the inc[] of keys in
// 16-key groups of more than 65535 values (the caller has read whatever it held).
//
// Only two key ranges take part: lower ends are keys with f(a) < K, so at most a_max, the
// key holding rank K - 1; upper ends hold rank f(a) + t - 1 >= t - 1, so they are at least
// m_min, the key holding rank t - 1.  (For ratios near 1 both ranges are short tails.)
// The distinct keys of the two ranges, with their inc[], are listed in LDS while they fit
// (every key below a candidate is below a_max, so the list holds each candidate's
// predecessor, and the keys left out between the ranges have inc[] <= t - 1, never an
// upper end); otherwise the merge search below runs over the two ranges.
__device__ void window_from_counts(uint32_t (&c)[kBinsPerThread], uint32_t* lds, uint32_t* inc_g, const HistArgs& a,
                                   int64_t bh) {
  uint32_t* ctl = lds;                                  // [kCtlWords] scan and reduction scratch
  uint32_t* inc_l = lds + kCtlWords;                    // [kWinCap] inc of each listed value
  uint16_t* key_l = reinterpret_cast<uint16_t*>(inc_l + kWinCap);  // [kWinCap] its key
  const int tid = static_cast<int>(threadIdx.x);
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const int bin0 = tid * kBinsPerThread;
  const bool f16 = a.f16 != 0;

  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < kBinsPerThread; ++i) sum += c[i];
  uint2 tot;
  const uint32_t pre0 = block_exclusive_scan2(make_uint2(sum, 0u), ctl, &tot).x;
  // the keys holding ranks K - 1 and t - 1: the first of the thread's keys whose inc[] passes
  // the rank is its (number of keys with inc[] <= rank)-th; the thread whose keys hold the
  // rank writes it
  {
    const uint32_t r0 = a.K - 1, r1 = a.t - 1;
    uint32_t run = pre0, n0 = 0, n1 = 0;
    // only the threads holding a rank count (inside a branch the unrolled loop keeps to its
    // own registers; in straight-line code it spilled)
    if ((pre0 <= r0 && r0 - pre0 < sum) || (pre0 <= r1 && r1 - pre0 < sum)) {
#pragma unroll
      for (int i = 0; i < kBinsPerThread; ++i) {
        run = opaque(run + c[i]);
        n0 += run <= r0 ? 1u : 0u;
        n1 += run <= r1 ? 1u : 0u;
      }
    }
    if (pre0 <= r0 && r0 < run) ctl[kCtlRanks] = static_cast<uint32_t>(bin0) + n0;
    if (pre0 <= r1 && r1 < run) ctl[kCtlRanks + 1] = static_cast<uint32_t>(bin0) + n1;
  }
  __syncthreads();
  const uint32_t a_max = ctl[kCtlRanks], m_min = ctl[kCtlRanks + 1];
  // the thread's listed keys: bin0 + i with i < cut_lo (at most a_max) or i >= cut_hi (at
  // least m_min); each loop below takes the cuts through opaque(), so that the compiler
  // does not keep 64 predicates live from one loop to the next
  const uint32_t ub0 = static_cast<uint32_t>(bin0);
  const uint32_t cut_lo = a_max >= ub0 ? min(a_max - ub0 + 1, static_cast<uint32_t>(kBinsPerThread)) : 0u;
  const uint32_t cut_hi = m_min > ub0 ? min(m_min - ub0, static_cast<uint32_t>(kBinsPerThread)) : 0u;
  // a thread whose keys hold no value, or all lie between the two ranges, lists nothing: it
  // skips the loops (most threads: values occupy a small part of the 65536 keys)
  const bool lists = sum > 0u && (cut_lo > 0u || cut_hi < static_cast<uint32_t>(kBinsPerThread));
  uint32_t nz = 0;
  if (lists) {
    const uint32_t lo = opaque(cut_lo), hi = opaque(cut_hi);
#pragma unroll
    for (int i = 0; i < kBinsPerThread; ++i)
      nz += (c[i] && (static_cast<uint32_t>(i) < lo || static_cast<uint32_t>(i) >= hi)) ? 1u : 0u;
  }
  const uint32_t j0 = block_exclusive_scan2(make_uint2(nz, 0u), ctl, &tot).x;
  const uint32_t distinct = tot.x;
  const bool in_lds = distinct <= static_cast<uint32_t>(kWinCap);

  uint64_t best = ~uint64_t{0};
  uint32_t best_hi = 0;
  if (in_lds) {
    if (nz) {
      uint32_t run = pre0, j = j0;
      const uint32_t lo = opaque(cut_lo), hi = opaque(cut_hi);
#pragma unroll
      for (int i = 0; i < kBinsPerThread; ++i) {
        run = opaque(run + c[i]);
        if (c[i] && (static_cast<uint32_t>(i) < lo || static_cast<uint32_t>(i) >= hi)) {
          inc_l[j] = run;
          key_l[j] = static_cast<uint16_t>(bin0 + i);
          ++j;
        }
      }
    }
    __syncthreads();
    // candidates: each listed value a whose first index f(a) is below K; the window's
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
    // Too many values for the list (float16 heads reach tens of thousands of distinct values
    // at ratios far from 1).  inc[] of every key goes to LDS as a 32-bit prefix per 16-key
    // group plus each key's 16-bit inclusive prefix inside its group; a group of more than
    // 65535 values keeps its keys' inc[] in inc_g instead.  The upper ends come from merging
    // two ascending sequences, A = inc[m] for keys m >= m_min and B = min(f(a), K) + t - 1
    // for keys a <= a_max: merged with A first on ties, B[a] is preceded by exactly the
    // A[m] <= B[a], so m_min plus their number is the smallest m with inc[m] > B[a], the
    // upper end of a's window (for a candidate, f(a) < K and B[a] = f(a) + t - 1 < N =
    // inc[65535]; clamping f(a) at K keeps B ascending and below 2^32; every A[m] left out
    // below m_min is <= t - 1 <= B[a]).  Each thread emits an equal share of the merge from
    // the split its diagonal gives (merge path).
    //
    // Both arrays are stored XOR-swizzled: in the search, the lanes of a wave sit a few dozen
    // keys apart, which unswizzled would put many lanes' 16-bit reads in one LDS bank.  Key k
    // lives at p16[k ^ (((k >> 6) & 31) << 1)] and group g's prefix at gpre[g ^ ((g >> 5) & 3)];
    // both permute only inside a thread's own 64 keys / 4 groups.
    uint16_t* p16 = reinterpret_cast<uint16_t*>(lds + kCtlWords);  // [65536] prefix inside the group
    uint32_t* gpre = lds + kCtlWords + kBins / 2;                    // [4097] values below each group; N
    {
      uint32_t run = pre0;
      const uint32_t m = (static_cast<uint32_t>(tid) & 31u) << 1;    // the swizzle of this thread's keys
      uint4* dst = reinterpret_cast<uint4*>(p16 + bin0);
#pragma unroll
      for (int q = 0; q < kBinsPerThread / 16; ++q) {  // the thread's four groups
        const uint32_t g0 = run;
        gpre[(tid * (kBinsPerThread / 16) + q) ^ ((tid >> 3) & 3)] = g0;
        uint32_t tsum = 0;
#pragma unroll
        for (int e = 0; e < 16; ++e) tsum += c[16 * q + e];
        const bool heavy = tsum > 0xffffu;
        uint32_t w[8];
        uint32_t in = 0;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          in = opaque(in + c[16 * q + e]);
          if (heavy) inc_g[bin0 + 16 * q + e] = g0 + in;
          w[e >> 1] = (e & 1) ? (w[e >> 1] | ((in & 0xffffu) << 16)) : (in & 0xffffu);
        }
        // keys 16q + 8h + e (h = 0, 1) go to the 8-key slot (2q + h) ^ (m >> 3), dword (e >> 1) ^ ((m >> 1) & 3)
        const uint32_t pd = (m >> 1) & 3u;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          uint32_t x0 = w[4 * h], x1 = w[4 * h + 1], x2 = w[4 * h + 2], x3 = w[4 * h + 3];
          if (pd & 1u) {  // dword p takes dword p ^ pd: swap pairs, then halves
            const uint32_t t0 = x0, t2 = x2;
            x0 = x1; x1 = t0; x2 = x3; x3 = t2;
          }
          if (pd & 2u) {
            const uint32_t t0 = x0, t1 = x1;
            x0 = x2; x1 = x3; x2 = t0; x3 = t1;
          }
          dst[(2 * q + h) ^ (m >> 3)] = make_uint4(x0, x1, x2, x3);
        }
        run = g0 + tsum;
      }
      if (tid == kHistThreads - 1) gpre[kBins / 16] = run;  // unswizzled: (4096 >> 5) & 3 == 0
    }
    // the barrier orders the workgroup's global stores too: no device-scope fence (on a chip
    // of several L2 caches that would write back and invalidate this one's L2)
    __syncthreads();
    // inc[k] in one LDS round trip (the three reads issue together; the empty asm keeps the
    // 16-bit read ahead of the rare branch to global memory)
    auto inc_at = [&](uint32_t k) -> uint32_t {
      const uint32_t g = k >> 4;
      const uint32_t e0 = gpre[g ^ ((g >> 5) & 3u)], e1 = gpre[(g + 1) ^ (((g + 1) >> 5) & 3u)];
      uint32_t v = e0 + static_cast<uint32_t>(p16[k ^ (((k >> 6) & 31u) << 1)]);
      __asm__ volatile("" : "+v"(v));
      if (e1 - e0 > 0xffffu) v = inc_g[k];
      return v;
    };
    auto b_of = [&](uint32_t exc) -> uint32_t { return min(exc, a.K) + a.t - 1; };
    const uint32_t nA = static_cast<uint32_t>(kBins) - m_min, nB = a_max + 1;
    const uint32_t total = nA + nB;
    const uint32_t per = (total + kHistThreads - 1) / kHistThreads;  // merge outputs per thread, <= 128
    const uint32_t d = min(static_cast<uint32_t>(tid) * per, total);
    const uint32_t steps = min(per, total - d);
    uint32_t lo_i = d > nB ? d - nB : 0u;
    uint32_t hi_i = min(d, nA);
    while (lo_i < hi_i) {  // the most A elements among the first d outputs
      const uint32_t mid = (lo_i + hi_i + 1) >> 1;
      const uint32_t y = d - mid;  // < nB, since mid > d - nB
      const uint32_t am = inc_at(m_min + mid - 1), by = inc_at(y ? y - 1 : 0u);
      if (am <= b_of(y ? by : 0u)) lo_i = mid; else hi_i = mid - 1;
    }
    // The walk: one merge output per step without divergence -- the step's choice picks the
    // key whose inc[] is read next (the next A key after an A, j + 1 after a B), so every
    // lane issues one read per step.  Within a thread's outputs A and B are never both
    // exhausted, so a B step always has j < nB, and a candidate's upper end is a key of A
    // since B[j] < inc[65535].
    uint32_t i = lo_i, j = d - lo_i;
    uint32_t ai = inc_at(min(m_min + i, static_cast<uint32_t>(kBins) - 1));
    uint32_t ej = j ? inc_at(j - 1) : 0u;                             // f(j): values below key j
    uint32_t ij = inc_at(min(j, static_cast<uint32_t>(kBins) - 1));   // inc[j]
    for (uint32_t step = 0; step < steps; ++step) {
      const bool take_a = i < nA && (j >= nB || ai <= b_of(ej));
      // a B step on a key that holds values with f(j) < K: a candidate window [key j, key m_min + i]
      const uint32_t ku = (m_min + i) & 0xffffu;
      const bool cand_ok = !take_a && ij > ej && ej < a.K;
      const float len = value16(ku, f16) - value16(j & 0xffffu, f16);
      const uint64_t cand = (static_cast<uint64_t>(__float_as_uint(len)) << 32) | j;
      if (cand_ok && cand < best) {
        best = cand;
        best_hi = (j << 16) | ku;
      }
      const uint32_t v = inc_at(min(take_a ? m_min + i + 1 : j + 1, static_cast<uint32_t>(kBins) - 1));
      if (take_a) {
        ++i;
        ai = v;  // past the end: never read again
      } else {
        ++j;
        ej = ij;
        ij = v;
      }
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
constexpr int kHistSmemWords = std::max<int>(std::max<int>(kBins / 2 + kMaxEvents + 16, kCtlWords + kWinCap + kWinCap / 2),
                                             kMergeWords);
static_assert(static_cast<size_t>(kHistSmemWords) * 4 <= kLdsLimit, "LDS budget");

// kWhole: one part per head (P = 1); the workgroup holds the head's whole histogram and
// finds the window itself.  Otherwise it writes its part's record for the window kernel.
// kRows: rows of at most kHistThreads vectors, parts of whole rows (stream_rows).  kF32:
// float32 input, counted by the high halves of its values (records only).
template <bool kWhole, bool kRows, bool kF32>
__global__ __launch_bounds__(kHistThreads) void calib_hist_kernel(HistArgs a) {
  static_assert(!(kWhole && kF32), "float32 heads are counted into records");
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

  CountVisit<kHistUnroll, kF32> f{hist, ev, nev};
  if constexpr (kRows) {
    const int64_t j0 = static_cast<int64_t>(part) * a.part_rows;
    stream_rows<kHistUnroll>(a, xb, h, j0, min(j0 + a.part_rows, a.nrows), f);
  } else {
    const int64_t q = static_cast<int64_t>(part) * a.part_vecs;
    stream_range<kHistUnroll>(a, xb, h, q, min(q + a.part_vecs, a.Qv), f);
  }
  __syncthreads();

  if constexpr (kWhole) {
    const int bin0 = tid * kBinsPerThread;
    const int dw0 = first_dword(bin0);
    uint32_t c[kBinsPerThread];
#pragma unroll
    for (int i = 0; i < kBinsPerThread; ++i) c[i] = 0;
    add_packed(c, hist, dw0, bin0 < 0x8000);
    const uint32_t ne = *nev;
    __syncthreads();  // every thread has its counts: the LDS is free again
    if (ne) {
      zero_hist(hist);
      __syncthreads();
      add_wraps(c, hist, dw0, bin0 < 0x8000, ev, ne);
    }
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

// Sums the part records of head blockIdx.x / kSumSlices over packed dwords [d_lo, d_lo +
// kSumDwords) of slice blockIdx.x % kSumSlices: thread t takes dword d_lo + t (two bins) of
// every record, kSumUnroll records in flight, and the logged wraps of every part that fall in
// the slice are added through LDS.  Writes the slice's counts, in pattern order, to the head's
// 65536 summed counts after its records.
__global__ __launch_bounds__(kSumThreads) void calib_hist_sum_kernel(HistArgs a) {
  __shared__ uint32_t wraps[2 * kSumDwords];  // wrap corrections of the slice's bins (rare)
  const int tid = static_cast<int>(threadIdx.x);
  const int64_t bh = blockIdx.x / kSumSlices;
  const int slice = static_cast<int>(blockIdx.x % kSumSlices);
  uint32_t* hs = a.hist + bh * a.head_words;
  const int d_lo = slice * kSumDwords;
  const uint32_t* src = hs + d_lo + tid;
  const uint32_t* hdr = hs + kPartPacked + kHdrEvents;
  uint32_t lo = 0, hi = 0, n_events = 0;  // n_events: the same for every thread
  int p = 0;
  for (; p + kSumUnroll <= a.P; p += kSumUnroll) {  // the records' dwords and headers load together
    uint32_t w[kSumUnroll], n[kSumUnroll];
#pragma unroll
    for (int u = 0; u < kSumUnroll; ++u) {
      w[u] = src[static_cast<int64_t>(p + u) * kPartWords];
      n[u] = hdr[static_cast<int64_t>(p + u) * kPartWords];
    }
#pragma unroll
    for (int u = 0; u < kSumUnroll; ++u) {
      lo += w[u] & 0xffffu;
      hi += w[u] >> 16;
      n_events += n[u];
    }
  }
  for (; p < a.P; ++p) {
    const uint32_t w = src[static_cast<int64_t>(p) * kPartWords];
    lo += w & 0xffffu;
    hi += w >> 16;
    n_events += hdr[static_cast<int64_t>(p) * kPartWords];
  }
  if (n_events) {
    // a lower wrap of dword d gave bin 2d 65536 more and carried one into bin 2d+1's field; an
    // upper wrap gave bin 2d+1 65536 more (modulo 2^32, as the counts are)
    for (int i = tid; i < 2 * kSumDwords; i += kSumThreads) wraps[i] = 0;
    __syncthreads();
    for (int q = 0; q < a.P; ++q) {
      const uint32_t* rec = hs + static_cast<int64_t>(q) * kPartWords;
      const uint32_t n = rec[kPartPacked + kHdrEvents];
      for (uint32_t e = tid; e < n; e += kSumThreads) {
        const uint32_t pat = rec[kPartPacked + 64 + e];
        const int d = static_cast<int>(pat >> 1);
        if (d < d_lo || d >= d_lo + kSumDwords) continue;
        const int i = 2 * (d - d_lo) + static_cast<int>(pat & 1u);
        atomicAdd(&wraps[i], 65536u);
        if (!(pat & 1u)) atomicSub(&wraps[i + 1], 1u);
      }
    }
    __syncthreads();
    lo += wraps[2 * tid];
    hi += wraps[2 * tid + 1];
  }
  *reinterpret_cast<uint2*>(hs + static_cast<int64_t>(a.P) * kPartWords + 2 * (d_lo + tid)) = make_uint2(lo, hi);
}

// The counts of the thread's 64 keys [64t, 64t+64) (key order) of the head whose region is
// hs: summed from its P part records, or read from the summed counts after them (P >=
// kSumMinParts).  cnt: 32768 words of LDS for the rare logged wraps.
__device__ __forceinline__ void head_counts(uint32_t (&c)[kBinsPerThread], const uint32_t* hs, int P, uint32_t* cnt) {
  const int tid = static_cast<int>(threadIdx.x);
  const int bin0 = tid * kBinsPerThread;
  const bool rev = bin0 < 0x8000;
  if (P >= kSumMinParts) {
    // patterns ascend with the keys for non-negative values (pattern = key ^ 0x8000) and
    // descend for negative ones (pattern = 0xffff - key); selects, not branches, pick the order
    const uint32_t* sums = hs + static_cast<int64_t>(P) * kPartWords + (rev ? 0xffc0 - bin0 : bin0 - 0x8000);
#pragma unroll
    for (int q = 0; q < kBinsPerThread / 4; ++q) {
      const uint4 v = reinterpret_cast<const uint4*>(sums)[rev ? kBinsPerThread / 4 - 1 - q : q];
      c[4 * q] = rev ? v.w : v.x;
      c[4 * q + 1] = rev ? v.z : v.y;
      c[4 * q + 2] = rev ? v.y : v.z;
      c[4 * q + 3] = rev ? v.x : v.w;
    }
    return;
  }
  const int dw0 = first_dword(bin0);
  uint32_t n_events = 0;
  // Each record goes through LDS: coalesced 16-byte loads in, then every thread takes its 32
  // dwords (read straight from global memory, a wave's loads would touch 64 lines each).
  // 16-byte chunk i sits at chunk i ^ ((i >> 3) & 7), so the eight chunks of a thread's block
  // land in different banks from its neighbours'.  (Loading two records at once spills: the
  // 64 counts hold half the registers.)
  constexpr int kChunks = kBins / 8 / kHistThreads;
  uint4* st = reinterpret_cast<uint4*>(cnt);
  const int blk = dw0 / 32;  // the thread's 8 chunks: blk * 8 + q
  auto stage = [&](const uint4 (&v)[kChunks]) {
#pragma unroll
    for (int k = 0; k < kChunks; ++k) {
      const int i = tid + k * kHistThreads;
      st[i ^ ((i >> 3) & 7)] = v[k];
    }
  };
  auto take = [&](bool first) {  // first: the counts start from this record
#pragma unroll
    for (int q = 0; q < kBinsPerThread / 8; ++q) {
      const int qq = rev ? 7 - q : q;
      const uint4 w4 = st[8 * blk + (qq ^ (blk & 7))];
      const uint32_t w[4] = {rev ? w4.w : w4.x, rev ? w4.z : w4.y, rev ? w4.y : w4.z, rev ? w4.x : w4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = w[e] & 0xffffu, hi = w[e] >> 16;
        c[8 * q + 2 * e] = (first ? 0u : c[8 * q + 2 * e]) + (rev ? hi : lo);
        c[8 * q + 2 * e + 1] = (first ? 0u : c[8 * q + 2 * e + 1]) + (rev ? lo : hi);
      }
    }
  };
  for (int p = 0; p < P; ++p) {
    const uint32_t* rec = hs + static_cast<int64_t>(p) * kPartWords;
    uint4 v[kChunks];
#pragma unroll
    for (int k = 0; k < kChunks; ++k) v[k] = reinterpret_cast<const uint4*>(rec)[tid + k * kHistThreads];
    n_events += rec[kPartPacked + kHdrEvents];
    stage(v);
    __syncthreads();
    take(p == 0);
    __syncthreads();
  }
  if (n_events) {
    // logged wraps (rare: a pattern past 65535 values in one part)
    for (int p = 0; p < P; ++p) {
      const uint32_t* rec = hs + static_cast<int64_t>(p) * kPartWords;
      zero_hist(cnt);
      __syncthreads();
      add_wraps(c, cnt, dw0, rev, rec + kPartPacked + 64, rec[kPartPacked + kHdrEvents]);
    }
  }
}

// One workgroup per head after the parts' records are written: their counts summed, the
// window found from them.
__global__ __launch_bounds__(kHistThreads) void calib_hist_window_kernel(HistArgs a) {
  extern __shared__ uint32_t lds[];
  const int64_t bh = blockIdx.x;
  uint32_t* hs = a.hist + bh * a.head_words;
  uint32_t c[kBinsPerThread];
  head_counts(c, hs, a.P, lds + kCtlWords);
  window_from_counts(c, lds, hs, a, bh);
}

// ---- float32 heads: the cut and the collected tails -------------------------------------
//
// A float32 head has too many distinct values for a histogram of its own, but the histogram
// of its values' leading 16 bits (the high halves of their 32-bit keys) says which leading
// keys hold ranks K - 1 and t - 1: a_max and m_min.  Every value of rank below K has a
// leading key <= a_max, every value of rank >= t - 1 one >= m_min, so the values whose
// leading key is <= a_max or >= m_min hold both tails of the sorted head; sorted, their first
// K are s[0 .. K-1] and their last K are s[t-1 .. N-1] (any other collected value lies
// between the two tails).  When a_max >= m_min that is every value of the head.

// One workgroup per head after the parts' records are written: the leading-key counts summed,
// a_max and m_min found, the number of collected values M, an empty list and no best window.
__global__ __launch_bounds__(kHistThreads) void calib_cut_kernel(HistArgs a, TailCut* cut, uint64_t* best) {
  extern __shared__ uint32_t lds[];
  uint32_t* ctl = lds;              // [kCtlWords] scan scratch, the ranks' keys and prefixes
  uint32_t* cnt = lds + kCtlWords;  // packed wrap counts (rare)
  const int tid = static_cast<int>(threadIdx.x);
  const int64_t bh = blockIdx.x;
  const int bin0 = tid * kBinsPerThread;
  uint32_t c[kBinsPerThread];
  head_counts(c, a.hist + bh * a.head_words, a.P, cnt);
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < kBinsPerThread; ++i) sum += c[i];
  uint2 tot;
  const uint32_t pre0 = block_exclusive_scan2(make_uint2(sum, 0u), ctl, &tot).x;
  // a_max with inc[a_max] (the first inclusive prefix past K - 1), m_min with inc[m_min - 1]
  // (the last prefix at most t - 1, or the values below the thread's first key)
  const uint32_t r0 = a.K - 1, r1 = a.t - 1;
  uint32_t run = pre0, n0 = 0, n1 = 0, inc_a = ~0u, exc_m = pre0;
  if ((pre0 <= r0 && r0 - pre0 < sum) || (pre0 <= r1 && r1 - pre0 < sum)) {
#pragma unroll
    for (int i = 0; i < kBinsPerThread; ++i) {
      run = opaque(run + c[i]);
      n0 += run <= r0 ? 1u : 0u;
      n1 += run <= r1 ? 1u : 0u;
      inc_a = min(inc_a, run > r0 ? run : ~0u);
      exc_m = max(exc_m, run <= r1 ? run : 0u);
    }
  }
  if (pre0 <= r0 && r0 < run) {
    ctl[kCtlRanks] = static_cast<uint32_t>(bin0) + n0;
    ctl[kCtlRanks + 2] = inc_a;
  }
  if (pre0 <= r1 && r1 < run) {
    ctl[kCtlRanks + 1] = static_cast<uint32_t>(bin0) + n1;
    ctl[kCtlRanks + 3] = exc_m;
  }
  __syncthreads();
  if (tid == 0) {
    TailCut tc;
    tc.a_max = ctl[kCtlRanks];
    tc.m_min = ctl[kCtlRanks + 1];
    tc.M = tc.a_max < tc.m_min ? ctl[kCtlRanks + 2] + (tot.x - ctl[kCtlRanks + 3]) : tot.x;
    tc.fill = 0;
    cut[bh] = tc;
    best[bh] = ~uint64_t{0};
  }
}
constexpr size_t kCutLds = (static_cast<size_t>(kCtlWords) + kBins / 2) * 4;
static_assert(kCutLds <= kLdsLimit, "LDS budget");

// keys a collecting workgroup stages in LDS; it writes them out once a round could overflow
constexpr uint32_t kCollectCap = 32768;
constexpr uint32_t kCollectRound = kHistThreads * kHistUnroll * 4;  // float32 values per round
constexpr uint32_t kCollectFlush = kCollectCap - kCollectRound;

// Unsigned key whose order is the float32 total order with -0.0 below +0.0.
__device__ __forceinline__ uint32_t key32(uint32_t b) { return (b & 0x80000000u) ? ~b : (b | 0x80000000u); }

// The collecting pass's visitor: the 32-bit keys of the values whose leading key is <= a_max or
// >= m_min are appended to the LDS stage (each thread's keys at its offset from a prefix sum
// over the wave, one LDS atomic per wave and round), which is written to the head's list (one
// global atomic per write) when another round might not fit.
template <int U>
struct CollectVisit {
  uint32_t* buf;    // LDS [kCollectCap]
  uint32_t* nbuf;   // LDS: keys staged
  uint32_t* gbase;  // LDS: list position of a write-out
  uint32_t a_max, m_min;
  uint32_t* fill;   // the head's append counter
  uint32_t* list;   // the head's list
  __device__ __forceinline__ void flush(uint32_t n) {
    if (threadIdx.x == 0) {
      *gbase = atomicAdd(fill, n);
      *nbuf = 0;
    }
    __syncthreads();
    const uint32_t g = *gbase;
    for (uint32_t i = threadIdx.x; i < n; i += kHistThreads) list[g + i] = buf[i];
    __syncthreads();
  }
  template <bool kAll>
  __device__ __forceinline__ void run(const uint4 (&v)[U], const bool (&valid)[U]) {
    uint32_t k[U][4];
    uint32_t sel = 0, c = 0;  // bit 4u+e: value e of vector u is collected
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        k[u][e] = key32(w[e]);
        const uint32_t lead = k[u][e] >> 16;
        const bool on = (kAll || valid[u]) && (lead <= a_max || lead >= m_min);
        sel |= on ? 1u << (4 * u + e) : 0u;
        c += on ? 1u : 0u;
      }
    }
    // the wave's inclusive prefix of the counts; its last lane holds the total
    const int lane = lane_id();
    uint32_t inc = c;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const uint32_t t = __shfl_up(inc, o);
      if (lane >= o) inc += t;
    }
    const uint32_t total = __builtin_amdgcn_readlane(inc, kWave - 1);
    if (total) {  // uniform over the wave
      uint32_t base = 0;
      if (lane == 0) base = atomicAdd(nbuf, total);
      uint32_t pos = __builtin_amdgcn_readfirstlane(base) + inc - c;
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (sel & (1u << (4 * u + e))) buf[pos++] = k[u][e];
    }
    __syncthreads();
    const uint32_t n = *nbuf;
    __syncthreads();  // every thread has read the count before the next round appends
    if (n > kCollectFlush) flush(n);
  }
};

// The parts of the counting pass again, one workgroup each: the head's tail values into its list.
template <bool kRows>
__global__ __launch_bounds__(kHistThreads) void calib_collect_kernel(HistArgs a, TailCut* cut, uint32_t* lists,
                                                                      int64_t stride) {
  __shared__ uint32_t buf[kCollectCap];
  __shared__ uint32_t misc[2];
  const int part = static_cast<int>(blockIdx.x) % a.P;
  const int bh = static_cast<int>(blockIdx.x) / a.P;  // one batch: the head
  const uint4* xb = static_cast<const uint4*>(a.x[0]);
  if (threadIdx.x == 0) misc[0] = 0;
  __syncthreads();
  CollectVisit<kHistUnroll> f{buf, misc, misc + 1, cut[bh].a_max, cut[bh].m_min, &cut[bh].fill,
                              lists + static_cast<int64_t>(bh) * stride};
  if constexpr (kRows) {
    const int64_t j0 = static_cast<int64_t>(part) * a.part_rows;
    stream_rows<kHistUnroll>(a, xb, bh, j0, min(j0 + a.part_rows, a.nrows), f);
  } else {
    const int64_t q = static_cast<int64_t>(part) * a.part_vecs;
    stream_range<kHistUnroll>(a, xb, bh, q, min(q + a.part_vecs, a.Qv), f);
  }
  const uint32_t n = misc[0];  // settled: the last round ended on a barrier
  if (n) f.flush(n);
}

}  // namespace

int hist_plan(int64_t nb, bool bshd, int vpv, int64_t B, int64_t H, int64_t S, int64_t D, HistPlan& hp) {
  if (nb <= 0 || nb > kHistMaxBatches || B <= 0 || H <= 0 || S <= 0 || D <= 0) return FA3Q_ERR_SHAPE;
  if (vpv != 4 && vpv != 8) return FA3Q_ERR_SHAPE;
  const int64_t row = bshd ? D : S * D;
  if (row % vpv != 0) return FA3Q_ERR_SHAPE;
  const int64_t N = B * S * D;
  if (N >= (int64_t{1} << 32)) return FA3Q_ERR_SHAPE;
  hp.vpv = vpv;
  hp.Lv = row / vpv;
  hp.nrows = bshd ? B * S : B;
  hp.Qv = hp.nrows * hp.Lv;
  hp.rows = hp.Lv <= kHistThreads;
  // parts per head: at least one workgroup per CU over the nb batches' heads, parts not so
  // small that their records cost more than their data, and small enough for the wrap log
  int64_t P = std::max<int64_t>(1, (256 + nb * H - 1) / (nb * H));
  P = std::min<int64_t>(P, std::max<int64_t>(1, N / kMinPartValues));
  P = std::max<int64_t>(P, (N + kMaxPartValues - 1) / kMaxPartValues);
  if (hp.rows) {
    // parts of whole rows; a row holds at most vpv * kHistThreads values, so the wrap log's
    // bound is kept by adding parts
    P = std::min<int64_t>(P, hp.nrows);
    int64_t per = (hp.nrows + P - 1) / P;
    while (per > 1 && per * hp.Lv * vpv > kMaxPartValues) {
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
  if (hp.part_vecs * vpv > kMaxPartValues) return FA3Q_ERR_SHAPE;
  if (kHistMaxBatches * H * hp.P > (int64_t{1} << 31) - 1) return FA3Q_ERR_SHAPE;
  // P records, then (many parts) the summed counts; at least 65536 words (the merge search's
  // inc[] of heavy groups reuses the start of the region)
  hp.head_words = hp.P >= kSumMinParts ? hp.P * kPartWords + kBins : std::max<int64_t>(hp.P * kPartWords, kBins);
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
      hipLaunchKernelGGL((calib_hist_kernel<true, true, false>), g, blk, 0, stream, ha);
    else
      hipLaunchKernelGGL((calib_hist_kernel<true, false, false>), g, blk, 0, stream, ha);
  } else {
    const dim3 g(static_cast<unsigned>(nb * H * hp.P));
    if (hp.rows)
      hipLaunchKernelGGL((calib_hist_kernel<false, true, false>), g, blk, 0, stream, ha);
    else
      hipLaunchKernelGGL((calib_hist_kernel<false, false, false>), g, blk, 0, stream, ha);
    if (hp.P >= kSumMinParts)
      hipLaunchKernelGGL(calib_hist_sum_kernel, dim3(static_cast<unsigned>(nb * H * kSumSlices)), dim3(kSumThreads), 0,
                         stream, ha);
    hipLaunchKernelGGL(calib_hist_window_kernel, dim3(static_cast<unsigned>(nb * H)), blk, kWinLds, stream, ha);
  }
  return launch_status();
}


int hist_f32_collect(const void* x, int64_t H, int64_t t, int64_t K, const HistPlan& hp, uint32_t* records,
                     TailCut* cut, uint64_t* best, uint32_t* lists, int64_t stride, hipStream_t stream) {
  if (hp.vpv != 4) return FA3Q_ERR_SHAPE;
  const int st = allow_dynamic_lds(reinterpret_cast<const void*>(calib_cut_kernel), kCutLds);
  if (st != FA3Q_OK) return st;
  HistArgs ha{};
  ha.x[0] = x;
  ha.hist = records;
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
  const dim3 blk(kHistThreads), g_parts(static_cast<unsigned>(H * hp.P));
  if (hp.rows)
    hipLaunchKernelGGL((calib_hist_kernel<false, true, true>), g_parts, blk, 0, stream, ha);
  else
    hipLaunchKernelGGL((calib_hist_kernel<false, false, true>), g_parts, blk, 0, stream, ha);
  if (hp.P >= kSumMinParts)
    hipLaunchKernelGGL(calib_hist_sum_kernel, dim3(static_cast<unsigned>(H * kSumSlices)), dim3(kSumThreads), 0, stream,
                       ha);
  hipLaunchKernelGGL(calib_cut_kernel, dim3(static_cast<unsigned>(H)), blk, kCutLds, stream, ha, cut, best);
  if (hp.rows)
    hipLaunchKernelGGL(calib_collect_kernel<true>, g_parts, blk, 0, stream, ha, cut, lists, stride);
  else
    hipLaunchKernelGGL(calib_collect_kernel<false>, g_parts, blk, 0, stream, ha, cut, lists, stride);
  return launch_status();
}

}  // namespace fa3q
