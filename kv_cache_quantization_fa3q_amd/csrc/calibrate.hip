// Per-head Recall Window calibration of one batch.
//
// msModelSlim page "FA3量化：Flash Attention 3激活量化算法说明", section 原理 -> 算法流程:
// head h of an activation x (B,H,S,D) owns N = B*S*D values; after sorting them
// (s[0] <= ... <= s[N-1]) and setting t = int(ratio*N), the window [s[i], s[i+t-1]]
// with the smallest length over i = 0 .. N-t is kept and its (min, max) reported.
//
// Only order statistics s[0..K-1] and s[t-1..N-1] (K = N-t+1) take part: the window
// starting at i is [L[i], U[i]] with L the K smallest values and U the K largest, both
// ascending.  So instead of sorting N values the library selects the two tails:
//
//   calib_sample_kernel  one workgroup per head reads a small sample spread over the
//                        head (32 runs of 256 16-byte vectors, one per 1/32 of the head at
//                        a fixed phase inside it, about 3% of a 2M-value head) and sets
//                        per-head bounds: the K-th smallest minimum of a
//                        group of sampled vectors (K-th largest maximum), which has at
//                        least K of the head's values at or beyond it.
//   calib_chunk_kernel   one HBM pass.  Each workgroup streams a contiguous chunk of one
//                        head (inside one (b,h) slab) and keeps, in LDS, a candidate
//                        buffer per side holding a superset of the chunk's part of the
//                        head's K smallest (K largest) values.  A value is a candidate
//                        only if it is within the head bound and beats the chunk's own
//                        threshold; when a buffer passes 2K entries an exact LDS radix
//                        select cuts it back to the K extreme values and tightens the
//                        threshold.  At most K values per side go to the workspace.
//   calib_merge_side_kernel  one workgroup per (head, side): the same select over the
//                        keys the chunks' lists hold gives the side's exact K extreme
//                        values, and a counting sort (or a bitonic one) orders them into
//                        the workspace;
//   calib_window_kernel  one workgroup per head, after both passes: the shortest float32
//                        window U[i]-L[i] over the two sorted sides, smallest i on ties.
//                        Heads whose lists fit in registers take calib_merge_wave_kernel
//                        instead: one wave per side and the window in the same workgroup.
//
// Estimated bounds.  A group-minimum bound is certain but loose: with a sampled fraction f
// of the head it lets about K/f values per side through.  When K is large against the
// sample (no certain bound at all once K exceeds the number of groups) the sample instead
// gives the r-th smallest group minimum with r = 2e + 4 sqrt(e) + 8, e = K f the expected
// number of sampled keys among the head's K smallest: about r/f values pass, a few times K.
// Such a bound is checked, exactly, by the merge: it holds at least K head values iff the
// chunk lists together hold at least K keys (a chunk that cut its buffer held K by
// itself; otherwise every value within the bound was kept).  Each chunk records how many
// keys its lists hold, so the check is a sum.  A side that fails sets its flag, and a head
// with either flag set is redone by a second chunk pass and merge that use no bound (their
// workgroups exit at once for every head that passed).
//
// Why the union of the chunk lists holds the head's K smallest values: a value v at or
// below the head's K-th smallest value is never dropped.  The head bound has at least K
// head values at or below it, so v is within it; a chunk's own K-th smallest value is at
// least the head's, so v is within that too (values equal to a threshold are kept until
// K values at or below it are held, as below).
//
// Values are compared through order-preserving unsigned keys (16-bit for bf16 input,
// 32-bit for float32), which realise the float total order with -0.0 below +0.0.
// Ties need no special care: a tail is a multiset of key values, and dropping a value
// equal to the K-th smallest once K values <= it are held never changes that multiset.
//
// Streaming filter of the chunk kernel.  Once the lo threshold is a negative value and
// the hi threshold a non-negative one (the usual case from the start), the test
// needs no key transform: among sign-magnitude patterns, "below a negative threshold"
// is an unsigned compare of the raw bits and "above a non-negative threshold" a signed
// one, so each dword of input costs one packed unsigned and one packed signed max.
// Only 16-byte vectors holding a candidate are copied to a per-wave LDS stage, from
// which the wave appends the qualifying keys; a round appends at most 64 vectors per
// wave, so the buffers need room for one round, not for a whole tile.
#include <cmath>
#include <type_traits>

#include "calib_hist.hpp"
#include "calib_sort.hpp"
#include "fa3q_internal.hpp"

namespace fa3q {
namespace {

constexpr int kChunkThreads = 256;
constexpr int kChunkWaves = kChunkThreads / kWave;
constexpr int kVec = 8;                // 16-byte vectors per thread per tile (chunk kernel)
constexpr int kStageVecs = 64;         // vectors one wave stages and appends per round
constexpr int kMergeThreads = 1024;
constexpr int kSampleThreads = 256;
constexpr int kSampleRuns = 32;       // runs of kSampleThreads vectors sampled per head
constexpr int kSampleGroupRuns = 4;   // a thread's vectors of this many runs form one group
constexpr int kSampleGroups = kSampleRuns / kSampleGroupRuns;  // groups per thread
constexpr int kMergePerThread = 4;     // keys per thread per tile (merge kernel)
constexpr int kMergeTile = kMergeThreads * kMergePerThread;
constexpr int64_t kTargetCUs = 256;    // MI355X compute units (sizes the chunk grid)
constexpr int64_t kChunkGroupsPerCU = 4;  // chunk workgroups resident per CU (VGPR-bound)
constexpr int kMinTilesPerChunk = 4;
constexpr int kMaxBatches = kHistMaxBatches;  // calibration batches one call can take (16)
// 16-bit heads of at least this many values take the histogram path for every K: from
// there on it streams faster than the tail lists (measured on MI355X: 4 batches of
// (8,128,2048,128) at ratio 0.9999 in 343 against 379 us, one (2,128,16384,128) tensor in
// 186-198 against 199-227 us over ratios 0.999-0.99999)
constexpr int64_t kHistMinValues = int64_t{1} << 20;

// Several batches of the same shape in one launch: workgroup i serves batch i / per, with
// that batch's input and its own region of the workspace (lists, bounds, flags).
struct Batches {
  const void* x[kMaxBatches];
  int64_t region;  // workspace bytes per batch
  int32_t per;     // workgroups per batch
};

template <typename T>
__device__ __forceinline__ T* in_region(T* p, int64_t off) {
  return p ? reinterpret_cast<T*>(reinterpret_cast<unsigned char*>(const_cast<std::remove_const_t<T>*>(p)) + off) : p;
}

// Control words at the start of dynamic LDS.
enum Ctl : int {
  kSlotLo = 0,   // [3] per-round append counters, lo side
  kSlotHi = 3,   // [3] hi side
  kThrLo = 6,    // threshold key after the latest compaction, lo side
  kThrHi = 7,    // hi side
  kTmpCnt = 8,
  kSelDigit = 9,
  kSelBefore = 10,
  kSelCount = 11,
  kBestLen = 12,
  kWaveTot = 16,  // [3][kChunkWaves] staged-vector totals per wave, one set per round slot
  kHist = 64,    // [256] radix histogram
  kWaveScratch = 64 + 256,  // [2 * 16] per-wave (length, index) pairs
  kCtlWords = 64 + 256 + 32
};
constexpr size_t kCtlBytes = 2048;
static_assert(kCtlWords * 4 <= kCtlBytes, "control block too small");
static_assert(kWaveScratch + 16 <= kCtlWords, "wave scratch holds a total per wave of 1024 threads");
static_assert(kWaveTot + 3 * kChunkWaves <= kHist, "wave totals overlap the histogram");
constexpr size_t kStageBytes = static_cast<size_t>(kChunkWaves) * kStageVecs * 16;

template <typename KeyT>
struct KeyInfo;
template <>
struct KeyInfo<uint16_t> {
  static constexpr uint32_t kMax = 0xffffu;
  static constexpr int kBits = 16;
};
template <>
struct KeyInfo<uint32_t> {
  static constexpr uint32_t kMax = 0xffffffffu;
  static constexpr int kBits = 32;
};

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Per input type: keys packed in dwords as they come from memory, the raw-bit maxima of
// the sign-split filter, and the limits that make that filter exact.
//   key(v)  = bits ^ (sign ? all-ones : sign-bit)       (order-preserving, unsigned)
//   Lim     signed type wide enough for key - 1 and key + 1
template <typename InT>
struct In;

template <>
struct In<uint16_t> {  // bf16 or float16 patterns (same sign-magnitude order), two per dword
  using KeyT = uint16_t;
  using Lim = int32_t;
  static constexpr int kPerDword = 2;
  static constexpr Lim kKeyZero = 0x8000;  // key of +0.0: smaller keys are negative values or -0.0
  __device__ static uint32_t keys(uint32_t w) {
    const s16x2 sg = __builtin_bit_cast(s16x2, w) >> (s16x2){15, 15};
    return w ^ ((__builtin_bit_cast(uint32_t, sg) & 0x7fff7fffu) | 0x80008000u);
  }
  __device__ static uint32_t at(uint32_t w, int i) { return i ? (w >> 16) : (w & 0xffffu); }
  __device__ static uint32_t umin(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2, a),
                                                                 __builtin_bit_cast(u16x2, b)));
  }
  __device__ static uint32_t umax(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                 __builtin_bit_cast(u16x2, b)));
  }
  __device__ static uint32_t smax(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(s16x2, a),
                                                                 __builtin_bit_cast(s16x2, b)));
  }
  __device__ static Lim ulane_min(uint32_t p) { return static_cast<Lim>(min(p & 0xffffu, p >> 16)); }
  __device__ static Lim ulane_max(uint32_t p) { return static_cast<Lim>(max(p & 0xffffu, p >> 16)); }
  __device__ static Lim slane_max(uint32_t p) {
    return max(static_cast<Lim>(static_cast<int16_t>(p & 0xffffu)), static_cast<Lim>(static_cast<int32_t>(p) >> 16));
  }
};

template <>
struct In<uint32_t> {  // float32 patterns, one per dword
  using KeyT = uint32_t;
  using Lim = int64_t;
  static constexpr int kPerDword = 1;
  static constexpr Lim kKeyZero = 0x80000000ll;
  __device__ static uint32_t keys(uint32_t w) {
    return w ^ ((w & 0x80000000u) ? 0xffffffffu : 0x80000000u);
  }
  __device__ static uint32_t at(uint32_t w, int) { return w; }
  __device__ static uint32_t umin(uint32_t a, uint32_t b) { return min(a, b); }
  __device__ static uint32_t umax(uint32_t a, uint32_t b) { return max(a, b); }
  __device__ static uint32_t smax(uint32_t a, uint32_t b) {
    return static_cast<uint32_t>(max(static_cast<int32_t>(a), static_cast<int32_t>(b)));
  }
  __device__ static Lim ulane_min(uint32_t p) { return static_cast<Lim>(p); }
  __device__ static Lim ulane_max(uint32_t p) { return static_cast<Lim>(p); }
  __device__ static Lim slane_max(uint32_t p) { return static_cast<Lim>(static_cast<int32_t>(p)); }
};

// Value of a key: 16-bit keys hold bf16 or (f16) float16 patterns, 32-bit keys float32 ones.
__device__ __forceinline__ float value_of_key(uint32_t k, uint16_t, bool f16) {
  const uint32_t b = (k & 0x8000u) ? (k ^ 0x8000u) : (k ^ 0xffffu);
  return f16 ? static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b))) : __uint_as_float(b << 16);
}
__device__ __forceinline__ float value_of_key(uint32_t k, uint32_t, bool) {
  const uint32_t b = (k & 0x80000000u) ? (k ^ 0x80000000u) : ~k;
  return __uint_as_float(b);
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
}

// Wave-aggregated append of `key` (where pred holds) at buf[*cnt ...]; all lanes of the
// wave must call it together.
template <typename KeyT>
__device__ __forceinline__ void wave_append(bool pred, uint32_t key, KeyT* buf, uint32_t* cnt) {
  const uint64_t m = __ballot(pred);
  if (m == 0) return;
  const int leader = __ffsll(static_cast<unsigned long long>(m)) - 1;
  uint32_t base = 0;
  if (lane_id() == leader) base = atomicAdd(cnt, static_cast<uint32_t>(__popcll(m)));
  base = __shfl(base, leader);
  if (pred) buf[base + lanes_below(m)] = static_cast<KeyT>(key);
}

// Same for two keys per lane with one counter update; every lane of the wave is active.
template <typename KeyT>
__device__ __forceinline__ void wave_append2(bool p0, uint32_t k0, bool p1, uint32_t k1, KeyT* buf,
                                             uint32_t* cnt) {
  const uint64_t m0 = __ballot(p0), m1 = __ballot(p1);
  if ((m0 | m1) == 0) return;
  const uint32_t c0 = static_cast<uint32_t>(__popcll(m0));
  uint32_t base = 0;
  if (lane_id() == 0) base = atomicAdd(cnt, c0 + static_cast<uint32_t>(__popcll(m1)));
  base = __builtin_amdgcn_readfirstlane(base);
  if (p0) buf[base + lanes_below(m0)] = static_cast<KeyT>(k0);
  if (p1) buf[base + c0 + lanes_below(m1)] = static_cast<KeyT>(k1);
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) {
  const int lane = lane_id();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint32_t u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  return v;
}

// Exact rank selection over buf[0..n): returns the key of rank `rank` (1-based, ascending)
// plus the number of keys below it and equal to it.  MSD radix, 8 bits per pass.
template <typename KeyT, int NT>
__device__ void block_select(const KeyT* buf, uint32_t n, uint32_t rank, uint32_t* ctl,
                             uint32_t& kth, uint32_t& less, uint32_t& eq) {
  const int tid = static_cast<int>(threadIdx.x);
  uint32_t* hist = ctl + kHist;
  uint32_t prefix = 0, pmask = 0, rem = rank;
  less = 0;
  eq = 0;
#pragma unroll 1
  for (int shift = KeyInfo<KeyT>::kBits - 8; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += NT) hist[i] = 0;
    lds_barrier();
    if (shift == KeyInfo<KeyT>::kBits - 8) {
      // top digit: tail keys share few values, so equal digits of a wave are counted with
      // one atomic per distinct digit instead of one per lane
      const uint32_t n_round = (n + NT - 1) / NT * NT;
      for (uint32_t i = tid; i < n_round; i += NT) {
        const bool act = i < n;
        const uint32_t d = act ? (static_cast<uint32_t>(buf[i]) >> shift) & 0xffu : 0u;
        uint64_t pending = __ballot(act);
        while (pending != 0) {
          const int leader = __ffsll(static_cast<unsigned long long>(pending)) - 1;
          const uint32_t dl = __builtin_amdgcn_readlane(d, leader);
          const uint64_t same = __ballot(act && d == dl);
          if (lane_id() == leader) atomicAdd(&hist[dl], static_cast<uint32_t>(__popcll(same)));
          pending &= ~same;
        }
      }
    } else {
      for (uint32_t i = tid; i < n; i += NT) {
        const uint32_t k = buf[i];
        if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & 0xffu], 1u);
      }
    }
    lds_barrier();
    if (tid < kWave) {
      const int lane = tid;
      const uint32_t c0 = hist[4 * lane], c1 = hist[4 * lane + 1], c2 = hist[4 * lane + 2],
                     c3 = hist[4 * lane + 3];
      const uint32_t sum = c0 + c1 + c2 + c3;
      const uint32_t incl = wave_inclusive_scan(sum);
      const uint32_t excl = incl - sum;
      if (excl < rem && rem <= incl) {
        uint32_t r = rem - excl, before = excl, d = 4 * lane, c = c0;
        if (r > c0) {
          r -= c0; before += c0; ++d; c = c1;
          if (r > c1) {
            r -= c1; before += c1; ++d; c = c2;
            if (r > c2) { r -= c2; before += c2; ++d; c = c3; }
          }
        }
        ctl[kSelDigit] = d;
        ctl[kSelBefore] = before;
        ctl[kSelCount] = c;
      }
    }
    lds_barrier();
    const uint32_t d = ctl[kSelDigit];
    const uint32_t before = ctl[kSelBefore];
    eq = ctl[kSelCount];
    prefix |= d << shift;
    pmask |= 0xffu << shift;
    rem -= before;
    less += before;
  }
  kth = prefix;
}

// Cut buf[0..n) (n > K) to exactly K entries: the K smallest (lo side) or the K largest
// (hi side) values as a multiset.  Sets the side's threshold to the K-th extreme key.
template <typename KeyT, int NT, bool kLo>
__device__ void compact(KeyT* buf, uint32_t n, uint32_t K, KeyT* tmp, uint32_t* ctl) {
  const int tid = static_cast<int>(threadIdx.x);
  uint32_t kth, less, eq;
  block_select<KeyT, NT>(buf, n, kLo ? K : n - K + 1, ctl, kth, less, eq);
  const uint32_t keep = kLo ? less : n - less - eq;  // strictly inside the tail
  if (tid == 0) ctl[kTmpCnt] = 0;
  lds_barrier();
  const uint32_t n_round = (n + NT - 1) / NT * NT;
  for (uint32_t i = tid; i < n_round; i += NT) {
    uint32_t k = 0;
    bool take = false;
    if (i < n) {
      k = buf[i];
      take = kLo ? (k < kth) : (k > kth);
    }
    wave_append<KeyT>(take, k, tmp, &ctl[kTmpCnt]);
  }
  lds_barrier();
  for (uint32_t i = tid; i < K; i += NT) buf[i] = (i < keep) ? tmp[i] : static_cast<KeyT>(kth);
  if (tid == 0) ctl[kLo ? kThrLo : kThrHi] = kth;
  lds_barrier();
}

// Candidate buffers of both sides and their bookkeeping (uniform across the workgroup).
template <typename KeyT, int NT>
struct TailState {
  KeyT* lo;
  KeyT* hi;
  KeyT* tmp;
  uint32_t* ctl;
  uint32_t K;
  uint32_t cap;       // entries per side buffer
  uint32_t room;      // most entries one round can append per side
  uint32_t base_lo;   // entries held before the current round
  uint32_t base_hi;
  uint32_t thr_lo;    // lo candidates: key < thr_lo
  uint32_t thr_hi;    // hi candidates: key > thr_hi
  int parity;         // round counter mod 3 (append-counter slot)

  __device__ void init() {
    const int tid = static_cast<int>(threadIdx.x);
    if (tid < 3) {
      ctl[kSlotLo + tid] = 0;
      ctl[kSlotHi + tid] = 0;
    }
    if (tid == 0) {
      ctl[kThrLo] = KeyInfo<KeyT>::kMax;
      ctl[kThrHi] = 0;
    }
    base_lo = base_hi = 0;
    thr_lo = KeyInfo<KeyT>::kMax;
    thr_hi = 0;
    parity = 0;
    lds_barrier();
  }

  __device__ __forceinline__ void append_lo(bool pred, uint32_t key) {
    wave_append<KeyT>(pred, key, lo + base_lo, &ctl[kSlotLo + parity]);
  }
  __device__ __forceinline__ void append_hi(bool pred, uint32_t key) {
    wave_append<KeyT>(pred, key, hi + base_hi, &ctl[kSlotHi + parity]);
  }

  // After every thread appended its share of one round.  Three rotating counter slots let
  // a single barrier per round separate "read this round's count" from the next round's
  // appends: slot p is filled in round i, read after barrier i, and cleared after
  // barrier i+1 (when every thread has read it), before round i+3 uses it again.
  // Returns the slot that was current before the barrier.
  __device__ int end_round() {
    lds_barrier();
    const int cur = parity;
    base_lo += ctl[kSlotLo + cur];
    base_hi += ctl[kSlotHi + cur];
    const int clear = cur == 0 ? 2 : cur - 1;
    if (threadIdx.x == 0) {
      ctl[kSlotLo + clear] = 0;
      ctl[kSlotHi + clear] = 0;
    }
    parity = cur == 2 ? 0 : cur + 1;
    if (base_lo > cap - room) {
      compact<KeyT, NT, true>(lo, base_lo, K, tmp, ctl);
      base_lo = K;
      thr_lo = ctl[kThrLo];
    }
    if (base_hi > cap - room) {
      compact<KeyT, NT, false>(hi, base_hi, K, tmp, ctl);
      base_hi = K;
      thr_hi = ctl[kThrHi];
    }
    return cur;
  }

  // Leave exactly min(K, held) entries per side.
  __device__ void finish() {
    if (base_lo > K) {
      compact<KeyT, NT, true>(lo, base_lo, K, tmp, ctl);
      base_lo = K;
    }
    if (base_hi > K) {
      compact<KeyT, NT, false>(hi, base_hi, K, tmp, ctl);
      base_hi = K;
    }
  }
};

struct ChunkArgs {
  const void* x;
  void* lists;        // [2][H][nch][K] keys; unused slots hold keys no filter lets through
  int64_t L;          // S*D, elements per (b,h) slab
  int64_t CL;         // elements per chunk (multiple of the vector width)
  int32_t H;
  int32_t cps;        // chunks per slab
  int32_t nch;        // chunks per head = B*cps
  uint32_t* counts;        // [2][H][nch] keys each list holds (the rest are unused slots)
  const uint32_t* bounds;  // [2][H] sampled bound keys per head (lo side, then hi side)
  const uint32_t* fail;    // fix-up pass: [2][H] check flags per side, a head is redone when
                           // either is set (nullptr: the first pass)
  uint32_t K;
  uint32_t cap;
  int32_t pad;             // fill the unused list slots (the merges that read every slot need it)
  // (B,S,H,D) input (kRows kernels): element e of slab (b, h) is at b*H*L + h*D + (e >> log2D) *
  // row_stride + (e & (D - 1)), with D a power of two and row_stride = H*D
  int32_t log2D;
  int64_t row_stride;
};

template <typename InT>
constexpr int chunk_tile() {
  return kChunkThreads * kVec * (16 / static_cast<int>(sizeof(InT)));
}
template <typename InT>
constexpr uint32_t chunk_room() {  // keys one round appends per side at most
  return static_cast<uint32_t>(kChunkWaves * kStageVecs * (16 / static_cast<int>(sizeof(InT))));
}

// One thread's 16-byte vector holds a candidate: some key < lo_lim or > hi_lim.
template <typename InT>
__device__ __forceinline__ bool vec_flag_keys(const u32x4& x, typename In<InT>::Lim lo_lim,
                                              typename In<InT>::Lim hi_lim) {
  using T = In<InT>;
  const uint32_t k0 = T::keys(x.x), k1 = T::keys(x.y), k2 = T::keys(x.z), k3 = T::keys(x.w);
  const uint32_t mn = T::umin(T::umin(k0, k1), T::umin(k2, k3));
  const uint32_t mx = T::umax(T::umax(k0, k1), T::umax(k2, k3));
  return T::ulane_min(mn) < lo_lim || T::ulane_max(mx) > hi_lim;
}
// Same test on raw bits; valid when lo_lim <= key(+0) and hi_lim >= key(+0) - 1, with
// rlo = key_max - lo_lim and rhi = hi_lim - key(+0) (see the file header).
template <typename InT>
__device__ __forceinline__ bool vec_flag_raw(const u32x4& x, typename In<InT>::Lim rlo,
                                             typename In<InT>::Lim rhi) {
  using T = In<InT>;
  const uint32_t mu = T::umax(T::umax(x.x, x.y), T::umax(x.z, x.w));
  const uint32_t ms = T::smax(T::smax(x.x, x.y), T::smax(x.z, x.w));
  return T::ulane_max(mu) > rlo || T::slane_max(ms) > rhi;
}

// Sum over the 64 lanes of a wave (uniform result): an inclusive scan with DPP row shifts
// and row broadcasts leaves the total in lane 63.
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
  v += __builtin_amdgcn_update_dpp(0u, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0u, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0u, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0u, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0u, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  v += __builtin_amdgcn_update_dpp(0u, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return __builtin_amdgcn_readlane(v, 63);
}

struct SampleArgs {
  const void* x;
  uint32_t* bounds;  // [2][H] out: lo bound keys, then hi bound keys
  int64_t Lv;        // 16-byte vectors per (b,h) slab
  int64_t run_off[kSampleRuns];  // element offset of each run's first vector in head 0
  uint32_t run_w[kSampleRuns];   // that vector's index inside its slab
  uint32_t run_n[kSampleRuns];   // vectors in the run (0 .. kSampleThreads)
  int32_t H;
  uint32_t M;        // sampled groups per head
  uint32_t K;
  // (B,S,H,D) input (kRows kernels): run j starts at head row run_row[j] (rows of D values, row R
  // of head h at (R*H + h)*D); thread t takes vector t & (Dv - 1) of row run_row[j] + (t >> log2Dv)
  int64_t run_row[kSampleRuns];
  int32_t log2Dv;
  int32_t D;
};

// Head bounds from a sample: kSampleRuns spread-out runs of kSampleThreads consecutive
// 16-byte vectors of the head (all of it when it is small).  A thread's vectors of
// kSampleGroupRuns runs form a group of keys; the K-th smallest of the M sampled group
// minima has at least K of the head's keys at or below it (one per group), so the head's
// K smallest keys all lie at or below it; symmetrically the K-th largest group maximum.
// With K a small fraction of M it sits near the head's K/(sampled keys) quantile.  Both
// ranks are found by one bisection over the key bits, counting with ballots and one
// barrier per bit.  M < K gives no bound (every key passes the chunk filter until the
// chunk itself holds K).
// kSmallSlab: slabs shorter than a run, so a run may cross several slab boundaries.
template <typename InT, bool kSmallSlab, bool kRows>
__global__ __launch_bounds__(kSampleThreads) void calib_sample_kernel(SampleArgs a, Batches bt) {
  using T = In<InT>;
  using KeyT = typename T::KeyT;
  constexpr int kPerVec = 16 / sizeof(InT);
  constexpr int kWaves = kSampleThreads / kWave;
  __shared__ uint32_t cnt[2][kWaves];  // [bit parity][wave]: lo count | hi count << 16
  const int batch = static_cast<int>(blockIdx.x) / bt.per;
  const int h = static_cast<int>(blockIdx.x) - batch * bt.per;
  a.bounds = in_region(a.bounds, batch * bt.region);
  const int tid = static_cast<int>(threadIdx.x);
  const int wave = tid / kWave;
  const int lane = lane_id();
  const InT* x = static_cast<const InT*>(bt.x[batch]);

  // every load of the sample is issued before the first is used
  u32x4 xs[kSampleRuns];
  uint32_t valid = 0;  // bit j: this thread's vector of run j lies inside the head
  const int64_t head_off = static_cast<int64_t>(h) * a.Lv * kPerVec;
  const int64_t jump = static_cast<int64_t>(a.H - 1) * a.Lv * kPerVec;  // slab end -> next slab of the head
#pragma unroll
  for (int j = 0; j < kSampleRuns; ++j) {
    const bool ok = static_cast<uint32_t>(tid) < a.run_n[j];
    valid |= static_cast<uint32_t>(ok) << j;
    int64_t e;
    if constexpr (kRows) {
      const int64_t row = a.run_row[j] + (tid >> a.log2Dv);
      e = (row * a.H + h) * a.D + static_cast<int64_t>(tid & ((1 << a.log2Dv) - 1)) * kPerVec;
    } else {
      const uint32_t w = a.run_w[j] + static_cast<uint32_t>(tid);
      // slab boundaries crossed inside the run: at most one unless slabs are short
      const uint32_t d = kSmallSlab ? w / static_cast<uint32_t>(a.Lv) : static_cast<uint32_t>(w >= a.Lv);
      e = a.run_off[j] + head_off + static_cast<int64_t>(tid) * kPerVec + d * jump;
    }
    xs[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + (ok ? e : 0)));
  }
  // A group is a thread's vectors of kSampleGroupRuns runs (any distinct keys make a
  // group); its extremes are taken over the vectors inside the head.  Groups with no such
  // vector count as the largest key, and are taken off again when a probe reaches it.
  uint32_t gmin[kSampleGroups], gmax[kSampleGroups];
#pragma unroll
  for (int g = 0; g < kSampleGroups; ++g) {
    uint32_t mn = KeyInfo<KeyT>::kMax, mx = 0;
    bool any = false;
#pragma unroll
    for (int q = 0; q < kSampleGroupRuns; ++q) {
      const int j = g * kSampleGroupRuns + q;
      const uint32_t k0 = T::keys(xs[j].x), k1 = T::keys(xs[j].y), k2 = T::keys(xs[j].z), k3 = T::keys(xs[j].w);
      const bool ok = (valid >> j) & 1u;
      any |= ok;
      mn = ok ? min(mn, T::ulane_min(T::umin(T::umin(k0, k1), T::umin(k2, k3)))) : mn;
      mx = ok ? max(mx, T::ulane_max(T::umax(T::umax(k0, k1), T::umax(k2, k3)))) : mx;
    }
    gmin[g] = any ? mn : KeyInfo<KeyT>::kMax;
    gmax[g] = any ? mx : KeyInfo<KeyT>::kMax;
  }

  // least t_lo with #{gmin <= t_lo} >= K, least t_hi with #{gmax <= t_hi} >= M-K+1, bit by
  // bit from the top: bit b is 0 exactly when the largest value agreeing with the bits
  // fixed so far and having bit b clear already reaches the rank.
  const bool have = a.M >= a.K;
  const uint32_t rank_lo = a.K, rank_hi = a.M - a.K + 1;
  const uint32_t n_out = static_cast<uint32_t>(kSampleGroups * kSampleThreads) - a.M;
  uint32_t t_lo = 0, t_hi = 0;
#pragma unroll 1
  for (int bit = KeyInfo<KeyT>::kBits - 1; bit >= 0 && have; --bit) {
    const uint32_t p_lo = t_lo | ((1u << bit) - 1u), p_hi = t_hi | ((1u << bit) - 1u);
    uint32_t c_lo = 0, c_hi = 0;  // wave counts: a ballot per register, popcounts on the scalar unit
#pragma unroll
    for (int g = 0; g < kSampleGroups; ++g) {
      c_lo += static_cast<uint32_t>(__popcll(__ballot(gmin[g] <= p_lo)));
      c_hi += static_cast<uint32_t>(__popcll(__ballot(gmax[g] <= p_hi)));
    }
    const uint32_t c = c_lo | (c_hi << 16);  // each at most kSampleGroups * 64
    const int par = bit & 1;  // a slot is rewritten two bits later, after every wave read it
    if (lane == 0) cnt[par][wave] = c;
    __syncthreads();
    uint32_t s_lo = 0, s_hi = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const uint32_t v = cnt[par][w];
      s_lo += v & 0xffffu;
      s_hi += v >> 16;
    }
    if (p_lo == KeyInfo<KeyT>::kMax) s_lo -= n_out;
    if (p_hi == KeyInfo<KeyT>::kMax) s_hi -= n_out;
    if (s_lo < rank_lo) t_lo |= 1u << bit;
    if (s_hi < rank_hi) t_hi |= 1u << bit;
  }
  if (tid == 0) {
    a.bounds[h] = have ? t_lo : KeyInfo<KeyT>::kMax;
    a.bounds[a.H + h] = have ? t_hi : 0u;
  }
}

template <typename InT, bool kRows>
__global__ __launch_bounds__(kChunkThreads) __attribute__((amdgpu_waves_per_eu(4, 8))) void calib_chunk_kernel(ChunkArgs a, Batches bt) {
  using T = In<InT>;
  using KeyT = typename T::KeyT;
  using Lim = typename T::Lim;
  constexpr int NT = kChunkThreads;
  constexpr int kPerVec = 16 / sizeof(InT);  // elements per 16-byte vector
  constexpr int kTile = chunk_tile<InT>();
  constexpr Lim kKeyMax = static_cast<Lim>(KeyInfo<KeyT>::kMax);
  extern __shared__ __align__(16) unsigned char smem[];
  uint32_t* ctl = reinterpret_cast<uint32_t*>(smem);
  const int tid = static_cast<int>(threadIdx.x);
  const int wave = tid / kWave;
  const int lane = lane_id();
  u32x4* stage = reinterpret_cast<u32x4*>(smem + kCtlBytes) + wave * kStageVecs;
  const uint32_t* stage_dw = reinterpret_cast<const uint32_t*>(stage);
  KeyT* lo = reinterpret_cast<KeyT*>(smem + kCtlBytes + kStageBytes);

  TailState<KeyT, NT> st;
  st.lo = lo;
  st.hi = lo + a.cap;
  st.tmp = lo + 2 * a.cap;
  st.ctl = ctl;
  st.K = a.K;
  st.cap = a.cap;
  st.room = chunk_room<InT>();
  st.init();

  // Blocks take chunks in address order (block i: slab i / cps, slab = b*H + h), so the
  // blocks the dispatcher deals round-robin to the XCDs read neighbouring chunks and every
  // XCD streams from all of memory at once; a block per (h, b) in head order would hand
  // each XCD one batch's contiguous range instead, which runs far below the HBM rate.
  const int batch = static_cast<int>(blockIdx.x) / bt.per;
  const int bid = static_cast<int>(blockIdx.x) - batch * bt.per;
  a.x = bt.x[batch];
  a.lists = in_region(a.lists, batch * bt.region);
  a.counts = in_region(a.counts, batch * bt.region);
  a.bounds = in_region(a.bounds, batch * bt.region);
  a.fail = in_region(a.fail, batch * bt.region);
  const int slab_i = bid / a.cps;
  const int part = bid - slab_i * a.cps;
  const int b = slab_i / a.H;
  const int h = slab_i - b * a.H;
  const int c = b * a.cps + part;
  // (b, h) slab: contiguous, or (kRows) S rows of D values a row_stride apart
  const InT* slab = static_cast<const InT*>(a.x) +
                    (kRows ? static_cast<int64_t>(b) * a.H * a.L + (static_cast<int64_t>(h) << a.log2D)
                           : (static_cast<int64_t>(b) * a.H + h) * a.L);
  const int64_t begin = static_cast<int64_t>(part) * a.CL;
  const int64_t end = min(a.L, begin + a.CL);

  u32x4 x[kVec];
  // Unconditional loads (a vector past the chunk end re-reads the chunk's last vector and
  // is masked out), so no load has to merge with the register's previous contents.
  const int64_t last = end - kPerVec;
  auto load_tile = [&](int64_t t0) {
#pragma unroll
    for (int v = 0; v < kVec; ++v) {
      const int64_t e = min(t0 + static_cast<int64_t>(v * NT + tid) * kPerVec, last);
      const int64_t off = kRows ? (e >> a.log2D) * a.row_stride + (e & ((int64_t{1} << a.log2D) - 1)) : e;
      x[v] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(slab + off));
    }
  };

  // Candidate limits: key < lo_lim or key > hi_lim.  The head's sampled bounds have at
  // least K of the head's keys at or beyond them, so the head's K extreme keys all lie
  // within them: the chunk keeps every key up to and including the bounds (it may hold
  // fewer than K such keys), then its own K-th extreme key once it holds K.
  Lim lo_lim = static_cast<Lim>(a.bounds[h]) + 1, hi_lim = static_cast<Lim>(a.bounds[a.H + h]) - 1;
  if (a.fail != nullptr) {  // fix-up pass: only flagged heads, and every key is a candidate
    if ((a.fail[h] | a.fail[a.H + h]) == 0) return;  // uniform over the workgroup
    lo_lim = kKeyMax + 1;
    hi_lim = -1;
  }
  if (begin < end) load_tile(begin);
  for (int64_t t0 = begin; t0 < end; t0 += kTile) {
    bool vv[kVec];
#pragma unroll
    for (int v = 0; v < kVec; ++v) vv[v] = t0 + static_cast<int64_t>(v * NT + tid) * kPerVec < end;

    bool f[kVec];
    if (lo_lim <= T::kKeyZero && hi_lim >= T::kKeyZero - 1) {
      const Lim rlo = kKeyMax - lo_lim, rhi = hi_lim - T::kKeyZero;
#pragma unroll
      for (int v = 0; v < kVec; ++v) f[v] = vv[v] & vec_flag_raw<InT>(x[v], rlo, rhi);  // no short-circuit branch
    } else {
#pragma unroll
      for (int v = 0; v < kVec; ++v) f[v] = vv[v] & vec_flag_keys<InT>(x[v], lo_lim, hi_lim);
    }
    uint64_t m[kVec];
    uint32_t off[kVec];
    uint32_t tot = 0;
#pragma unroll
    for (int v = 0; v < kVec; ++v) {
      m[v] = __ballot(f[v]);
      off[v] = tot;
      tot += static_cast<uint32_t>(__popcll(m[v]));
    }
    if (lane == 0) ctl[kWaveTot + st.parity * kChunkWaves + wave] = tot;

    const int64_t tn = t0 + kTile;
    uint32_t rounds = 1;
    for (uint32_t r = 0; r < rounds; ++r) {
      const uint32_t r0 = r * kStageVecs;
      if (tot > r0) {
        // stage this round's vectors: the wave's flagged vectors ranked r0 .. r0+63
#pragma unroll
        for (int v = 0; v < kVec; ++v) {
          if (m[v] != 0) {
            const uint32_t rank = off[v] + lanes_below(m[v]);
            if (f[v] && rank >= r0 && rank < r0 + kStageVecs) stage[rank - r0] = x[v];
          }
        }
        // the registers are free once the last round of this wave is staged
        if (tot <= r0 + kStageVecs && tn < end) load_tile(tn);
        __asm__ volatile("" ::: "memory");  // stage writes before the reads below (same wave)
        const uint32_t dwords = min(tot - r0, static_cast<uint32_t>(kStageVecs)) * 4;
        for (uint32_t j0 = 0; j0 < dwords; j0 += kWave) {
          const uint32_t j = j0 + lane;
          const bool ok = j < dwords;
          const uint32_t w = T::keys(ok ? stage_dw[j] : 0u);
          if constexpr (T::kPerDword == 2) {
            const Lim k0 = static_cast<Lim>(w & 0xffffu), k1 = static_cast<Lim>(w >> 16);
            wave_append2<KeyT>(ok && k0 < lo_lim, w & 0xffffu, ok && k1 < lo_lim, w >> 16,
                               st.lo + st.base_lo, &ctl[kSlotLo + st.parity]);
            wave_append2<KeyT>(ok && k0 > hi_lim, w & 0xffffu, ok && k1 > hi_lim, w >> 16,
                               st.hi + st.base_hi, &ctl[kSlotHi + st.parity]);
          } else {
            const Lim k = static_cast<Lim>(w);
            wave_append2<KeyT>(ok && k < lo_lim, w, false, 0u, st.lo + st.base_lo, &ctl[kSlotLo + st.parity]);
            wave_append2<KeyT>(ok && k > hi_lim, w, false, 0u, st.hi + st.base_hi, &ctl[kSlotHi + st.parity]);
          }
        }
        __asm__ volatile("" ::: "memory");
      } else if (r == 0 && tn < end) {
        load_tile(tn);
      }
      const uint32_t thr_lo0 = st.thr_lo, thr_hi0 = st.thr_hi;
      const int slot = st.end_round();
      if (r == 0) {
        uint32_t most = 0;
#pragma unroll
        for (int w = 0; w < kChunkWaves; ++w) most = max(most, ctl[kWaveTot + slot * kChunkWaves + w]);
        rounds = (most + kStageVecs - 1) / kStageVecs;
      }
      if (st.thr_lo != thr_lo0) lo_lim = min(lo_lim, static_cast<Lim>(st.thr_lo));
      if (st.thr_hi != thr_hi0) hi_lim = max(hi_lim, static_cast<Lim>(st.thr_hi));
    }
  }
  st.finish();

  // Fixed-size list per chunk and its count; with `pad`, slots past the held count get keys
  // that fail both filters (the side merge with a count prefix reads only the held keys).
  const int64_t list = static_cast<int64_t>(h) * a.nch + c;
  const int64_t heads_lists = static_cast<int64_t>(a.H) * a.nch;
  KeyT* out_lo = static_cast<KeyT*>(a.lists) + list * a.K;
  KeyT* out_hi = static_cast<KeyT*>(a.lists) + (heads_lists + list) * a.K;
  const uint32_t n_out = a.pad ? a.K : max(st.base_lo, st.base_hi);
  for (uint32_t i = tid; i < n_out; i += NT) {
    if (a.pad || i < st.base_lo) out_lo[i] = i < st.base_lo ? st.lo[i] : static_cast<KeyT>(KeyInfo<KeyT>::kMax);
    if (a.pad || i < st.base_hi) out_hi[i] = i < st.base_hi ? st.hi[i] : static_cast<KeyT>(0);
  }
  if (tid == 0) {
    a.counts[list] = st.base_lo;
    a.counts[heads_lists + list] = st.base_hi;
  }
}

struct MergeArgs {
  const void* lists;
  const uint32_t* counts;  // [2][H][nch] keys each list holds
  void* sorted;            // [2][H][K] each side's K extreme keys, ascending (hi side complemented)
  float* win_min;
  float* win_max;
  uint32_t* fail;  // [2][H] with an estimated bound: written by the check pass, read by the fix-up
  int32_t fixup;   // 0: check pass (verifies the bound when fail != nullptr), 1: fix-up pass
  int32_t H;
  int32_t nch;
  uint32_t K;
  uint32_t cap;
  uint32_t P;  // next power of two >= K
  int32_t f16;  // 16-bit keys: 1 float16 patterns, 0 bf16
};

constexpr int kMaxPrefixLists = 2048;  // list counts the side merge keeps as an LDS prefix

// Ascending bitonic sort of buf[0..P), P = kMergeThreads * E.  Thread t holds elements
// t*E .. t*E+E-1 in registers: compare-exchange distances below E stay in registers,
// distances below 64*E go through lane shuffles, and only the wider ones through LDS (one
// barrier each) -- 10 barriers instead of 91 for P = 8192.
template <typename KeyT, int E>
__device__ void bitonic_sort_regs(KeyT* buf, int tid) {
  constexpr int NT = kMergeThreads;
  constexpr uint32_t P = static_cast<uint32_t>(NT) * E;
  constexpr uint32_t kWide = static_cast<uint32_t>(kWave) * E;  // distances from here on cross waves
  uint32_t a[E];
  const uint32_t base = static_cast<uint32_t>(tid) * E;
#pragma unroll
  for (int e = 0; e < E; ++e) a[e] = buf[base + e];
#pragma unroll
  for (uint32_t k = 2; k <= P; k <<= 1) {
    uint32_t j = k >> 1;
    if (j >= kWide) {
#pragma unroll
      for (int e = 0; e < E; ++e) buf[base + e] = static_cast<KeyT>(a[e]);
      lds_barrier();
      for (; j >= kWide; j >>= 1) {
        for (uint32_t i = static_cast<uint32_t>(tid); i < P / 2; i += NT) {
          const uint32_t l = ((i & ~(j - 1)) << 1) | (i & (j - 1));
          const uint32_t r = l + j;
          const bool up = (l & k) == 0;
          const KeyT a0 = buf[l], a1 = buf[r];
          if ((a0 > a1) == up) { buf[l] = a1; buf[r] = a0; }
        }
        lds_barrier();
      }
#pragma unroll
      for (int e = 0; e < E; ++e) a[e] = buf[base + e];  // each thread reads back only its own elements
    }
#pragma unroll
    for (; j >= static_cast<uint32_t>(E); j >>= 1) {
      const int lm = static_cast<int>(j / E);  // partner lane = lane ^ lm
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const uint32_t oa = static_cast<uint32_t>(__shfl_xor(static_cast<int>(a[e]), lm));
        const uint32_t i = base + e;
        const bool keep_min = ((i & k) == 0) == ((i & j) == 0);
        a[e] = keep_min ? min(a[e], oa) : max(a[e], oa);
      }
    }
#pragma unroll
    for (; j > 0; j >>= 1) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if ((e & j) == 0) {
          const bool up = ((base + e) & k) == 0;
          const uint32_t x0 = a[e], x1 = a[e ^ j];
          const bool sa = (x0 > x1) == up;
          a[e] = sa ? x1 : x0;
          a[e ^ j] = sa ? x0 : x1;
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) buf[base + e] = static_cast<KeyT>(a[e]);
  lds_barrier();
}

// Ascending sort of buf[0..P), P a power of two.
template <typename KeyT>
__device__ void bitonic_sort(KeyT* buf, uint32_t P, int tid) {
  constexpr int NT = kMergeThreads;
  switch (P / NT) {  // P >= NT: registers, shuffles and LDS; smaller: all in LDS
    case 1: bitonic_sort_regs<KeyT, 1>(buf, tid); break;
    case 2: bitonic_sort_regs<KeyT, 2>(buf, tid); break;
    case 4: bitonic_sort_regs<KeyT, 4>(buf, tid); break;
    case 8: bitonic_sort_regs<KeyT, 8>(buf, tid); break;
    case 16: bitonic_sort_regs<KeyT, 16>(buf, tid); break;
    default:
      for (uint32_t k = 2; k <= P; k <<= 1) {
        for (uint32_t j = k >> 1; j > 0; j >>= 1) {
          for (uint32_t i = tid; i < P / 2; i += NT) {
            const uint32_t l = ((i & ~(j - 1)) << 1) | (i & (j - 1));
            const uint32_t r = l + j;
            const bool up = (l & k) == 0;
            const KeyT a0 = buf[l], a1 = buf[r];
            if ((a0 > a1) == up) { buf[l] = a1; buf[r] = a0; }
          }
          lds_barrier();
        }
      }
  }
}

constexpr int kSortBuckets = 16;  // top-byte buckets the counting sort of 16-bit keys takes
constexpr int kSortBins = kSortBuckets * 256;
constexpr size_t kSortLdsBytes = (kSortBins + 256 + kSortBuckets) * 4;  // bins, bucket of each top byte, top byte of each bucket
static_assert(kSortBins == 4 * kMergeThreads, "the prefix takes four bins per thread");

// The K smallest of the n >= K 16-bit keys buf[0..n), in ascending order, into dst (device
// memory), by counting: equal keys are indistinguishable, so the sorted sequence follows
// from how many times each key value occurs.  A top-byte histogram locates the top byte of
// the K-th smallest key; the keys at or below it are counted per (top byte, low byte)
// over the top bytes present, and output slot i < K holds the key of the bin whose prefix
// range contains i.  Returns false (nothing written) when those keys span more than
// kSortBuckets top bytes.
__device__ bool value_select_sort16(const uint16_t* buf, uint32_t n, uint32_t K, uint32_t* sort_lds, uint32_t* ctl,
                                    uint16_t* dst, int tid) {
  constexpr int NT = kMergeThreads;
  uint32_t* bins = sort_lds;                 // [kSortBins]
  uint32_t* bidx = sort_lds + kSortBins;     // [256] bucket of each counted top byte
  uint32_t* btop = bidx + 256;               // [kSortBuckets] top byte of each bucket
  uint32_t* hist = ctl + kHist;              // [256] keys per top byte
  for (int i = tid; i < 256; i += NT) hist[i] = 0;
  for (int i = tid; i < kSortBins; i += NT) bins[i] = 0;
  lds_barrier();
  // tail keys share few top bytes: one atomic per distinct top byte of a wave
  const uint32_t n_round = (n + NT - 1) / NT * NT;
  for (uint32_t i = tid; i < n_round; i += NT) {
    const bool act = i < n;
    const uint32_t d = act ? static_cast<uint32_t>(buf[i]) >> 8 : 0u;
    uint64_t pending = __ballot(act);
    while (pending != 0) {
      const int leader = __ffsll(static_cast<unsigned long long>(pending)) - 1;
      const uint32_t dl = __builtin_amdgcn_readlane(d, leader);
      const uint64_t same = __ballot(act && d == dl);
      if (lane_id() == leader) atomicAdd(&hist[dl], static_cast<uint32_t>(__popcll(same)));
      pending &= ~same;
    }
  }
  lds_barrier();
  if (tid < kWave) {
    // the top byte t* holding the K-th smallest key, then the buckets: top bytes <= t* present
    uint32_t c[4], sum = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      c[q] = hist[4 * tid + q];
      sum += c[q];
    }
    const uint32_t incl = wave_inclusive_scan(sum);
    uint32_t cum = incl - sum;
    uint32_t tk = 0;
    bool mine = false;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (!mine && cum < K && K <= cum + c[q]) {
        tk = 4 * tid + q;
        mine = true;
      }
      cum += c[q];
    }
    const uint64_t who = __ballot(mine);  // one lane (n >= K); none would count every key
    const uint32_t t_star = who ? __builtin_amdgcn_readlane(tk, __ffsll(static_cast<unsigned long long>(who)) - 1) : 255u;
    uint32_t f[4], m = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f[q] = (c[q] != 0 && static_cast<uint32_t>(4 * tid + q) <= t_star) ? 1u : 0u;
      m += f[q];
    }
    const uint32_t mincl = wave_inclusive_scan(m);
    uint32_t idx = mincl - m;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (f[q]) {
        bidx[4 * tid + q] = idx;
        if (idx < kSortBuckets) btop[idx] = 4 * tid + q;
        ++idx;
      }
    }
    if (tid == kWave - 1) {
      ctl[kSelCount] = mincl;
      ctl[kSelDigit] = t_star;
    }
  }
  lds_barrier();
  const uint32_t nbk = ctl[kSelCount];
  const uint32_t t_star = ctl[kSelDigit];
  if (nbk > kSortBuckets) return false;  // uniform
  for (uint32_t i = tid; i < n; i += NT) {
    const uint32_t k = buf[i];
    if ((k >> 8) <= t_star) atomicAdd(&bins[bidx[k >> 8] * 256 + (k & 255u)], 1u);
  }
  lds_barrier();
  // exclusive prefix over the nbk * 256 bins, four consecutive bins per thread
  const uint32_t nbins = nbk * 256;
  uint32_t c[4], sum = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t j = 4 * static_cast<uint32_t>(tid) + q;
    c[q] = j < nbins ? bins[j] : 0u;
    sum += c[q];
  }
  const uint32_t incl = wave_inclusive_scan(sum);
  uint32_t* wsum = ctl + kWaveScratch;  // [NT / kWave] wave totals
  const int wave = tid / kWave;
  if (lane_id() == kWave - 1) wsum[wave] = incl;
  lds_barrier();
  uint32_t run = incl - sum;
  for (int w = 0; w < wave; ++w) run += wsum[w];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t j = 4 * static_cast<uint32_t>(tid) + q;
    if (j < nbins) bins[j] = run;
    run += c[q];
  }
  lds_barrier();
  // slot i: the largest bin j with prefix[j] <= i (empty bins share the next bin's prefix);
  // the counted keys number at least K, so every slot i < K lies in a bin
  for (uint32_t i = tid; i < K; i += NT) {
    uint32_t lo = 0, hi = nbins;
    while (hi - lo > 1) {
      const uint32_t mid = (lo + hi) >> 1;
      if (bins[mid] <= i) lo = mid; else hi = mid;
    }
    dst[i] = static_cast<uint16_t>((btop[lo >> 8] << 8) | (lo & 255u));
  }
  return true;
}

// One side of one head (workgroup = batch, side, head; the hi side works on complemented
// keys kMax - key, so both sides look for their K smallest keys): the keys the chunk lists
// hold go through the chunk kernel's filter and cuts, and the K smallest are sorted into
// the workspace.  Only the lists' real keys are read: an LDS prefix of the list counts maps
// a flat index to (list, slot); past kMaxPrefixLists lists every slot is read and the
// unused ones fail the filter.
template <typename KeyT>
__global__ __launch_bounds__(kMergeThreads) void calib_merge_side_kernel(MergeArgs a, Batches bt) {
  constexpr int NT = kMergeThreads;
  constexpr uint32_t kMax = KeyInfo<KeyT>::kMax;
  extern __shared__ __align__(16) unsigned char smem[];
  uint32_t* ctl = reinterpret_cast<uint32_t*>(smem);
  uint32_t* pre = reinterpret_cast<uint32_t*>(smem + kCtlBytes);  // [nch + 1] when nch <= kMaxPrefixLists
  const bool use_pre = a.nch <= kMaxPrefixLists;
  const size_t pre_bytes = use_pre ? (static_cast<size_t>(a.nch + 1) * 4 + 15) / 16 * 16 : 0;  // as the plan sizes it
  KeyT* buf = reinterpret_cast<KeyT*>(smem + kCtlBytes + pre_bytes);
  // counting-sort scratch (16-bit keys) after the buffer and cut scratch
  uint32_t* sort_lds = reinterpret_cast<uint32_t*>(
      smem + kCtlBytes + pre_bytes + (static_cast<size_t>(a.cap + a.K) * sizeof(KeyT) + 15) / 16 * 16);

  const int batch = static_cast<int>(blockIdx.x) / bt.per;
  const int r = static_cast<int>(blockIdx.x) - batch * bt.per;
  const int side = r / a.H;
  const int h = r - side * a.H;
  a.lists = in_region(a.lists, batch * bt.region);
  a.counts = in_region(a.counts, batch * bt.region);
  a.sorted = in_region(a.sorted, batch * bt.region);
  a.fail = in_region(a.fail, batch * bt.region);
  const int tid = static_cast<int>(threadIdx.x);
  if (a.fixup && (a.fail[h] | a.fail[a.H + h]) == 0) return;  // uniform over the workgroup

  TailState<KeyT, NT> st;
  st.lo = buf;
  st.hi = buf;  // one side only: nothing is appended to the hi buffer
  st.tmp = buf + a.cap;
  st.ctl = ctl;
  st.K = a.K;
  st.cap = a.cap;
  st.room = kMergeTile;
  st.init();

  const int64_t lists0 = (static_cast<int64_t>(side) * a.H + h) * a.nch;
  const KeyT* src = static_cast<const KeyT*>(a.lists) + lists0 * a.K;
  const uint32_t* cnt = a.counts + lists0;
  const uint32_t flip = side == 0 ? 0u : kMax;
  uint32_t total = static_cast<uint32_t>(a.nch) * a.K;
  if (use_pre) {
    if (tid < kWave) {
      uint32_t carry = 0;
      for (int c0 = 0; c0 < a.nch; c0 += kWave) {
        const int c = c0 + tid;
        const uint32_t v = c < a.nch ? cnt[c] : 0u;
        const uint32_t incl = wave_inclusive_scan(v);
        if (c < a.nch) pre[c] = carry + incl - v;
        carry += __shfl(incl, kWave - 1);
      }
      if (tid == 0) pre[a.nch] = carry;
    }
    lds_barrier();
    total = pre[a.nch];
  }
  if (!a.fixup && a.fail != nullptr) {
    // the estimated bound holds iff the lists hold at least K keys (a list that was cut
    // holds K by itself); the hi-side workgroup writes the hi flag
    uint32_t held = total;
    if (!use_pre) {
      held = 0;
      for (int c = tid; c < a.nch; c += NT) held += cnt[c];
      held = wave_sum(held);
      uint32_t* acc = ctl + kWaveScratch;
      if (tid == 0) acc[0] = 0;
      lds_barrier();
      if (lane_id() == 0) atomicAdd(&acc[0], held);
      lds_barrier();
      held = acc[0];
    }
    const bool ok = held >= a.K;
    if (tid == 0) a.fail[side * a.H + h] = ok ? 0u : 1u;
    if (!ok) return;  // uniform: the fix-up pass redoes this head
  }

  // Every list key fits the buffer (the usual case under a sampled bound): copy them as they
  // are and let the counting sort select the K smallest; else filter and cut as the chunk
  // kernel does.
  const bool direct = sizeof(KeyT) == 2 && use_pre && total <= a.cap;
  if (direct) {
    for (uint32_t i = tid; i < total; i += NT) {
      int c = 0, hi = a.nch;  // largest c with pre[c] <= i
      while (hi - c > 1) {
        const int mid = (c + hi) >> 1;
        if (pre[mid] <= i) c = mid; else hi = mid;
      }
      buf[i] = static_cast<KeyT>(static_cast<uint32_t>(src[static_cast<int64_t>(c) * a.K + (i - pre[c])]) ^ flip);
    }
    lds_barrier();
    st.base_lo = total;
  }
  for (uint32_t t0 = 0; !direct && t0 < total; t0 += kMergeTile) {
    uint32_t k[kMergePerThread];
#pragma unroll
    for (int e = 0; e < kMergePerThread; ++e) {
      const uint32_t i = t0 + static_cast<uint32_t>(e * NT + tid);
      k[e] = kMax;
      if (i < total) {
        int64_t at = i;
        if (use_pre) {
          int c = 0, hi = a.nch;  // largest c with pre[c] <= i
          while (hi - c > 1) {
            const int mid = (c + hi) >> 1;
            if (pre[mid] <= i) c = mid; else hi = mid;
          }
          at = static_cast<int64_t>(c) * a.K + (i - pre[c]);
        }
        k[e] = static_cast<uint32_t>(src[at]) ^ flip;  // an unused slot (kMax lo, 0 hi) reads as kMax
      }
    }
#pragma unroll
    for (int e = 0; e < kMergePerThread; ++e) st.append_lo(k[e] < st.thr_lo, k[e]);
    st.end_round();
  }
  // The side's K smallest keys, ascending, into the workspace: by counting for 16-bit keys
  // spanning few top bytes (straight from the held keys), else a cut to exactly K and a
  // bitonic sort padded to P with the largest key.
  const uint32_t K = a.K, P = a.P;
  KeyT* dst = static_cast<KeyT*>(a.sorted) + (static_cast<int64_t>(side) * a.H + h) * K;
  bool sorted = false;
  if constexpr (sizeof(KeyT) == 2) sorted = value_select_sort16(buf, st.base_lo, K, sort_lds, ctl, dst, tid);
  if (!sorted) {
    st.finish();  // now exactly K (every head holds at least K values)
    for (uint32_t i = K + tid; i < P; i += NT) buf[i] = static_cast<KeyT>(kMax);
    lds_barrier();
    bitonic_sort<KeyT>(buf, P, tid);
    for (uint32_t i = tid; i < K; i += NT) dst[i] = buf[i];
  }

}

// Shortest window U[i] - L[i] (float32), smallest i on ties, over the two sorted sides of
// a head: L[i] = lo[i], U[i] = kMax - hi_c[K-1-i] (hi_c: the complemented hi keys in
// ascending order).  One launch after the fix-up pass, so it reads each head's final lists.
template <typename KeyT>
__global__ __launch_bounds__(256) void calib_window_kernel(MergeArgs a, Batches bt) {
  constexpr uint32_t kMax = KeyInfo<KeyT>::kMax;
  constexpr int NT = 256;
  __shared__ float wl[NT / kWave];
  __shared__ uint32_t wi[NT / kWave];
  const int batch = static_cast<int>(blockIdx.x) / bt.per;
  const int h = static_cast<int>(blockIdx.x) - batch * bt.per;
  a.sorted = in_region(a.sorted, batch * bt.region);
  a.win_min += static_cast<int64_t>(batch) * a.H;
  a.win_max += static_cast<int64_t>(batch) * a.H;
  const uint32_t K = a.K;
  const KeyT* lo = static_cast<const KeyT*>(a.sorted) + static_cast<int64_t>(h) * K;
  const KeyT* hic = static_cast<const KeyT*>(a.sorted) + (static_cast<int64_t>(a.H) + h) * K;
  const int tid = static_cast<int>(threadIdx.x);
  float bl = __uint_as_float(0x7f800000u);
  uint32_t bi = 0xffffffffu;
  for (uint32_t i = static_cast<uint32_t>(tid); i < K; i += NT) {
    const float len = value_of_key(kMax - hic[K - 1 - i], KeyT{}, a.f16 != 0) - value_of_key(lo[i], KeyT{}, a.f16 != 0);
    if (len < bl || bi == 0xffffffffu) {
      bl = len;
      bi = i;
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float ol = __shfl_xor(bl, o);
    const uint32_t oi = static_cast<uint32_t>(__shfl_xor(static_cast<int>(bi), o));
    if (ol < bl || (ol == bl && oi < bi)) {
      bl = ol;
      bi = oi;
    }
  }
  const int wave = tid / kWave;
  if (lane_id() == 0) {
    wl[wave] = bl;
    wi[wave] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < NT / kWave; ++w) {
      if (wl[w] < bl || (wl[w] == bl && wi[w] < bi)) {
        bl = wl[w];
        bi = wi[w];
      }
    }
    a.win_min[h] = value_of_key(lo[bi], KeyT{}, a.f16 != 0);
    a.win_max[h] = value_of_key(kMax - hic[K - 1 - bi], KeyT{}, a.f16 != 0);
  }
}

// Merge for heads whose lists fit in registers (nch*K <= 64*R, K <= 64*E):
// wave 0 takes the lo side, wave 1 the hi side with its keys complemented (kMax - key), so
// that both look for their side's K smallest keys in ascending order.  Each wave alone,
// with no barrier: the K-th smallest key by a search over the key bits (counts in
// registers, summed with DPP), the K keys below it (ballot appends, then copies of the
// K-th key up to K), and a bitonic sort of them, E keys per lane (element lane*E + e),
// exchanging registers across lanes for the wide steps.  One barrier, then the window.
// Up to 32 union keys per lane.  Larger unions (64 per lane at K = 421 on the long-context
// shape) took 32 us against 13 us (plus the window kernel) for the side merge.
constexpr int kWaveMergeRegs = 32;  // most union keys per lane
constexpr int kWaveMergeThreads = 2 * kWave;

template <typename KeyT, int R, int E>
__global__ __launch_bounds__(kWaveMergeThreads) void calib_merge_wave_kernel(MergeArgs a, Batches bt) {
  constexpr uint32_t kMax = KeyInfo<KeyT>::kMax;
  constexpr int P = kWave * E;
  __shared__ uint32_t sorted[2][P];
  __shared__ float best_l[2];
  __shared__ uint32_t best_at[2];
  const int batch = static_cast<int>(blockIdx.x) / bt.per;
  const int h = static_cast<int>(blockIdx.x) - batch * bt.per;
  a.lists = in_region(a.lists, batch * bt.region);
  a.fail = in_region(a.fail, batch * bt.region);
  a.win_min += static_cast<int64_t>(batch) * a.H;
  a.win_max += static_cast<int64_t>(batch) * a.H;
  const int tid = static_cast<int>(threadIdx.x);
  const int side = tid / kWave;
  const uint32_t lane = static_cast<uint32_t>(lane_id());
  const uint32_t K = a.K;
  const uint32_t n = static_cast<uint32_t>(a.nch) * K;
  const KeyT* src = static_cast<const KeyT*>(a.lists) +
                    (static_cast<int64_t>(side) * a.H + h) * static_cast<int64_t>(n);
  const uint32_t flip = side == 0 ? 0u : kMax;  // hi side: complemented keys
  if (a.fixup && (a.fail[h] | a.fail[a.H + h]) == 0) return;  // uniform over the workgroup

  uint32_t k[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t i = static_cast<uint32_t>(r) * kWave + lane;
    k[r] = i < n ? (static_cast<uint32_t>(src[i]) ^ flip) : kMax;
  }
  if (!a.fixup && a.fail != nullptr) {
    // the estimated bound holds iff the lists hold at least K keys per side (unused
    // slots hold kMax after the complement)
    uint32_t c = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) c += k[r] != kMax ? 1u : 0u;
    c = wave_sum(c);
    if (lane == 0) best_at[side] = c;
    __syncthreads();
    const bool ok = best_at[0] >= K && best_at[1] >= K;
    __syncthreads();  // both waves have read best_at before it is reused
    if (tid < 2) a.fail[tid * a.H + h] = ok ? 0u : 1u;  // the head's result in both side flags
    if (!ok) return;  // uniform: the fix-up pass redoes this head
  }
  // least t with #{k <= t} >= K (entries past n hold kMax and never change that answer,
  // since the n list entries already reach K at kMax)
  uint32_t t = 0;
#pragma unroll 1
  for (int bit = KeyInfo<KeyT>::kBits - 1; bit >= 0; --bit) {
    const uint32_t probe = t | ((1u << bit) - 1u);
    uint32_t c = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) c += k[r] <= probe ? 1u : 0u;
    if (wave_sum(c) < K) t |= 1u << bit;
  }
  // the keys below t, then copies of t up to K
  uint32_t* out = sorted[side];
  uint32_t less = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const bool take = k[r] < t;
    const uint64_t m = __ballot(take);
    if (take) out[less + lanes_below(m)] = k[r];
    less += static_cast<uint32_t>(__popcll(m));
  }
  for (uint32_t i = less + lane; i < static_cast<uint32_t>(P); i += kWave) out[i] = i < K ? t : kMax;
  __asm__ volatile("" ::: "memory");  // the wave reads back what it wrote (in order)
  uint32_t v[E];
#pragma unroll
  for (int e = 0; e < E; ++e) v[e] = out[lane * E + e];
  // bitonic network over P = 64*E elements, element lane*E + e
#pragma unroll
  for (int kk = 2; kk <= P; kk <<= 1) {
#pragma unroll
    for (int j = kk >> 1; j > 0; j >>= 1) {
      if (j < E) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          if ((e & j) == 0) {
            const bool up = ((lane * E + e) & kk) == 0;
            const uint32_t x0 = v[e], x1 = v[e ^ j];
            const bool sw = (x0 > x1) == up;
            v[e] = sw ? x1 : x0;
            v[e ^ j] = sw ? x0 : x1;
          }
        }
      } else {
        const int lm = j / E;  // partner lane = lane ^ lm
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const uint32_t o = static_cast<uint32_t>(__shfl_xor(static_cast<int>(v[e]), lm));
          const uint32_t i = lane * E + e;
          const bool up = (i & kk) == 0;
          const bool low = (i & j) == 0;
          v[e] = (low == up) ? min(v[e], o) : max(v[e], o);
        }
      }
    }
  }
  __asm__ volatile("" ::: "memory");
#pragma unroll
  for (int e = 0; e < E; ++e) out[lane * E + e] = v[e];
  __syncthreads();

  // Shortest window U[i] - L[i] (float32), smallest i on ties; U[i] is the (K-1-i)-th
  // complemented hi key.
  float bl = __uint_as_float(0x7f800000u);
  uint32_t bi = 0xffffffffu;
  for (uint32_t i = static_cast<uint32_t>(tid); i < K; i += kWaveMergeThreads) {
    const float len =
        value_of_key(sorted[1][K - 1 - i] ^ kMax, KeyT{}, a.f16 != 0) - value_of_key(sorted[0][i], KeyT{}, a.f16 != 0);
    if (len < bl || bi == 0xffffffffu) {
      bl = len;
      bi = i;
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float ol = __shfl_xor(bl, o);
    const uint32_t oi = static_cast<uint32_t>(__shfl_xor(static_cast<int>(bi), o));
    if (ol < bl || (ol == bl && oi < bi)) {
      bl = ol;
      bi = oi;
    }
  }
  if (lane == 0) {
    best_l[side] = bl;
    best_at[side] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    if (best_l[1] < best_l[0] || (best_l[1] == best_l[0] && best_at[1] < best_at[0])) {
      bl = best_l[1];
      bi = best_at[1];
    } else {
      bl = best_l[0];
      bi = best_at[0];
    }
    a.win_min[h] = value_of_key(sorted[0][bi], KeyT{}, a.f16 != 0);
    a.win_max[h] = value_of_key(sorted[1][K - 1 - bi] ^ kMax, KeyT{}, a.f16 != 0);
  }
}

// ----------------------------------------------------------------------------- host side

struct CalibPlan {
  int64_t N = 0, t = 0, K = 0;
  int64_t L = 0, CL = 0;
  int32_t cps = 0, nch = 0;
  int64_t sample_off[kSampleRuns] = {};
  uint32_t sample_w[kSampleRuns] = {}, sample_n[kSampleRuns] = {}, sample_m = 0;
  uint32_t cap_chunk = 0, cap_merge = 0, P = 0;
  size_t lds_chunk = 0, lds_merge = 0;
  size_t key_bytes = 0;
  int wave_merge_e = 0;  // > 0: the two-wave merge with this many sorted keys per lane
  uint32_t rank = 0;     // rank of the sampled group minimum used as the bound
  bool estimate = false; // rank < K: the bound is checked by the merge, failures redone
  // workspace per batch: lists | counts | sorted | bounds | fail
  size_t lists_bytes = 0, counts_bytes = 0, sorted_bytes = 0, bounds_bytes = 0, fail_bytes = 0, total_bytes = 0;
  bool hist = false;     // the histogram path (16-bit keys)
  bool f16 = false;      // 16-bit keys are float16 patterns (else bf16)
  HistPlan hp;
  bool sort = false;     // the collect-and-sort path (float32 keys); its workspace serves every batch in turn
  SortPlan sp;
  // tail lists over (B,S,H,D) rows (float32, D a power of two): the sample runs start at head
  // rows sample_row[], and the chunk kernel addresses slab element e through its row
  bool rows = false;
  int64_t D = 0;
  int32_t log2D = 0, log2Dv = 0;
  int64_t sample_row[kSampleRuns] = {};
};

int32_t log2_exact(int64_t v) {  // v a power of two
  int32_t l = 0;
  while ((int64_t{1} << l) < v) ++l;
  return l;
}

int64_t next_pow2(int64_t v) {
  int64_t p = 1;
  while (p < v) p <<= 1;
  return p;
}

// Validates everything except pointers and computes the launch plan.  The plan depends
// only on the arguments (not on the device), so the workspace query is reproducible.
int make_plan(int dtype, int layout, int64_t nb, int64_t B, int64_t H, int64_t S, int64_t D, double ratio,
              CalibPlan& p) {
  if (dtype != FA3Q_F32 && dtype != FA3Q_BF16 && dtype != FA3Q_F16) return FA3Q_ERR_DTYPE;
  if (layout != FA3Q_BHSD && layout != FA3Q_BSHD) return FA3Q_ERR_LAYOUT;
  if (B <= 0 || H <= 0 || S <= 0 || D <= 0) return FA3Q_ERR_SHAPE;
  const bool k16 = dtype != FA3Q_F32;
  const int vec = k16 ? 8 : 4;
  if (S > (int64_t{1} << 40) / D) return FA3Q_ERR_SHAPE;
  p.L = S * D;
  // 16-byte vectors never straddle a head's rows: (b, h) slabs of S*D values, or (BSHD) rows of D
  if ((layout == FA3Q_BHSD ? p.L : D) % vec != 0) return FA3Q_ERR_SHAPE;
  if (B > (int64_t{1} << 40) / p.L || B * H > (int64_t{1} << 31)) return FA3Q_ERR_SHAPE;
  if (B * H > (int64_t{1} << 50) / p.L) return FA3Q_ERR_SHAPE;
  p.N = B * p.L;
  if (p.N >= (int64_t{1} << 32)) return FA3Q_ERR_SHAPE;  // values per head
  if (!(ratio > 0.0 && ratio <= 1.0)) return FA3Q_ERR_RATIO;  // also rejects NaN
  p.t = static_cast<int64_t>(ratio * static_cast<double>(p.N));  // truncation toward zero
  if (p.t < 1) return FA3Q_ERR_RATIO;
  p.K = p.N - p.t + 1;
  p.f16 = dtype == FA3Q_F16;
  // float32 (B,S,H,D) rows with D a power of two take the tail lists like (B,H,S,D) slabs
  const bool rows_ok = layout == FA3Q_BSHD && !k16 && (D & (D - 1)) == 0 && D >= vec;
  if (p.K > fa3q_calibrate_max_windows(dtype) || (layout == FA3Q_BSHD && !rows_ok) || (k16 && p.N >= kHistMinValues)) {
    if (!k16) {
      // float32: both tails collected through a histogram of their leading 16 bits and sorted
      p.sort = true;
      p.key_bytes = 4;
      const int st = sort_plan(layout == FA3Q_BSHD, B, H, S, D, p.K, p.sp);
      if (st != FA3Q_OK) return st;
      p.total_bytes = p.sp.bytes;
      return FA3Q_OK;
    }
    // 16-bit keys: the whole head as one histogram, any K and either layout
    p.hist = true;
    p.key_bytes = 2;
    const int st = hist_plan(nb, layout == FA3Q_BSHD, 8, B, H, S, D, p.hp);
    if (st != FA3Q_OK) return st;
    p.total_bytes = p.hp.bytes;
    return FA3Q_OK;
  }

  // Sample runs: one per 1/32 of the head's B*L/vec vectors, or back to back (covering
  // the whole head) when it has fewer than kSampleRuns runs' worth.
  const int64_t Lv = p.L / vec, Q = B * Lv;
  // Run j starts at a fixed pseudo-random phase inside its stride (an odd multiple of a
  // 16-bit golden-ratio step, as a fraction of the free range), so that runs do not line up
  // with slab starts or any other period of the data: an over-sampled structure (large
  // first tokens of every sequence, say) would make an estimated bound fail for every head.
  // (B,S,H,D) rows: strides and phases are whole rows of Dv vectors, so every run starts at a
  // row and the runs stay disjoint (the group-minimum bound needs distinct values).
  p.rows = layout == FA3Q_BSHD;
  const int64_t Dv = p.rows ? D / vec : 1;
  p.D = D;
  if (p.rows) {
    p.log2D = log2_exact(D);
    p.log2Dv = log2_exact(Dv);
  }
  int64_t stride = std::max<int64_t>(kSampleThreads, Q / kSampleRuns);
  stride = (stride + Dv - 1) / Dv * Dv;
  int64_t m = 0;
  for (int j = 0; j < kSampleRuns; ++j) {
    int64_t phase = ((((2 * j + 1) * 40503) & 0xffff) * std::max<int64_t>(0, stride - kSampleThreads) >> 16) &
                    ~int64_t{7};  // whole lines
    phase = phase / Dv * Dv;
    const int64_t q0 = j * stride + phase;
    p.sample_n[j] = static_cast<uint32_t>(std::min<int64_t>(kSampleThreads, std::max<int64_t>(0, Q - q0)));
    const int64_t b = p.sample_n[j] ? q0 / Lv : 0, w = p.sample_n[j] ? q0 - b * Lv : 0;
    p.sample_off[j] = (b * H * Lv + w) * vec;
    p.sample_w[j] = static_cast<uint32_t>(w);
    p.sample_row[j] = p.sample_n[j] ? q0 / Dv : 0;
  }
  // a thread's group holds a vector inside the head when its lane is below the largest
  // run length among the group's runs
  for (int g = 0; g < kSampleGroups; ++g) {
    uint32_t most = 0;
    for (int q = 0; q < kSampleGroupRuns; ++q) most = std::max(most, p.sample_n[g * kSampleGroupRuns + q]);
    m += most;
  }
  p.sample_m = static_cast<uint32_t>(m);

  // Rank of the bound: K gives a certain bound (while the sample has K groups); the
  // estimate r = 2e + 4 sqrt(e) + 8 (e: expected sampled keys among the head's K extremes)
  // is used, with the merge's check, when it is far tighter or the only bound there is.
  int64_t sampled = 0;
  for (int j = 0; j < kSampleRuns; ++j) sampled += p.sample_n[j];
  sampled *= vec;
  const double e = static_cast<double>(p.K) * static_cast<double>(sampled) / static_cast<double>(p.N);
  const double r = std::ceil(2.0 * e + 4.0 * std::sqrt(e) + 8.0);
  const int64_t r_est = r < static_cast<double>(p.K) ? static_cast<int64_t>(r) : p.K;
  p.estimate = r_est < p.K && r_est <= static_cast<int64_t>(p.sample_m) &&
               (4 * r_est <= p.K || static_cast<int64_t>(p.sample_m) < p.K);  // 4: measured (K = 211 gains, K = 43 would lose)
  p.rank = static_cast<uint32_t>(p.estimate ? r_est : p.K);

  p.key_bytes = k16 ? 2 : 4;
  const int64_t tile = k16 ? chunk_tile<uint16_t>() : chunk_tile<uint32_t>();
  const int64_t room = k16 ? chunk_room<uint16_t>() : chunk_room<uint32_t>();
  const size_t tmp_keys = static_cast<size_t>(p.K);
  p.cap_chunk = static_cast<uint32_t>(2 * p.K + room);
  if (p.estimate) {
    // candidates are sparse under an estimated bound: a buffer that still leaves room to
    // cut (at least K + one round) but lets kChunkGroupsPerCU workgroups share a CU
    const int64_t fit = (static_cast<int64_t>(kLdsLimit / kChunkGroupsPerCU) - static_cast<int64_t>(kCtlBytes + kStageBytes)) /
                            static_cast<int64_t>(p.key_bytes) - p.K;
    const int64_t cap = std::min<int64_t>(2 * p.K + room, fit / 2);
    if (cap >= p.K + room + 64) p.cap_chunk = static_cast<uint32_t>(cap);
  }
  p.cap_merge = static_cast<uint32_t>(2 * p.K + kMergeTile);
  p.P = static_cast<uint32_t>(next_pow2(p.K));
  p.lds_chunk = kCtlBytes + kStageBytes + (2 * static_cast<size_t>(p.cap_chunk) + tmp_keys) * p.key_bytes;
  if (p.lds_chunk > kLdsLimit) return FA3Q_ERR_UNSUPPORTED;

  // Workgroups resident per CU (bound by LDS and by registers) times 256 CUs: one round of
  // chunks, each as long as possible, never shorter than kMinTilesPerChunk tiles.
  const int64_t per_cu = std::max<int64_t>(
      1, std::min<int64_t>(kChunkGroupsPerCU, static_cast<int64_t>(kLdsLimit / p.lds_chunk)));
  const int64_t want = (kTargetCUs * per_cu + B * H - 1) / (B * H);
  const int64_t most = std::max<int64_t>(1, p.L / (kMinTilesPerChunk * tile));
  p.cps = static_cast<int32_t>(std::max<int64_t>(1, std::min(want, most)));
  p.CL = (p.L + p.cps - 1) / p.cps;
  p.CL = (p.CL + vec - 1) / vec * vec;
  p.cps = static_cast<int32_t>((p.L + p.CL - 1) / p.CL);
  if (B * p.cps > (int64_t{1} << 30) || H * B * p.cps > (int64_t{1} << 31) - 1) return FA3Q_ERR_SHAPE;
  p.nch = static_cast<int32_t>(B * p.cps);
  if (static_cast<int64_t>(p.nch) * p.K <= static_cast<int64_t>(kWave) * kWaveMergeRegs) {
    for (int e = 1; e <= 16; e <<= 1) {
      if (p.K <= static_cast<int64_t>(kWave) * e) {
        p.wave_merge_e = e;
        break;
      }
    }
  }

  // the side merge: control block, the list-count prefix, one side's buffer and cut
  // scratch, and the counting-sort bins (16-bit keys)
  const size_t pre_bytes = p.nch <= kMaxPrefixLists ? round_up(static_cast<size_t>(p.nch + 1) * 4, 16) : 0;
  const size_t sort_bytes = p.key_bytes == 2 ? kSortLdsBytes : 0;
  {
    // a buffer of up to 4K + one tile where the LDS allows: the estimated bounds let a few
    // times K keys through per head, which then need no cut before the last
    const int64_t fit = (static_cast<int64_t>(kLdsLimit) - static_cast<int64_t>(kCtlBytes + pre_bytes + sort_bytes) - 16) /
                            static_cast<int64_t>(p.key_bytes) - p.K;
    const int64_t want = std::min<int64_t>(4 * p.K + kMergeTile, fit);
    if (want > static_cast<int64_t>(p.cap_merge)) p.cap_merge = static_cast<uint32_t>(want);
  }
  p.lds_merge = kCtlBytes + pre_bytes + round_up((static_cast<size_t>(p.cap_merge) + p.K) * p.key_bytes, 16) + sort_bytes;
  if (p.wave_merge_e == 0 && p.lds_merge > kLdsLimit) return FA3Q_ERR_UNSUPPORTED;

  const size_t lists = static_cast<size_t>(H) * p.nch;
  p.lists_bytes = round_up(2 * lists * static_cast<size_t>(p.K) * p.key_bytes, 256);
  p.counts_bytes = round_up(2 * lists * sizeof(uint32_t), 256);
  p.sorted_bytes = p.wave_merge_e > 0 ? 0 : round_up(2 * static_cast<size_t>(H) * p.K * p.key_bytes, 256);
  p.bounds_bytes = round_up(2 * static_cast<size_t>(H) * sizeof(uint32_t), 256);
  p.fail_bytes = round_up(2 * static_cast<size_t>(H) * sizeof(uint32_t), 256);
  p.total_bytes = p.lists_bytes + p.counts_bytes + p.sorted_bytes + p.bounds_bytes + p.fail_bytes;

  return FA3Q_OK;
}

template <typename KeyT, int R>
void launch_wave_merge(int e, int64_t groups, const MergeArgs& ma, const Batches& bt, hipStream_t stream) {
  const dim3 g(static_cast<unsigned>(groups)), blk(kWaveMergeThreads);
  switch (e) {
    case 1: hipLaunchKernelGGL((calib_merge_wave_kernel<KeyT, R, 1>), g, blk, 0, stream, ma, bt); break;
    case 2: hipLaunchKernelGGL((calib_merge_wave_kernel<KeyT, R, 2>), g, blk, 0, stream, ma, bt); break;
    case 4: hipLaunchKernelGGL((calib_merge_wave_kernel<KeyT, R, 4>), g, blk, 0, stream, ma, bt); break;
    case 8: hipLaunchKernelGGL((calib_merge_wave_kernel<KeyT, R, 8>), g, blk, 0, stream, ma, bt); break;
    default: hipLaunchKernelGGL((calib_merge_wave_kernel<KeyT, R, 16>), g, blk, 0, stream, ma, bt); break;
  }
}

// Windows of nb batches (x[b], each (B,H,S,D)) into win_min/win_max [nb][H]; batch b uses
// the workspace region b (p.total_bytes each).
template <typename InT>
int launch(const void* const* x, int64_t nb, int64_t H, const CalibPlan& p, float* win_min, float* win_max,
           void* workspace, hipStream_t stream) {
  using KeyT = InT;
  const auto chunk_kernel = p.rows ? calib_chunk_kernel<InT, true> : calib_chunk_kernel<InT, false>;
  int st = allow_dynamic_lds(reinterpret_cast<const void*>(chunk_kernel), p.lds_chunk);
  if (st != FA3Q_OK) return st;
  if (p.wave_merge_e == 0) {
    st = allow_dynamic_lds(reinterpret_cast<const void*>(calib_merge_side_kernel<KeyT>), p.lds_merge);
    if (st != FA3Q_OK) return st;
  }

  Batches bt;
  for (int b = 0; b < kMaxBatches; ++b) bt.x[b] = b < nb ? x[b] : nullptr;
  bt.region = static_cast<int64_t>(p.total_bytes);
  unsigned char* w0 = static_cast<unsigned char*>(workspace);
  uint32_t* counts = reinterpret_cast<uint32_t*>(w0 + p.lists_bytes);
  void* sorted = w0 + p.lists_bytes + p.counts_bytes;
  uint32_t* bounds = reinterpret_cast<uint32_t*>(w0 + p.lists_bytes + p.counts_bytes + p.sorted_bytes);
  uint32_t* fail = reinterpret_cast<uint32_t*>(w0 + p.total_bytes - p.fail_bytes);
  SampleArgs sa;
  sa.x = nullptr;
  sa.bounds = bounds;
  sa.Lv = p.L / (16 / static_cast<int64_t>(p.key_bytes));
  for (int j = 0; j < kSampleRuns; ++j) {
    sa.run_off[j] = p.sample_off[j];
    sa.run_w[j] = p.sample_w[j];
    sa.run_n[j] = p.sample_n[j];
  }
  sa.H = static_cast<int32_t>(H);
  sa.M = p.sample_m;
  sa.K = p.rank;
  for (int j = 0; j < kSampleRuns; ++j) sa.run_row[j] = p.sample_row[j];
  sa.log2Dv = p.log2Dv;
  sa.D = static_cast<int32_t>(p.D);
  bt.per = static_cast<int32_t>(H);
  const dim3 g_heads(static_cast<unsigned>(nb * H));
  if (p.rows)
    hipLaunchKernelGGL((calib_sample_kernel<InT, false, true>), g_heads, dim3(kSampleThreads), 0, stream, sa, bt);
  else if (sa.Lv >= kSampleThreads)
    hipLaunchKernelGGL((calib_sample_kernel<InT, false, false>), g_heads, dim3(kSampleThreads), 0, stream, sa, bt);
  else
    hipLaunchKernelGGL((calib_sample_kernel<InT, true, false>), g_heads, dim3(kSampleThreads), 0, stream, sa, bt);

  ChunkArgs ca;
  ca.x = nullptr;
  ca.lists = workspace;
  ca.counts = counts;
  ca.bounds = bounds;
  ca.fail = nullptr;
  ca.L = p.L;
  ca.CL = p.CL;
  ca.H = static_cast<int32_t>(H);
  ca.cps = p.cps;
  ca.nch = p.nch;
  ca.K = static_cast<uint32_t>(p.K);
  ca.cap = p.cap_chunk;
  ca.pad = (p.wave_merge_e > 0 || p.nch > kMaxPrefixLists) ? 1 : 0;
  ca.log2D = p.log2D;
  ca.row_stride = H * p.D;
  Batches bc = bt;
  bc.per = static_cast<int32_t>(H * p.nch);
  const dim3 g_chunks(static_cast<unsigned>(nb * H * p.nch));
  hipLaunchKernelGGL(chunk_kernel, g_chunks, dim3(kChunkThreads), p.lds_chunk, stream, ca, bc);
  MergeArgs ma;
  ma.lists = workspace;
  ma.counts = counts;
  ma.sorted = sorted;
  ma.win_min = win_min;
  ma.win_max = win_max;
  ma.fail = p.estimate ? fail : nullptr;
  ma.fixup = 0;
  ma.H = static_cast<int32_t>(H);
  ma.nch = p.nch;
  ma.K = static_cast<uint32_t>(p.K);
  ma.cap = p.cap_merge;
  ma.P = p.P;
  ma.f16 = p.f16 ? 1 : 0;
  auto merge = [&](const MergeArgs& m) {
    if (p.wave_merge_e > 0)
      launch_wave_merge<KeyT, kWaveMergeRegs>(p.wave_merge_e, nb * H, m, bt, stream);
    else {
      Batches bs = bt;
      bs.per = static_cast<int32_t>(2 * H);
      hipLaunchKernelGGL(calib_merge_side_kernel<KeyT>, dim3(static_cast<unsigned>(2 * nb * H)),
                         dim3(kMergeThreads), p.lds_merge, stream, m, bs);
    }
  };
  merge(ma);
  if (p.estimate) {
    // heads whose estimated bound held fewer than K values: again with no bound
    ChunkArgs cf = ca;
    cf.fail = fail;
    hipLaunchKernelGGL(chunk_kernel, g_chunks, dim3(kChunkThreads), p.lds_chunk, stream, cf, bc);
    MergeArgs mf = ma;
    mf.fixup = 1;
    merge(mf);
  }
  if (p.wave_merge_e == 0)  // the windows of every head from its final sorted sides
    hipLaunchKernelGGL(calib_window_kernel<KeyT>, g_heads, dim3(256), 0, stream, ma, bt);
  return launch_status();
}

// Unsigned key whose order is the float32 total order with -0.0 below +0.0.
__device__ __forceinline__ uint32_t total_order_key(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Running min/max over nb batches' windows, head by head, in batch order (the same
// comparisons as nb accumulate calls); init starts from the identity (+inf, -inf).
__global__ __launch_bounds__(256) void accumulate_batches_kernel(float* __restrict__ run_min, float* __restrict__ run_max,
                                                                 const float* __restrict__ win_min,
                                                                 const float* __restrict__ win_max, int64_t nb,
                                                                 int64_t H, int init) {
  const int64_t h = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (h >= H) return;
  float mn = init ? __uint_as_float(0x7f800000u) : run_min[h];
  float mx = init ? __uint_as_float(0xff800000u) : run_max[h];
  for (int64_t b = 0; b < nb; ++b) {
    const float c = win_min[b * H + h], d = win_max[b * H + h];
    mn = total_order_key(c) < total_order_key(mn) ? c : mn;
    mx = total_order_key(d) > total_order_key(mx) ? d : mx;
  }
  run_min[h] = mn;
  run_max[h] = mx;
}

}  // namespace
}  // namespace fa3q

using namespace fa3q;

extern "C" int64_t fa3q_calibrate_max_windows(int dtype) {
  // The chunk kernel keeps 2*cap + K keys (cap = 2K + one round of appends) after its
  // control block and stage; the side merge cap + K keys (cap = 2K + one merge tile) after
  // its control block and a list-count prefix of up to kMaxPrefixLists + 1 words, then the
  // counting-sort bins for 16-bit keys.  Largest K for which both fit the 160 KiB a gfx950
  // workgroup may use.
  if (dtype != FA3Q_F32 && dtype != FA3Q_BF16 && dtype != FA3Q_F16) return 0;
  const int64_t kb = dtype == FA3Q_F32 ? 4 : 2;
  const int64_t round = kb == 2 ? chunk_room<uint16_t>() : chunk_room<uint32_t>();
  const int64_t lds = static_cast<int64_t>(kLdsLimit);
  const int64_t chunk = (lds - static_cast<int64_t>(kCtlBytes + kStageBytes) - 2 * round * kb) / (5 * kb);
  const int64_t pre = static_cast<int64_t>(round_up(static_cast<size_t>(kMaxPrefixLists + 1) * 4, 16));
  const int64_t sort = kb == 2 ? static_cast<int64_t>(kSortLdsBytes) : 0;
  const int64_t merge = (lds - static_cast<int64_t>(kCtlBytes) - pre - sort - 16 - kMergeTile * kb) / (3 * kb);
  return std::min(chunk, merge);
}

namespace fa3q {
namespace {

// Windows of nb batches into win_min/win_max [nb][H] on the path the plan chose.
int launch_windows(const void* const* xs, int64_t nb, int64_t H, const CalibPlan& p, float* win_min, float* win_max,
                   void* workspace, hipStream_t s) {
  if (p.hist) return hist_launch(xs, nb, H, p.f16, p.t, p.K, p.hp, win_min, win_max, workspace, s);
  if (p.sort) return sort_launch(xs, nb, H, p.t, p.K, p.sp, win_min, win_max, workspace, s);
  if (p.key_bytes == 2) return launch<uint16_t>(xs, nb, H, p, win_min, win_max, workspace, s);
  return launch<uint32_t>(xs, nb, H, p, win_min, win_max, workspace, s);
}

size_t batches_workspace_bytes(int dtype, int layout, int64_t nb, int64_t B, int64_t H, int64_t S, int64_t D,
                               double ratio) {
  CalibPlan p;
  if (nb <= 0 || nb > kMaxBatches || make_plan(dtype, layout, nb, B, H, S, D, ratio, p) != FA3Q_OK) return 0;
  if (!p.hist && !p.sort && nb * B * H * p.nch > (int64_t{1} << 31) - 1) return 0;
  return static_cast<size_t>(p.sort ? 1 : nb) * p.total_bytes + round_up(2 * static_cast<size_t>(nb * H) * sizeof(float), 256);
}

// Validation and launches of the several-batch entry points: run_min/run_max may both be
// null when win_min/win_max are given (windows only, no running statistics).
int calibrate_batches(const void* const* xs, int64_t nb, int dtype, int layout, int64_t B, int64_t H, int64_t S,
                      int64_t D, double ratio, float* run_min, float* run_max, int init, float* win_min,
                      float* win_max, void* workspace, size_t workspace_bytes, void* stream) {
  if (!xs || (!run_min != !run_max) || (!win_min != !win_max) || (!run_min && !win_min)) return FA3Q_ERR_NULL;
  if (nb <= 0 || nb > kMaxBatches) return FA3Q_ERR_SHAPE;
  for (int64_t b = 0; b < nb; ++b)
    if (!xs[b]) return FA3Q_ERR_NULL;
  CalibPlan p;
  const int st = make_plan(dtype, layout, nb, B, H, S, D, ratio, p);
  if (st != FA3Q_OK) return st;
  if (!p.hist && !p.sort && nb * H * p.nch > (int64_t{1} << 31) - 1) return FA3Q_ERR_SHAPE;
  for (int64_t b = 0; b < nb; ++b)
    if (!is_aligned(xs[b], 16)) return FA3Q_ERR_ALIGN;
  if ((run_min && (!is_aligned(run_min, 4) || !is_aligned(run_max, 4))) ||
      (win_min && (!is_aligned(win_min, 4) || !is_aligned(win_max, 4))))
    return FA3Q_ERR_ALIGN;
  const size_t need = batches_workspace_bytes(dtype, layout, nb, B, H, S, D, ratio);
  if (!workspace || workspace_bytes < need) return FA3Q_ERR_WORKSPACE;
  if (!is_aligned(workspace, 256)) return FA3Q_ERR_ALIGN;
  float* wins = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) +
                                        static_cast<size_t>(p.sort ? 1 : nb) * p.total_bytes);
  float* wmin = win_min ? win_min : wins;
  float* wmax = win_max ? win_max : wins + nb * H;
  hipStream_t s = as_stream(stream);
  const int lst = launch_windows(xs, nb, H, p, wmin, wmax, workspace, s);
  if (lst != FA3Q_OK || !run_min) return lst;
  hipLaunchKernelGGL(accumulate_batches_kernel, dim3(static_cast<unsigned>((H + 255) / 256)), dim3(256), 0, s, run_min,
                     run_max, wmin, wmax, nb, H, init ? 1 : 0);
  return launch_status();
}

}  // namespace
}  // namespace fa3q

extern "C" size_t fa3q_calibrate_workspace_bytes(int dtype, int64_t B, int64_t H, int64_t S,
                                                 int64_t D, double ratio) {
  CalibPlan p;
  if (make_plan(dtype, FA3Q_BHSD, 1, B, H, S, D, ratio, p) != FA3Q_OK) return 0;
  return p.total_bytes;
}

extern "C" int fa3q_calibrate_perhead(const void* x, int dtype, int64_t B, int64_t H, int64_t S,
                                      int64_t D, double ratio, float* win_min, float* win_max,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  if (!x || !win_min || !win_max) return FA3Q_ERR_NULL;
  CalibPlan p;
  const int st = make_plan(dtype, FA3Q_BHSD, 1, B, H, S, D, ratio, p);
  if (st != FA3Q_OK) return st;
  if (!is_aligned(x, 16) || !is_aligned(win_min, 4) || !is_aligned(win_max, 4))
    return FA3Q_ERR_ALIGN;
  if (!workspace || workspace_bytes < p.total_bytes) return FA3Q_ERR_WORKSPACE;
  if (!is_aligned(workspace, 256)) return FA3Q_ERR_ALIGN;
  const void* xs[1] = {x};
  return launch_windows(xs, 1, H, p, win_min, win_max, workspace, as_stream(stream));
}

extern "C" size_t fa3q_calibrate_batches_workspace_bytes(int dtype, int64_t nb, int64_t B, int64_t H, int64_t S,
                                                         int64_t D, double ratio) {
  return batches_workspace_bytes(dtype, FA3Q_BHSD, nb, B, H, S, D, ratio);
}

extern "C" int fa3q_calibrate_batches(const void* const* xs, int64_t nb, int dtype, int64_t B, int64_t H, int64_t S,
                                      int64_t D, double ratio, float* run_min, float* run_max, int init,
                                      float* win_min, float* win_max, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  if (!run_min || !run_max) return FA3Q_ERR_NULL;
  return calibrate_batches(xs, nb, dtype, FA3Q_BHSD, B, H, S, D, ratio, run_min, run_max, init, win_min, win_max,
                           workspace, workspace_bytes, stream);
}

extern "C" size_t fa3q_calibrate_ex_workspace_bytes(int dtype, int layout, int64_t nb, int64_t B, int64_t H,
                                                    int64_t S, int64_t D, double ratio) {
  return batches_workspace_bytes(dtype, layout, nb, B, H, S, D, ratio);
}

extern "C" int fa3q_calibrate_ex(const void* const* xs, int64_t nb, int dtype, int layout, int64_t B, int64_t H,
                                 int64_t S, int64_t D, double ratio, float* run_min, float* run_max, int init,
                                 float* win_min, float* win_max, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  return calibrate_batches(xs, nb, dtype, layout, B, H, S, D, ratio, run_min, run_max, init, win_min, win_max,
                           workspace, workspace_bytes, stream);
}
