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
//   calib_chunk_kernel   one HBM pass.  Each workgroup streams a contiguous chunk of one
//                        head (inside one (b,h) slab) and keeps, in LDS, a candidate
//                        buffer per side holding a superset of the chunk's K smallest
//                        (K largest) values.  A value enters only if it beats the side's
//                        threshold; when a buffer passes 2K entries an exact LDS radix
//                        select cuts it back to the K extreme values and tightens the
//                        threshold.  The chunk's exact tails go to the workspace.
//   calib_merge_kernel   one workgroup per head: the same select over the chunks' tails
//                        gives the head's exact K smallest and K largest values, a
//                        bitonic sort orders them, and a block reduction finds the
//                        shortest float32 window U[i]-L[i], smallest i on ties.
//
// Values are compared through order-preserving unsigned keys (16-bit for bf16 input,
// 32-bit for float32), which realise the float total order with -0.0 below +0.0.
// Ties need no special care: a tail is a multiset of key values, and dropping a value
// equal to the K-th smallest once K values <= it are held never changes that multiset.
#include "fa3q_internal.hpp"

namespace fa3q {
namespace {

constexpr int kChunkThreads = 256;
constexpr int kMergeThreads = 1024;
constexpr int kVecPerThread = 4;       // 16-byte vectors per thread per tile (chunk kernel)
constexpr int kMergePerThread = 4;     // keys per thread per tile (merge kernel)
constexpr int kMergeTile = kMergeThreads * kMergePerThread;
constexpr int64_t kTargetCUs = 256;    // MI355X compute units (sizes the chunk grid)
constexpr int kMinTilesPerChunk = 8;

// Control words at the start of dynamic LDS.
enum Ctl : int {
  kSlotLo = 0,   // [3] per-tile append counters, lo side
  kSlotHi = 3,   // [3] hi side
  kThrLo = 6,    // current lo threshold key: candidates are keys < thrLo
  kThrHi = 7,    // current hi threshold key: candidates are keys > thrHi
  kTmpCnt = 8,
  kSelDigit = 9,
  kSelBefore = 10,
  kSelCount = 11,
  kBestLen = 12,
  kHist = 64,    // [256] radix histogram
  kWaveScratch = 64 + 256,  // [2 * 16] per-wave (length, index) pairs
  kCtlWords = 64 + 256 + 32
};
constexpr size_t kCtlBytes = 2048;
static_assert(kCtlWords * 4 <= kCtlBytes, "control block too small");

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

// Order-preserving key of a bf16 pattern (low 16 bits) and of a float32 pattern.
__device__ __forceinline__ uint32_t key_bf16(uint32_t b) {
  return b ^ ((b & 0x8000u) ? 0xffffu : 0x8000u);
}
__device__ __forceinline__ uint32_t key_f32(uint32_t b) {
  return b ^ ((b & 0x80000000u) ? 0xffffffffu : 0x80000000u);
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));

// Keys held in dwords as they come from memory: two 16-bit keys per dword for bf16
// input (transformed in place with packed 16-bit ops), one 32-bit key for float32.
template <typename InT>
struct Pack;
template <>
struct Pack<uint16_t> {
  static constexpr int kPerDword = 2;
  static constexpr uint32_t kMinInit = 0xffffffffu;
  static constexpr uint32_t kMaxInit = 0u;
  __device__ static uint32_t keys(uint32_t w) {  // key_bf16 on both halves
    const s16x2 sg = __builtin_bit_cast(s16x2, w) >> (s16x2){15, 15};
    return w ^ ((__builtin_bit_cast(uint32_t, sg) & 0x7fff7fffu) | 0x80008000u);
  }
  __device__ static uint32_t at(uint32_t w, int i) { return i ? (w >> 16) : (w & 0xffffu); }
  __device__ static uint32_t pmin(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2, a),
                                                                 __builtin_bit_cast(u16x2, b)));
  }
  __device__ static uint32_t pmax(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                 __builtin_bit_cast(u16x2, b)));
  }
  __device__ static uint32_t hmin(uint32_t p) { return min(p & 0xffffu, p >> 16); }
  __device__ static uint32_t hmax(uint32_t p) { return max(p & 0xffffu, p >> 16); }
};
template <>
struct Pack<uint32_t> {
  static constexpr int kPerDword = 1;
  static constexpr uint32_t kMinInit = 0xffffffffu;
  static constexpr uint32_t kMaxInit = 0u;
  __device__ static uint32_t keys(uint32_t w) { return key_f32(w); }
  __device__ static uint32_t at(uint32_t w, int) { return w; }
  __device__ static uint32_t pmin(uint32_t a, uint32_t b) { return min(a, b); }
  __device__ static uint32_t pmax(uint32_t a, uint32_t b) { return max(a, b); }
  __device__ static uint32_t hmin(uint32_t p) { return p; }
  __device__ static uint32_t hmax(uint32_t p) { return p; }
};

__device__ __forceinline__ float value_of_key(uint32_t k, uint16_t) {
  const uint32_t b = (k & 0x8000u) ? (k ^ 0x8000u) : (k ^ 0xffffu);
  return __uint_as_float(b << 16);
}
__device__ __forceinline__ float value_of_key(uint32_t k, uint32_t) {
  const uint32_t b = (k & 0x80000000u) ? (k ^ 0x80000000u) : ~k;
  return __uint_as_float(b);
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
  const uint32_t below = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
  if (pred) buf[base + below] = static_cast<KeyT>(key);
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
    for (uint32_t i = tid; i < n; i += NT) {
      const uint32_t k = buf[i];
      if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & 0xffu], 1u);
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
  uint32_t tile;      // most entries one tile can append per side
  uint32_t base_lo;   // entries held before the current tile
  uint32_t base_hi;
  uint32_t thr_lo;    // lo candidates: key < thr_lo
  uint32_t thr_hi;    // hi candidates: key > thr_hi
  int parity;         // tile counter mod 3 (append-counter slot)

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

  // After every thread appended its share of one tile.  Three rotating counter slots let
  // a single barrier per tile separate "read this tile's count" from the next tile's
  // appends: slot p is filled in tile i, read after barrier i, and cleared after
  // barrier i+1 (when every thread has read it), before tile i+3 uses it again.
  __device__ void end_tile() {
    lds_barrier();
    base_lo += ctl[kSlotLo + parity];
    base_hi += ctl[kSlotHi + parity];
    const int clear = parity == 0 ? 2 : parity - 1;
    if (threadIdx.x == 0) {
      ctl[kSlotLo + clear] = 0;
      ctl[kSlotHi + clear] = 0;
    }
    parity = parity == 2 ? 0 : parity + 1;
    if (base_lo > cap - tile) {
      compact<KeyT, NT, true>(lo, base_lo, K, tmp, ctl);
      base_lo = K;
      thr_lo = ctl[kThrLo];
    }
    if (base_hi > cap - tile) {
      compact<KeyT, NT, false>(hi, base_hi, K, tmp, ctl);
      base_hi = K;
      thr_hi = ctl[kThrHi];
    }
  }

  // Filter one tile into both buffers.  kw holds W dwords of packed keys per thread, in
  // groups of 4 dwords (one 16-byte vector each); vv[] marks vectors inside the chunk.
  template <typename InT, int W>
  __device__ __forceinline__ void filter_tile(const uint32_t (&kw)[W], const bool (&vv)[W / 4]) {
    using P = Pack<InT>;
    uint32_t pmn = P::kMinInit, pmx = P::kMaxInit;
#pragma unroll
    for (int j = 0; j < W; ++j) {
      if (vv[j / 4]) {
        pmn = P::pmin(pmn, kw[j]);
        pmx = P::pmax(pmx, kw[j]);
      }
    }
    const uint32_t kmin = P::hmin(pmn), kmax = P::hmax(pmx);
    if (__ballot(kmin < thr_lo) != 0) {
#pragma unroll
      for (int j = 0; j < W; ++j)
#pragma unroll
        for (int i = 0; i < P::kPerDword; ++i) {
          const uint32_t k = P::at(kw[j], i);
          append_lo(vv[j / 4] && k < thr_lo, k);
        }
    }
    if (__ballot(kmax > thr_hi) != 0) {
#pragma unroll
      for (int j = 0; j < W; ++j)
#pragma unroll
        for (int i = 0; i < P::kPerDword; ++i) {
          const uint32_t k = P::at(kw[j], i);
          append_hi(vv[j / 4] && k > thr_hi, k);
        }
    }
    end_tile();
  }

  // First tile of a chunk, all of it real data: split every thread's keys into `groups`
  // groups of consecutive keys.  The K-th smallest group minimum has at least K keys at
  // or below it (one per group), so it is a valid lo threshold from the start and only
  // keys at or below it enter the buffer; symmetrically for the K-th largest group
  // maximum.  Needs NT * groups >= K and groups dividing the keys per thread.
  template <typename InT, int W>
  __device__ void bootstrap(const uint32_t (&kw)[W], int groups) {
    using P = Pack<InT>;
    constexpr int E = W * P::kPerDword;
    const int tid = static_cast<int>(threadIdx.x);
    const int gs = E / groups;
    uint32_t mn = KeyInfo<KeyT>::kMax, mx = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint32_t k = P::at(kw[e / P::kPerDword], e % P::kPerDword);
      mn = min(mn, k);
      mx = max(mx, k);
      if (((e + 1) % gs) == 0) {
        const int g = tid * groups + (e + 1) / gs - 1;
        lo[g] = static_cast<KeyT>(mn);
        hi[g] = static_cast<KeyT>(mx);
        mn = KeyInfo<KeyT>::kMax;
        mx = 0;
      }
    }
    const uint32_t n = static_cast<uint32_t>(NT * groups);
    lds_barrier();
    uint32_t t_lo, t_hi, less, eq;
    block_select<KeyT, NT>(lo, n, K, ctl, t_lo, less, eq);
    block_select<KeyT, NT>(hi, n, n - K + 1, ctl, t_hi, less, eq);
    // block_select returns after its last barrier: nobody reads lo[]/hi[] any more
#pragma unroll
    for (int j = 0; j < W; ++j)
#pragma unroll
      for (int i = 0; i < P::kPerDword; ++i) {
        const uint32_t k = P::at(kw[j], i);
        append_lo(k <= t_lo, k);
      }
#pragma unroll
    for (int j = 0; j < W; ++j)
#pragma unroll
      for (int i = 0; i < P::kPerDword; ++i) {
        const uint32_t k = P::at(kw[j], i);
        append_hi(k >= t_hi, k);
      }
    thr_lo = t_lo;
    thr_hi = t_hi;
    end_tile();
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
  int32_t boot_groups;  // groups per thread for the first-tile bootstrap (0: none)
  uint32_t K;
  uint32_t cap;
};

template <typename InT>
constexpr int chunk_tile() {
  return kChunkThreads * kVecPerThread * 4 * Pack<InT>::kPerDword;
}

template <typename InT>
__global__ __launch_bounds__(kChunkThreads, 4) void calib_chunk_kernel(ChunkArgs a) {
  using KeyT = InT;  // 16-bit keys for bf16 input, 32-bit keys for float32 input
  constexpr int NT = kChunkThreads;
  constexpr int kPerVec = 16 / sizeof(InT);  // elements per 16-byte vector
  constexpr int W = kVecPerThread * 4;        // dwords per thread per tile
  constexpr int kTile = chunk_tile<InT>();
  extern __shared__ __align__(16) unsigned char smem[];
  uint32_t* ctl = reinterpret_cast<uint32_t*>(smem);
  KeyT* lo = reinterpret_cast<KeyT*>(smem + kCtlBytes);

  TailState<KeyT, NT> st;
  st.lo = lo;
  st.hi = lo + a.cap;
  st.tmp = lo + 2 * a.cap;
  st.ctl = ctl;
  st.K = a.K;
  st.cap = a.cap;
  st.tile = kTile;
  st.init();

  const int h = static_cast<int>(blockIdx.x) / a.nch;
  const int c = static_cast<int>(blockIdx.x) - h * a.nch;
  const int b = c / a.cps;
  const int part = c - b * a.cps;
  const InT* slab = static_cast<const InT*>(a.x) + (static_cast<int64_t>(b) * a.H + h) * a.L;
  const int64_t begin = static_cast<int64_t>(part) * a.CL;
  const int64_t end = min(a.L, begin + a.CL);
  const int tid = static_cast<int>(threadIdx.x);

  uint4 cur[kVecPerThread], nxt[kVecPerThread];
#pragma unroll
  for (int v = 0; v < kVecPerThread; ++v) {
    cur[v] = make_uint4(0, 0, 0, 0);
    nxt[v] = make_uint4(0, 0, 0, 0);
  }
  auto load_tile = [&](int64_t t0, uint4 (&dst)[kVecPerThread]) {
#pragma unroll
    for (int v = 0; v < kVecPerThread; ++v) {
      const int64_t e = t0 + static_cast<int64_t>(v * NT + tid) * kPerVec;
      if (e < end) dst[v] = *reinterpret_cast<const uint4*>(slab + e);
    }
  };
  if (begin < end) load_tile(begin, cur);
  bool first = true;
  for (int64_t t0 = begin; t0 < end; t0 += kTile) {
    if (t0 + kTile < end) load_tile(t0 + kTile, nxt);
    uint32_t kw[W];
    bool vv[kVecPerThread];
#pragma unroll
    for (int v = 0; v < kVecPerThread; ++v) {
      kw[4 * v + 0] = Pack<InT>::keys(cur[v].x);
      kw[4 * v + 1] = Pack<InT>::keys(cur[v].y);
      kw[4 * v + 2] = Pack<InT>::keys(cur[v].z);
      kw[4 * v + 3] = Pack<InT>::keys(cur[v].w);
      vv[v] = t0 + static_cast<int64_t>(v * NT + tid) * kPerVec < end;
    }
    if (first && a.boot_groups > 0 && t0 + kTile <= end) {
      st.template bootstrap<InT, W>(kw, a.boot_groups);
    } else {
      st.template filter_tile<InT, W>(kw, vv);
    }
    first = false;
#pragma unroll
    for (int v = 0; v < kVecPerThread; ++v) cur[v] = nxt[v];
  }
  st.finish();

  // Fixed-size list per chunk; slots past the held count get keys that fail both filters.
  const int64_t list = static_cast<int64_t>(h) * a.nch + c;
  const int64_t heads_lists = static_cast<int64_t>(a.H) * a.nch;
  KeyT* out_lo = static_cast<KeyT*>(a.lists) + list * a.K;
  KeyT* out_hi = static_cast<KeyT*>(a.lists) + (heads_lists + list) * a.K;
  for (uint32_t i = tid; i < a.K; i += NT) {
    out_lo[i] = i < st.base_lo ? st.lo[i] : static_cast<KeyT>(KeyInfo<KeyT>::kMax);
    out_hi[i] = i < st.base_hi ? st.hi[i] : static_cast<KeyT>(0);
  }
}

struct MergeArgs {
  const void* lists;
  float* win_min;
  float* win_max;
  int32_t H;
  int32_t nch;
  uint32_t K;
  uint32_t cap;
  uint32_t P;  // next power of two >= K
};

template <typename KeyT>
__global__ __launch_bounds__(kMergeThreads) void calib_merge_kernel(MergeArgs a) {
  constexpr int NT = kMergeThreads;
  extern __shared__ __align__(16) unsigned char smem[];
  uint32_t* ctl = reinterpret_cast<uint32_t*>(smem);
  KeyT* lo = reinterpret_cast<KeyT*>(smem + kCtlBytes);

  TailState<KeyT, NT> st;
  st.lo = lo;
  st.hi = lo + a.cap;
  st.tmp = lo + 2 * a.cap;
  st.ctl = ctl;
  st.K = a.K;
  st.cap = a.cap;
  st.tile = kMergeTile;
  st.init();

  const int h = static_cast<int>(blockIdx.x);
  const int tid = static_cast<int>(threadIdx.x);
  const int64_t per_head = static_cast<int64_t>(a.nch) * a.K;
  const KeyT* src_lo = static_cast<const KeyT*>(a.lists) + h * per_head;
  const KeyT* src_hi = static_cast<const KeyT*>(a.lists) + (static_cast<int64_t>(a.H) + h) * per_head;

  // Stream the head's chunk tails (one flat array per side) through the same filter.
  for (int64_t t0 = 0; t0 < per_head; t0 += kMergeTile) {
    uint32_t klo[kMergePerThread], khi[kMergePerThread];
    bool ev[kMergePerThread];
#pragma unroll
    for (int e = 0; e < kMergePerThread; ++e) {
      const int64_t i = t0 + e * NT + tid;
      ev[e] = i < per_head;
      klo[e] = ev[e] ? static_cast<uint32_t>(src_lo[i]) : KeyInfo<KeyT>::kMax;
      khi[e] = ev[e] ? static_cast<uint32_t>(src_hi[i]) : 0u;
    }
#pragma unroll
    for (int e = 0; e < kMergePerThread; ++e) st.append_lo(klo[e] < st.thr_lo, klo[e]);
#pragma unroll
    for (int e = 0; e < kMergePerThread; ++e) st.append_hi(khi[e] > st.thr_hi, khi[e]);
    st.end_tile();
  }
  st.finish();  // now exactly K per side (every head holds at least K values)

  // Ascending bitonic sort of both tails, padded to P with the largest key.
  const uint32_t K = a.K, P = a.P;
  for (uint32_t i = K + tid; i < P; i += NT) {
    st.lo[i] = static_cast<KeyT>(KeyInfo<KeyT>::kMax);
    st.hi[i] = static_cast<KeyT>(KeyInfo<KeyT>::kMax);
  }
  lds_barrier();
  for (uint32_t k = 2; k <= P; k <<= 1) {
    for (uint32_t j = k >> 1; j > 0; j >>= 1) {
      for (uint32_t i = tid; i < P / 2; i += NT) {
        const uint32_t l = ((i & ~(j - 1)) << 1) | (i & (j - 1));
        const uint32_t r = l + j;
        const bool up = (l & k) == 0;
        const KeyT a0 = st.lo[l], a1 = st.lo[r];
        if ((a0 > a1) == up) { st.lo[l] = a1; st.lo[r] = a0; }
        const KeyT b0 = st.hi[l], b1 = st.hi[r];
        if ((b0 > b1) == up) { st.hi[l] = b1; st.hi[r] = b0; }
      }
      lds_barrier();
    }
  }

  // Shortest window U[i] - L[i] (float32), smallest i on ties.
  float best_len = __uint_as_float(0x7f800000u);
  uint32_t best_i = 0xffffffffu;
  for (uint32_t i = tid; i < K; i += NT) {
    const float len = value_of_key(st.hi[i], KeyT{}) - value_of_key(st.lo[i], KeyT{});
    if (len < best_len || best_i == 0xffffffffu) {
      best_len = len;
      best_i = i;
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float ol = __shfl_xor(best_len, o);
    const uint32_t oi = __shfl_xor(best_i, o);
    if (ol < best_len || (ol == best_len && oi < best_i)) {
      best_len = ol;
      best_i = oi;
    }
  }
  float* wl = reinterpret_cast<float*>(ctl + kWaveScratch);
  uint32_t* wi = ctl + kWaveScratch + 16;
  const int wave = tid / kWave;
  if (lane_id() == 0) {
    wl[wave] = best_len;
    wi[wave] = best_i;
  }
  lds_barrier();
  if (tid == 0) {
    float bl = wl[0];
    uint32_t bi = wi[0];
    for (int w = 1; w < NT / kWave; ++w) {
      if (wl[w] < bl || (wl[w] == bl && wi[w] < bi)) {
        bl = wl[w];
        bi = wi[w];
      }
    }
    a.win_min[h] = value_of_key(st.lo[bi], KeyT{});
    a.win_max[h] = value_of_key(st.hi[bi], KeyT{});
  }
}

// ----------------------------------------------------------------------------- host side

struct CalibPlan {
  int64_t N = 0, t = 0, K = 0;
  int64_t L = 0, CL = 0;
  int32_t cps = 0, nch = 0, boot_groups = 0;
  uint32_t cap_chunk = 0, cap_merge = 0, P = 0;
  size_t lds_chunk = 0, lds_merge = 0;
  size_t key_bytes = 0;
  size_t lists_bytes = 0, total_bytes = 0;
};

int64_t next_pow2(int64_t v) {
  int64_t p = 1;
  while (p < v) p <<= 1;
  return p;
}

// Validates everything except pointers and computes the launch plan.  The plan depends
// only on the arguments (not on the device), so the workspace query is reproducible.
int make_plan(int dtype, int64_t B, int64_t H, int64_t S, int64_t D, double ratio, CalibPlan& p) {
  if (dtype != FA3Q_F32 && dtype != FA3Q_BF16) return FA3Q_ERR_DTYPE;
  if (B <= 0 || H <= 0 || S <= 0 || D <= 0) return FA3Q_ERR_SHAPE;
  const int vec = dtype == FA3Q_BF16 ? 8 : 4;
  if (S > (int64_t{1} << 40) / D) return FA3Q_ERR_SHAPE;
  p.L = S * D;
  if (p.L % vec != 0) return FA3Q_ERR_SHAPE;
  if (B > (int64_t{1} << 40) / p.L || B * H > (int64_t{1} << 31)) return FA3Q_ERR_SHAPE;
  if (B * H > (int64_t{1} << 50) / p.L) return FA3Q_ERR_SHAPE;
  p.N = B * p.L;
  if (!(ratio > 0.0 && ratio <= 1.0)) return FA3Q_ERR_RATIO;  // also rejects NaN
  p.t = static_cast<int64_t>(ratio * static_cast<double>(p.N));  // truncation toward zero
  if (p.t < 1) return FA3Q_ERR_RATIO;
  p.K = p.N - p.t + 1;
  if (p.K > fa3q_calibrate_max_windows(dtype)) return FA3Q_ERR_UNSUPPORTED;

  p.key_bytes = dtype == FA3Q_BF16 ? 2 : 4;
  const int64_t tile = dtype == FA3Q_BF16 ? chunk_tile<uint16_t>() : chunk_tile<uint32_t>();
  const int E = static_cast<int>(tile / kChunkThreads);
  p.cap_chunk = static_cast<uint32_t>(2 * p.K + tile);
  p.cap_merge = static_cast<uint32_t>(2 * p.K + kMergeTile);
  p.P = static_cast<uint32_t>(next_pow2(p.K));
  p.lds_chunk = kCtlBytes + (2 * static_cast<size_t>(p.cap_chunk) + p.K) * p.key_bytes;
  p.lds_merge = kCtlBytes + (2 * static_cast<size_t>(p.cap_merge) + p.K) * p.key_bytes;
  if (p.lds_chunk > kLdsLimit || p.lds_merge > kLdsLimit) return FA3Q_ERR_UNSUPPORTED;

  // Workgroups resident per CU (LDS-bound, at most 8) times 256 CUs: one round of chunks,
  // each as long as possible, never shorter than kMinTilesPerChunk tiles.
  const int64_t per_cu = std::max<int64_t>(1, std::min<int64_t>(8, static_cast<int64_t>(kLdsLimit / p.lds_chunk)));
  const int64_t want = (kTargetCUs * per_cu + B * H - 1) / (B * H);
  const int64_t most = std::max<int64_t>(1, p.L / (kMinTilesPerChunk * tile));
  p.cps = static_cast<int32_t>(std::max<int64_t>(1, std::min(want, most)));
  p.CL = (p.L + p.cps - 1) / p.cps;
  p.CL = (p.CL + vec - 1) / vec * vec;
  p.cps = static_cast<int32_t>((p.L + p.CL - 1) / p.CL);
  if (B * p.cps > (int64_t{1} << 30) || H * B * p.cps > (int64_t{1} << 31) - 1) return FA3Q_ERR_SHAPE;
  p.nch = static_cast<int32_t>(B * p.cps);

  // First-tile bootstrap: groups per thread so that NT * groups >= K (only for K <= tile).
  p.boot_groups = 0;
  if (p.K <= tile) {
    int64_t g = next_pow2((p.K + kChunkThreads - 1) / kChunkThreads);
    if (g <= E) p.boot_groups = static_cast<int32_t>(g);
  }

  const size_t lists = static_cast<size_t>(H) * p.nch;
  p.lists_bytes = round_up(2 * lists * static_cast<size_t>(p.K) * p.key_bytes, 256);
  p.total_bytes = p.lists_bytes;
  return FA3Q_OK;
}

template <typename InT>
int launch(const void* x, int64_t H, const CalibPlan& p, float* win_min, float* win_max,
           void* workspace, hipStream_t stream) {
  using KeyT = InT;
  int st = allow_dynamic_lds(reinterpret_cast<const void*>(calib_chunk_kernel<InT>), p.lds_chunk);
  if (st != FA3Q_OK) return st;
  st = allow_dynamic_lds(reinterpret_cast<const void*>(calib_merge_kernel<KeyT>), p.lds_merge);
  if (st != FA3Q_OK) return st;

  ChunkArgs ca;
  ca.x = x;
  ca.lists = workspace;
  ca.L = p.L;
  ca.CL = p.CL;
  ca.H = static_cast<int32_t>(H);
  ca.cps = p.cps;
  ca.nch = p.nch;
  ca.boot_groups = p.boot_groups;
  ca.K = static_cast<uint32_t>(p.K);
  ca.cap = p.cap_chunk;
  hipLaunchKernelGGL(calib_chunk_kernel<InT>, dim3(static_cast<unsigned>(H * p.nch)), dim3(kChunkThreads),
                     p.lds_chunk, stream, ca);
  MergeArgs ma;
  ma.lists = workspace;
  ma.win_min = win_min;
  ma.win_max = win_max;
  ma.H = static_cast<int32_t>(H);
  ma.nch = p.nch;
  ma.K = static_cast<uint32_t>(p.K);
  ma.cap = p.cap_merge;
  ma.P = p.P;
  hipLaunchKernelGGL(calib_merge_kernel<KeyT>, dim3(static_cast<unsigned>(H)), dim3(kMergeThreads),
                     p.lds_merge, stream, ma);
  return launch_status();
}

}  // namespace
}  // namespace fa3q

using namespace fa3q;

extern "C" int64_t fa3q_calibrate_max_windows(int dtype) {
  // Each kernel keeps 2*cap + K keys in LDS with cap = 2K + tile.  Largest K for which
  // both fit the 160 KiB a gfx950 workgroup may use.
  if (dtype != FA3Q_F32 && dtype != FA3Q_BF16) return 0;
  const int64_t kb = dtype == FA3Q_BF16 ? 2 : 4;
  const int64_t tile = std::max<int64_t>(dtype == FA3Q_BF16 ? chunk_tile<uint16_t>() : chunk_tile<uint32_t>(),
                                         kMergeTile);
  const int64_t room = (static_cast<int64_t>(kLdsLimit) - static_cast<int64_t>(kCtlBytes)) / kb;
  return (room - 2 * tile) / 5;
}

extern "C" size_t fa3q_calibrate_workspace_bytes(int dtype, int64_t B, int64_t H, int64_t S,
                                                 int64_t D, double ratio) {
  CalibPlan p;
  if (make_plan(dtype, B, H, S, D, ratio, p) != FA3Q_OK) return 0;
  return p.total_bytes;
}

extern "C" int fa3q_calibrate_perhead(const void* x, int dtype, int64_t B, int64_t H, int64_t S,
                                      int64_t D, double ratio, float* win_min, float* win_max,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  if (!x || !win_min || !win_max) return FA3Q_ERR_NULL;
  CalibPlan p;
  const int st = make_plan(dtype, B, H, S, D, ratio, p);
  if (st != FA3Q_OK) return st;
  if (!is_aligned(x, 16) || !is_aligned(win_min, 4) || !is_aligned(win_max, 4))
    return FA3Q_ERR_ALIGN;
  if (!workspace || workspace_bytes < p.total_bytes) return FA3Q_ERR_WORKSPACE;
  if (!is_aligned(workspace, 256)) return FA3Q_ERR_ALIGN;
  if (dtype == FA3Q_BF16)
    return launch<uint16_t>(x, H, p, win_min, win_max, workspace, as_stream(stream));
  return launch<uint32_t>(x, H, p, win_min, win_max, workspace, as_stream(stream));
}
