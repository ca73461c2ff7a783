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
constexpr int kVecPerThread = 2;       // 16-byte vectors per thread per tile (chunk kernel)
constexpr int kMergePerThread = 4;     // keys per thread per tile (merge kernel)
constexpr int kMergeTile = kMergeThreads * kMergePerThread;
constexpr int64_t kTargetChunkGroups = 2048;
constexpr int kMinTilesPerChunk = 16;

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

// Order-preserving key of a bf16 pattern (low 16 bits of w).
__device__ __forceinline__ uint32_t key_bf16(uint32_t b) {
  return b ^ ((b & 0x8000u) ? 0xffffu : 0x8000u);
}
__device__ __forceinline__ uint32_t key_f32(uint32_t b) {
  return b ^ ((b & 0x80000000u) ? 0xffffffffu : 0x80000000u);
}
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
  uint32_t thr_lo;
  uint32_t thr_hi;
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
  uint32_t* counts;   // [2][H][nch]
  void* lists;        // [2][H][nch][K] keys
  int64_t L;          // S*D, elements per (b,h) slab
  int64_t CL;         // elements per chunk (multiple of the vector width)
  int32_t H;
  int32_t cps;        // chunks per slab
  int32_t nch;        // chunks per head = B*cps
  uint32_t K;
  uint32_t cap;
};

// One 16-byte vector of input -> up to 8 keys (8 for bf16, 4 for float32).
template <typename InT>
struct VecKeys;
template <>
struct VecKeys<uint16_t> {
  static constexpr int kPerVec = 8;
  __device__ static void get(const uint4& v, uint32_t (&k)[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      k[2 * i] = key_bf16(w[i] & 0xffffu);
      k[2 * i + 1] = key_bf16(w[i] >> 16);
    }
  }
};
template <>
struct VecKeys<uint32_t> {
  static constexpr int kPerVec = 4;
  __device__ static void get(const uint4& v, uint32_t (&k)[8]) {
    k[0] = key_f32(v.x);
    k[1] = key_f32(v.y);
    k[2] = key_f32(v.z);
    k[3] = key_f32(v.w);
  }
};

template <typename InT>
__global__ __launch_bounds__(kChunkThreads) void calib_chunk_kernel(ChunkArgs a) {
  using KeyT = InT;  // 16-bit keys for bf16 input, 32-bit keys for float32 input
  constexpr int NT = kChunkThreads;
  constexpr int kPerVec = VecKeys<InT>::kPerVec;
  constexpr int kTile = NT * kVecPerThread * kPerVec;
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
  auto load_tile = [&](int64_t t0, uint4 (&dst)[kVecPerThread]) {
#pragma unroll
    for (int v = 0; v < kVecPerThread; ++v) {
      const int64_t e = t0 + static_cast<int64_t>(v * NT + tid) * kPerVec;
      if (e < end) dst[v] = *reinterpret_cast<const uint4*>(slab + e);
    }
  };
  if (begin < end) load_tile(begin, cur);
  for (int64_t t0 = begin; t0 < end; t0 += kTile) {
    if (t0 + kTile < end) load_tile(t0 + kTile, nxt);
    uint32_t keys[kVecPerThread][8];
    bool valid[kVecPerThread];
    uint32_t kmin = KeyInfo<KeyT>::kMax, kmax = 0;
#pragma unroll
    for (int v = 0; v < kVecPerThread; ++v) {
      valid[v] = t0 + static_cast<int64_t>(v * NT + tid) * kPerVec < end;
      VecKeys<InT>::get(cur[v], keys[v]);
      if (valid[v]) {
#pragma unroll
        for (int i = 0; i < kPerVec; ++i) {
          kmin = min(kmin, keys[v][i]);
          kmax = max(kmax, keys[v][i]);
        }
      }
    }
    if (__ballot(kmin < st.thr_lo) != 0) {
#pragma unroll
      for (int v = 0; v < kVecPerThread; ++v)
#pragma unroll
        for (int i = 0; i < kPerVec; ++i) st.append_lo(valid[v] && keys[v][i] < st.thr_lo, keys[v][i]);
    }
    if (__ballot(kmax > st.thr_hi) != 0) {
#pragma unroll
      for (int v = 0; v < kVecPerThread; ++v)
#pragma unroll
        for (int i = 0; i < kPerVec; ++i) st.append_hi(valid[v] && keys[v][i] > st.thr_hi, keys[v][i]);
    }
    st.end_tile();
#pragma unroll
    for (int v = 0; v < kVecPerThread; ++v) cur[v] = nxt[v];
  }
  st.finish();

  const int64_t list = static_cast<int64_t>(h) * a.nch + c;
  const int64_t heads_lists = static_cast<int64_t>(a.H) * a.nch;
  KeyT* out_lo = static_cast<KeyT*>(a.lists) + list * a.K;
  KeyT* out_hi = static_cast<KeyT*>(a.lists) + (heads_lists + list) * a.K;
  for (uint32_t i = tid; i < st.base_lo; i += NT) out_lo[i] = st.lo[i];
  for (uint32_t i = tid; i < st.base_hi; i += NT) out_hi[i] = st.hi[i];
  if (tid == 0) {
    a.counts[list] = st.base_lo;
    a.counts[heads_lists + list] = st.base_hi;
  }
}

struct MergeArgs {
  const uint32_t* counts;
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
  const int64_t heads_lists = static_cast<int64_t>(a.H) * a.nch;
  const KeyT* lists = static_cast<const KeyT*>(a.lists);

  // Stream the chunk tails of head h through the same two-sided filter.
  for (int c = 0; c < a.nch; ++c) {
    const int64_t list = static_cast<int64_t>(h) * a.nch + c;
    const uint32_t n_lo = a.counts[list];
    const uint32_t n_hi = a.counts[heads_lists + list];
    const KeyT* src_lo = lists + list * a.K;
    const KeyT* src_hi = lists + (heads_lists + list) * a.K;
    const uint32_t n = max(n_lo, n_hi);
    for (uint32_t t0 = 0; t0 < n; t0 += kMergeTile) {
      uint32_t klo[kMergePerThread], khi[kMergePerThread];
      bool vlo[kMergePerThread], vhi[kMergePerThread];
#pragma unroll
      for (int e = 0; e < kMergePerThread; ++e) {
        const uint32_t i = t0 + e * NT + tid;
        vlo[e] = i < n_lo;
        vhi[e] = i < n_hi;
        klo[e] = vlo[e] ? static_cast<uint32_t>(src_lo[i]) : 0u;
        khi[e] = vhi[e] ? static_cast<uint32_t>(src_hi[i]) : 0u;
      }
#pragma unroll
      for (int e = 0; e < kMergePerThread; ++e) st.append_lo(vlo[e] && klo[e] < st.thr_lo, klo[e]);
#pragma unroll
      for (int e = 0; e < kMergePerThread; ++e) st.append_hi(vhi[e] && khi[e] > st.thr_hi, khi[e]);
      st.end_tile();
    }
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
  int32_t cps = 0, nch = 0;
  uint32_t cap_chunk = 0, cap_merge = 0, P = 0;
  size_t lds_chunk = 0, lds_merge = 0;
  size_t key_bytes = 0;
  size_t counts_bytes = 0, lists_bytes = 0, total_bytes = 0;
};

int64_t next_pow2(int64_t v) {
  int64_t p = 1;
  while (p < v) p <<= 1;
  return p;
}

// Validates everything except pointers and computes the launch plan.
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

  const int64_t tile = static_cast<int64_t>(kChunkThreads) * kVecPerThread * vec;
  const int64_t pairs = B * H;
  const int64_t want = (kTargetChunkGroups + pairs - 1) / pairs;
  const int64_t most = std::max<int64_t>(1, p.L / (kMinTilesPerChunk * tile));
  p.cps = static_cast<int32_t>(std::max<int64_t>(1, std::min(want, most)));
  p.CL = (p.L + p.cps - 1) / p.cps;
  p.CL = (p.CL + vec - 1) / vec * vec;
  p.cps = static_cast<int32_t>((p.L + p.CL - 1) / p.CL);
  if (B * p.cps > (int64_t{1} << 30) || H * B * p.cps > (int64_t{1} << 31) - 1) return FA3Q_ERR_SHAPE;
  p.nch = static_cast<int32_t>(B * p.cps);

  p.key_bytes = dtype == FA3Q_BF16 ? 2 : 4;
  p.cap_chunk = static_cast<uint32_t>(2 * p.K + tile);
  p.cap_merge = static_cast<uint32_t>(2 * p.K + kMergeTile);
  p.P = static_cast<uint32_t>(next_pow2(p.K));
  p.lds_chunk = kCtlBytes + (2 * static_cast<size_t>(p.cap_chunk) + p.K) * p.key_bytes;
  p.lds_merge = kCtlBytes + (2 * static_cast<size_t>(p.cap_merge) + p.K) * p.key_bytes;
  if (p.lds_chunk > kLdsLimit || p.lds_merge > kLdsLimit) return FA3Q_ERR_UNSUPPORTED;

  const size_t lists = static_cast<size_t>(H) * p.nch;
  p.counts_bytes = round_up(2 * lists * sizeof(uint32_t), 256);
  p.lists_bytes = round_up(2 * lists * static_cast<size_t>(p.K) * p.key_bytes, 256);
  p.total_bytes = p.counts_bytes + p.lists_bytes;
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

  uint32_t* counts = static_cast<uint32_t*>(workspace);
  void* lists = static_cast<char*>(workspace) + p.counts_bytes;
  ChunkArgs ca;
  ca.x = x;
  ca.counts = counts;
  ca.lists = lists;
  ca.L = p.L;
  ca.CL = p.CL;
  ca.H = static_cast<int32_t>(H);
  ca.cps = p.cps;
  ca.nch = p.nch;
  ca.K = static_cast<uint32_t>(p.K);
  ca.cap = p.cap_chunk;
  hipLaunchKernelGGL(calib_chunk_kernel<InT>, dim3(static_cast<unsigned>(H * p.nch)), dim3(kChunkThreads),
                     p.lds_chunk, stream, ca);
  MergeArgs ma;
  ma.counts = counts;
  ma.lists = lists;
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
  // Both kernels keep 2*cap + K keys in LDS with cap = 2K + tile; the merge tile (4096
  // keys) is the larger one.  Largest K whose LDS fits the 160 KiB of a gfx950 workgroup.
  if (dtype != FA3Q_F32 && dtype != FA3Q_BF16) return 0;
  const int64_t kb = dtype == FA3Q_BF16 ? 2 : 4;
  const int64_t room = (static_cast<int64_t>(kLdsLimit) - static_cast<int64_t>(kCtlBytes)) / kb;
  return (room - 2 * static_cast<int64_t>(kMergeTile)) / 5;
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
