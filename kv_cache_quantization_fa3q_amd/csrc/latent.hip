// Decode attention over a shared-latent (absorbed MLA) cache on the matrix cores.
//
// MindIE LLM page "FA3 quantization", overview: in MLA attention only the non-RoPE part of
// K goes to 8 bits and the RoPE part stays floating point, to shrink the KV cache of the
// decode phase.  With the up-projections absorbed into the query, every query head of a
// sequence reads the same cache rows [c | k_rope]: a latent c of Dl features (INT8 codes
// with one scale s, the per-head method applied with one head) and Dr bf16 RoPE features.
// For query q = [q_abs | q_rope] of head h:
//   score_t = sm * (s * <q_abs, c_t> + <q_rope, r_t>),  out = s * sum_t softmax(score)_t c_t
// (the latent-space output; the value up-projection is outside this path).
//
// Sharing the rows across heads makes both products dense [heads x tokens] contractions,
// so they run on MFMA (v_mfma_f32_16x16x32_bf16, float32 accumulation):
//   S^T (16 tokens x 16 heads) = K (tokens x dims) . Q^T (dims x heads)
//   O^T (16 dims x 16 heads)  += V^T (dims x tokens) . P^T (tokens x heads)
// The transposed forms put one head in each lane's accumulator column (lane % 16), so the
// running max, sum and rescale of the online softmax are per lane, and the probabilities
// a lane holds after the softmax are exactly the B operand of the second product: over a
// 32-token tile, lane group g = lane / 16 holds tokens {4g + 0..3} and {16 + 4g + 0..3},
// which become k-slots 8g .. 8g+7; V^T is stored in LDS with its tokens in that order, so
// one 8-byte read gives the matching A operand.
//
// A workgroup is eight waves of one sequence over one run of tokens (a split): four pairs
// of waves, 16 heads per pair (64 heads).  The two waves of a pair split the work of their
// heads in halves: each computes the first product over half of the k-steps (half the
// latent dims and half the RoPE dims) and exchanges its partial scores with the other
// through LDS, so both hold the same scores and weights; each then accumulates half of the
// output dims.  Two waves run on every SIMD, so one computes while the other waits, and
// each wave holds half the query and half the output tiles in registers.  Per tile of 32
// tokens the workgroup widens the INT8 latent rows to bf16 (exact) once and stages them
// twice in LDS, row-major for the first product and transposed for the second (a 4x4 byte
// transpose in registers), plus the bf16 RoPE rows (the latent units and the RoPE chunks
// go to different threads); the next tile's global loads are issued before the current
// tile is computed.  The
// output is rescaled only when a head's running max grows by more than 2^8.  Splits leave
// (max reference, sum, s * unnormalised output) in the workspace; a combine kernel merges
// them.
//
// With 128 heads or more, latent_wide_kernel (below) takes 128 heads per workgroup, one wave
// of 32 heads per SIMD on the 32x32 MFMA, from one staged copy of each tile that the second
// product reads with the LDS transpose load; this kernel then only recomputes the splits
// that the wide kernel gave up.
//
// Probabilities enter the second product as two bf16 terms, p = hi + lo with hi = bf16(p)
// and lo = bf16(p - hi), through two MFMAs that share the V operand: the weight error is
// below 2^-17 relative instead of the 2^-9 of a single bf16 term, whose error bound
// 2^-9 * max|v| would exceed 1e-4 of the output when the weights are spread out.
#include <cmath>

#include "fa3q_internal.hpp"

namespace fa3q {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kLatThreads = 512;  // eight waves: four pairs of 16 heads
constexpr int kLatHeads = 64;     // heads per workgroup
constexpr int kTT = 32;           // tokens per tile
// A workgroup's two LDS buffers (157 KB at the MLA shape) leave room for one per CU, so
// 256 workgroups fill the chip in a single wave; more splits would only add a second,
// partial wave and more partial rows for the combine to read.
constexpr int64_t kLatTargetGroups = 256;
constexpr int64_t kLatMinSplit = 64;

struct LatentArgs {
  const uint16_t* q;      // (B,H,Dl+Dr) bf16
  const int8_t* cq;       // (B,T,Dl) latent codes
  const float* scale;     // [1]
  const uint16_t* kr;     // (B,T,Dr) bf16
  float* out;             // (B,H,Dl)
  float* ws_ml;           // [B*H*nsplit][2]
  float* ws_o;            // [B*H*nsplit][Dl]
  // wide kernel: [B][ceil(H/128)][nsplit][4] one word per wave, 1 when the wave gave up its
  // split; the split kernel, given them, recomputes only the 64-head groups of such waves
  uint32_t* flags;
  int64_t T;
  int32_t H;
  int32_t groups;         // ceil(H / 64)
  int32_t nsplit;
  int32_t split_len;      // multiple of kTT
  float sm_log2;          // sm_scale * log2(e)
};

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// Staged operands of one tile: 2 tokens x 16 latent dims and one 16-byte RoPE chunk.
struct LatentStage {
  u32x4v x[2];
  u32x4v r;
};

// Max over lanes i, i^16, i^32 and i^48 (the four lane groups that hold one head), in
// VALU lane swaps instead of LDS permutes.  permlane16_swap(x, x) returns (a, b) with row
// pairs (0,1) and (2,3) of 16 lanes holding x's even rows in a and odd rows in b, so
// max(a, b) is the max over i and i^16; permlane32_swap does the same for halves (i^32).
__device__ __forceinline__ float max_over_lane_groups(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Two bf16 (packed) from two float32 (exact here: small integers).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// Code `e` (0..3) of a dword of INT8 codes as float32 (one byte-select conversion).
__device__ __forceinline__ float code_f32(uint32_t w, int e) {
  return static_cast<float>(static_cast<int8_t>(w >> (8 * e)));
}

template <int DL, int DR>
__global__ __launch_bounds__(kLatThreads) void latent_split_kernel(LatentArgs a) {
  constexpr int KL = DL / 32;          // k-steps of the latent part of S
  constexpr int KR = DR / 32;          // k-steps of the RoPE part
  constexpr int MT = DL / 16;          // 16-dim tiles of the output
  // each wave of a pair: latent k-steps [half*KLH, (half+1)*KLH), RoPE k-steps
  // [half*KRH, ...) (an odd KR leaves the last one to the second wave), output tiles
  // [half*MTH, (half+1)*MTH)
  constexpr int KLH = KL / 2;
  constexpr int KRH = (KR + 1) / 2;    // RoPE k-step registers per wave
  constexpr int MTH = MT / 2;
  static_assert(KL % 2 == 0 && MT % 2 == 0, "the pair splits the latent k-steps and the output tiles in halves");
  constexpr int KROW = DL + 8;         // bf16 per row-major latent row in LDS
  constexpr int RROW = DR + 8;         // bf16 per RoPE row in LDS
  constexpr int VROW = kTT;            // bf16 per transposed latent row in LDS (unpadded: measured
                                       // 1.6% faster than kTT + 8; rows of Dl + 8 keep their pad)
  constexpr int DC = DL / 16;          // 16-byte chunks per latent row
  constexpr int UNITS = (kTT / 2) * DC;  // (2 tokens x 16 dims) staging units per tile
  constexpr int UPT = (UNITS + kLatThreads - 1) / kLatThreads;  // units per thread
  constexpr int RCH = kTT * DR / 8;    // 16-byte RoPE chunks per tile
  static_assert(RCH <= kLatThreads, "one RoPE chunk per thread");
  // the RoPE chunks go to the last RCH threads, past the latent units when both fit
  constexpr int RT0 = kLatThreads - RCH;
  constexpr float kLazy = 8.0f;        // log2 headroom before the output is rescaled
  // two buffers: the next tile is staged while this one is read
  __shared__ __align__(16) uint16_t klat_buf[2][kTT * KROW];
  __shared__ __align__(16) uint16_t vt_buf[2][DL * VROW];
  __shared__ __align__(16) uint16_t krope_buf[2][DR > 0 ? kTT * RROW : 8];
  // each wave's partial scores for its pair partner: [wave][value][lane], 16 KiB
  __shared__ __align__(16) float xch[kLatThreads / kWave][8][kWave];

  const int tid = static_cast<int>(threadIdx.x);
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int hl = lane & 15, lg = lane >> 4;

  const int split = static_cast<int>(blockIdx.x % a.nsplit);
  const int rest = static_cast<int>(blockIdx.x / a.nsplit);
  const int grp = rest % a.groups;
  const int b = rest / a.groups;
  if (a.flags != nullptr) {
    // recompute only what the wide kernel gave up: 64-head group grp is waves 2(grp%2) and
    // 2(grp%2)+1 of the wide workgroup (b, grp/2, split) (uniform over the workgroup)
    const uint32_t* f = a.flags + ((static_cast<int64_t>(b) * ((a.groups + 1) / 2) + grp / 2) * a.nsplit + split) * 4 +
                        2 * (grp % 2);
    if ((f[0] | f[1]) == 0u) return;
  }
  const int pair = wave & 3, half = wave >> 2;  // the partner is wave ^ 4
  const int head = grp * kLatHeads + pair * 16 + hl;
  const bool hv = head < a.H;
  const int64_t t_begin = static_cast<int64_t>(split) * a.split_len;
  const int64_t t_end = min(a.T, t_begin + a.split_len);

  const int8_t* cbase = a.cq + static_cast<int64_t>(b) * a.T * DL;
  const uint16_t* rbase = a.kr + static_cast<int64_t>(b) * a.T * DR;

  // global -> registers for tile t0 (rows past the end re-read the last row; masked later)
  auto fetch = [&](int64_t t0, LatentStage (&st)[UPT]) {
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
      const int u = tid + k * kLatThreads;
      if (UNITS % kLatThreads == 0 || u < UNITS) {  // folds when every thread has a unit
        const int tg = u % (kTT / 2), dc = u / (kTT / 2);  // token pair fastest
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const int64_t tok = min(t0 + 2 * tg + r, t_end - 1);
          st[k].x[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(cbase + tok * DL + 16 * dc));
        }
      }
    }
    if constexpr (DR > 0) {
      if (tid >= RT0) {
        const int rt = tid - RT0;
        const int r = rt / (DR / 8), k8 = rt - r * (DR / 8);
        const int64_t tok = min(t0 + r, t_end - 1);
        st[0].r = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(rbase + tok * DR + 8 * k8));
      }
    }
  };
  // registers -> LDS buffer `buf`: latent rows widened to bf16, row-major and transposed; RoPE rows
  auto stage = [&](const LatentStage (&st)[UPT], int buf) {
    uint16_t* klat = klat_buf[buf];
    uint16_t* vt = vt_buf[buf];
    uint16_t* krope = krope_buf[buf];
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
      const int u = tid + k * kLatThreads;
      if (UNITS % kLatThreads == 0 || u < UNITS) {  // folds when every thread has a unit
        const int tg = u % (kTT / 2), dc = u / (kTT / 2);  // token pair fastest
        // each code is converted once; the row-major copy pairs neighbouring dims of a
        // token, the transposed copy the two tokens of a dim
        float f[2][16];
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
          for (int j = 0; j < 16; ++j) f[r][j] = code_f32(st[k].x[r][j / 4], j % 4);
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          uint32_t h[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) h[i] = pack_bf16(f[r][2 * i], f[r][2 * i + 1]);
          uint16_t* row = klat + (2 * tg + r) * KROW + 16 * dc;
          *reinterpret_cast<uint4*>(row) = make_uint4(h[0], h[1], h[2], h[3]);
          *reinterpret_cast<uint4*>(row + 8) = make_uint4(h[4], h[5], h[6], h[7]);
        }
        // token t = 2tg + r sits at k-slot position 8*((t >> 2) & 3) + 4*(t >> 4) + (t & 3) of
        // its transposed row; the row's 16-byte chunks are XOR-swizzled by (row >> 4) & 3
        // (= dc & 3), so the four rows a wave writes at once fall in different banks
        const int pos = 8 * ((tg >> 1) & 3) + 4 * (tg >> 3) + 2 * (tg & 1);
        const int spos = (((pos >> 3) ^ (dc & 3)) << 3) | (pos & 7);
#pragma unroll
        for (int j = 0; j < 16; ++j)
          *reinterpret_cast<uint32_t*>(vt + (16 * dc + j) * VROW + spos) = pack_bf16(f[0][j], f[1][j]);
      }
    }
    if constexpr (DR > 0) {
      if (tid >= RT0) {
        const int rt = tid - RT0;
        const int r = rt / (DR / 8), k8 = rt - r * (DR / 8);
        *reinterpret_cast<u32x4v*>(krope + r * RROW + 8 * k8) = st[0].r;
      }
    }
  };

  // the wave's half of the query as B operands (Q^T: dims x heads): lane holds dims
  // 32kk + 8lg .. +7 of its k-steps; a RoPE k-step past KR (odd KR, first wave) stays zero
  const int kl0 = half * KLH, kr0 = half * (KR / 2);
  const int nkr = half ? KR - KR / 2 : KR / 2;  // RoPE k-steps of this wave
  bf16x8 ql[KLH];
  bf16x8 qr[KRH > 0 ? KRH : 1];
  {
    const uint16_t* qrow = a.q + (static_cast<int64_t>(b) * a.H + (hv ? head : 0)) * (DL + DR);
#pragma unroll
    for (int kk = 0; kk < KLH; ++kk) {
      const uint4 u = hv ? *reinterpret_cast<const uint4*>(qrow + 32 * (kl0 + kk) + 8 * lg) : make_uint4(0, 0, 0, 0);
      ql[kk] = as_bf16x8(u);
    }
#pragma unroll
    for (int kk = 0; kk < KRH; ++kk) {
      const uint4 u = hv && kk < nkr ? *reinterpret_cast<const uint4*>(qrow + DL + 32 * (kr0 + kk) + 8 * lg)
                                     : make_uint4(0, 0, 0, 0);
      qr[kk] = as_bf16x8(u);
    }
  }
  const float s = a.scale[0];

  f32x4 o[MTH];  // output dims 16 (half*MTH + mt) + 4lg .. +3
#pragma unroll
  for (int mt = 0; mt < MTH; ++mt) o[mt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  // mu: the reference the weights are taken against (p = 2^(score - mu)); it lags the
  // running max by at most kLazy, so the output is rescaled only when the max has grown
  // by more than that (weights stay <= 2^kLazy, far inside float32 and bf16 range)
  float mu = -INFINITY, l = 0.0f;

  // ---- softmax weights of one tile against mu, then O^T += V^T . P^T
  // (k-slot 8lg + i holds token 4lg + i for i < 4, 16 + 4lg + i - 4 otherwise)
  auto accumulate = [&](float (&p)[8], const uint16_t* vt) {
    float rsum = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // the hardware exp2 alone: exponents are <= kLazy, and only weights below 2^-126
      // (against a head total >= 1) lose their denormal tail
      p[i] = __builtin_amdgcn_exp2f(p[i] - mu);
      rsum += p[i];
    }
    l += rsum;  // this lane's part: the four lanes of a head are summed once, at the end
    bf16x8 phi, plo;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      phi[i] = static_cast<__bf16>(p[i]);
      plo[i] = static_cast<__bf16>(p[i] - static_cast<float>(phi[i]));  // the difference is exact in float32
    }
#pragma unroll
    for (int mt = 0; mt < MTH; ++mt) {
      // (the transposed rows' 16-byte chunks are swizzled by (row >> 4) & 3, uniform here)
      const uint4 w = *reinterpret_cast<const uint4*>(vt + (16 * (half * MTH + mt) + hl) * VROW +
                                                      8 * (lg ^ ((half * MTH + mt) & 3)));
      o[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(w), phi, o[mt], 0, 0, 0);
      o[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(w), plo, o[mt], 0, 0, 0);
    }
  };

  LatentStage st[UPT];
  fetch(t_begin, st);
  stage(st, 0);
  if (t_begin + kTT < t_end) fetch(t_begin + kTT, st);
  __syncthreads();
  int64_t t0 = t_begin;
  int buf = 0;
  float p[8];
  float rmax = -INFINITY;
  // The tile loop leaves early when a head's max outgrows mu + kLazy (the first tile, then
  // rarely): the output is rescaled outside it, so the hot loop holds no operation on the
  // accumulators other than the MFMAs.  Each pass computes tile t0 from buffer `buf` while
  // tile t0 + 32 (already in registers) is staged into the other buffer and tile t0 + 64 is
  // fetched; one barrier per tile.
  for (;;) {
    for (; t0 < t_end; t0 += kTT, buf ^= 1) {
      const uint16_t* klat = klat_buf[buf];
      const uint16_t* krope = krope_buf[buf];
      // ---- S^T = K . Q^T for tokens 16tt .. 16tt+15 (latent and RoPE parts apart)
      f32x4 sl[2], sr[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        sl[tt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        sr[tt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kk = 0; kk < KLH; ++kk) {
          const uint4 w = *reinterpret_cast<const uint4*>(klat + (16 * tt + hl) * KROW + 32 * (kl0 + kk) + 8 * lg);
          sl[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(w), ql[kk], sl[tt], 0, 0, 0);
        }
#pragma unroll
        for (int kk = 0; kk < KRH; ++kk) {
          // (an odd KR: the first wave's last slot reads a valid row and multiplies zeros)
          const int kr = min(kr0 + kk, KR - 1);
          const uint4 w = *reinterpret_cast<const uint4*>(krope + (16 * tt + hl) * RROW + 32 * kr + 8 * lg);
          sr[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(w), qr[kk], sr[tt], 0, 0, 0);
        }
      }
      {
        // keep kSDepth operand reads in flight ahead of the score MFMAs (left alone, the
        // scheduler issues each read one MFMA before its use)
        constexpr int NS = 2 * (KLH + KRH);
        constexpr int kSDepth = NS < 6 ? NS : 6;
        __builtin_amdgcn_sched_group_barrier(0x100, kSDepth, 0);  // DS reads
#pragma unroll
        for (int i = 0; i < NS - kSDepth; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one DS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kSDepth, 0);
      }
      // the other buffer was last read before the previous barrier.  Staged and fetched
      // unconditionally, so that the score MFMAs and the staging share one basic block and
      // the scheduler interleaves them: past the end the fetch re-reads the last row (in
      // bounds) and the staged buffer is never read.
      stage(st, buf ^ 1);
      fetch(t0 + 2 * kTT, st);
      // ---- the pair's partial scores: each wave's s <q_abs, c> + <q_rope, r> over its
      // k-steps, exchanged through LDS; both waves add the two in the same order
      float x[8];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          x[4 * tt + j] = fmaf(s, sl[tt][j], sr[tt][j]);
          xch[wave][4 * tt + j][lane] = x[4 * tt + j];
        }
      __syncthreads();
      // ---- scores (log2 domain) of the lane's head over its 8 tokens (16tt + 4lg + j)
      rmax = -INFINITY;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t tok = t0 + 16 * tt + 4 * lg + j;
          const float other = xch[wave ^ 4][4 * tt + j][lane];
          const float sc = (half ? other + x[4 * tt + j] : x[4 * tt + j] + other) * a.sm_log2;
          p[4 * tt + j] = tok < t_end ? sc : -INFINITY;
          rmax = fmaxf(rmax, p[4 * tt + j]);
        }
      rmax = max_over_lane_groups(rmax);  // finite: every tile holds a valid token
      if (__builtin_amdgcn_ballot_w64(rmax > mu + kLazy) != 0) break;
      accumulate(p, vt_buf[buf]);
      __syncthreads();
    }
    if (t0 >= t_end) break;
    // rescale to the new reference, then finish the tile the loop left; a lane moves its
    // reference only when its own max outgrew it (alpha is then exactly 1 elsewhere), so a
    // head's arithmetic does not depend on the other heads of its wave
    const float mu_new = rmax > mu + kLazy ? rmax : mu;
    const float alpha = exp2f(mu - mu_new);
    l *= alpha;
#pragma unroll
    for (int mt = 0; mt < MTH; ++mt) o[mt] *= alpha;
    mu = mu_new;
    accumulate(p, vt_buf[buf]);
    __syncthreads();
    t0 += kTT;
    buf ^= 1;
  }

  // a head's reference mu is the same in its four lanes, so their partial sums share scale
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  // ---- lane holds O^T[dims 16mt + 4lg + j][head]
  if (!hv) return;
  const int64_t row = static_cast<int64_t>(b) * a.H + head;
  const float f = a.nsplit == 1 ? s / l : s;
  float* dst = a.nsplit == 1 ? a.out + row * DL : a.ws_o + (row * a.nsplit + split) * DL;
#pragma unroll
  for (int mt = 0; mt < MTH; ++mt)
    *reinterpret_cast<float4*>(dst + 16 * (half * MTH + mt) + 4 * lg) =
        make_float4(o[mt][0] * f, o[mt][1] * f, o[mt][2] * f, o[mt][3] * f);
  if (a.nsplit > 1 && lg == 0 && half == 0) {
    const int64_t slot = row * a.nsplit + split;
    a.ws_ml[2 * slot] = mu;
    a.ws_ml[2 * slot + 1] = l;
  }
}

// ---- 128 heads per workgroup: one wave of 32 heads per SIMD on v_mfma_f32_32x32x16_bf16.
//   S^T (32 tokens x 32 heads) = K (tokens x 16 dims) . Q^T (16 dims x heads), per k-step
//   O^T (32 dims x 32 heads)  += V^T (dims x 16 tokens) . P^T (16 tokens x heads)
// A lane holds head lane % 32; its half hh = lane / 32 holds the scores of tokens
// 8i + 4hh + j (i, j < 4) of a tile, which are k-slots 8hh .. 8hh+7 of the two PV k-steps
// (i < 2, then i >= 2).  Each staged operand read feeds a 32-head MFMA, so a tile is read from
// LDS once per 32 heads, and no scores are exchanged between waves.  The RoPE part of the
// query sits in LDS (the latent part and the 512 output dims fill the registers).
//
// One staged copy: the codes are widened to bf16 once, into token rows.  The score product
// reads them as they are; the PV product reads V^T from the same rows with the LDS transpose
// read (ds_read_b64_tr_b16): within each group of 16 lanes, lane i receives, as its v-th
// value, element i % 4 of the 8 bytes addressed by lane 4v + i / 4.  So lanes 4v .. 4v+3
// address 16 consecutive dims of token row v, and lane i comes back with dim i of the four
// tokens: two such reads give a lane its 8 k-values.  The 16-byte chunks of a row are XORed
// with ((t & 3) << 2) | ((t >> 2) & 3) of its token t, which keeps both kinds of read free of
// bank conflicts (16 consecutive rows at one chunk; 4 consecutive rows of 64 bytes each).
//
// Three buffers: while tile j's scores are computed from one, tile j+1 is staged into the
// next, and the PV product of tile j-1 -- whose weights the previous pass left in registers --
// reads the third, alongside tile j's softmax.  So the widening overlaps the score MFMAs and
// the softmax overlaps the PV MFMAs.  One barrier per tile.
//
// No rescale in the tile loop: a head's reference mu is the max of its split's first tile,
// and weights 2^(score - mu) stay within float32 and bf16 range while no later score exceeds
// mu + 64.  Scaling the 256 output accumulators on the rare tile that breaks this would need
// registers the loop does not have, so a wave whose head meets such a tile marks its split
// in `flags` and runs on (its output is then not used): the split kernel, launched after this
// one with the flags, recomputes those splits.
constexpr int kWideThreads = 256;  // four waves, one per SIMD
constexpr int kWideHeads = 128;    // 32 heads per wave

typedef short i16x4 __attribute__((ext_vector_type(4)));

// 8 bytes at LDS byte address `p`, transposed across each group of 16 lanes (see above)
__device__ __forceinline__ uint2 lds_read_tr16(const void* p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(const_cast<void*>(p)));
  return __builtin_bit_cast(uint2, v);
}

// chunk swizzle of staged token row t
__device__ __forceinline__ int wide_swz(int t) { return ((t & 3) << 2) | ((t >> 2) & 3); }

template <int DL, int DR>
__global__ __launch_bounds__(kWideThreads) void latent_wide_kernel(LatentArgs a) {
  constexpr int KS = DL / 16;          // latent k-steps of the score product
  constexpr int RS = DR / 16;          // RoPE k-steps
  constexpr int OT = DL / 32;          // 32-dim output tiles
  constexpr int ROWB = 2 * DL;         // bytes per staged latent row (chunks swizzled, no padding)
  constexpr int RROW = DR + 8;         // bf16 per RoPE row in LDS
  constexpr int DC = DL / 16;          // 16-code chunks per latent row
  constexpr int UNITS = (kTT / 4) * DC;  // staging units of 4 tokens x 16 dims
  static_assert(UNITS <= kWideThreads, "at most one staging unit per thread");
  static_assert(DL >= 128, "the chunk swizzle spans 16 chunks");
  constexpr int RPR = DR > 0 ? DR / 8 : 1;  // 16-byte RoPE chunks per row
  constexpr int RCH = kTT * DR / 8;
  static_assert(RCH <= kWideThreads, "at most one RoPE chunk per thread");
  constexpr float kLazy = 64.0f;       // log2 headroom of the weights over the reference
  constexpr int QROW = DR + 8;         // bf16 per RoPE query row in LDS (padded: 128-byte rows conflict)
  // three buffers of each staged operand, as distinct arrays (accesses to different buffers
  // are then known to be disjoint)
  __shared__ __align__(16) uint16_t klb[3][kTT * DL];
  __shared__ __align__(16) uint16_t krb[3][DR > 0 ? kTT * RROW : 8];
  __shared__ __align__(16) uint16_t qrope[DR > 0 ? kWideHeads * QROW : 8];  // [head][QROW]
  auto klat = [&](int bc) __attribute__((always_inline)) -> uint16_t* { return klb[bc]; };
  auto krope = [&](int bc) __attribute__((always_inline)) -> uint16_t* { return krb[bc]; };

  const int tid = static_cast<int>(threadIdx.x);
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int hc = lane & 31, hh = lane >> 5;

  const int split = static_cast<int>(blockIdx.x % a.nsplit);
  const int rest = static_cast<int>(blockIdx.x / a.nsplit);
  const int grp = rest % a.groups;
  const int b = rest / a.groups;
  const int head = grp * kWideHeads + wave * 32 + hc;
  const bool hv = head < a.H;
  const int64_t t_begin = static_cast<int64_t>(split) * a.split_len;
  const int64_t t_end = min(a.T, t_begin + a.split_len);

  const int8_t* cbase = a.cq + static_cast<int64_t>(b) * a.T * DL;
  const uint16_t* rbase = a.kr + static_cast<int64_t>(b) * a.T * DR;

  // this thread's staging unit: tokens 4tg .. 4tg+3, latent dims 16dc .. 16dc+15
  const int tg = tid % 8, dc = tid / 8;
  const bool has_unit = UNITS == kWideThreads || tid < UNITS;
  const int rr = tid / RPR, rk = tid % RPR;
  const bool has_rope = DR > 0 && (RCH == kWideThreads || tid < RCH);

  u32x4v xs[4];
  u32x4v xr;
  // global -> registers for tile t0 (rows past the end re-read the last row; masked later)
  auto fetch = [&](int64_t t0) __attribute__((always_inline)) {
    if (has_unit) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t tok = min(t0 + 4 * tg + r, t_end - 1);
        xs[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(cbase + tok * DL + 16 * dc));
      }
    }
    if (has_rope) {
      const int64_t tok = min(t0 + rr, t_end - 1);
      xr = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(rbase + tok * DR + 8 * rk));
    }
  };
  // registers -> buffer B: the codes widened to bf16 (exact) in token rows, chunk-swizzled
  auto stage = [&](int bc) __attribute__((always_inline)) {
    if (has_unit) {
      char* kb = reinterpret_cast<char*>(klat(bc));
      float f[4][16];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < 16; ++j) f[r][j] = code_f32(xs[r][j / 4], j % 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        uint32_t h[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) h[i] = pack_bf16(f[r][2 * i], f[r][2 * i + 1]);
        const int t = 4 * tg + r;
        const int sw = wide_swz(t);
        char* row = kb + t * ROWB;
        *reinterpret_cast<uint4*>(row + 16 * ((2 * dc) ^ sw)) = make_uint4(h[0], h[1], h[2], h[3]);
        *reinterpret_cast<uint4*>(row + 16 * ((2 * dc + 1) ^ sw)) = make_uint4(h[4], h[5], h[6], h[7]);
      }
    }
    if constexpr (DR > 0) {
      if (has_rope) *reinterpret_cast<u32x4v*>(krope(bc) + rr * RROW + 8 * rk) = xr;
    }
  };

  // the latent part of the query as B operands (Q^T: dims x heads): lane holds dims
  // 16kk + 8hh .. +7 of its head; heads past H read as zero
  bf16x8 ql[KS];
  {
    const uint16_t* qrow = a.q + (static_cast<int64_t>(b) * a.H + (hv ? head : 0)) * (DL + DR);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const uint4 u = hv ? *reinterpret_cast<const uint4*>(qrow + 16 * kk + 8 * hh) : make_uint4(0, 0, 0, 0);
      ql[kk] = as_bf16x8(u);
    }
  }
  if constexpr (DR > 0) {
    for (int c = tid; c < kWideHeads * DR / 8; c += kWideThreads) {
      const int hq = c / (DR / 8), k8 = c % (DR / 8);
      const int hg = grp * kWideHeads + hq;
      const uint4 u = hg < a.H ? *reinterpret_cast<const uint4*>(a.q + (static_cast<int64_t>(b) * a.H + hg) * (DL + DR) +
                                                                 DL + 8 * k8)
                               : make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(qrope + hq * QROW + 8 * k8) = u;
    }
  }
  const float s = a.scale[0];

  // score operand: row hc, chunk (2kk + hh) ^ swz(hc) = 2kk ^ qx
  const int qx = wide_swz(hc) ^ hh;
  const int qrow_b = hc * ROWB;
  // PV operand, as the supplier lane of the transpose read: group pg, token row pv of the
  // group's four, 4-dim piece pq; read s (0, 1) covers tokens 16ks + 8s + 4(pg/2) + pv and the
  // dims 32dt + 16(pg%2) + 4pq .. +3, whose chunk is 4dt + 2(pg%2) + pq/2 and whose swizzle is
  // (pv << 2) | ((2s + pg/2) & 3).  Split into a lane part for each (s, dt % 4) and
  // compile-time offsets.
  const int pg = lane >> 4, pv = (lane >> 2) & 3, pq = lane & 3;
  int pbase[2][4];
#pragma unroll
  for (int sr = 0; sr < 2; ++sr)
#pragma unroll
    for (int d3 = 0; d3 < 4; ++d3)
      pbase[sr][d3] = (4 * (pg >> 1) + pv) * ROWB + 8 * (pq & 1) +
                      16 * ((2 * (pg & 1) + (pq >> 1)) ^ ((2 * sr + (pg >> 1)) & 3)) + 64 * (d3 ^ pv);

  f32x16 o[OT];  // output dims 32dt + 8i + 4hh + j at o[dt][4i + j]
#pragma unroll
  for (int dt = 0; dt < OT; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[dt][v] = 0.0f;
  float mu = -INFINITY, l = 0.0f;
  bool gave_up = false;

  // s <q_abs, c> + <q_rope, r> of the lane's head over its 16 tokens, from buffer B
  auto scores = [&](int bc) __attribute__((always_inline)) {
    const char* kb = reinterpret_cast<const char*>(klat(bc)) + qrow_b;
    f32x16 sc;
#pragma unroll
    for (int v = 0; v < 16; ++v) sc[v] = 0.0f;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const uint4 w = *reinterpret_cast<const uint4*>(kb + 256 * (kk >> 3) + 16 * ((2 * (kk & 7)) ^ qx));
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(w), ql[kk], sc, 0, 0, 0);
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) sc[v] *= s;
    if constexpr (DR > 0) {
      const uint16_t* kr = krope(bc);
#pragma unroll
      for (int kk = 0; kk < RS; ++kk) {
        const uint4 w = *reinterpret_cast<const uint4*>(kr + hc * RROW + 16 * kk + 8 * hh);
        const uint4 qv = *reinterpret_cast<const uint4*>(qrope + (wave * 32 + hc) * QROW + 16 * kk + 8 * hh);
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(w), as_bf16x8(qv), sc, 0, 0, 0);
      }
    }
    return sc;
  };
  // weights of tile t0 against mu as two bf16 terms (the first tile of a split sets mu; on a
  // later tile a wave whose head outgrows mu by more than kLazy gives its split up)
  auto weights = [&](const f32x16& sc, int64_t t0, auto firstc, bf16x8 (&phi)[2], bf16x8 (&plo)[2]) __attribute__((always_inline)) {
    float p[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) p[v] = sc[v] * a.sm_log2;
    if (t_end - t0 < kTT) {  // a split's last tile may be partial (uniform branch)
      const int nv = static_cast<int>(t_end - t0);
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (8 * (v / 4) + 4 * hh + (v % 4) >= nv) p[v] = -INFINITY;
    }
    float rmax = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; ++v) rmax = fmaxf(rmax, p[v]);
    {
      const auto m = __builtin_amdgcn_permlane32_swap(__float_as_uint(rmax), __float_as_uint(rmax), false, false);
      rmax = fmaxf(__uint_as_float(m[0]), __uint_as_float(m[1]));  // finite: a tile holds a valid token
    }
    if constexpr (decltype(firstc)::value)
      mu = rmax;
    else
      gave_up = gave_up || __builtin_amdgcn_ballot_w64(rmax > mu + kLazy) != 0;
    float rsum = 0.0f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      p[v] = __builtin_amdgcn_exp2f(p[v] - mu);
      rsum += p[v];
    }
    l += rsum;  // this lane's part; the two lanes of a head are summed once, at the end
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        phi[ks][e] = static_cast<__bf16>(p[8 * ks + e]);
        plo[ks][e] = static_cast<__bf16>(p[8 * ks + e] - static_cast<float>(phi[ks][e]));  // exact in float32
      }
  };
  // O^T += V^T . P^T for the tile in buffer B, four output tiles at a time (one tile's MFMAs
  // back to back would wait on each other's results)
  auto pv_product = [&](int bc, const bf16x8 (&phi)[2], const bf16x8 (&plo)[2]) __attribute__((always_inline)) {
    const char* kb = reinterpret_cast<const char*>(klat(bc));
    constexpr int kG = OT < 4 ? OT : 4;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int d0 = 0; d0 < OT; d0 += kG) {
        bf16x8 w[kG];
#pragma unroll
        for (int i = 0; i < kG; ++i) {
          const int dt = d0 + i;
          const uint2 lo = lds_read_tr16(kb + pbase[0][dt & 3] + 16 * ks * ROWB + 256 * (dt >> 2));
          const uint2 hi = lds_read_tr16(kb + pbase[1][dt & 3] + (16 * ks + 8) * ROWB + 256 * (dt >> 2));
          w[i] = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
        }
#pragma unroll
        for (int i = 0; i < kG; ++i)
          o[d0 + i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w[i], phi[ks], o[d0 + i], 0, 0, 0);
#pragma unroll
        for (int i = 0; i < kG; ++i)
          o[d0 + i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w[i], plo[ks], o[d0 + i], 0, 0, 0);
      }
  };

  bf16x8 phi[2], plo[2];  // weights of the previous tile, for its PV product
  // one pass: scores of tile t0 from buffer Bq while tile t0+32 is staged into Bs and tile
  // t0+64 fetched; then the weights of tile t0 and the PV product of the previous tile (buffer
  // Bp); staged and fetched unconditionally (past the end the fetch re-reads the last row and
  // the staged buffer is never read)
  auto pass = [&](int64_t t0, int bq, int bs, int bp, auto firstc) __attribute__((always_inline)) {
    const f32x16 sc = scores(bq);
    stage(bs);
    fetch(t0 + 2 * kTT);
    bf16x8 nhi[2], nlo[2];
    weights(sc, t0, firstc, nhi, nlo);
    if constexpr (!decltype(firstc)::value) pv_product(bp, phi, plo);
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      phi[ks] = nhi[ks];
      plo[ks] = nlo[ks];
    }
  };

  fetch(t_begin);
  stage(0);
  if (t_begin + kTT < t_end) fetch(t_begin + kTT);
  __syncthreads();
  pass(t_begin, 0, 1, 2, std::true_type{});  // a split is never empty
  int bq = 1;  // buffer of the next tile
  for (int64_t t0 = t_begin + kTT; t0 < t_end; t0 += kTT) {
    const int bs = bq == 2 ? 0 : bq + 1, bp = bq == 0 ? 2 : bq - 1;
    pass(t0, bq, bs, bp, std::false_type{});
    bq = bs;
  }
  pv_product(bq == 0 ? 2 : bq - 1, phi, plo);  // the last tile's

  l += __shfl_xor(l, 32);
  if (lane == 0)
    a.flags[((static_cast<int64_t>(b) * a.groups + grp) * a.nsplit + split) * 4 + wave] = gave_up ? 1u : 0u;
  if (!hv || gave_up) return;
  const int64_t row = static_cast<int64_t>(b) * a.H + head;
  const float f = a.nsplit == 1 ? s / l : s;
  float* dst = a.nsplit == 1 ? a.out + row * DL : a.ws_o + (row * a.nsplit + split) * DL;
#pragma unroll
  for (int dt = 0; dt < OT; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<float4*>(dst + 32 * dt + 8 * i + 4 * hh) =
          make_float4(o[dt][4 * i] * f, o[dt][4 * i + 1] * f, o[dt][4 * i + 2] * f, o[dt][4 * i + 3] * f);
  if (a.nsplit > 1 && hh == 0) {
    const int64_t slot = row * a.nsplit + split;
    a.ws_ml[2 * slot] = mu;
    a.ws_ml[2 * slot + 1] = l;
  }
}

// out = sum_s w_s o_s / sum_s w_s l_s with w_s = 2^(m_s - max m), per (b, h).  A workgroup
// of 256 threads takes 256 / (dl/4) rows, four dims per thread, with the splits' partials
// loaded four at a time.
constexpr int kCombineThreads = 256;

__global__ __launch_bounds__(kCombineThreads) void latent_combine_kernel(LatentArgs a, int dl, int64_t rows) {
  const int per_row = dl / 4;  // threads per row (dl is 128, 256 or 512)
  const int64_t row = static_cast<int64_t>(blockIdx.x) * (kCombineThreads / per_row) + threadIdx.x / per_row;
  if (row >= rows) return;
  const int d = 4 * (static_cast<int>(threadIdx.x) % per_row);
  const int ns = a.nsplit;
  const float* ml = a.ws_ml + 2 * row * ns;
  float mmax = -INFINITY;
  for (int s = 0; s < ns; ++s) mmax = fmaxf(mmax, ml[2 * s]);
  float den = 0.0f;
  float4 num = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  const float* src = a.ws_o + row * ns * dl + d;
  int s = 0;
  for (; s + 4 <= ns; s += 4) {
    float4 o[4];
    float w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) o[u] = *reinterpret_cast<const float4*>(src + static_cast<int64_t>(s + u) * dl);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      w[u] = exp2f(ml[2 * (s + u)] - mmax);
      den += w[u] * ml[2 * (s + u) + 1];
      num.x += w[u] * o[u].x;
      num.y += w[u] * o[u].y;
      num.z += w[u] * o[u].z;
      num.w += w[u] * o[u].w;
    }
  }
  for (; s < ns; ++s) {
    const float4 o = *reinterpret_cast<const float4*>(src + static_cast<int64_t>(s) * dl);
    const float w = exp2f(ml[2 * s] - mmax);
    den += w * ml[2 * s + 1];
    num.x += w * o.x;
    num.y += w * o.y;
    num.z += w * o.z;
    num.w += w * o.w;
  }
  *reinterpret_cast<float4*>(a.out + row * dl + d) = make_float4(num.x / den, num.y / den, num.z / den, num.w / den);
}

struct LatentPlan {
  bool wide;  // 128 heads per workgroup (latent_wide_kernel), else 64 (latent_split_kernel)
  int32_t groups, nsplit, split_len;
};

LatentPlan plan_latent(int64_t B, int64_t H, int64_t T) {
  LatentPlan p;
  p.wide = H >= kWideHeads;
  const int64_t per = p.wide ? kWideHeads : kLatHeads;
  p.groups = static_cast<int32_t>((H + per - 1) / per);
  const int64_t base = B * p.groups;
  int64_t ns = (kLatTargetGroups + base - 1) / base;
  ns = std::max<int64_t>(1, std::min(ns, (T + kLatMinSplit - 1) / kLatMinSplit));
  int64_t len = (T + ns - 1) / ns;
  len = (len + kTT - 1) / kTT * kTT;
  ns = (T + len - 1) / len;  // no empty split
  p.nsplit = static_cast<int32_t>(ns);
  p.split_len = static_cast<int32_t>(len);
  return p;
}

bool latent_dims_ok(int64_t Dl, int64_t Dr) {
  return (Dl == 128 || Dl == 256 || Dl == 512) && (Dr == 0 || Dr == 32 || Dr == 64);
}

bool latent_shape_ok(int64_t B, int64_t H, int64_t T, int64_t Dl) {
  if (B <= 0 || H <= 0 || T <= 0) return false;
  if (H > 65536 || B > (int64_t{1} << 24) || T > (int64_t{1} << 31)) return false;
  if (B * ((H + kLatHeads - 1) / kLatHeads) > (int64_t{1} << 24)) return false;
  return B <= (int64_t{1} << 62) / (T * (Dl + 128));
}

using LatentFn = void (*)(LatentArgs);

template <int DL, int DR>
LatentFn pick_kernel(bool wide) {
  return wide ? latent_wide_kernel<DL, DR> : latent_split_kernel<DL, DR>;
}

template <int DL>
LatentFn pick_dr(int64_t dr, bool wide) {
  switch (dr) {
    case 0: return pick_kernel<DL, 0>(wide);
    case 32: return pick_kernel<DL, 32>(wide);
    default: return pick_kernel<DL, 64>(wide);
  }
}

LatentFn pick_latent(int64_t dl, int64_t dr, bool wide) {
  switch (dl) {
    case 128: return pick_dr<128>(dr, wide);
    case 256: return pick_dr<256>(dr, wide);
    default: return pick_dr<512>(dr, wide);
  }
}

// Workspace layout: (reference, sum) per split slot and the unnormalised split outputs when
// there are several splits; then the wide kernel's per-wave flags.
struct LatentWs {
  size_t ml, o, flags, bytes;
};

LatentWs latent_ws(int64_t B, int64_t H, int64_t Dl, const LatentPlan& p) {
  LatentWs w{0, 0, 0, 0};
  if (p.nsplit > 1) {
    const size_t slots = static_cast<size_t>(B * H) * p.nsplit;
    w.o = round_up(slots * 2 * sizeof(float), 256);
    w.bytes = w.o + round_up(slots * static_cast<size_t>(Dl) * sizeof(float), 256);
  }
  if (p.wide) {
    w.flags = w.bytes;
    w.bytes += round_up(static_cast<size_t>(B) * p.groups * p.nsplit * 4 * sizeof(uint32_t), 256);
  }
  return w;
}

}  // namespace
}  // namespace fa3q

using namespace fa3q;

extern "C" size_t fa3q_decode_latent_workspace_bytes(int64_t B, int64_t H, int64_t T, int64_t Dl) {
  if (!latent_shape_ok(B, H, T, Dl) || !(Dl == 128 || Dl == 256 || Dl == 512)) return 0;
  return latent_ws(B, H, Dl, plan_latent(B, H, T)).bytes;
}

extern "C" int fa3q_decode_latent(const uint16_t* q, const int8_t* c_q, const float* scale, const uint16_t* k_rope,
                                  int64_t B, int64_t H, int64_t T, int64_t Dl, int64_t Dr, float sm_scale,
                                  float* out, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !c_q || !scale || !out || (Dr > 0 && !k_rope)) return FA3Q_ERR_NULL;
  if (!latent_dims_ok(Dl, Dr) || !latent_shape_ok(B, H, T, Dl)) return FA3Q_ERR_SHAPE;
  if (!std::isfinite(sm_scale)) return FA3Q_ERR_SHAPE;
  if (!is_aligned(q, 16) || !is_aligned(c_q, 16) || !is_aligned(scale, 4) || !is_aligned(out, 16) ||
      (Dr > 0 && !is_aligned(k_rope, 16)))
    return FA3Q_ERR_ALIGN;
  const LatentPlan p = plan_latent(B, H, T);
  const LatentWs w = latent_ws(B, H, Dl, p);
  if (w.bytes > 0) {
    if (!workspace || workspace_bytes < w.bytes) return FA3Q_ERR_WORKSPACE;
    if (!is_aligned(workspace, 256)) return FA3Q_ERR_ALIGN;
  }
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  LatentArgs a;
  a.q = q;
  a.cq = c_q;
  a.scale = scale;
  a.kr = k_rope;
  a.out = out;
  a.ws_ml = p.nsplit > 1 ? reinterpret_cast<float*>(ws) : nullptr;
  a.ws_o = p.nsplit > 1 ? reinterpret_cast<float*>(ws + w.o) : nullptr;
  a.flags = nullptr;
  a.T = T;
  a.H = static_cast<int32_t>(H);
  a.groups = p.groups;
  a.nsplit = p.nsplit;
  a.split_len = p.split_len;
  a.sm_log2 = sm_scale * 1.4426950408889634f;
  hipStream_t s = as_stream(stream);
  // Dl = 512 with a RoPE part of 32 features spills in the wide kernel's tile loop: that one
  // takes the split kernel over the same splits (the workspace is the same)
  if (p.wide && (Dl < 512 || Dr != 32)) {
    a.flags = reinterpret_cast<uint32_t*>(ws + w.flags);
    hipLaunchKernelGGL(pick_latent(Dl, Dr, true), dim3(static_cast<unsigned>(B * p.groups * p.nsplit)),
                       dim3(kWideThreads), 0, s, a);
    // the splits a wave gave up, recomputed by the split kernel over the same splits (its
    // workgroups exit at once elsewhere)
    LatentArgs f = a;
    f.groups = static_cast<int32_t>((H + kLatHeads - 1) / kLatHeads);
    hipLaunchKernelGGL(pick_latent(Dl, Dr, false), dim3(static_cast<unsigned>(B * f.groups * p.nsplit)),
                       dim3(kLatThreads), 0, s, f);
  } else {
    a.groups = static_cast<int32_t>((H + kLatHeads - 1) / kLatHeads);
    hipLaunchKernelGGL(pick_latent(Dl, Dr, false), dim3(static_cast<unsigned>(B * a.groups * p.nsplit)),
                       dim3(kLatThreads), 0, s, a);
  }
  if (p.nsplit > 1) {
    const int64_t rows = B * H, per_wg = kCombineThreads / (Dl / 4);
    hipLaunchKernelGGL(latent_combine_kernel, dim3(static_cast<unsigned>((rows + per_wg - 1) / per_wg)),
                       dim3(kCombineThreads), 0, s, a, static_cast<int>(Dl), rows);
  }
  return launch_status();
}
