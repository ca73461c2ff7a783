// Decode-phase attention over the quantised cache: INT8 K-nope (per-head scale),
// bf16 K-rope and bf16 V, one query token per (b, h).
//
// MindIE LLM page "FA3 quantization", overview: the INT8 K-nope / float K-rope cache is
// there to cut KV-cache memory and speed up decode-phase attention.  The pages show no
// operator; this is softmax attention over the cache dequantised per head:
//   s_t = sm * (scale[h] * <q_nope, code_t> + <q_rope, k_rope_t>),  out = sum_t softmax(s)_t v_t
// with scale[h] factored out of the nope dot product (equal to dequantising each code).
//
// Shape of the work: a single query per (b, h) makes QK^T a matrix-vector product over
// T rows of 2*Dn + 2*Dr + 2*Dv bytes (512 B for the MLA shape), at about 1.25 flop per
// byte; it is bound by HBM, so it runs on the vector ALUs (a 16x16 MFMA tile would be
// 15/16 empty).  Each workgroup owns (b, h, split) and a run of up to kMaxSplitLen tokens:
//   phase 1  LK lanes per token, 16 int8 nope codes + 8 rope values per lane (two
//            16-byte loads), eight tokens in flight per lane, DPP row reductions;
//            scores (log2 domain) go to LDS;
//   phase 2  block max and exp2 -> probabilities in LDS, block sum;
//   phase 3  LV = Dv/8 lanes per token, one 16-byte V load per lane, probability-weighted
//            sums, eight tokens in flight per lane.
// Splits of one (b, h) leave (max, sum, unnormalised output) in the workspace and a
// combine kernel merges them; with one split the output is written directly.
// Cache loads carry the nontemporal hint: each byte is read once (about 10% more bandwidth
// than plain loads on MI355X at the MLA shape).
//
// Decode step with append and ragged lengths (fa3q_decode_append_attn): sequence b holds
// kv_len[b] cached tokens out of a capacity of T.  With a new token, the split that owns
// position kv_len[b] quantises the new K-nope row exactly as fa3q_quantize_k does (same
// per-head scale, correctly rounded quotient, round half to even, clamp to +-127), stores
// it with the new K-rope and V rows at that position, and scores and weights the token
// from registers; attention then covers kv_len[b] + 1 tokens.  Without one it covers
// kv_len[b].  Splits past a sequence's end leave an empty softmax state.
//
// Q, K and V all INT8 (fa3q_decode_attn_qkv8): Q's non-RoPE part and V carry per-head
// codes too (from fa3q_quantize_k).  The non-RoPE score is scale_q[h]*scale_k[h] times an
// exact integer dot product (v_dot4 over four code pairs per instruction), the RoPE part
// stays bf16, and V is weighted as codes with scale_v[h] applied once at the end: 384
// bytes per cached token instead of 512 at the MLA shape.
//
// Asymmetric K cache (fa3q_decode_attn_asym): K-nope codes with a scale and an offset per
// (head, dim) (fa3q_quantize_asym), the value of a code being (code - o[h,d]) * s[h,d].
// The per-dim scale folds into the query (q'_d = q_d * s[h,d]) and the offsets into one
// constant per (b, h) (sum_d q'_d * o[h,d]), so the score is the same code dot product.
#include <cmath>
#include <mutex>
#include <unordered_map>

#include "fa3q_internal.hpp"

// Scratch of fa3q_decode_attn_noalloc: the split softmax states (max, sum, unnormalised
// output per split) live in this file-scope device array instead of a caller workspace.
// Each GPU holds its own copy, at its own address, until the process ends; host code must
// use the address hipGetSymbolAddress gives on that device, never the array's name (on the
// host the name is a stand-in, not a device address).  Every split writes its whole state
// before the combine kernel reads it, so nothing needs clearing between calls.
static __device__ __align__(256) unsigned char scratch[FA3Q_NOALLOC_SCRATCH_BYTES];

namespace fa3q {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxSplitLen = 4096;  // scores of one split are kept in LDS (16 KiB)
constexpr int kMinSplitLen = 256;
constexpr int64_t kTargetGroups = 2048;  // enough workgroups to fill 256 CUs several times
constexpr int kUk = 8;  // tokens per lane in flight, phase 1
constexpr int kUv = 8;  // tokens per lane in flight, phase 3

struct DecodeArgs {
  const uint16_t* q;
  const int8_t* kq;
  const float* scale;
  const uint16_t* kr;
  const uint16_t* v;
  float* out;
  const int32_t* kv_len;   // [B] cached tokens per sequence (ragged kernels only)
  const int32_t* block_table;  // [B][max_pages] physical page of each logical page (paged kernels)
  int64_t num_pages;           // pages in each pool (paged kernels)
  int32_t max_pages;           // block-table row length; T = max_pages << page_shift
  int32_t page_shift;          // log2 of the page size
  const uint16_t* k_new;   // (B,H,Dn+Dr) token to append, or null
  const uint16_t* v_new;   // (B,H,Dv)
  const int8_t* qq;        // (B,H,Dn) query codes (INT8 kernels; q is then the (B,H,Dr) RoPE part)
  const int8_t* vq;        // (B,H,T,Dv) value codes (INT8 kernels)
  const float* scale_q;    // [H]
  const float* scale_v;    // [H]
  const uint16_t* k_scale_hd;   // [H][Dn] bf16 or float16 (asymmetric kernels)
  const uint16_t* k_offset_hd;  // [H][Dn]
  int32_t params_f16;           // 1: the tables are float16, 0: bfloat16
  float* ws_ml;  // [B*H*nsplit][2] (max, sum)
  float* ws_o;   // [B*H*nsplit][Dv]
  int64_t hs;    // cache rows from one head to the next: T (B,H,T,.) or 1 (B,T,H,.)
  int64_t ts;    // cache rows from one token to the next: 1 (B,H,T,.) or H (B,T,H,.)
  int64_t T;
  int32_t H;
  int32_t Dn;
  int32_t Dr;
  int32_t Dv;
  int32_t nsplit;
  int32_t split_len;
  float sm_log2;  // sm_scale * log2(e)
};

// Sum over lanes of one wave that share (lane % LV): lane bits at and above log2(LV).
template <int LV>
__device__ __forceinline__ float slot_sum(float v) {
#pragma unroll
  for (int o = LV; o < kWave; o <<= 1) v += __shfl_xor(v, o);
  return v;
}

// <q, code> over 16 int8 codes held in a uint4, using unsigned bytes code+128 and the
// precomputed sum of q (v_cvt_f32_ubyte* reads the offset codes directly).
__device__ __forceinline__ float dot16_i8(const float (&qn)[16], float qsum, uint4 w) {
  const uint32_t d[4] = {w.x ^ 0x80808080u, w.y ^ 0x80808080u, w.z ^ 0x80808080u, w.w ^ 0x80808080u};
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc = fmaf(qn[4 * i + 0], static_cast<float>(d[i] & 0xffu), acc);
    acc = fmaf(qn[4 * i + 1], static_cast<float>((d[i] >> 8) & 0xffu), acc);
    acc = fmaf(qn[4 * i + 2], static_cast<float>((d[i] >> 16) & 0xffu), acc);
    acc = fmaf(qn[4 * i + 3], static_cast<float>(d[i] >> 24), acc);
  }
  return fmaf(-128.0f, qsum, acc);
}

// <q_rope, k_rope> over 8 bf16 (or, kF16, float16) values held in a uint4.
template <bool kF16>
__device__ __forceinline__ float dot8_16(const float (&qr)[8], uint4 w) {
  float acc = 0.0f;
  acc = fmaf(qr[0], lo16<kF16>(w.x), acc);
  acc = fmaf(qr[1], hi16<kF16>(w.x), acc);
  acc = fmaf(qr[2], lo16<kF16>(w.y), acc);
  acc = fmaf(qr[3], hi16<kF16>(w.y), acc);
  acc = fmaf(qr[4], lo16<kF16>(w.z), acc);
  acc = fmaf(qr[5], hi16<kF16>(w.z), acc);
  acc = fmaf(qr[6], lo16<kF16>(w.w), acc);
  acc = fmaf(qr[7], hi16<kF16>(w.w), acc);
  return acc;
}

typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
// 16-byte load with the nontemporal hint (the cache is streamed once).
__device__ __forceinline__ uint4 load_nt(const void* p) {
  const u32x4v v = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// 4 bf16 (kF16: float16) values (two dwords) -> 4 INT8 codes in one dword, little-endian
// element order: clamp(round_half_even(fl32(x / s)), -127, 127) with the IEEE quotient; 0
// when s == 0.
template <bool kF16>
__device__ __forceinline__ uint32_t quant4_exact(uint32_t w0, uint32_t w1, float s) {
  const float xv[4] = {lo16<kF16>(w0), hi16<kF16>(w0), lo16<kF16>(w1), hi16<kF16>(w1)};
  uint32_t o = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = s == 0.0f ? 0 : static_cast<int>(__builtin_amdgcn_fmed3f(rintf(xv[i] / s), -127.0f, 127.0f));
    o |= (static_cast<uint32_t>(c) & 0xffu) << (8 * i);
  }
  return o;
}

// float32 value of a bf16 or float16 parameter pattern.
__device__ __forceinline__ float param_f32(uint16_t bits, bool f16) {
  return f16 ? static_cast<float>(__builtin_bit_cast(_Float16, bits)) : __uint_as_float(static_cast<uint32_t>(bits) << 16);
}

constexpr int kFmtBf16 = 0;  // bf16 query and values, per-head symmetric K-nope codes
constexpr int kFmtQkv8 = 1;  // INT8 query (non-RoPE part) and values; LV is then Dv/16
constexpr int kFmtAsym = 2;  // bf16 query and values, per-(head, dim) asymmetric K-nope codes
constexpr int kFmtF16 = 3;   // float16 query and values, per-head symmetric K-nope codes

constexpr int kVarFixed = 0;  // every sequence holds T tokens at (b, h, t)
constexpr int kVarRagged = 1; // kv_len[] tokens, optional append, contiguous (B,H,T,.) or (B,T,H,.) cache
constexpr int kVarPaged = 2;  // kVarRagged through a block table over (pages,H,P,.) pools

// Pages of one split that a paged kernel stages in LDS: enough for split_len tokens starting
// anywhere inside a page.
__host__ __device__ constexpr int split_pages(int64_t split_len, int page_shift) {
  return static_cast<int>(split_len >> page_shift) + 2;
}

// Float offset of the paged kernels' page rows in dynamic LDS, after the scores, the
// reduction scratch and the per-wave partials, rounded up to 8 bytes.
__host__ __device__ constexpr int64_t prow_offset(int64_t split_len, int64_t Dv) {
  return (split_len + kWaves + kWaves * Dv + 1) & ~int64_t{1};
}

// kVar: kVarFixed, kVarRagged (ragged lengths from kv_len[] and, when k_new is set, the
// appended token) or kVarPaged (the same through a block table).
template <int LK, int LV, int kVar, int kFmt>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecodeArgs a) {
  constexpr bool kQ8 = kFmt == kFmtQkv8;
  constexpr bool kAsym = kFmt == kFmtAsym;
  constexpr bool kPaged = kVar == kVarPaged;
  constexpr bool kH = kFmt == kFmtF16;  // float16 query, K-rope and V
  static_assert(!kVar || kFmt == kFmtBf16 || kFmt == kFmtF16, "the append step takes the per-head symmetric cache");
  extern __shared__ float smem[];
  float* sc = smem;                       // [split_len] scores, then probabilities
  float* red = smem + a.split_len;        // [kWaves] block reduction scratch
  float* part = red + kWaves;             // [kWaves][Dv] per-wave output partials
  // paged kernels: row index (page * H + h) * P of each page the split touches
  int64_t* prow = reinterpret_cast<int64_t*>(smem + prow_offset(a.split_len, a.Dv));

  const int bh = static_cast<int>(blockIdx.x) / a.nsplit;
  const int sp = static_cast<int>(blockIdx.x) - bh * a.nsplit;
  const int h = bh % a.H;
  const int64_t t0 = static_cast<int64_t>(sp) * a.split_len;
  const int tid = static_cast<int>(threadIdx.x);
  const int lane = lane_id();
  const int wave = tid / kWave;
  // tokens this split attends to: n from the cache, plus the new one when it owns it
  int n = static_cast<int>(min(a.T - t0, static_cast<int64_t>(a.split_len)));
  bool own_new = false;
  int64_t pos_new = 0;
  if constexpr (kVar) {
    // lengths out of range are clamped, so no access leaves the cache
    int64_t len = a.kv_len[bh / a.H];
    if (a.k_new) {
      pos_new = min(max(len, int64_t{0}), a.T - 1);
      len = pos_new;
      own_new = pos_new >= t0 && pos_new < t0 + a.split_len;
    } else {
      len = min(max(len, int64_t{1}), a.T);
    }
    n = static_cast<int>(max(int64_t{0}, min(len - t0, static_cast<int64_t>(a.split_len))));
    if (n == 0 && !own_new) {
      // past the sequence's end: an empty softmax state for the combine
      const int64_t row = static_cast<int64_t>(bh) * a.nsplit + sp;
      for (int dim = tid; dim < a.Dv; dim += kThreads) a.ws_o[row * a.Dv + dim] = 0.0f;
      if (tid == 0) {
        a.ws_ml[2 * row] = -INFINITY;
        a.ws_ml[2 * row + 1] = 0.0f;
      }
      return;
    }
  }
  const int n_all = n + (own_new ? 1 : 0);  // scores in LDS: the cached tokens, then the new one
  // Row of logical token t0 + tt in the (B,H,T,.) cache, or in the pools through the page rows
  // staged below.  Page indices out of [0, num_pages) are clamped, so no access leaves a pool.
  const int64_t pg0 = kPaged ? (t0 >> a.page_shift) : 0;
  const int64_t pmask = (int64_t{1} << a.page_shift) - 1;
  if constexpr (kPaged) {
    const int b = bh / a.H;
    const int np = static_cast<int>(((t0 + n_all - 1) >> a.page_shift) - pg0) + 1;
    for (int i = tid; i < np; i += kThreads) {
      const int64_t pg = min(max(static_cast<int64_t>(a.block_table[static_cast<int64_t>(b) * a.max_pages + pg0 + i]),
                                 int64_t{0}), a.num_pages - 1);
      prow[i] = (pg * a.H + h) << a.page_shift;
    }
    lds_barrier();
  }
  // row of the split's first token in a contiguous cache: (b, h, t0) in either layout
  const int64_t row0 = static_cast<int64_t>(bh / a.H) * a.H * a.T + static_cast<int64_t>(h) * a.hs + t0 * a.ts;
  auto row_of = [&](int tt) -> int64_t {
    if constexpr (kPaged) {
      const int64_t t = t0 + tt;
      return prow[(t >> a.page_shift) - pg0] + (t & pmask);
    } else {
      return row0 + static_cast<int64_t>(tt) * a.ts;
    }
  };

  // ---------------------------------------------------------------- phase 1: scores
  {
    constexpr int kSlots = kWave / LK;
    const int j = lane % LK;
    const int slot = lane / LK;
    const bool has_n = j < (a.Dn >> 4);
    const bool has_r = j < (a.Dr >> 3);
    const int Dk = a.Dn + a.Dr;
    const uint16_t* qrow = a.q + static_cast<int64_t>(bh) * Dk;  // bf16 query row (bf16 kernels)
    // RoPE part of the query: inside that row, or its own (B,H,Dr) tensor (INT8 kernels)
    const uint16_t* qrope = kQ8 ? a.q + static_cast<int64_t>(bh) * a.Dr : qrow + a.Dn;
    float qn[16], qr[8];
    float qsum = 0.0f;
    uint4 qc = make_uint4(0, 0, 0, 0);  // query codes (INT8 kernels)
    if (kQ8) {
      if (has_n) qc = *reinterpret_cast<const uint4*>(a.qq + static_cast<int64_t>(bh) * a.Dn + 16 * j);
    } else if (has_n) {
      const uint4* p = reinterpret_cast<const uint4*>(qrow + 16 * j);
      const uint4 u0 = p[0], u1 = p[1];
      const uint32_t w[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        qn[2 * i] = lo16<kH>(w[i]);
        qn[2 * i + 1] = hi16<kH>(w[i]);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) qsum += qn[i];
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) qn[i] = 0.0f;
    }
    if (has_r) {
      const uint4 u = *reinterpret_cast<const uint4*>(qrope + 8 * j);
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        qr[2 * i] = lo16<kH>(w[i]);
        qr[2 * i + 1] = hi16<kH>(w[i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) qr[i] = 0.0f;
    }
    const float head_scale = kQ8 ? a.scale_q[h] * a.scale[h] : (kAsym ? 1.0f : a.scale[h]);
    float c0 = 0.0f;  // asymmetric cache: this lane's share of sum_d q'_d * o[h,d]
    if constexpr (kAsym) {
      if (has_n) {
        const bool f16 = a.params_f16 != 0;
        const uint4* sp = reinterpret_cast<const uint4*>(a.k_scale_hd + static_cast<int64_t>(h) * a.Dn + 16 * j);
        const uint4* op = reinterpret_cast<const uint4*>(a.k_offset_hd + static_cast<int64_t>(h) * a.Dn + 16 * j);
        const uint4 s0 = sp[0], s1 = sp[1], o0 = op[0], o1 = op[1];
        const uint32_t sw[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
        const uint32_t ow[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
        qsum = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          qn[2 * i] *= param_f32(static_cast<uint16_t>(sw[i] & 0xffffu), f16);
          qn[2 * i + 1] *= param_f32(static_cast<uint16_t>(sw[i] >> 16), f16);
          c0 = fmaf(qn[2 * i], param_f32(static_cast<uint16_t>(ow[i] & 0xffffu), f16), c0);
          c0 = fmaf(qn[2 * i + 1], param_f32(static_cast<uint16_t>(ow[i] >> 16), f16), c0);
          qsum += qn[2 * i] + qn[2 * i + 1];
        }
      }
    }
    // contiguous caches: the split's first row and the rows' token stride; paged: whole rows
    const int8_t* kq = a.kq + (kPaged ? 0 : row0 * a.Dn) + 16 * j;
    const uint16_t* kr = a.kr + (kPaged ? 0 : row0 * a.Dr) + 8 * j;
    const int64_t kq_tok = a.ts * a.Dn, kr_tok = a.ts * a.Dr;
    const int step = kWaves * kSlots;
    for (int base = wave * kSlots + slot; base < n; base += step * kUk) {
      uint4 wn[kUk], wr[kUk];
#pragma unroll
      for (int u = 0; u < kUk; ++u) {
        const int tt = base + u * step;
        wn[u] = make_uint4(0, 0, 0, 0);
        wr[u] = make_uint4(0, 0, 0, 0);
        if (tt < n) {
          if constexpr (kPaged) {
            const int64_t r = row_of(tt);
            if (has_n) wn[u] = load_nt(kq + r * a.Dn);
            if (has_r) wr[u] = load_nt(kr + r * a.Dr);
          } else {
            if (has_n) wn[u] = load_nt(kq + tt * kq_tok);
            if (has_r) wr[u] = load_nt(kr + tt * kr_tok);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < kUk; ++u) {
        const int tt = base + u * step;
        float s = 0.0f;
        if (has_n) {
          if constexpr (kQ8) {
            int d = __builtin_amdgcn_sdot4(static_cast<int>(qc.x), static_cast<int>(wn[u].x), 0, false);
            d = __builtin_amdgcn_sdot4(static_cast<int>(qc.y), static_cast<int>(wn[u].y), d, false);
            d = __builtin_amdgcn_sdot4(static_cast<int>(qc.z), static_cast<int>(wn[u].z), d, false);
            d = __builtin_amdgcn_sdot4(static_cast<int>(qc.w), static_cast<int>(wn[u].w), d, false);
            s = head_scale * static_cast<float>(d);  // |d| <= 16*127*127: exact in float32
          } else if constexpr (kAsym) {
            s = dot16_i8(qn, qsum, wn[u]) - c0;
          } else {
            s = head_scale * dot16_i8(qn, qsum, wn[u]);
          }
        }
        if (has_r) s += dot8_16<kH>(qr, wr[u]);
        s = group_sum<LK>(s);
        if (j == 0 && tt < n) sc[tt] = s * a.sm_log2;
      }
    }
    if constexpr (kVar) {
      if (own_new && wave == 0) {
        // every slot of wave 0 quantises the same new row; slot 0 stores it and its score
        const uint16_t* knew = a.k_new + static_cast<int64_t>(bh) * Dk;
        const int64_t at = row_of(static_cast<int>(pos_new - t0));
        uint4 cn = make_uint4(0, 0, 0, 0), rn = make_uint4(0, 0, 0, 0);
        if (has_n) {
          const uint4* p = reinterpret_cast<const uint4*>(knew + 16 * j);
          const uint4 u0 = p[0], u1 = p[1];
          cn = make_uint4(quant4_exact<kH>(u0.x, u0.y, head_scale), quant4_exact<kH>(u0.z, u0.w, head_scale),
                          quant4_exact<kH>(u1.x, u1.y, head_scale), quant4_exact<kH>(u1.z, u1.w, head_scale));
          if (slot == 0) *reinterpret_cast<uint4*>(const_cast<int8_t*>(a.kq) + at * a.Dn + 16 * j) = cn;
        }
        if (has_r) {
          rn = *reinterpret_cast<const uint4*>(knew + a.Dn + 8 * j);
          if (slot == 0) *reinterpret_cast<uint4*>(const_cast<uint16_t*>(a.kr) + at * a.Dr + 8 * j) = rn;
        }
        float s = 0.0f;
        if (has_n) s = head_scale * dot16_i8(qn, qsum, cn);
        if (has_r) s += dot8_16<kH>(qr, rn);
        s = group_sum<LK>(s);
        if (j == 0 && slot == 0) sc[n] = s * a.sm_log2;
      }
    }
  }
  lds_barrier();

  // ---------------------------------------------------------------- phase 2: softmax
  float m = -INFINITY;
  for (int i = tid; i < n_all; i += kThreads) m = fmaxf(m, sc[i]);
  m = wave_max(m);
  if (lane == 0) red[wave] = m;
  lds_barrier();
  m = red[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) m = fmaxf(m, red[w]);
  float l = 0.0f;
  for (int i = tid; i < n_all; i += kThreads) {
    const float p = exp2f(sc[i] - m);
    sc[i] = p;
    l += p;
  }
  l = wave_sum(l);
  lds_barrier();  // every wave has read red[] (max) before it is reused for the sum
  if (lane == 0) red[wave] = l;
  lds_barrier();
  l = 0.0f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) l += red[w];

  // ---------------------------------------------------------------- phase 3: P . V
  constexpr int kVSlots = kWave / LV;
  constexpr int kVD = kQ8 ? 16 : 8;  // value dims per lane: one 16-byte load per token
  const int jv = lane % LV;
  const int vslot = lane / LV;
  float acc[kVD];
#pragma unroll
  for (int d = 0; d < kVD; ++d) acc[d] = 0.0f;
  float psum = 0.0f;  // INT8 values: sum of the weights, for the +128 offset of the byte reads
  {
    const int64_t vrow = kQ8 ? a.Dv : 2 * static_cast<int64_t>(a.Dv);  // bytes per cache row
    const char* vp = (kQ8 ? reinterpret_cast<const char*>(a.vq + 16 * jv) : reinterpret_cast<const char*>(a.v + 8 * jv)) +
                     (kPaged ? 0 : row0 * vrow);
    const int64_t v_tok = a.ts * vrow;  // contiguous caches: bytes from one token to the next
    const int step = kWaves * kVSlots;
    for (int base = wave * kVSlots + vslot; base < n; base += step * kUv) {
      uint4 wv[kUv];
      float p[kUv];
#pragma unroll
      for (int u = 0; u < kUv; ++u) {
        const int tt = base + u * step;
        wv[u] = make_uint4(0, 0, 0, 0);
        p[u] = 0.0f;
        if (tt < n) {
          wv[u] = load_nt(kPaged ? vp + row_of(tt) * vrow : vp + tt * v_tok);
          p[u] = sc[tt];
        }
      }
#pragma unroll
      for (int u = 0; u < kUv; ++u) {
        if constexpr (kQ8) {
          const uint32_t d[4] = {wv[u].x ^ 0x80808080u, wv[u].y ^ 0x80808080u, wv[u].z ^ 0x80808080u,
                                 wv[u].w ^ 0x80808080u};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[4 * i + 0] = fmaf(p[u], static_cast<float>(d[i] & 0xffu), acc[4 * i + 0]);
            acc[4 * i + 1] = fmaf(p[u], static_cast<float>((d[i] >> 8) & 0xffu), acc[4 * i + 1]);
            acc[4 * i + 2] = fmaf(p[u], static_cast<float>((d[i] >> 16) & 0xffu), acc[4 * i + 2]);
            acc[4 * i + 3] = fmaf(p[u], static_cast<float>(d[i] >> 24), acc[4 * i + 3]);
          }
          psum += p[u];
        } else {
          acc[0] = fmaf(p[u], lo16<kH>(wv[u].x), acc[0]);
          acc[1] = fmaf(p[u], hi16<kH>(wv[u].x), acc[1]);
          acc[2] = fmaf(p[u], lo16<kH>(wv[u].y), acc[2]);
          acc[3] = fmaf(p[u], hi16<kH>(wv[u].y), acc[3]);
          acc[4] = fmaf(p[u], lo16<kH>(wv[u].z), acc[4]);
          acc[5] = fmaf(p[u], hi16<kH>(wv[u].z), acc[5]);
          acc[6] = fmaf(p[u], lo16<kH>(wv[u].w), acc[6]);
          acc[7] = fmaf(p[u], hi16<kH>(wv[u].w), acc[7]);
        }
      }
    }
  }
  if constexpr (kQ8) {
    // codes were read as unsigned bytes code + 128; the head scale comes in once
    const float sv = a.scale_v[h];
#pragma unroll
    for (int d = 0; d < kVD; ++d) acc[d] = fmaf(-128.0f, psum, acc[d]) * sv;
  }
  if constexpr (kVar) {
    if (own_new && wave == 0 && vslot == 0) {
      const uint4 wv = *reinterpret_cast<const uint4*>(a.v_new + static_cast<int64_t>(bh) * a.Dv + 8 * jv);
      *reinterpret_cast<uint4*>(const_cast<uint16_t*>(a.v) + row_of(static_cast<int>(pos_new - t0)) * a.Dv + 8 * jv) = wv;
      const float p = sc[n];
      acc[0] = fmaf(p, lo16<kH>(wv.x), acc[0]);
      acc[1] = fmaf(p, hi16<kH>(wv.x), acc[1]);
      acc[2] = fmaf(p, lo16<kH>(wv.y), acc[2]);
      acc[3] = fmaf(p, hi16<kH>(wv.y), acc[3]);
      acc[4] = fmaf(p, lo16<kH>(wv.z), acc[4]);
      acc[5] = fmaf(p, hi16<kH>(wv.z), acc[5]);
      acc[6] = fmaf(p, lo16<kH>(wv.w), acc[6]);
      acc[7] = fmaf(p, hi16<kH>(wv.w), acc[7]);
    }
  }
#pragma unroll
  for (int d = 0; d < kVD; ++d) acc[d] = slot_sum<LV>(acc[d]);
  if (vslot == 0) {
#pragma unroll
    for (int d = 0; d < kVD; ++d) part[wave * a.Dv + kVD * jv + d] = acc[d];
  }
  lds_barrier();
  const int64_t row = static_cast<int64_t>(bh) * a.nsplit + sp;
  for (int dim = tid; dim < a.Dv; dim += kThreads) {
    float o = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) o += part[w * a.Dv + dim];
    if (a.nsplit == 1) {
      a.out[static_cast<int64_t>(bh) * a.Dv + dim] = o / l;
    } else {
      a.ws_o[row * a.Dv + dim] = o;
    }
  }
  if (a.nsplit > 1 && tid == 0) {
    a.ws_ml[2 * row] = m;
    a.ws_ml[2 * row + 1] = l;
  }
}

// Merge the per-split softmax states of one (b, h): out = sum_s w_s o_s / sum_s w_s l_s,
// w_s = 2^(m_s - max_s m_s).
__global__ __launch_bounds__(128) void decode_combine_kernel(DecodeArgs a) {
  const int64_t bh = blockIdx.x;
  const float* ml = a.ws_ml + 2 * bh * a.nsplit;
  float mmax = -INFINITY;
  for (int s = 0; s < a.nsplit; ++s) mmax = fmaxf(mmax, ml[2 * s]);
  float den = 0.0f;
  for (int s = 0; s < a.nsplit; ++s) den += exp2f(ml[2 * s] - mmax) * ml[2 * s + 1];
  for (int dim = threadIdx.x; dim < a.Dv; dim += blockDim.x) {
    float num = 0.0f;
    for (int s = 0; s < a.nsplit; ++s)
      num += exp2f(ml[2 * s] - mmax) * a.ws_o[(bh * a.nsplit + s) * a.Dv + dim];
    a.out[bh * a.Dv + dim] = num / den;
  }
}

struct SplitPlan {
  int32_t nsplit;
  int32_t split_len;
};

SplitPlan plan_splits(int64_t B, int64_t H, int64_t T) {
  const int64_t pairs = B * H;
  int64_t ns = (T + kMaxSplitLen - 1) / kMaxSplitLen;
  const int64_t want = (kTargetGroups + pairs - 1) / pairs;
  const int64_t cap = std::max<int64_t>(1, T / kMinSplitLen);
  ns = std::max(ns, std::min(want, cap));
  const int64_t len = (T + ns - 1) / ns;
  ns = (T + len - 1) / len;  // no empty split
  return {static_cast<int32_t>(ns), static_cast<int32_t>(len)};
}

bool pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

int64_t next_pow2(int64_t v) {
  int64_t p = 1;
  while (p < v) p <<= 1;
  return p;
}

using KernelFn = void (*)(DecodeArgs);

template <int LK, int kVar, int kFmt>
KernelFn pick_lv(int lv) {
  switch (lv) {
    case 1: return decode_split_kernel<LK, 1, kVar, kFmt>;
    case 2: return decode_split_kernel<LK, 2, kVar, kFmt>;
    case 4: return decode_split_kernel<LK, 4, kVar, kFmt>;
    case 8: return decode_split_kernel<LK, 8, kVar, kFmt>;
    case 16: return decode_split_kernel<LK, 16, kVar, kFmt>;
    case 32: return decode_split_kernel<LK, 32, kVar, kFmt>;
    case 64:
      if constexpr (kFmt == kFmtQkv8) return nullptr;  // Dv = 1024 is past the supported range
      else return decode_split_kernel<LK, 64, kVar, kFmt>;
    default: return nullptr;
  }
}

template <int kVar, int kFmt>
KernelFn pick_kernel(int lk, int lv) {
  switch (lk) {
    case 1: return pick_lv<1, kVar, kFmt>(lv);
    case 2: return pick_lv<2, kVar, kFmt>(lv);
    case 4: return pick_lv<4, kVar, kFmt>(lv);
    case 8: return pick_lv<8, kVar, kFmt>(lv);
    case 16: return pick_lv<16, kVar, kFmt>(lv);
    case 32: return pick_lv<32, kVar, kFmt>(lv);
    case 64: return pick_lv<64, kVar, kFmt>(lv);
    default: return nullptr;
  }
}

bool valid_dims(int64_t Dn, int64_t Dr, int64_t Dv) {
  if (Dn <= 0 || Dn % 16 != 0 || Dn > 1024) return false;
  if (Dr < 0 || Dr % 8 != 0 || Dr > 512) return false;
  if (!pow2(Dv) || Dv < 8 || Dv > 512) return false;
  return true;
}

}  // namespace
}  // namespace fa3q

using namespace fa3q;

extern "C" size_t fa3q_decode_attn_workspace_bytes(int64_t B, int64_t H, int64_t T, int64_t Dv) {
  if (B <= 0 || H <= 0 || T <= 0 || !pow2(Dv) || Dv < 8 || Dv > 512) return 0;
  if (B > (int64_t{1} << 31) / H || T > (int64_t{1} << 40)) return 0;
  const SplitPlan p = plan_splits(B, H, T);
  if (p.nsplit <= 1) return 0;
  return round_up(static_cast<size_t>(B * H * p.nsplit) * 2 * sizeof(float), 256) +
         static_cast<size_t>(B * H * p.nsplit) * static_cast<size_t>(Dv) * sizeof(float);
}

namespace fa3q {
namespace {

constexpr size_t kScratchBytes = FA3Q_NOALLOC_SCRATCH_BYTES;

// Device address of the current device's scratch array, looked up once per device.
int scratch_address(void** out) {
  static std::mutex mu;
  static std::unordered_map<int, void*> addr;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FA3Q_ERR_HIP;
  std::lock_guard<std::mutex> lock(mu);
  auto it = addr.find(dev);
  if (it == addr.end()) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return FA3Q_ERR_HIP;
    it = addr.emplace(dev, p).first;
  }
  *out = it->second;
  return FA3Q_OK;
}

// INT8 query and values of fa3q_decode_attn_qkv8, and the asymmetric K tables of
// fa3q_decode_attn_asym (unused by the other entry points).
struct Int8QV {
  const int8_t* qq = nullptr;
  const int8_t* vq = nullptr;
  const float* scale_q = nullptr;
  const float* scale_v = nullptr;
  const uint16_t* k_scale_hd = nullptr;
  const uint16_t* k_offset_hd = nullptr;
  int params_f16 = 0;
};

// Block table of the paged entry point (unused by the others).
struct PagedKV {
  const int32_t* block_table = nullptr;
  int64_t num_pages = 0;
  int64_t page_size = 0;
  int64_t max_pages = 0;
};

int log2_exact(int64_t v) {
  int s = 0;
  while ((int64_t{1} << s) < v) ++s;
  return s;
}

// Shared validation and launch of the decode entry points (kVar: kVarFixed, kVarRagged or
// kVarPaged, the last with T = max_pages * page_size and the cache pointers being pools;
// kFmt: kFmtQkv8 takes INT8 query and values, with q the (B,H,Dr) RoPE part and v unused;
// kFmtAsym takes the per-(head, dim) K tables instead of the per-head scale; kFmtF16 is
// kFmtBf16 with float16 query, K-rope and V).  bshd: contiguous caches are (B,T,H,.).
template <int kVar, int kFmt>
int decode_launch(const uint16_t* q, const int8_t* k_nope_q, const float* scale, const uint16_t* k_rope,
                  const uint16_t* v, const int32_t* kv_len, const uint16_t* k_new, const uint16_t* v_new,
                  const Int8QV& i8, int64_t B, int64_t H, int64_t T, int64_t Dn, int64_t Dr, int64_t Dv,
                  float sm_scale, float* out, void* workspace, size_t workspace_bytes, void* stream,
                  const PagedKV& pk = PagedKV{}, bool use_scratch = false, bool bshd = false) {
  constexpr bool kQ8 = kFmt == kFmtQkv8;
  constexpr bool kAsym = kFmt == kFmtAsym;
  constexpr bool kPaged = kVar == kVarPaged;
  if (kQ8) {
    if (!i8.qq || !i8.vq || !i8.scale_q || !i8.scale_v || !k_nope_q || !scale || !out || (Dr > 0 && (!q || !k_rope)))
      return FA3Q_ERR_NULL;
  } else if (!q || !k_nope_q || (!kAsym && !scale) || !v || !out || (Dr > 0 && !k_rope)) {
    return FA3Q_ERR_NULL;
  }
  if (kAsym && (!i8.k_scale_hd || !i8.k_offset_hd)) return FA3Q_ERR_NULL;
  if (kAsym && i8.params_f16 != 0 && i8.params_f16 != 1) return FA3Q_ERR_DTYPE;
  if (kVar && (!kv_len || (k_new != nullptr) != (v_new != nullptr))) return FA3Q_ERR_NULL;
  if (kPaged && !pk.block_table) return FA3Q_ERR_NULL;
  if (kPaged) {
    // pages: a power of two from 16 to 65536 tokens; pools of num_pages pages of H * P rows
    if (B <= 0 || H <= 0 || H > (int64_t{1} << 20)) return FA3Q_ERR_SHAPE;
    if (pk.page_size < 16 || pk.page_size > 65536 || !pow2(pk.page_size)) return FA3Q_ERR_SHAPE;
    if (pk.num_pages <= 0 || pk.max_pages <= 0 || pk.max_pages > (int64_t{1} << 24)) return FA3Q_ERR_SHAPE;
    if (pk.num_pages > (int64_t{1} << 62) / (H * pk.page_size * 1024)) return FA3Q_ERR_SHAPE;  // pool bytes
    if (B > (int64_t{1} << 31) / pk.max_pages) return FA3Q_ERR_SHAPE;  // block-table entries
    T = pk.max_pages * pk.page_size;
  }
  if (B <= 0 || H <= 0 || T <= 0) return FA3Q_ERR_SHAPE;
  if (!valid_dims(Dn, Dr, Dv) || (kQ8 && Dv < 16)) return FA3Q_ERR_SHAPE;
  if (B > (int64_t{1} << 31) / H || T > (int64_t{1} << 40)) return FA3Q_ERR_SHAPE;
  if (B * H * T > (int64_t{1} << 62) / (Dn + Dr + Dv)) return FA3Q_ERR_SHAPE;
  if (!std::isfinite(sm_scale)) return FA3Q_ERR_SHAPE;
  if ((Dr > 0 && !is_aligned(q, 16)) || !is_aligned(k_nope_q, 16) || (Dr > 0 && !is_aligned(k_rope, 16)) ||
      !is_aligned(out, 16) || (!kAsym && !is_aligned(scale, 4)))
    return FA3Q_ERR_ALIGN;
  if (kAsym && (!is_aligned(i8.k_scale_hd, 16) || !is_aligned(i8.k_offset_hd, 16))) return FA3Q_ERR_ALIGN;
  if (kQ8 ? (!is_aligned(i8.qq, 16) || !is_aligned(i8.vq, 16) || !is_aligned(i8.scale_q, 4) ||
             !is_aligned(i8.scale_v, 4))
          : (!is_aligned(q, 16) || !is_aligned(v, 16)))
    return FA3Q_ERR_ALIGN;
  if (kVar && (!is_aligned(kv_len, 4) || (k_new && (!is_aligned(k_new, 16) || !is_aligned(v_new, 16)))))
    return FA3Q_ERR_ALIGN;
  if (kPaged && !is_aligned(pk.block_table, 4)) return FA3Q_ERR_ALIGN;
  const SplitPlan p = plan_splits(B, H, T);
  if (B * H * p.nsplit > (int64_t{1} << 31) - 1) return FA3Q_ERR_SHAPE;
  const size_t need = fa3q_decode_attn_workspace_bytes(B, H, T, Dv);
  if (use_scratch) {
    if (need > kScratchBytes) return FA3Q_ERR_SCRATCH;
  } else if (need > 0) {
    if (!workspace || workspace_bytes < need) return FA3Q_ERR_WORKSPACE;
    if (!is_aligned(workspace, 256)) return FA3Q_ERR_ALIGN;
  }
  const int lk = static_cast<int>(next_pow2(std::max<int64_t>(Dn / 16, Dr / 8)));
  const int lv = static_cast<int>(Dv / (kQ8 ? 16 : 8));
  KernelFn fn = pick_kernel<kVar, kFmt>(lk, lv);
  if (!fn) return FA3Q_ERR_UNSUPPORTED;
  if (use_scratch && need > 0) {
    // every argument is valid: only now touch the runtime for this device's copy of the array
    const int st = scratch_address(&workspace);
    if (st != FA3Q_OK) return st;
  }

  DecodeArgs a;
  a.q = q;
  a.kq = k_nope_q;
  a.scale = scale;
  a.kr = k_rope;
  a.v = v;
  a.out = out;
  a.kv_len = kv_len;
  a.block_table = pk.block_table;
  a.num_pages = pk.num_pages;
  a.max_pages = static_cast<int32_t>(pk.max_pages);
  a.page_shift = kPaged ? log2_exact(pk.page_size) : 0;
  a.k_new = k_new;
  a.v_new = v_new;
  a.qq = i8.qq;
  a.vq = i8.vq;
  a.scale_q = i8.scale_q;
  a.scale_v = i8.scale_v;
  a.k_scale_hd = i8.k_scale_hd;
  a.k_offset_hd = i8.k_offset_hd;
  a.params_f16 = i8.params_f16;
  a.ws_ml = need ? static_cast<float*>(workspace) : nullptr;
  a.ws_o = need ? reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                           round_up(static_cast<size_t>(B * H * p.nsplit) * 2 * sizeof(float), 256))
                : nullptr;
  a.hs = bshd ? 1 : T;
  a.ts = bshd ? H : 1;
  a.T = T;
  a.H = static_cast<int32_t>(H);
  a.Dn = static_cast<int32_t>(Dn);
  a.Dr = static_cast<int32_t>(Dr);
  a.Dv = static_cast<int32_t>(Dv);
  a.nsplit = p.nsplit;
  a.split_len = p.split_len;
  a.sm_log2 = static_cast<float>(static_cast<double>(sm_scale) * 1.4426950408889634);
  const size_t lds = kPaged ? static_cast<size_t>(prow_offset(p.split_len, Dv)) * sizeof(float) +
                                  static_cast<size_t>(split_pages(p.split_len, a.page_shift)) * sizeof(int64_t)
                            : (static_cast<size_t>(p.split_len) + kWaves + kWaves * static_cast<size_t>(Dv)) * sizeof(float);
  hipLaunchKernelGGL(fn, dim3(static_cast<unsigned>(B * H * p.nsplit)), dim3(kThreads), lds,
                     as_stream(stream), a);
  if (p.nsplit > 1) {
    hipLaunchKernelGGL(decode_combine_kernel, dim3(static_cast<unsigned>(B * H)), dim3(128), 0,
                       as_stream(stream), a);
  }
  return launch_status();
}

}  // namespace
}  // namespace fa3q

extern "C" int fa3q_decode_attn(const uint16_t* q, const int8_t* k_nope_q, const float* scale,
                                const uint16_t* k_rope, const uint16_t* v, int64_t B, int64_t H,
                                int64_t T, int64_t Dn, int64_t Dr, int64_t Dv, float sm_scale,
                                float* out, void* workspace, size_t workspace_bytes,
                                void* stream) {
  return decode_launch<kVarFixed, kFmtBf16>(q, k_nope_q, scale, k_rope, v, nullptr, nullptr, nullptr, Int8QV{}, B, H, T,
                                     Dn, Dr, Dv, sm_scale, out, workspace, workspace_bytes, stream);
}

extern "C" int fa3q_decode_append_attn(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                                       const float* scale, int8_t* k_nope_q, uint16_t* k_rope,
                                       uint16_t* v, const int32_t* kv_len, int64_t B, int64_t H,
                                       int64_t T, int64_t Dn, int64_t Dr, int64_t Dv, float sm_scale,
                                       float* out, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  return decode_launch<kVarRagged, kFmtBf16>(q, k_nope_q, scale, k_rope, v, kv_len, k_new, v_new, Int8QV{}, B, H, T, Dn,
                                    Dr, Dv, sm_scale, out, workspace, workspace_bytes, stream);
}

extern "C" int fa3q_decode_paged_attn(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                                      const float* scale, int8_t* k_nope_pool, uint16_t* k_rope_pool,
                                      uint16_t* v_pool, const int32_t* block_table, const int32_t* kv_len,
                                      int64_t B, int64_t H, int64_t num_pages, int64_t page_size,
                                      int64_t max_pages, int64_t Dn, int64_t Dr, int64_t Dv, float sm_scale,
                                      float* out, void* workspace, size_t workspace_bytes, void* stream) {
  PagedKV pk;
  pk.block_table = block_table;
  pk.num_pages = num_pages;
  pk.page_size = page_size;
  pk.max_pages = max_pages;
  return decode_launch<kVarPaged, kFmtBf16>(q, k_nope_pool, scale, k_rope_pool, v_pool, kv_len, k_new, v_new,
                                            Int8QV{}, B, H, 0, Dn, Dr, Dv, sm_scale, out, workspace,
                                            workspace_bytes, stream, pk);
}

extern "C" int fa3q_decode_attn_qkv8(const int8_t* q_nope_q, const uint16_t* q_rope, const float* scale_q,
                                     const int8_t* k_nope_q, const float* scale_k, const uint16_t* k_rope,
                                     const int8_t* v_q, const float* scale_v, int64_t B, int64_t H, int64_t T,
                                     int64_t Dn, int64_t Dr, int64_t Dv, float sm_scale, float* out,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  Int8QV i8;
  i8.qq = q_nope_q;
  i8.vq = v_q;
  i8.scale_q = scale_q;
  i8.scale_v = scale_v;
  return decode_launch<kVarFixed, kFmtQkv8>(q_rope, k_nope_q, scale_k, k_rope, nullptr, nullptr, nullptr, nullptr, i8, B,
                                        H, T, Dn, Dr, Dv, sm_scale, out, workspace, workspace_bytes, stream);
}

extern "C" int fa3q_decode_attn_asym(const uint16_t* q, const int8_t* k_nope_q, const uint16_t* k_scale,
                                     const uint16_t* k_offset, int params_dtype, const uint16_t* k_rope,
                                     const uint16_t* v, int64_t B, int64_t H, int64_t T, int64_t Dn, int64_t Dr,
                                     int64_t Dv, float sm_scale, float* out, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  Int8QV i8;
  i8.k_scale_hd = k_scale;
  i8.k_offset_hd = k_offset;
  i8.params_f16 = params_dtype == FA3Q_BF16 ? 0 : (params_dtype == FA3Q_F16 ? 1 : -1);
  return decode_launch<kVarFixed, kFmtAsym>(q, k_nope_q, nullptr, k_rope, v, nullptr, nullptr, nullptr, i8, B, H, T, Dn,
                                        Dr, Dv, sm_scale, out, workspace, workspace_bytes, stream);
}

extern "C" int fa3q_decode_attn_noalloc(const uint16_t* q, const int8_t* k_nope_q, const float* scale,
                                        const uint16_t* k_rope, const uint16_t* v, int64_t B, int64_t H, int64_t T,
                                        int64_t Dn, int64_t Dr, int64_t Dv, float sm_scale, float* out,
                                        void* stream) {
  return decode_launch<kVarFixed, kFmtBf16>(q, k_nope_q, scale, k_rope, v, nullptr, nullptr, nullptr, Int8QV{}, B, H, T,
                                            Dn, Dr, Dv, sm_scale, out, nullptr, 0, stream, PagedKV{}, true);
}

namespace fa3q {
namespace {

// dtype and layout codes of the _ex entry points -> (float16?, (B,T,H,.)?), or a status.
int ex_codes(int dtype, int layout, bool& f16, bool& bshd) {
  if (dtype != FA3Q_BF16 && dtype != FA3Q_F16) return FA3Q_ERR_DTYPE;
  if (layout != FA3Q_BHSD && layout != FA3Q_BSHD) return FA3Q_ERR_LAYOUT;
  f16 = dtype == FA3Q_F16;
  bshd = layout == FA3Q_BSHD;
  return FA3Q_OK;
}

}  // namespace
}  // namespace fa3q

extern "C" int fa3q_decode_attn_ex(const void* q, const int8_t* k_nope_q, const float* scale, const void* k_rope,
                                   const void* v, int dtype, int layout, int64_t B, int64_t H, int64_t T, int64_t Dn,
                                   int64_t Dr, int64_t Dv, float sm_scale, float* out, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  bool f16 = false, bshd = false;
  const int st = ex_codes(dtype, layout, f16, bshd);
  if (st != FA3Q_OK) return st;
  const auto* q16 = static_cast<const uint16_t*>(q);
  const auto* r16 = static_cast<const uint16_t*>(k_rope);
  const auto* v16 = static_cast<const uint16_t*>(v);
  if (f16)
    return decode_launch<kVarFixed, kFmtF16>(q16, k_nope_q, scale, r16, v16, nullptr, nullptr, nullptr, Int8QV{}, B, H,
                                             T, Dn, Dr, Dv, sm_scale, out, workspace, workspace_bytes, stream,
                                             PagedKV{}, false, bshd);
  return decode_launch<kVarFixed, kFmtBf16>(q16, k_nope_q, scale, r16, v16, nullptr, nullptr, nullptr, Int8QV{}, B, H, T,
                                            Dn, Dr, Dv, sm_scale, out, workspace, workspace_bytes, stream, PagedKV{},
                                            false, bshd);
}

extern "C" int fa3q_decode_append_attn_ex(const void* q, const void* k_new, const void* v_new, const float* scale,
                                          int8_t* k_nope_q, void* k_rope, void* v, const int32_t* kv_len, int dtype,
                                          int layout, int64_t B, int64_t H, int64_t T, int64_t Dn, int64_t Dr,
                                          int64_t Dv, float sm_scale, float* out, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  bool f16 = false, bshd = false;
  const int st = ex_codes(dtype, layout, f16, bshd);
  if (st != FA3Q_OK) return st;
  const auto* q16 = static_cast<const uint16_t*>(q);
  const auto* kn16 = static_cast<const uint16_t*>(k_new);
  const auto* vn16 = static_cast<const uint16_t*>(v_new);
  const auto* r16 = static_cast<const uint16_t*>(k_rope);
  const auto* v16 = static_cast<const uint16_t*>(v);
  if (f16)
    return decode_launch<kVarRagged, kFmtF16>(q16, k_nope_q, scale, r16, v16, kv_len, kn16, vn16, Int8QV{}, B, H, T, Dn,
                                              Dr, Dv, sm_scale, out, workspace, workspace_bytes, stream, PagedKV{},
                                              false, bshd);
  return decode_launch<kVarRagged, kFmtBf16>(q16, k_nope_q, scale, r16, v16, kv_len, kn16, vn16, Int8QV{}, B, H, T, Dn,
                                             Dr, Dv, sm_scale, out, workspace, workspace_bytes, stream, PagedKV{},
                                             false, bshd);
}
