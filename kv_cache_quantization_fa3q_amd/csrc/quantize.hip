// K-cache quantisation: non-RoPE part of K -> per-head symmetric INT8, RoPE part kept in bf16.
//
// MindIE LLM page "FA3 quantization", overview: only the non-RoPE slice of K is quantised
// to 8 bits, per head; the RoPE slice of K is left as it is.  msModelSlim page "FA3量化",
// section 适用要求: symmetric INT8 only, with scale[h] = abs_max[h] / 127 (section 算法流程).
//
// code = clamp(round_half_even(fl32(x / scale[h])), -127, 127); 0 for a head with scale 0.
//
// Pure streaming: per (token, head) row the kernel reads (Dn + Dr) bf16 and writes Dn int8
// plus Dr bf16.  Layout in HBM: k (B,H,S,Dn+Dr), k_nope_q (B,H,S,Dn), k_rope (B,H,S,Dr),
// all row-major.  A work item is one (b,h) and a block of up to kRowsPerItem rows, so
// scale[h] is one scalar load.  Every thread moves whole 16-byte vectors of 8 elements;
// consecutive lanes take consecutive vectors of a row part, so each load instruction of a
// wave covers whole 128-byte lines (16 lanes per 256-byte nope row, 8 per 128-byte rope
// row) and the 8-byte code stores of a row are contiguous.  Loads and stores carry the
// nontemporal hint: every byte is touched once.
//
// The quotient: with r = fl32(1/s) and y = fl32(x*r), |y - x/s| <= |x/s| * 2^-23 (1 + 2^-25),
// at most 1.53e-5 below 128, and the IEEE quotient fl32(x/s) is within half an ulp (7.6e-6)
// of x/s.  So rint(y) equals rint(fl32(x/s)) unless y lies within 2.3e-5 of a half-integer;
// such elements (and every element of a head whose scale is not a moderate normal number)
// take the correctly rounded division.  Above 127.5 both clamp to 127.
//
// Asymmetric variant (fa3q_quantize_asym).  MindIE Turbo page "Attention量化", tables 1
// and 2: the K activation carries a scale and an offset per (head, dim), stored as float16
// or bfloat16; the pages give no formula, so the plain asymmetric INT8 code is used:
//   code = clamp(round_half_even(fl32(fl32(x / s[h,d]) + o[h,d])), -128, 127),
// 0 for a channel whose scale is 0, the value of a code being (code - o) * s.  Same
// streaming layout and item shape; each lane also holds the 8 scales, reciprocals and
// offsets of the dims it covers.  The quotient: with r = v_rcp(s) (at most 1 ulp off 1/s)
// and y' = x*r, |y' - fl32(x/s)| <= |y'| * 2^-22 (1 + 2^-20); both sums are rounded to
// float32 below 256 with an ulp of at most 2^-16, so the two codes agree unless z' = y' + o
// lies within |y'| * 2^-20 + 2^-15 of a half-integer (checked; the correctly rounded
// division then decides), and for |z'| >= 200 both saturate the same way while |y'| <= 2^24
// (the margin check sends larger |y'| to the division).  A scale outside [2^-100, 2^100]
// sends its channel to the division too.
#include "fa3q_internal.hpp"

namespace fa3q {
namespace {

// One single-wave workgroup per item of 16 rows, a grid of all items.  On MI355X that
// streams this read+write mix about 15% faster than a grid-stride loop over a few
// workgroups per CU (3.6 ms against 4.1-4.4 ms for the (64,128,4096,128+64) K); 64 to
// 512 threads with 16 to 128 rows per item all measured within 6% of each other.  The
// item loop remains for grids past the cap.
constexpr int kThreads = 64;
constexpr int kRowsPerItem = 16;
constexpr int64_t kMaxGrid = int64_t{1} << 30;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

struct QuantArgs {
  const uint16_t* k;
  const float* scale;
  int8_t* kq;
  uint16_t* kr;
  int64_t S;
  int64_t rows;           // B*S*H (token-major items)
  int64_t items;          // B*H*chunks_per_bh, or ceil(rows / kRowsPerItem) (token-major)
  int32_t chunks_per_bh;  // ceil(S / kRowsPerItem)
  int32_t H;
  int32_t Dn;
  int32_t Dr;
};

__device__ __forceinline__ int code_exact(float x, float s) {
  const float y = __builtin_amdgcn_fmed3f(rintf(x / s), -127.0f, 127.0f);  // IEEE division
  return static_cast<int>(y);
}

// 8 bf16 (kF16: float16) values, one 16-byte vector -> their 8 codes.
template <bool kF16 = false>
__device__ __forceinline__ void codes8(const u32x4& w, float s, float r, bool fast, int (&c)[8]) {
  float xv[8];
  xv[0] = lo16<kF16>(w.x); xv[1] = hi16<kF16>(w.x); xv[2] = lo16<kF16>(w.y); xv[3] = hi16<kF16>(w.y);
  xv[4] = lo16<kF16>(w.z); xv[5] = hi16<kF16>(w.z); xv[6] = lo16<kF16>(w.w); xv[7] = hi16<kF16>(w.w);
  bool amb = !fast;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float y = xv[i] * r;
    const float n = rintf(y);
    amb |= fabsf(y - n) > 0.5f - 0x1p-14f;
    c[i] = static_cast<int>(__builtin_amdgcn_fmed3f(n, -127.0f, 127.0f));
  }
  if (__ballot(amb) != 0) {
    if (amb) {
#pragma unroll
      for (int i = 0; i < 8; ++i) c[i] = code_exact(xv[i], s);
    }
  }
}

// 8 bf16 (kF16: float16) -> 8 codes in two dwords (little-endian element order).
template <bool kF16>
__device__ __forceinline__ u32x2 quant8(const u32x4& w, float s, float r, bool fast) {
  int c[8];
  codes8<kF16>(w, s, r, fast, c);
  u32x2 o;
  o.x = (c[0] & 0xff) | ((c[1] & 0xff) << 8) | ((c[2] & 0xff) << 16) | (static_cast<uint32_t>(c[3]) << 24);
  o.y = (c[4] & 0xff) | ((c[5] & 0xff) << 8) | ((c[6] & 0xff) << 16) | (static_cast<uint32_t>(c[7]) << 24);
  return o;
}

// 8 bf16 -> the bf16 values of their codes: round_half_even_to_bf16(fl32(code * s)).
__device__ __forceinline__ u32x4 fake8(const u32x4& w, float s, float r, bool fast) {
  int c[8];
  codes8(w, s, r, fast, c);
  uint32_t h[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(__fmul_rn(static_cast<float>(c[i]), s)));
  return u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
}

// Quotient parameters of one head's scale: the reciprocal, whether the fast quotient
// applies (a moderate normal scale: 1/s normal, x*(1/s) free of overflow), and a zero scale.
struct HeadQ {
  float s, r;
  bool fast, zero;
};

__device__ __forceinline__ HeadQ head_q(float s) {
  return HeadQ{s, 1.0f / s, fabsf(s) >= 0x1p-100f && fabsf(s) <= 0x1p100f, s == 0.0f};
}

// UN / UR: 8-element units per nope / rope row when known at compile time (0: runtime).
// kF16: float16 K (the RoPE copy is float16 too), else bf16.  kTok: (B,S,H,Dn+Dr) rows; an
// item is kRowsPerItem consecutive rows, row g belonging to head g % H, so every vector
// carries its own head's scale.  Otherwise (B,H,S,.) rows; an item is a run of rows of one
// (b, h) and the scale one scalar.
template <int UN, int UR, bool kF16, bool kTok>
__global__ __launch_bounds__(kThreads) void quantize_k_kernel(QuantArgs a) {
  const int tid = static_cast<int>(threadIdx.x);
  const int Dk = a.Dn + a.Dr;
  const int Un = UN ? UN : a.Dn >> 3;
  const int Ur = UR ? UR : a.Dr >> 3;
  constexpr int kNope = UN ? kRowsPerItem * UN / kThreads : 4;  // nope vectors per thread per pass
  constexpr int kRope = UR ? (kRowsPerItem * UR + kThreads - 1) / kThreads : 2;

  for (int64_t item = blockIdx.x; item < a.items; item += gridDim.x) {
    int64_t row0;
    int nr, hh;
    if constexpr (kTok) {
      row0 = item * kRowsPerItem;
      nr = static_cast<int>(min(static_cast<int64_t>(kRowsPerItem), a.rows - row0));
      hh = __builtin_amdgcn_readfirstlane(static_cast<int>(row0 % a.H));  // head of the item's first row
    } else {
      const int64_t bh = item / a.chunks_per_bh;
      const int64_t chunk = item - bh * a.chunks_per_bh;
      hh = __builtin_amdgcn_readfirstlane(static_cast<int>(bh % a.H));  // uniform: scalar read
      const int64_t r_begin = chunk * kRowsPerItem;
      nr = static_cast<int>(min(static_cast<int64_t>(kRowsPerItem), a.S - r_begin));
      row0 = bh * a.S + r_begin;
    }
    const uint16_t* __restrict__ kin = a.k + row0 * Dk;
    int8_t* __restrict__ qout = a.kq + row0 * a.Dn;
    uint16_t* __restrict__ rout = a.kr + row0 * a.Dr;
    const int nn = nr * Un, nrp = nr * Ur;

    for (int pass = 0; pass * kThreads * kNope < nn || pass * kThreads * kRope < nrp; ++pass) {
      u32x4 xn[kNope], xr[kRope];
      int on[kNope], orr[kRope];
      int rv[kNope];  // token-major: each nope vector's row in the item
      // Loads are unconditional (a vector past the item's end re-reads its last vector and is
      // not stored), so they issue back to back instead of one exec-masked block at a time.
#pragma unroll
      for (int j = 0; j < kNope; ++j) {
        const int q = (pass * kNope + j) * kThreads + tid;
        const int qc = min(q, nn - 1);
        const int row = qc / Un, unit = qc - row * Un;
        on[j] = q < nn ? row * a.Dn + unit * 8 : -1;
        rv[j] = row;
        xn[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kin + static_cast<int64_t>(row) * Dk + unit * 8));
      }
      if (Ur > 0) {
#pragma unroll
        for (int j = 0; j < kRope; ++j) {
          const int q = (pass * kRope + j) * kThreads + tid;
          const int qc = min(q, nrp - 1);
          const int row = qc / Ur, unit = qc - row * Ur;
          orr[j] = q < nrp ? row * a.Dr + unit * 8 : -1;
          xr[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kin + static_cast<int64_t>(row) * Dk + a.Dn + unit * 8));
        }
      }
      // the scales are read after the data loads are issued, so their latency hides behind theirs
      if constexpr (kTok) {
        // lane l < kRowsPerItem takes row l's head (rows of one item are consecutive, row g of
        // head g % H): one scale load and one reciprocal per lane, which each vector then
        // fetches from its row's lane
        const int hr = hh + (tid & (kRowsPerItem - 1));  // < H + kRowsPerItem
        const float s_row = a.scale[hr < a.H ? hr : hr % a.H];
        const float r_row = 1.0f / s_row;
#pragma unroll
        for (int j = 0; j < kNope; ++j) {
          if (on[j] >= 0) {
            const float sj = __shfl(s_row, rv[j]);
            const float rj = __shfl(r_row, rv[j]);
            const bool fast = fabsf(sj) >= 0x1p-100f && fabsf(sj) <= 0x1p100f;  // as head_q
            const u32x2 o = sj == 0.0f ? u32x2{0u, 0u} : quant8<kF16>(xn[j], sj, rj, fast);
            __builtin_nontemporal_store(o, reinterpret_cast<u32x2*>(qout + on[j]));
          }
        }
      } else {
        const HeadQ hq = head_q(a.scale[hh]);
#pragma unroll
        for (int j = 0; j < kNope; ++j) {
          if (on[j] >= 0) {
            const u32x2 o = hq.zero ? u32x2{0u, 0u} : quant8<kF16>(xn[j], hq.s, hq.r, hq.fast);
            __builtin_nontemporal_store(o, reinterpret_cast<u32x2*>(qout + on[j]));
          }
        }
      }
      if (Ur > 0) {
#pragma unroll
        for (int j = 0; j < kRope; ++j)
          if (orr[j] >= 0) __builtin_nontemporal_store(xr[j], reinterpret_cast<u32x4*>(rout + orr[j]));
      }
    }
  }
}

struct FakeArgs {
  const uint16_t* x;
  const float* scale;
  uint16_t* y;
  int64_t S;
  int64_t items;
  int32_t chunks_per_bh;
  int32_t H;
  int32_t Dn;
  int32_t Dr;
  int32_t copy_rope;  // 0 when y is x: the RoPE part is already in place
};

// Fake quantisation: the same items, loads and code decision as quantize_k_kernel; the
// codes are turned back into bf16 values (scale[h] * code) and written over a copy of the
// row layout, the RoPE part copied unchanged.
template <int UN, int UR>
__global__ __launch_bounds__(kThreads) void fake_quant_kernel(FakeArgs a) {
  const int tid = static_cast<int>(threadIdx.x);
  const int Dk = a.Dn + a.Dr;
  const int Un = UN ? UN : a.Dn >> 3;
  const int Ur = a.copy_rope ? (UR ? UR : a.Dr >> 3) : 0;
  constexpr int kNope = UN ? kRowsPerItem * UN / kThreads : 4;
  constexpr int kRope = UR ? (kRowsPerItem * UR + kThreads - 1) / kThreads : 2;

  for (int64_t item = blockIdx.x; item < a.items; item += gridDim.x) {
    const int64_t bh = item / a.chunks_per_bh;
    const int64_t chunk = item - bh * a.chunks_per_bh;
    const int hh = __builtin_amdgcn_readfirstlane(static_cast<int>(bh % a.H));
    const int64_t r_begin = chunk * kRowsPerItem;
    const int nr = static_cast<int>(min(static_cast<int64_t>(kRowsPerItem), a.S - r_begin));
    const int64_t row0 = bh * a.S + r_begin;
    const uint16_t* xin = a.x + row0 * Dk;  // may be the same memory as yout (in place)
    uint16_t* yout = a.y + row0 * Dk;
    const int nn = nr * Un, nrp = nr * Ur;

    for (int pass = 0; pass * kThreads * kNope < nn || pass * kThreads * kRope < nrp; ++pass) {
      u32x4 xn[kNope], xr[kRope];
      int on[kNope], orr[kRope];
#pragma unroll
      for (int j = 0; j < kNope; ++j) {
        const int q = (pass * kNope + j) * kThreads + tid;
        const int qc = min(q, nn - 1);
        const int row = qc / Un, unit = qc - row * Un;
        on[j] = q < nn ? row * Dk + unit * 8 : -1;
        xn[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(xin + static_cast<int64_t>(row) * Dk + unit * 8));
      }
      if (Ur > 0) {
#pragma unroll
        for (int j = 0; j < kRope; ++j) {
          const int q = (pass * kRope + j) * kThreads + tid;
          const int qc = min(q, nrp - 1);
          const int row = qc / Ur, unit = qc - row * Ur;
          orr[j] = q < nrp ? row * Dk + a.Dn + unit * 8 : -1;
          xr[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(xin + static_cast<int64_t>(row) * Dk + a.Dn + unit * 8));
        }
      }
      const float s = a.scale[hh];
      const bool zero = (s == 0.0f);
      const bool fast = fabsf(s) >= 0x1p-100f && fabsf(s) <= 0x1p100f;
      const float r = 1.0f / s;
#pragma unroll
      for (int j = 0; j < kNope; ++j) {
        if (on[j] >= 0) {
          const u32x4 o = zero ? u32x4{0u, 0u, 0u, 0u} : fake8(xn[j], s, r, fast);
          __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(yout + on[j]));
        }
      }
      if (Ur > 0) {
#pragma unroll
        for (int j = 0; j < kRope; ++j)
          if (orr[j] >= 0) __builtin_nontemporal_store(xr[j], reinterpret_cast<u32x4*>(yout + orr[j]));
      }
    }
  }
}

struct AsymArgs {
  const uint16_t* k;
  const uint16_t* scale;   // [H][Dn] bf16 or float16 patterns
  const uint16_t* offset;  // [H][Dn]
  int8_t* kq;
  uint16_t* kr;
  int64_t S;
  int64_t items;
  int32_t chunks_per_bh;
  int32_t H;
  int32_t Dn;
  int32_t Dr;
  int32_t f16;  // 1: float16 tables, 0: bfloat16
};

__device__ __forceinline__ float param_value(uint32_t bits16, bool f16) {
  return f16 ? static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16)))
             : __uint_as_float(bits16 << 16);
}

// The 8 channels of one 16-byte unit: scale, fast-path reciprocal (NaN for a scale the fast
// path does not take, which forces the division) and offset.
struct AsymUnit {
  float s[8], r[8], o[8];
};

__device__ __forceinline__ AsymUnit load_asym_unit(const uint16_t* scale, const uint16_t* offset, bool f16) {
  const u32x4 sw = *reinterpret_cast<const u32x4*>(scale);
  const u32x4 ow = *reinterpret_cast<const u32x4*>(offset);
  const uint32_t sv[4] = {sw.x, sw.y, sw.z, sw.w}, ov[4] = {ow.x, ow.y, ow.z, ow.w};
  AsymUnit u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    u.s[2 * i] = param_value(sv[i] & 0xffffu, f16);
    u.s[2 * i + 1] = param_value(sv[i] >> 16, f16);
    u.o[2 * i] = param_value(ov[i] & 0xffffu, f16);
    u.o[2 * i + 1] = param_value(ov[i] >> 16, f16);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float m = fabsf(u.s[i]);
    u.r[i] = (m >= 0x1p-100f && m <= 0x1p100f) ? __builtin_amdgcn_rcpf(u.s[i]) : __builtin_nanf("");
  }
  return u;
}

__device__ __forceinline__ int asym_code_exact(float x, float s, float o) {
  if (s == 0.0f) return 0;
  const float z = x / s + o;  // IEEE division, then one float32 addition
  return static_cast<int>(__builtin_amdgcn_fmed3f(rintf(z), -128.0f, 127.0f));
}

__device__ __forceinline__ u32x2 quant8_asym(const u32x4& w, const AsymUnit& p) {
  float xv[8];
  xv[0] = bf16_lo(w.x); xv[1] = bf16_hi(w.x); xv[2] = bf16_lo(w.y); xv[3] = bf16_hi(w.y);
  xv[4] = bf16_lo(w.z); xv[5] = bf16_hi(w.z); xv[6] = bf16_lo(w.w); xv[7] = bf16_hi(w.w);
  int c[8];
  bool amb = false;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float y = __fmul_rn(xv[i], p.r[i]);
    const float z = __fadd_rn(y, p.o[i]);
    const float n = rintf(z);
    const float thr = fmaf(-fabsf(y), 0x1p-20f, 0.5f - 0x1p-15f);
    amb |= !(fabsf(z - n) <= thr);  // NaN anywhere (skipped scale, non-finite input) -> division
    c[i] = static_cast<int>(__builtin_amdgcn_fmed3f(n, -128.0f, 127.0f));
  }
  if (__ballot(amb) != 0) {
    if (amb) {
#pragma unroll
      for (int i = 0; i < 8; ++i) c[i] = asym_code_exact(xv[i], p.s[i], p.o[i]);
    }
  }
  u32x2 o;
  o.x = (c[0] & 0xff) | ((c[1] & 0xff) << 8) | ((c[2] & 0xff) << 16) | (static_cast<uint32_t>(c[3]) << 24);
  o.y = (c[4] & 0xff) | ((c[5] & 0xff) << 8) | ((c[6] & 0xff) << 16) | (static_cast<uint32_t>(c[7]) << 24);
  return o;
}

// UN / UR as in quantize_k_kernel.  When UN divides the block size every nope vector of a
// lane lies in the same unit (q % UN == tid % UN), so the lane loads its 8 channels' tables
// once per item; otherwise per vector.
template <int UN, int UR>
__global__ __launch_bounds__(kThreads) void quantize_asym_kernel(AsymArgs a) {
  const int tid = static_cast<int>(threadIdx.x);
  const int Dk = a.Dn + a.Dr;
  const int Un = UN ? UN : a.Dn >> 3;
  const int Ur = UR ? UR : a.Dr >> 3;
  constexpr bool kFixedUnit = UN != 0 && kThreads % UN == 0;
  constexpr int kNope = UN ? kRowsPerItem * UN / kThreads : 4;
  constexpr int kRope = UR ? (kRowsPerItem * UR + kThreads - 1) / kThreads : 2;
  const bool f16 = a.f16 != 0;

  for (int64_t item = blockIdx.x; item < a.items; item += gridDim.x) {
    const int64_t bh = item / a.chunks_per_bh;
    const int64_t chunk = item - bh * a.chunks_per_bh;
    const int64_t h = bh % a.H;
    const uint16_t* stab = a.scale + h * a.Dn;
    const uint16_t* otab = a.offset + h * a.Dn;
    const int64_t r_begin = chunk * kRowsPerItem;
    const int nr = static_cast<int>(min(static_cast<int64_t>(kRowsPerItem), a.S - r_begin));
    const int64_t row0 = bh * a.S + r_begin;
    const uint16_t* __restrict__ kin = a.k + row0 * Dk;
    int8_t* __restrict__ qout = a.kq + row0 * a.Dn;
    uint16_t* __restrict__ rout = a.kr + row0 * a.Dr;
    const int nn = nr * Un, nrp = nr * Ur;

    for (int pass = 0; pass * kThreads * kNope < nn || pass * kThreads * kRope < nrp; ++pass) {
      u32x4 xn[kNope], xr[kRope];
      int on[kNope], un[kNope], orr[kRope];
      // Loads are unconditional (a vector past the item's end re-reads its last vector and is
      // not stored), so they issue back to back instead of one exec-masked block at a time.
#pragma unroll
      for (int j = 0; j < kNope; ++j) {
        const int q = (pass * kNope + j) * kThreads + tid;
        const int qc = min(q, nn - 1);
        const int row = qc / Un, unit = qc - row * Un;
        on[j] = q < nn ? row * a.Dn + unit * 8 : -1;
        un[j] = unit;
        xn[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kin + static_cast<int64_t>(row) * Dk + unit * 8));
      }
      if (Ur > 0) {
#pragma unroll
        for (int j = 0; j < kRope; ++j) {
          const int q = (pass * kRope + j) * kThreads + tid;
          const int qc = min(q, nrp - 1);
          const int row = qc / Ur, unit = qc - row * Ur;
          orr[j] = q < nrp ? row * a.Dr + unit * 8 : -1;
          xr[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kin + static_cast<int64_t>(row) * Dk + a.Dn + unit * 8));
        }
      }
      // tables after the data loads (their latency hides behind the data's)
      AsymUnit fixed;
      if constexpr (kFixedUnit) fixed = load_asym_unit(stab + (tid % UN) * 8, otab + (tid % UN) * 8, f16);
#pragma unroll
      for (int j = 0; j < kNope; ++j) {
        if (on[j] >= 0) {
          u32x2 o;
          if constexpr (kFixedUnit) {
            o = quant8_asym(xn[j], fixed);
          } else {
            const AsymUnit p = load_asym_unit(stab + un[j] * 8, otab + un[j] * 8, f16);
            o = quant8_asym(xn[j], p);
          }
          __builtin_nontemporal_store(o, reinterpret_cast<u32x2*>(qout + on[j]));
        }
      }
      if (Ur > 0) {
#pragma unroll
        for (int j = 0; j < kRope; ++j)
          if (orr[j] >= 0) __builtin_nontemporal_store(xr[j], reinterpret_cast<u32x4*>(rout + orr[j]));
      }
    }
  }
}

}  // namespace
}  // namespace fa3q

using namespace fa3q;

namespace fa3q {
namespace {

template <bool kF16, bool kTok>
void launch_quantize_k(const QuantArgs& a, dim3 g, hipStream_t s) {
  if (a.Dn == 128 && a.Dr == 64)
    hipLaunchKernelGGL((quantize_k_kernel<16, 8, kF16, kTok>), g, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((quantize_k_kernel<0, 0, kF16, kTok>), g, dim3(kThreads), 0, s, a);
}

int quantize_k(const uint16_t* k, const float* scale, int8_t* k_nope_q, uint16_t* k_rope, bool f16, bool tok,
               int64_t B, int64_t H, int64_t S, int64_t Dn, int64_t Dr, void* stream) {
  if (!k || !scale || !k_nope_q || (Dr > 0 && !k_rope)) return FA3Q_ERR_NULL;
  if (B <= 0 || H <= 0 || S <= 0) return FA3Q_ERR_SHAPE;
  if (Dn <= 0 || Dn % 16 != 0 || Dn > 4096) return FA3Q_ERR_SHAPE;
  if (Dr < 0 || Dr % 8 != 0 || Dr > 2048) return FA3Q_ERR_SHAPE;
  if (B > (int64_t{1} << 31) / H) return FA3Q_ERR_SHAPE;
  const int64_t chunks = (S + kRowsPerItem - 1) / kRowsPerItem;
  if (chunks > (int64_t{1} << 30) || B * H > (int64_t{1} << 62) / (chunks * kRowsPerItem * (Dn + Dr)))
    return FA3Q_ERR_SHAPE;
  if (!is_aligned(k, 16) || !is_aligned(k_nope_q, 16) || (Dr > 0 && !is_aligned(k_rope, 16)) ||
      !is_aligned(scale, 4))
    return FA3Q_ERR_ALIGN;

  QuantArgs a;
  a.k = k;
  a.scale = scale;
  a.kq = k_nope_q;
  a.kr = k_rope;
  a.S = S;
  a.rows = B * S * H;
  a.chunks_per_bh = static_cast<int32_t>(chunks);
  a.items = tok ? (a.rows + kRowsPerItem - 1) / kRowsPerItem : B * H * chunks;
  a.H = static_cast<int32_t>(H);
  a.Dn = static_cast<int32_t>(Dn);
  a.Dr = static_cast<int32_t>(Dr);
  const dim3 g(static_cast<unsigned>(std::min<int64_t>(a.items, kMaxGrid)));
  hipStream_t s = as_stream(stream);
  if (f16) {
    if (tok) launch_quantize_k<true, true>(a, g, s);
    else launch_quantize_k<true, false>(a, g, s);
  } else {
    if (tok) launch_quantize_k<false, true>(a, g, s);
    else launch_quantize_k<false, false>(a, g, s);
  }
  return launch_status();
}

}  // namespace
}  // namespace fa3q

extern "C" int fa3q_quantize_k(const uint16_t* k, const float* scale, int8_t* k_nope_q,
                               uint16_t* k_rope, int64_t B, int64_t H, int64_t S, int64_t Dn,
                               int64_t Dr, void* stream) {
  return quantize_k(k, scale, k_nope_q, k_rope, false, false, B, H, S, Dn, Dr, stream);
}

extern "C" int fa3q_quantize_k_ex(const void* k, const float* scale, int8_t* k_nope_q, void* k_rope, int dtype,
                                  int layout, int64_t B, int64_t H, int64_t S, int64_t Dn, int64_t Dr, void* stream) {
  if (dtype != FA3Q_BF16 && dtype != FA3Q_F16) return FA3Q_ERR_DTYPE;
  if (layout != FA3Q_BHSD && layout != FA3Q_BSHD) return FA3Q_ERR_LAYOUT;
  return quantize_k(static_cast<const uint16_t*>(k), scale, k_nope_q, static_cast<uint16_t*>(k_rope),
                    dtype == FA3Q_F16, layout == FA3Q_BSHD, B, H, S, Dn, Dr, stream);
}

extern "C" int fa3q_fake_quant(const uint16_t* x, const float* scale, uint16_t* y, int64_t B, int64_t H,
                               int64_t S, int64_t Dn, int64_t Dr, void* stream) {
  if (!x || !scale || !y) return FA3Q_ERR_NULL;
  if (B <= 0 || H <= 0 || S <= 0) return FA3Q_ERR_SHAPE;
  if (Dn <= 0 || Dn % 16 != 0 || Dn > 4096) return FA3Q_ERR_SHAPE;
  if (Dr < 0 || Dr % 8 != 0 || Dr > 2048) return FA3Q_ERR_SHAPE;
  if (B > (int64_t{1} << 31) / H) return FA3Q_ERR_SHAPE;
  const int64_t chunks = (S + kRowsPerItem - 1) / kRowsPerItem;
  if (chunks > (int64_t{1} << 30) || B * H > (int64_t{1} << 62) / (chunks * kRowsPerItem * (Dn + Dr)))
    return FA3Q_ERR_SHAPE;
  if (!is_aligned(x, 16) || !is_aligned(y, 16) || !is_aligned(scale, 4)) return FA3Q_ERR_ALIGN;
  // y is x (in place) or does not overlap it
  const size_t bytes = static_cast<size_t>(B * H * S * (Dn + Dr)) * 2;
  const uintptr_t xb = reinterpret_cast<uintptr_t>(x), yb = reinterpret_cast<uintptr_t>(y);
  if (xb != yb && xb < yb + bytes && yb < xb + bytes) return FA3Q_ERR_ALIAS;

  FakeArgs a;
  a.x = x;
  a.scale = scale;
  a.y = y;
  a.S = S;
  a.chunks_per_bh = static_cast<int32_t>(chunks);
  a.items = B * H * chunks;
  a.H = static_cast<int32_t>(H);
  a.Dn = static_cast<int32_t>(Dn);
  a.Dr = static_cast<int32_t>(Dr);
  a.copy_rope = xb != yb ? 1 : 0;
  const int64_t grid = std::min<int64_t>(a.items, kMaxGrid);
  const dim3 g(static_cast<unsigned>(grid)), blk(kThreads);
  if (Dn == 128 && Dr == 64)
    hipLaunchKernelGGL((fake_quant_kernel<16, 8>), g, blk, 0, as_stream(stream), a);
  else
    hipLaunchKernelGGL((fake_quant_kernel<0, 0>), g, blk, 0, as_stream(stream), a);
  return launch_status();
}

extern "C" int fa3q_quantize_asym(const uint16_t* k, const uint16_t* scale, const uint16_t* offset,
                                  int params_dtype, int8_t* k_nope_q, uint16_t* k_rope, int64_t B,
                                  int64_t H, int64_t S, int64_t Dn, int64_t Dr, void* stream) {
  if (!k || !scale || !offset || !k_nope_q || (Dr > 0 && !k_rope)) return FA3Q_ERR_NULL;
  if (params_dtype != FA3Q_BF16 && params_dtype != FA3Q_F16) return FA3Q_ERR_DTYPE;
  if (B <= 0 || H <= 0 || S <= 0) return FA3Q_ERR_SHAPE;
  if (Dn <= 0 || Dn % 16 != 0 || Dn > 4096) return FA3Q_ERR_SHAPE;
  if (Dr < 0 || Dr % 8 != 0 || Dr > 2048) return FA3Q_ERR_SHAPE;
  if (B > (int64_t{1} << 31) / H) return FA3Q_ERR_SHAPE;
  const int64_t chunks = (S + kRowsPerItem - 1) / kRowsPerItem;
  if (chunks > (int64_t{1} << 30) || B * H > (int64_t{1} << 62) / (chunks * kRowsPerItem * (Dn + Dr)))
    return FA3Q_ERR_SHAPE;
  if (!is_aligned(k, 16) || !is_aligned(k_nope_q, 16) || (Dr > 0 && !is_aligned(k_rope, 16)) ||
      !is_aligned(scale, 16) || !is_aligned(offset, 16))
    return FA3Q_ERR_ALIGN;

  AsymArgs a;
  a.k = k;
  a.scale = scale;
  a.offset = offset;
  a.kq = k_nope_q;
  a.kr = k_rope;
  a.S = S;
  a.chunks_per_bh = static_cast<int32_t>(chunks);
  a.items = B * H * chunks;
  a.H = static_cast<int32_t>(H);
  a.Dn = static_cast<int32_t>(Dn);
  a.Dr = static_cast<int32_t>(Dr);
  a.f16 = params_dtype == FA3Q_F16 ? 1 : 0;
  const int64_t grid = std::min<int64_t>(a.items, kMaxGrid);
  const dim3 g(static_cast<unsigned>(grid)), blk(kThreads);
  if (Dn == 128 && Dr == 64)
    hipLaunchKernelGGL((quantize_asym_kernel<16, 8>), g, blk, 0, as_stream(stream), a);
  else
    hipLaunchKernelGGL((quantize_asym_kernel<0, 0>), g, blk, 0, as_stream(stream), a);
  return launch_status();
}
