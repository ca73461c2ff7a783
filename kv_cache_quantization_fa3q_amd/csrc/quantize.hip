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
#include "fa3q_internal.hpp"

namespace fa3q {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerItem = 64;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

struct QuantArgs {
  const uint16_t* k;
  const float* scale;
  int8_t* kq;
  uint16_t* kr;
  int64_t S;
  int64_t items;          // B*H*chunks_per_bh
  int32_t chunks_per_bh;  // ceil(S / kRowsPerItem)
  int32_t H;
  int32_t Dn;
  int32_t Dr;
};

__device__ __forceinline__ int code_exact(float x, float s) {
  const float y = __builtin_amdgcn_fmed3f(rintf(x / s), -127.0f, 127.0f);  // IEEE division
  return static_cast<int>(y);
}

// 8 bf16 (one 16-byte vector) -> 8 codes in two dwords (little-endian element order).
__device__ __forceinline__ u32x2 quant8(const u32x4& w, float s, float r, bool fast) {
  float xv[8];
  xv[0] = bf16_lo(w.x); xv[1] = bf16_hi(w.x); xv[2] = bf16_lo(w.y); xv[3] = bf16_hi(w.y);
  xv[4] = bf16_lo(w.z); xv[5] = bf16_hi(w.z); xv[6] = bf16_lo(w.w); xv[7] = bf16_hi(w.w);
  int c[8];
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
  u32x2 o;
  o.x = (c[0] & 0xff) | ((c[1] & 0xff) << 8) | ((c[2] & 0xff) << 16) | (static_cast<uint32_t>(c[3]) << 24);
  o.y = (c[4] & 0xff) | ((c[5] & 0xff) << 8) | ((c[6] & 0xff) << 16) | (static_cast<uint32_t>(c[7]) << 24);
  return o;
}

// UN / UR: 8-element units per nope / rope row when known at compile time (0: runtime).
template <int UN, int UR>
__global__ __launch_bounds__(kThreads) void quantize_k_kernel(QuantArgs a) {
  const int tid = static_cast<int>(threadIdx.x);
  const int Dk = a.Dn + a.Dr;
  const int Un = UN ? UN : a.Dn >> 3;
  const int Ur = UR ? UR : a.Dr >> 3;
  constexpr int kNope = UN ? kRowsPerItem * UN / kThreads : 4;  // nope vectors per thread per pass
  constexpr int kRope = UR ? (kRowsPerItem * UR + kThreads - 1) / kThreads : 2;

  for (int64_t item = blockIdx.x; item < a.items; item += gridDim.x) {
    const int64_t bh = item / a.chunks_per_bh;
    const int64_t chunk = item - bh * a.chunks_per_bh;
    const float s = a.scale[bh % a.H];
    const bool zero = (s == 0.0f);
    // fast quotient only for a moderate normal scale (1/s normal, x*(1/s) free of overflow)
    const bool fast = fabsf(s) >= 0x1p-100f && fabsf(s) <= 0x1p100f;
    const float r = 1.0f / s;
    const int64_t r_begin = chunk * kRowsPerItem;
    const int nr = static_cast<int>(min(static_cast<int64_t>(kRowsPerItem), a.S - r_begin));
    const int64_t row0 = bh * a.S + r_begin;
    const uint16_t* __restrict__ kin = a.k + row0 * Dk;
    int8_t* __restrict__ qout = a.kq + row0 * a.Dn;
    uint16_t* __restrict__ rout = a.kr + row0 * a.Dr;
    const int nn = nr * Un, nrp = nr * Ur;

    for (int pass = 0; pass * kThreads * kNope < nn || pass * kThreads * kRope < nrp; ++pass) {
      u32x4 xn[kNope], xr[kRope];
      int on[kNope], orr[kRope];
#pragma unroll
      for (int j = 0; j < kNope; ++j) {
        const int q = (pass * kNope + j) * kThreads + tid;
        const int row = q / Un, unit = q - row * Un;
        on[j] = q < nn ? row * a.Dn + unit * 8 : -1;
        if (q < nn) xn[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kin + static_cast<int64_t>(row) * Dk + unit * 8));
      }
      if (Ur > 0) {
#pragma unroll
        for (int j = 0; j < kRope; ++j) {
          const int q = (pass * kRope + j) * kThreads + tid;
          const int row = q / Ur, unit = q - row * Ur;
          orr[j] = q < nrp ? row * a.Dr + unit * 8 : -1;
          if (q < nrp)
            xr[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kin + static_cast<int64_t>(row) * Dk + a.Dn + unit * 8));
        }
      }
#pragma unroll
      for (int j = 0; j < kNope; ++j) {
        if (on[j] >= 0) {
          const u32x2 o = zero ? u32x2{0u, 0u} : quant8(xn[j], s, r, fast);
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

extern "C" int fa3q_quantize_k(const uint16_t* k, const float* scale, int8_t* k_nope_q,
                               uint16_t* k_rope, int64_t B, int64_t H, int64_t S, int64_t Dn,
                               int64_t Dr, void* stream) {
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
  a.chunks_per_bh = static_cast<int32_t>(chunks);
  a.items = B * H * chunks;
  a.H = static_cast<int32_t>(H);
  a.Dn = static_cast<int32_t>(Dn);
  a.Dr = static_cast<int32_t>(Dr);
  const int64_t grid = std::min<int64_t>(a.items, static_cast<int64_t>(device_cu_count()) * 8);
  const dim3 g(static_cast<unsigned>(grid)), blk(kThreads);
  if (Dn == 128 && Dr == 64)
    hipLaunchKernelGGL((quantize_k_kernel<16, 8>), g, blk, 0, as_stream(stream), a);
  else
    hipLaunchKernelGGL((quantize_k_kernel<0, 0>), g, blk, 0, as_stream(stream), a);
  return launch_status();
}
