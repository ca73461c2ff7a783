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
// all row-major.  A workgroup takes one (b,h) and a block of up to kRowsPerItem rows, so
// scale[h] is one scalar load; threads own fixed 16-element (nope) or 8-element (rope)
// column units, so every load and store is a 16-byte vector and a wave covers whole
// 128-byte lines.
#include "fa3q_internal.hpp"

namespace fa3q {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerItem = 128;
constexpr int kUnroll = 4;

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

__device__ __forceinline__ uint32_t code_byte(float x, float s, bool zero) {
  float y = x / s;  // correctly rounded float32 division
  y = rintf(y);     // round half to even
  y = fminf(fmaxf(y, -127.0f), 127.0f);
  const int c = zero ? 0 : static_cast<int>(y);
  return static_cast<uint32_t>(c) & 0xffu;
}

// 4 bf16 (two dwords) -> 4 int8 codes in one dword (little-endian element order).
__device__ __forceinline__ uint32_t quant4(uint32_t w0, uint32_t w1, float s, bool zero) {
  return code_byte(bf16_lo(w0), s, zero) | (code_byte(bf16_hi(w0), s, zero) << 8) |
         (code_byte(bf16_lo(w1), s, zero) << 16) | (code_byte(bf16_hi(w1), s, zero) << 24);
}

__global__ __launch_bounds__(kThreads) void quantize_k_kernel(QuantArgs a) {
  const int tid = static_cast<int>(threadIdx.x);
  const int Dk = a.Dn + a.Dr;
  const int Un = a.Dn >> 4;  // 16-wide nope units per row
  const int Ur = a.Dr >> 3;  // 8-wide rope units per row
  const int un = tid % Un, rn0 = tid / Un, rstep_n = kThreads / Un;
  const int ur = Ur ? tid % Ur : 0, rr0 = Ur ? tid / Ur : kThreads, rstep_r = Ur ? kThreads / Ur : 1;

  for (int64_t item = blockIdx.x; item < a.items; item += gridDim.x) {
    const int64_t bh = item / a.chunks_per_bh;
    const int64_t chunk = item - bh * a.chunks_per_bh;
    const float s = a.scale[bh % a.H];
    const bool zero = (s == 0.0f);
    const int64_t r_begin = chunk * kRowsPerItem;
    const int nr = static_cast<int>(min(static_cast<int64_t>(kRowsPerItem), a.S - r_begin));
    const int64_t row0 = bh * a.S + r_begin;
    const uint16_t* __restrict__ kin = a.k + row0 * Dk;
    int8_t* __restrict__ qout = a.kq + row0 * a.Dn;
    uint16_t* __restrict__ rout = a.kr + row0 * a.Dr;

    if (rn0 < rstep_n) {
      for (int rb = rn0; rb < nr; rb += rstep_n * kUnroll) {
        uint4 x0[kUnroll], x1[kUnroll];
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) {
          const int r = rb + j * rstep_n;
          if (r < nr) {
            const uint4* src = reinterpret_cast<const uint4*>(kin + static_cast<int64_t>(r) * Dk + un * 16);
            x0[j] = src[0];
            x1[j] = src[1];
          }
        }
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) {
          const int r = rb + j * rstep_n;
          if (r < nr) {
            uint4 o;
            o.x = quant4(x0[j].x, x0[j].y, s, zero);
            o.y = quant4(x0[j].z, x0[j].w, s, zero);
            o.z = quant4(x1[j].x, x1[j].y, s, zero);
            o.w = quant4(x1[j].z, x1[j].w, s, zero);
            *reinterpret_cast<uint4*>(qout + static_cast<int64_t>(r) * a.Dn + un * 16) = o;
          }
        }
      }
    }
    if (rr0 < rstep_r) {
      for (int rb = rr0; rb < nr; rb += rstep_r * kUnroll) {
        uint4 x[kUnroll];
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) {
          const int r = rb + j * rstep_r;
          if (r < nr)
            x[j] = *reinterpret_cast<const uint4*>(kin + static_cast<int64_t>(r) * Dk + a.Dn + ur * 8);
        }
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) {
          const int r = rb + j * rstep_r;
          if (r < nr) *reinterpret_cast<uint4*>(rout + static_cast<int64_t>(r) * a.Dr + ur * 8) = x[j];
        }
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
  hipLaunchKernelGGL(quantize_k_kernel, dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0,
                     as_stream(stream), a);
  return launch_status();
}
