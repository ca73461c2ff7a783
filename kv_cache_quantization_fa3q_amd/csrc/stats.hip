// Cross-batch accumulation and symmetric per-head scale.
//
// msModelSlim page "FA3量化：Flash Attention 3激活量化算法说明", section 原理 -> 算法流程:
// every calibration batch yields a per-head window; the running statistics keep the
// smallest window minimum and the largest window maximum seen so far, and the
// quantisation parameter of head h is abs_max[h] / 127 with
// abs_max[h] = max(|min_values[h]|, |max_values[h]|) (symmetric INT8, section 适用要求).
// These are H-element operations; one small launch each.
#include "fa3q_internal.hpp"

namespace fa3q {
namespace {

// Unsigned key whose order is the float32 total order with -0.0 below +0.0.
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__global__ __launch_bounds__(256) void init_minmax_kernel(float* __restrict__ run_min,
                                                          float* __restrict__ run_max, int64_t H) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < H) {
    run_min[i] = __uint_as_float(0x7f800000u);  // +inf
    run_max[i] = __uint_as_float(0xff800000u);  // -inf
  }
}

__global__ __launch_bounds__(256) void accumulate_kernel(float* __restrict__ run_min,
                                                         float* __restrict__ run_max,
                                                         const float* __restrict__ cur_min,
                                                         const float* __restrict__ cur_max,
                                                         int64_t H) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < H) {
    const float a = run_min[i], b = cur_min[i];
    const float c = run_max[i], d = cur_max[i];
    run_min[i] = order_key(b) < order_key(a) ? b : a;
    run_max[i] = order_key(d) > order_key(c) ? d : c;
  }
}

__global__ __launch_bounds__(256) void qparams_kernel(const float* __restrict__ run_min,
                                                      const float* __restrict__ run_max,
                                                      float* __restrict__ scale, int64_t H) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < H) {
    const float abs_max = fmaxf(fabsf(run_min[i]), fabsf(run_max[i]));
    scale[i] = abs_max / 127.0f;  // IEEE correctly rounded division (no fast-math in this build)
  }
}

inline unsigned blocks_for(int64_t H) { return static_cast<unsigned>((H + 255) / 256); }

}  // namespace
}  // namespace fa3q

using namespace fa3q;

extern "C" int fa3q_init_minmax(float* run_min, float* run_max, int64_t H, void* stream) {
  if (!run_min || !run_max) return FA3Q_ERR_NULL;
  if (H <= 0 || H > (int64_t{1} << 31)) return FA3Q_ERR_SHAPE;
  if (!is_aligned(run_min, 4) || !is_aligned(run_max, 4)) return FA3Q_ERR_ALIGN;
  hipLaunchKernelGGL(init_minmax_kernel, dim3(blocks_for(H)), dim3(256), 0, as_stream(stream),
                     run_min, run_max, H);
  return launch_status();
}

extern "C" int fa3q_accumulate_minmax(float* run_min, float* run_max, const float* cur_min,
                                      const float* cur_max, int64_t H, void* stream) {
  if (!run_min || !run_max || !cur_min || !cur_max) return FA3Q_ERR_NULL;
  if (H <= 0 || H > (int64_t{1} << 31)) return FA3Q_ERR_SHAPE;
  if (!is_aligned(run_min, 4) || !is_aligned(run_max, 4) || !is_aligned(cur_min, 4) ||
      !is_aligned(cur_max, 4))
    return FA3Q_ERR_ALIGN;
  hipLaunchKernelGGL(accumulate_kernel, dim3(blocks_for(H)), dim3(256), 0, as_stream(stream),
                     run_min, run_max, cur_min, cur_max, H);
  return launch_status();
}

extern "C" int fa3q_qparams(const float* run_min, const float* run_max, float* scale, int64_t H,
                            void* stream) {
  if (!run_min || !run_max || !scale) return FA3Q_ERR_NULL;
  if (H <= 0 || H > (int64_t{1} << 31)) return FA3Q_ERR_SHAPE;
  if (!is_aligned(run_min, 4) || !is_aligned(run_max, 4) || !is_aligned(scale, 4))
    return FA3Q_ERR_ALIGN;
  hipLaunchKernelGGL(qparams_kernel, dim3(blocks_for(H)), dim3(256), 0, as_stream(stream),
                     run_min, run_max, scale, H);
  return launch_status();
}
