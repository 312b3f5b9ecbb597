// Flow-matching Euler update ("Cosmos 3 方法原理全解" §7.2):
//     x <- x + (sigma_next - sigma) * v
// A pure streaming kernel: 8 elements per lane per trip (two 16-byte x loads,
// one 16-byte bf16 v load), grid-stride over the buffer, fp32 FMA.
// Optionally also stores bf16(x_new) for the next step's packed input.
#include "common.hpp"

namespace mot {

struct alignas(16) f32x4s { float a, b, c, d; };

template <bool V_BF16, bool MIRROR>
__global__ __launch_bounds__(256) void euler_kernel(float* __restrict__ x,
                                                    const void* __restrict__ v_,
                                                    int64_t n8, float dt,
                                                    bf16_t* __restrict__ xb) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < n8; c += stride) {
    float4 x0 = reinterpret_cast<const float4*>(x)[2 * c];
    float4 x1 = reinterpret_cast<const float4*>(x)[2 * c + 1];
    float vv[8];
    if (V_BF16) {
      uint4 w = reinterpret_cast<const uint4*>(v_)[c];
      uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vv[2 * e] = __uint_as_float(ws[e] << 16);
        vv[2 * e + 1] = __uint_as_float(ws[e] & 0xFFFF0000u);
      }
    } else {
      float4 a = reinterpret_cast<const float4*>(v_)[2 * c];
      float4 b = reinterpret_cast<const float4*>(v_)[2 * c + 1];
      vv[0] = a.x; vv[1] = a.y; vv[2] = a.z; vv[3] = a.w;
      vv[4] = b.x; vv[5] = b.y; vv[6] = b.z; vv[7] = b.w;
    }
    float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) xs[e] = __builtin_fmaf(dt, vv[e], xs[e]);
    reinterpret_cast<float4*>(x)[2 * c] = make_float4(xs[0], xs[1], xs[2], xs[3]);
    reinterpret_cast<float4*>(x)[2 * c + 1] = make_float4(xs[4], xs[5], xs[6], xs[7]);
    if (MIRROR) {
      uint32_t p[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        p[e] = (uint32_t)f32_to_bf16(xs[2 * e]) | ((uint32_t)f32_to_bf16(xs[2 * e + 1]) << 16);
      reinterpret_cast<uint4*>(xb)[c] = make_uint4(p[0], p[1], p[2], p[3]);
    }
  }
}

// Scalar tail (fewer than 8 trailing elements).
template <bool V_BF16, bool MIRROR>
__global__ void euler_tail(float* x, const void* v_, int64_t start, int64_t n, float dt,
                           bf16_t* xb) {
  int64_t e = start + threadIdx.x;
  if (e >= n) return;
  float vv = V_BF16 ? bf16_to_f32(reinterpret_cast<const bf16_t*>(v_)[e])
                    : reinterpret_cast<const float*>(v_)[e];
  float r = __builtin_fmaf(dt, vv, x[e]);
  x[e] = r;
  if (MIRROR) xb[e] = f32_to_bf16(r);
}

template <bool V_BF16, bool MIRROR>
static void launch(float* x, const void* v, int64_t n, float dt, bf16_t* xb, hipStream_t s) {
  int64_t n8 = n / 8;
  if (n8 > 0) {
    int64_t blocks = (n8 + 255) / 256;
    // a few resident blocks per CU saturate HBM; more only adds scheduling
    if (blocks > 256 * 16) blocks = 256 * 16;
    hipLaunchKernelGGL((euler_kernel<V_BF16, MIRROR>), dim3((unsigned)blocks), dim3(256), 0, s,
                       x, v, n8, dt, xb);
  }
  if (n8 * 8 < n)
    hipLaunchKernelGGL((euler_tail<V_BF16, MIRROR>), dim3(1), dim3(8), 0, s, x, v, n8 * 8, n, dt,
                       xb);
}

}  // namespace mot

extern "C" mot_status flow_euler_step(float* x, const void* v, int32_t v_dt, int64_t n,
                                      float sigma, float sigma_next, void* x_bf16,
                                      void* stream) {
  using namespace mot;
  if (n < 0) return MOT_ERR_INVALID_ARG;
  if (n == 0) return MOT_OK;
  if (!x || !v) return MOT_ERR_INVALID_ARG;
  if (v_dt != MOT_BF16 && v_dt != MOT_FP32) return MOT_ERR_INVALID_ARG;
  if (((uintptr_t)x | (uintptr_t)v | (uintptr_t)x_bf16) & 15) return MOT_ERR_INVALID_ARG;
  const float dt = sigma_next - sigma;
  hipStream_t s = (hipStream_t)stream;
  bf16_t* xb = (bf16_t*)x_bf16;
  if (v_dt == MOT_BF16) {
    if (xb) launch<true, true>(x, v, n, dt, xb, s);
    else launch<true, false>(x, v, n, dt, xb, s);
  } else {
    if (xb) launch<false, true>(x, v, n, dt, xb, s);
    else launch<false, false>(x, v, n, dt, xb, s);
  }
  MOT_CHECK_LAUNCH();
  return MOT_OK;
}
