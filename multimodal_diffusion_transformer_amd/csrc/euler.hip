// Flow-matching Euler update ("Cosmos 3 方法原理全解" §7.2):
//     x <- x + (sigma_next - sigma) * v
// and its guided form (§7.2 CFG equation, §7.3 generation loop), which
// combines the condition and baseline predictions in the same pass:
//     x <- x + (sigma_next - sigma) * (v_base + w (v_cond - v_base))
// Pure streaming kernels: 8 elements per lane per trip (two 16-byte x loads,
// one 16-byte bf16 load per velocity), grid-stride over the buffer, fp32
// fused multiply-adds.  Optionally also stores bf16(x_new) for the next
// step's packed input.
#include <math.h>

#include "common.hpp"

namespace mot {

// 8 consecutive velocity values from element 8c of a bf16 or fp32 buffer.
template <bool V_BF16>
__device__ __forceinline__ void load8(const void* __restrict__ v_, int64_t c, float (&vv)[8]) {
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
}

__device__ __forceinline__ float load1(const void* v_, bool bf16, int64_t e) {
  return bf16 ? bf16_to_f32(reinterpret_cast<const bf16_t*>(v_)[e]) : reinterpret_cast<const float*>(v_)[e];
}

// GUIDED: v = v_base + w (v_cond - v_base), formed as fma(w, v_cond -
// v_base, v_base); otherwise v = v_cond (v_base unused).
template <bool V_BF16, bool MIRROR, bool GUIDED>
__global__ __launch_bounds__(256) void euler_kernel(float* __restrict__ x,
                                                    const void* __restrict__ v_,
                                                    const void* __restrict__ vb_,
                                                    int64_t n8, float w, float dt,
                                                    bf16_t* __restrict__ xb) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < n8; c += stride) {
    float4 x0 = reinterpret_cast<const float4*>(x)[2 * c];
    float4 x1 = reinterpret_cast<const float4*>(x)[2 * c + 1];
    float vv[8];
    load8<V_BF16>(v_, c, vv);
    if (GUIDED) {
      float vb[8];
      load8<V_BF16>(vb_, c, vb);
#pragma unroll
      for (int e = 0; e < 8; ++e) vv[e] = __builtin_fmaf(w, vv[e] - vb[e], vb[e]);
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

// Scalar tail (fewer than 8 trailing elements), the same arithmetic.
__global__ void euler_tail(float* x, const void* v_, const void* vb_, bool v_bf16, bool guided,
                           int64_t start, int64_t n, float w, float dt, bf16_t* xb) {
  int64_t e = start + threadIdx.x;
  if (e >= n) return;
  float vv = load1(v_, v_bf16, e);
  if (guided) {
    const float vb = load1(vb_, v_bf16, e);
    vv = __builtin_fmaf(w, vv - vb, vb);
  }
  float r = __builtin_fmaf(dt, vv, x[e]);
  x[e] = r;
  if (xb) xb[e] = f32_to_bf16(r);
}

template <bool V_BF16, bool MIRROR, bool GUIDED>
static void launch(float* x, const void* v, const void* vb, int64_t n, float w, float dt, bf16_t* xb,
                   hipStream_t s) {
  int64_t n8 = n / 8;
  if (n8 > 0) {
    int64_t blocks = (n8 + 255) / 256;
    // a few resident blocks per CU saturate HBM; more only adds scheduling
    if (blocks > 256 * 16) blocks = 256 * 16;
    hipLaunchKernelGGL((euler_kernel<V_BF16, MIRROR, GUIDED>), dim3((unsigned)blocks), dim3(256), 0, s,
                       x, v, vb, n8, w, dt, xb);
  }
  if (n8 * 8 < n)
    hipLaunchKernelGGL(euler_tail, dim3(1), dim3(8), 0, s, x, v, vb, V_BF16, GUIDED, n8 * 8, n, w, dt,
                       MIRROR ? xb : (bf16_t*)nullptr);
}

template <bool GUIDED>
static void dispatch(float* x, const void* v, const void* vb, bool v_bf16, int64_t n, float w, float dt,
                     bf16_t* xb, hipStream_t s) {
  if (v_bf16) {
    if (xb) launch<true, true, GUIDED>(x, v, vb, n, w, dt, xb, s);
    else launch<true, false, GUIDED>(x, v, vb, n, w, dt, xb, s);
  } else {
    if (xb) launch<false, true, GUIDED>(x, v, vb, n, w, dt, xb, s);
    else launch<false, false, GUIDED>(x, v, vb, n, w, dt, xb, s);
  }
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
  dispatch<false>(x, v, nullptr, v_dt == MOT_BF16, n, 0.f, dt, (bf16_t*)x_bf16, (hipStream_t)stream);
  MOT_CHECK_LAUNCH();
  return MOT_OK;
}

extern "C" mot_status flow_cfg_euler_step(float* x, const void* v_cond, const void* v_base,
                                          int32_t v_dt, int64_t n, float guidance, float sigma,
                                          float sigma_next, void* x_bf16, void* stream) {
  using namespace mot;
  if (n < 0) return MOT_ERR_INVALID_ARG;
  if (n == 0) return MOT_OK;
  if (!x || !v_cond || !v_base) return MOT_ERR_INVALID_ARG;
  if (v_dt != MOT_BF16 && v_dt != MOT_FP32) return MOT_ERR_INVALID_ARG;
  if (!isfinite(guidance)) return MOT_ERR_INVALID_ARG;
  if (((uintptr_t)x | (uintptr_t)v_cond | (uintptr_t)v_base | (uintptr_t)x_bf16) & 15)
    return MOT_ERR_INVALID_ARG;
  const float dt = sigma_next - sigma;
  dispatch<true>(x, v_cond, v_base, v_dt == MOT_BF16, n, guidance, dt, (bf16_t*)x_bf16, (hipStream_t)stream);
  MOT_CHECK_LAUNCH();
  return MOT_OK;
}
