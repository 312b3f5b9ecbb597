// Region-split LayerNorm ("Cosmos 3 方法原理全解" §3: each room has its own
// LayerNorm): y[r] = (x[r] - mean) / sqrt(var + eps) * gamma + beta over the
// hidden dimension, with the Reasoner's (gamma, beta) for rows r < n_ar and
// the Generator's for the rest.
//
// One wave per row, 4 rows per workgroup.  A lane holds its share of the row
// in registers (8 consecutive elements per 16-byte chunk, chunks strided by
// the wave), so the row is read once and written once: HBM-bound at 4 bytes
// per element in bf16.  Mean and variance are fp32 wave sums in a fixed order
// (butterfly), the variance taken about the mean (two passes over the
// registers).
#include <math.h>

#include "common.hpp"

namespace mot {

constexpr int LN_ROWS = 4;  // rows (waves) per workgroup

// Wave-wide sum, the same order in every lane.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <bool IN_BF16>
__device__ __forceinline__ void ln_load8(const void* x, int64_t e, float (&v)[8]) {
  if (IN_BF16) {
    const uint4 w = *reinterpret_cast<const uint4*>(reinterpret_cast<const bf16_t*>(x) + e);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(ws[i] << 16);
      v[2 * i + 1] = __uint_as_float(ws[i] & 0xFFFF0000u);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + e);
    const float4 b = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + e + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

template <bool OUT_BF16>
__device__ __forceinline__ void ln_store8(void* y, int64_t e, const float (&v)[8]) {
  if (OUT_BF16) {
    uint32_t p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = (uint32_t)f32_to_bf16(v[2 * i]) | ((uint32_t)f32_to_bf16(v[2 * i + 1]) << 16);
    *reinterpret_cast<uint4*>(reinterpret_cast<bf16_t*>(y) + e) = make_uint4(p[0], p[1], p[2], p[3]);
  } else {
    float* d = reinterpret_cast<float*>(y) + e;
    *reinterpret_cast<float4*>(d) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(d + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
}

// C = chunks of 8 elements per lane (hidden <= 512 C).
template <int C, bool IN_BF16, bool OUT_BF16>
__global__ __launch_bounds__(64 * LN_ROWS) void layernorm_kernel(const void* __restrict__ x, void* __restrict__ y,
                                                                 int64_t n_rows, int64_t n_ar, int hidden,
                                                                 const float* __restrict__ g_ar,
                                                                 const float* __restrict__ b_ar,
                                                                 const float* __restrict__ g_dm,
                                                                 const float* __restrict__ b_dm, float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * LN_ROWS + (threadIdx.x >> 6);
  if (row >= n_rows) return;  // whole waves leave together
  const int nch = hidden / 8;
  const int64_t base = row * hidden;
  float v[C][8];
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int ch = lane + 64 * c;
    if (ch < nch) {
      ln_load8<IN_BF16>(x, base + 8 * ch, v[c]);
#pragma unroll
      for (int i = 0; i < 8; ++i) s += v[c][i];
    }
  }
  const float mean = wave_sum(s) / (float)hidden;
  float q = 0.f;
#pragma unroll
  for (int c = 0; c < C; ++c)
    if (lane + 64 * c < nch)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float t = v[c][i] - mean;
        q = __builtin_fmaf(t, t, q);
      }
  const float rstd = 1.0f / sqrtf(wave_sum(q) / (float)hidden + eps);
  const bool ar = row < n_ar;
  const float* g = ar ? g_ar : g_dm;
  const float* b = ar ? b_ar : b_dm;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int ch = lane + 64 * c;
    if (ch < nch) {
      const float4 g0 = *reinterpret_cast<const float4*>(g + 8 * ch);
      const float4 g1 = *reinterpret_cast<const float4*>(g + 8 * ch + 4);
      const float4 b0 = *reinterpret_cast<const float4*>(b + 8 * ch);
      const float4 b1 = *reinterpret_cast<const float4*>(b + 8 * ch + 4);
      const float gg[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
      const float bb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
      float o[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = __builtin_fmaf((v[c][i] - mean) * rstd, gg[i], bb[i]);
      ln_store8<OUT_BF16>(y, base + 8 * ch, o);
    }
  }
}

template <int C>
static void launch_ln(const void* x, void* y, int64_t n_rows, int64_t n_ar, int hidden, const float* ga,
                      const float* ba, const float* gd, const float* bd, float eps, bool in_bf16, bool out_bf16,
                      hipStream_t s) {
  const dim3 grid((unsigned)((n_rows + LN_ROWS - 1) / LN_ROWS)), block(64 * LN_ROWS);
  if (in_bf16 && out_bf16)
    hipLaunchKernelGGL((layernorm_kernel<C, true, true>), grid, block, 0, s, x, y, n_rows, n_ar, hidden, ga, ba, gd, bd, eps);
  else if (in_bf16)
    hipLaunchKernelGGL((layernorm_kernel<C, true, false>), grid, block, 0, s, x, y, n_rows, n_ar, hidden, ga, ba, gd, bd, eps);
  else if (out_bf16)
    hipLaunchKernelGGL((layernorm_kernel<C, false, true>), grid, block, 0, s, x, y, n_rows, n_ar, hidden, ga, ba, gd, bd, eps);
  else
    hipLaunchKernelGGL((layernorm_kernel<C, false, false>), grid, block, 0, s, x, y, n_rows, n_ar, hidden, ga, ba, gd, bd, eps);
}

}  // namespace mot

extern "C" mot_status mot_layernorm_region(const void* x, void* y, int64_t n_rows, int64_t n_ar,
                                           int64_t hidden, const float* gamma_ar, const float* beta_ar,
                                           const float* gamma_dm, const float* beta_dm, float eps,
                                           int32_t in_dt, int32_t out_dt, void* stream) {
  using namespace mot;
  if (n_rows < 0 || n_ar < 0 || n_ar > n_rows) return MOT_ERR_INVALID_ARG;
  if (n_rows == 0) return MOT_OK;
  if (!x || !y) return MOT_ERR_INVALID_ARG;
  if (n_ar > 0 && (!gamma_ar || !beta_ar)) return MOT_ERR_INVALID_ARG;
  if (n_ar < n_rows && (!gamma_dm || !beta_dm)) return MOT_ERR_INVALID_ARG;
  if ((in_dt != MOT_BF16 && in_dt != MOT_FP32) || (out_dt != MOT_BF16 && out_dt != MOT_FP32))
    return MOT_ERR_INVALID_ARG;
  if (!(eps > 0.f) || !isfinite(eps)) return MOT_ERR_INVALID_ARG;
  if (((uintptr_t)x | (uintptr_t)y | (uintptr_t)gamma_ar | (uintptr_t)beta_ar | (uintptr_t)gamma_dm |
       (uintptr_t)beta_dm) & 15)
    return MOT_ERR_INVALID_ARG;
  if (hidden <= 0 || hidden % 8) return MOT_ERR_INVALID_ARG;
  if (hidden > 8192) return MOT_ERR_UNSUPPORTED;
  // one 64-lane wave per row, 4 per workgroup, within one dispatch
  if (n_rows > ((int64_t)UINT32_MAX - 255) / 64) return MOT_ERR_UNSUPPORTED;
  const int h = (int)hidden;
  const int chunks = (h / 8 + 63) / 64;
  const bool ib = in_dt == MOT_BF16, ob = out_dt == MOT_BF16;
  hipStream_t s = (hipStream_t)stream;
  if (chunks <= 1) launch_ln<1>(x, y, n_rows, n_ar, h, gamma_ar, beta_ar, gamma_dm, beta_dm, eps, ib, ob, s);
  else if (chunks <= 2) launch_ln<2>(x, y, n_rows, n_ar, h, gamma_ar, beta_ar, gamma_dm, beta_dm, eps, ib, ob, s);
  else if (chunks <= 4) launch_ln<4>(x, y, n_rows, n_ar, h, gamma_ar, beta_ar, gamma_dm, beta_dm, eps, ib, ob, s);
  else if (chunks <= 8) launch_ln<8>(x, y, n_rows, n_ar, h, gamma_ar, beta_ar, gamma_dm, beta_dm, eps, ib, ob, s);
  else launch_ln<16>(x, y, n_rows, n_ar, h, gamma_ar, beta_ar, gamma_dm, beta_dm, eps, ib, ob, s);
  MOT_CHECK_LAUNCH();
  return MOT_OK;
}
