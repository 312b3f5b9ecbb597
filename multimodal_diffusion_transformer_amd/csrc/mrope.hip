// Unified 3D mRoPE, standalone and in place ("Cosmos 3 方法原理全解" §5).
//
// Pair k of the P = D/2 rotary pairs rotates (x_k, x_{k+P}) by
// a = pos[axis(k)] * theta^(-2k/D); axis = t, h or w by contiguous sections.
// One lane owns 4 consecutive pairs of one token: it evaluates their angles
// and cos/sin once in fp64 (DM time coordinates sit near 1.5e4, where a fp32
// angle would already be off by ~1e-3 rad) and applies them to every head of
// the token.  HBM-bound: each element is read and written once.
#include <math.h>

#include "common.hpp"

namespace mot {

struct RopeFreqs {
  double inv_freq[64];  // theta^(-2k/D), k < P
};

template <typename T, int D>
__global__ __launch_bounds__(256) void mrope_kernel(T* __restrict__ x, int64_t n_tok, int n_heads,
                                                    int64_t tok_stride, int64_t head_stride,
                                                    const float* __restrict__ pos, int sec_t,
                                                    int sec_th, RopeFreqs fr) {
  constexpr int P = D / 2;
  constexpr int TPT = P / 4;              // lanes per token
  constexpr int TOK_PER_BLOCK = 256 / TPT;
  const int lane_in_tok = threadIdx.x % TPT;
  // D = 80: 10 lanes per token leave the workgroup's last 6 lanes idle
  if (256 % TPT != 0 && threadIdx.x >= TOK_PER_BLOCK * TPT) return;
  const int64_t tok = (int64_t)blockIdx.x * TOK_PER_BLOCK + threadIdx.x / TPT;
  if (tok >= n_tok) return;
  const int k0 = 4 * lane_in_tok;
  float cs[4], sn[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    int k = k0 + e;
    int axis = k < sec_t ? 0 : (k < sec_th ? 1 : 2);
    double a = (double)pos[3 * tok + axis] * fr.inv_freq[k];
    double s, c;
    sincos(a, &s, &c);
    cs[e] = (float)c;
    sn[e] = (float)s;
  }
  T* base = x + tok * tok_stride;
  for (int h = 0; h < n_heads; ++h) {
    T* p = base + (int64_t)h * head_stride;
    float x1[4], x2[4];
    if constexpr (sizeof(T) == 2) {
      uint2 a = *reinterpret_cast<const uint2*>(p + k0);
      uint2 b = *reinterpret_cast<const uint2*>(p + k0 + P);
      x1[0] = __uint_as_float(a.x << 16); x1[1] = __uint_as_float(a.x & 0xFFFF0000u);
      x1[2] = __uint_as_float(a.y << 16); x1[3] = __uint_as_float(a.y & 0xFFFF0000u);
      x2[0] = __uint_as_float(b.x << 16); x2[1] = __uint_as_float(b.x & 0xFFFF0000u);
      x2[2] = __uint_as_float(b.y << 16); x2[3] = __uint_as_float(b.y & 0xFFFF0000u);
    } else {
      float4 a = *reinterpret_cast<const float4*>(p + k0);
      float4 b = *reinterpret_cast<const float4*>(p + k0 + P);
      x1[0] = a.x; x1[1] = a.y; x1[2] = a.z; x1[3] = a.w;
      x2[0] = b.x; x2[1] = b.y; x2[2] = b.z; x2[3] = b.w;
    }
    float y1[4], y2[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      y1[e] = __builtin_fmaf(x1[e], cs[e], -x2[e] * sn[e]);
      y2[e] = __builtin_fmaf(x1[e], sn[e], x2[e] * cs[e]);
    }
    if constexpr (sizeof(T) == 2) {
      uint2 a, b;
      a.x = (uint32_t)f32_to_bf16(y1[0]) | ((uint32_t)f32_to_bf16(y1[1]) << 16);
      a.y = (uint32_t)f32_to_bf16(y1[2]) | ((uint32_t)f32_to_bf16(y1[3]) << 16);
      b.x = (uint32_t)f32_to_bf16(y2[0]) | ((uint32_t)f32_to_bf16(y2[1]) << 16);
      b.y = (uint32_t)f32_to_bf16(y2[2]) | ((uint32_t)f32_to_bf16(y2[3]) << 16);
      *reinterpret_cast<uint2*>(p + k0) = a;
      *reinterpret_cast<uint2*>(p + k0 + P) = b;
    } else {
      *reinterpret_cast<float4*>(p + k0) = make_float4(y1[0], y1[1], y1[2], y1[3]);
      *reinterpret_cast<float4*>(p + k0 + P) = make_float4(y2[0], y2[1], y2[2], y2[3]);
    }
  }
}

template <typename T, int D>
static void launch_rope(void* x, int64_t n_tok, int n_heads, int64_t ts, int64_t hs,
                        const float* pos, int sec_t, int sec_th, const RopeFreqs& fr,
                        hipStream_t s) {
  constexpr int TOK_PER_BLOCK = 256 / (D / 8);
  int64_t blocks = (n_tok + TOK_PER_BLOCK - 1) / TOK_PER_BLOCK;
  hipLaunchKernelGGL((mrope_kernel<T, D>), dim3((unsigned)blocks), dim3(256), 0, s, (T*)x, n_tok,
                     n_heads, ts, hs, pos, sec_t, sec_th, fr);
}

}  // namespace mot

extern "C" mot_status mrope_apply(void* x, int32_t dt, int64_t n_tok, int32_t n_heads,
                                  int32_t head_dim, int64_t tok_stride, int64_t head_stride,
                                  const float* pos_thw, int32_t sec_t, int32_t sec_h,
                                  int32_t sec_w, float theta, void* stream) {
  using namespace mot;
  if (n_tok < 0 || n_heads <= 0) return MOT_ERR_INVALID_ARG;
  if (n_tok == 0) return MOT_OK;
  if (!x || !pos_thw) return MOT_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 80 && head_dim != 128) return MOT_ERR_INVALID_ARG;
  if (sec_t < 0 || sec_h < 0 || sec_w < 0 || sec_t + sec_h + sec_w != head_dim / 2)
    return MOT_ERR_INVALID_ARG;
  if (dt != MOT_BF16 && dt != MOT_FP32) return MOT_ERR_INVALID_ARG;
  if (!(theta > 0.0f)) return MOT_ERR_INVALID_ARG;
  const int64_t align = dt == MOT_BF16 ? 8 : 4;
  if (((uintptr_t)x & 15) || ((uintptr_t)pos_thw & 3)) return MOT_ERR_INVALID_ARG;
  if (tok_stride % align || head_stride % align || tok_stride <= 0 || head_stride <= 0)
    return MOT_ERR_INVALID_ARG;
  // head_dim/8 lanes per token, floor(256 / (head_dim/8)) tokens per
  // 256-lane workgroup, within one dispatch's 2^32 - 1 work-items
  const int64_t tpb = 256 / (head_dim / 8);
  if ((n_tok + tpb - 1) / tpb > (int64_t)(UINT32_MAX / 256)) return MOT_ERR_UNSUPPORTED;
  RopeFreqs fr;
  for (int k = 0; k < head_dim / 2; ++k) fr.inv_freq[k] = pow((double)theta, -2.0 * k / head_dim);
  const int sec_th = sec_t + sec_h;
  hipStream_t s = (hipStream_t)stream;
  if (dt == MOT_BF16) {
    if (head_dim == 128) launch_rope<bf16_t, 128>(x, n_tok, n_heads, tok_stride, head_stride, pos_thw, sec_t, sec_th, fr, s);
    else if (head_dim == 80) launch_rope<bf16_t, 80>(x, n_tok, n_heads, tok_stride, head_stride, pos_thw, sec_t, sec_th, fr, s);
    else launch_rope<bf16_t, 64>(x, n_tok, n_heads, tok_stride, head_stride, pos_thw, sec_t, sec_th, fr, s);
  } else {
    if (head_dim == 128) launch_rope<float, 128>(x, n_tok, n_heads, tok_stride, head_stride, pos_thw, sec_t, sec_th, fr, s);
    else if (head_dim == 80) launch_rope<float, 80>(x, n_tok, n_heads, tok_stride, head_stride, pos_thw, sec_t, sec_th, fr, s);
    else launch_rope<float, 64>(x, n_tok, n_heads, tok_stride, head_stride, pos_thw, sec_t, sec_th, fr, s);
  }
  MOT_CHECK_LAUNCH();
  return MOT_OK;
}
