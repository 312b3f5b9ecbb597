// Merge of attention over disjoint key sets into attention over their union
// (the softmax of the method page's §3 equations taken over all keys): with
// L = log sum_b exp(L_b),
//     O = sum_b exp(L_b - L) O_b,   LSE = L.
// This lets one query tile's keys be split over several workgroups (a batch
// of launches over key ranges) when one tile per head leaves the chip idle,
// as the streaming call's 1,440-row chunks do.
//
// One lane per (row, head, 8 dims): it reads the parts' LSE of its row and
// head and their 16-byte runs of O, and writes one merged run.  A part with
// no key for the row (LSE = -inf) gets weight 0 and its O is not read into
// the sum (it may be NaN).  HBM-bound.
#include <math.h>

#include "common.hpp"

namespace mot {

constexpr int MERGE_MAX_PARTS = 16;

template <bool BF16>
__device__ __forceinline__ void mload8(const void* p, int64_t e, float (&v)[8]) {
  if (BF16) {
    const uint4 w = *reinterpret_cast<const uint4*>(reinterpret_cast<const bf16_t*>(p) + e);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(ws[i] << 16);
      v[2 * i + 1] = __uint_as_float(ws[i] & 0xFFFF0000u);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p) + e);
    const float4 b = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p) + e + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

template <bool BF16>
__global__ __launch_bounds__(256) void attn_merge_kernel(const void* __restrict__ op, const float* __restrict__ lp,
                                                         int n_parts, int64_t part_stride, int64_t p_ts,
                                                         int64_t p_hs, void* __restrict__ o, int64_t o_ts,
                                                         int64_t o_hs, float* __restrict__ lse, int64_t nq,
                                                         int n_heads, int chunks) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_row = (int64_t)n_heads * chunks;
  const int64_t row = idx / per_row;
  if (row >= nq) return;
  const int rem = (int)(idx - row * per_row);
  const int head = rem / chunks, c = rem % chunks;
  const int64_t lrow = (int64_t)head * nq + row;  // [part][head][row]
  float m = -INFINITY;
  for (int b = 0; b < n_parts; ++b) m = fmaxf(m, lp[(int64_t)b * n_heads * nq + lrow]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float tot = 0.f;
  for (int b = 0; b < n_parts; ++b) {
    const float w = expf(lp[(int64_t)b * n_heads * nq + lrow] - m);
    if (!(w > 0.f)) continue;  // no key of this part for the row
    tot += w;
    float v[8];
    mload8<BF16>(op, (int64_t)b * part_stride + row * p_ts + (int64_t)head * p_hs + 8 * c, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(w, v[i], acc[i]);
  }
  const float inv = 1.0f / tot;
  const int64_t e = row * o_ts + (int64_t)head * o_hs + 8 * c;
  if (BF16) {
    uint32_t p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      p[i] = (uint32_t)f32_to_bf16(acc[2 * i] * inv) | ((uint32_t)f32_to_bf16(acc[2 * i + 1] * inv) << 16);
    *reinterpret_cast<uint4*>(reinterpret_cast<bf16_t*>(o) + e) = make_uint4(p[0], p[1], p[2], p[3]);
  } else {
    float* d = reinterpret_cast<float*>(o) + e;
    *reinterpret_cast<float4*>(d) = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
    *reinterpret_cast<float4*>(d + 4) = make_float4(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
  }
  if (lse && c == 0) lse[lrow] = m + logf(tot);
}

}  // namespace mot

extern "C" mot_status mot_attention_merge(const void* o_parts, const float* lse_parts, int32_t n_parts,
                                          int64_t part_stride, int64_t nq, int32_t n_heads, int32_t head_dim,
                                          int64_t p_ts, int64_t p_hs, void* o, int64_t o_ts, int64_t o_hs,
                                          float* lse, int32_t dt, void* stream) {
  using namespace mot;
  if (nq < 0 || n_heads <= 0 || (head_dim != 64 && head_dim != 80 && head_dim != 128)) return MOT_ERR_INVALID_ARG;
  if (n_parts < 1 || n_parts > MERGE_MAX_PARTS) return MOT_ERR_INVALID_ARG;
  if (dt != MOT_BF16 && dt != MOT_FP32) return MOT_ERR_INVALID_ARG;
  if (nq == 0) return MOT_OK;
  if (!o_parts || !lse_parts || !o) return MOT_ERR_INVALID_ARG;
  const int64_t al = dt == MOT_BF16 ? 8 : 4;
  if (part_stride < 0 || part_stride % al || p_ts <= 0 || p_ts % al || p_hs <= 0 || p_hs % al ||
      o_ts <= 0 || o_ts % al || o_hs <= 0 || o_hs % al)
    return MOT_ERR_INVALID_ARG;
  if (((uintptr_t)o_parts | (uintptr_t)o) & 15) return MOT_ERR_INVALID_ARG;
  if (((uintptr_t)lse_parts | (uintptr_t)lse) & 3) return MOT_ERR_INVALID_ARG;
  const int chunks = head_dim / 8;
  // one lane per (row, head, 8 dims), 256 per workgroup, in one dispatch
  if (nq > ((int64_t)UINT32_MAX - 255) / ((int64_t)n_heads * chunks)) return MOT_ERR_UNSUPPORTED;
  const int64_t lanes = nq * n_heads * chunks;
  const dim3 grid((unsigned)((lanes + 255) / 256)), block(256);
  hipStream_t s = (hipStream_t)stream;
  if (dt == MOT_BF16)
    hipLaunchKernelGGL(attn_merge_kernel<true>, grid, block, 0, s, o_parts, lse_parts, (int)n_parts, part_stride,
                       p_ts, p_hs, o, o_ts, o_hs, lse, nq, (int)n_heads, chunks);
  else
    hipLaunchKernelGGL(attn_merge_kernel<false>, grid, block, 0, s, o_parts, lse_parts, (int)n_parts, part_stride,
                       p_ts, p_hs, o, o_ts, o_hs, lse, nq, (int)n_heads, chunks);
  MOT_CHECK_LAUNCH();
  return MOT_OK;
}
