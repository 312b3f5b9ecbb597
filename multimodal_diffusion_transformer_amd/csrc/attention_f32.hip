// Masked attention in fp32 on the vector ALUs (for fp32 workloads).
//
// Same definition as the MFMA kernel ("Cosmos 3 方法原理全解" §3; chunk mode
// from "流式生成如何工作"), evaluated in fp32 throughout: one lane per query
// row holds q and its output accumulator in registers; 32-key K/V tiles are
// staged in LDS (rotated by mRoPE while staged when key positions are given)
// and read as broadcasts; the softmax is the streaming (online) form.
// Grid: x = 64-row query tiles, y = heads, z = batch items; query head h
// reads key/value head h / kv_group.
#include "common.hpp"
#include "rope_dev.hpp"

namespace mot {

struct AttnF32Params {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  int64_t q_ts, q_hs, k_ts, k_hs, v_ts, v_hs, o_ts, o_hs;
  MaskSpec m;
  int n_heads;
  int kv_group;
  int64_t q_bs, k_bs, v_bs, o_bs;
  float scale;
  const float* q_pos;
  const float* k_pos;
  RopeTable rope;
};

constexpr int F32_BQ = 64;  // queries per block (one wave)
constexpr int F32_BK = 32;  // keys per LDS tile

template <int D>
__global__ __launch_bounds__(64) void attn_fwd_f32(AttnF32Params p) {
  constexpr int P = D / 2;
  __shared__ float ks[F32_BK][D];
  __shared__ float vs[F32_BK][D];
  const int head = blockIdx.y;
  const int kvh = head / p.kv_group;
  const int64_t b = blockIdx.z;
  const float* ksrc = p.k + b * p.k_bs + (int64_t)kvh * p.k_hs;  // this item's key/value head
  const float* vsrc = p.v + b * p.v_bs + (int64_t)kvh * p.v_hs;
  const int64_t row = (int64_t)blockIdx.x * F32_BQ + threadIdx.x;
  const bool ok = row < p.m.nq;
  const int64_t i_abs = p.m.q0 + row;

  float q[D], o[D];
  const float* qs = p.q + b * p.q_bs + (ok ? row : 0) * p.q_ts + (int64_t)head * p.q_hs;
#pragma unroll
  for (int d = 0; d < D; ++d) { q[d] = ok ? qs[d] : 0.f; o[d] = 0.f; }
  if (p.q_pos && ok) {
    const float* pp = p.q_pos + 3 * row;
#pragma unroll
    for (int kk = 0; kk < P; ++kk) {
      float c, s;
      rope_cs(pp[rope_axis(p.rope, kk)], p.rope.inv_freq[kk], c, s);
      float x1 = q[kk], x2 = q[kk + P];
      q[kk] = __builtin_fmaf(x1, c, -x2 * s);
      q[kk + P] = __builtin_fmaf(x1, s, x2 * c);
    }
  }

  const int64_t r_last = ((int64_t)blockIdx.x + 1) * F32_BQ - 1 < p.m.nq
                             ? ((int64_t)blockIdx.x + 1) * F32_BQ - 1 : p.m.nq - 1;
  const int64_t kend = key_end(p.m, p.m.q0 + (int64_t)blockIdx.x * F32_BQ, p.m.q0 + r_last);
  float m_run = -INFINITY, l_run = 0.f;
  for (int64_t kb = 0; kb < kend; kb += F32_BK) {
    __syncthreads();
    for (int e = threadIdx.x; e < F32_BK * D; e += 64) {
      int kr = e / D, d = e % D;
      int64_t j = kb + kr;
      float kv = 0.f, vv = 0.f;
      if (j < p.m.nk) {
        kv = ksrc[j * p.k_ts + d];
        vv = vsrc[j * p.v_ts + d];
      }
      ks[kr][d] = kv;
      vs[kr][d] = vv;
    }
    __syncthreads();
    if (p.k_pos) {
      for (int e = threadIdx.x; e < F32_BK * P; e += 64) {
        int kr = e / P, kk = e % P;
        int64_t j = kb + kr;
        if (j < p.m.nk) {
          float c, s;
          rope_cs(p.k_pos[3 * j + rope_axis(p.rope, kk)], p.rope.inv_freq[kk], c, s);
          float x1 = ks[kr][kk], x2 = ks[kr][kk + P];
          ks[kr][kk] = __builtin_fmaf(x1, c, -x2 * s);
          ks[kr][kk + P] = __builtin_fmaf(x1, s, x2 * c);
        }
      }
      __syncthreads();
    }
    if (!ok) continue;
    for (int kr = 0; kr < F32_BK; ++kr) {
      int64_t j = kb + kr;
      if (j >= p.m.nk || !mask_allowed(p.m, i_abs, j)) continue;
      float sdot = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) sdot = __builtin_fmaf(q[d], ks[kr][d], sdot);
      float sc = sdot * p.scale;
      if (sc > m_run) {
        float corr = expf(m_run - sc);
        l_run *= corr;
#pragma unroll
        for (int d = 0; d < D; ++d) o[d] *= corr;
        m_run = sc;
      }
      float pr = expf(sc - m_run);
      l_run += pr;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] = __builtin_fmaf(pr, vs[kr][d], o[d]);
    }
  }
  if (ok) {
    float inv = 1.f / l_run;
    float* dst = p.o + b * p.o_bs + row * p.o_ts + (int64_t)head * p.o_hs;
#pragma unroll
    for (int d = 0; d < D; ++d) dst[d] = o[d] * inv;
    if (p.lse) p.lse[(b * p.n_heads + head) * p.m.nq + row] = m_run + logf(l_run);
  }
}

hipError_t attention_f32_valu(const mot_attn_args* a, const RopeTable& rt, hipStream_t s) {
  AttnF32Params p;
  p.q = (const float*)a->q; p.k = (const float*)a->k; p.v = (const float*)a->v;
  p.o = (float*)a->o; p.lse = a->lse;
  p.q_ts = a->q_ts; p.q_hs = a->q_hs; p.k_ts = a->k_ts; p.k_hs = a->k_hs;
  p.v_ts = a->v_ts; p.v_hs = a->v_hs; p.o_ts = a->o_ts; p.o_hs = a->o_hs;
  p.m.mode = a->mask; p.m.nq = a->nq; p.m.nk = a->nk; p.m.q0 = a->q0;
  p.m.n_ar = a->n_ar; p.m.n_prefix = a->n_prefix; p.m.chunk_len = a->chunk_len > 0 ? a->chunk_len : 1;
  p.n_heads = a->n_heads;
  p.kv_group = a->n_heads / (a->n_kv_heads > 0 ? a->n_kv_heads : a->n_heads);
  const int n_batch = a->n_batch > 1 ? a->n_batch : 1;
  p.q_bs = n_batch > 1 ? a->q_bs : 0;
  p.k_bs = n_batch > 1 ? a->k_bs : 0;
  p.v_bs = n_batch > 1 ? a->v_bs : 0;
  p.o_bs = n_batch > 1 ? a->o_bs : 0;
  p.scale = a->scale != 0.f ? a->scale : 1.f / sqrtf((float)a->head_dim);
  p.q_pos = a->q_pos; p.k_pos = a->k_pos; p.rope = rt;
  dim3 grid((unsigned)((a->nq + F32_BQ - 1) / F32_BQ), (unsigned)a->n_heads, (unsigned)n_batch);
  if (a->head_dim == 128)
    hipLaunchKernelGGL(attn_fwd_f32<128>, grid, dim3(64), 0, s, p);
  else if (a->head_dim == 80)
    hipLaunchKernelGGL(attn_fwd_f32<80>, grid, dim3(64), 0, s, p);
  else
    hipLaunchKernelGGL(attn_fwd_f32<64>, grid, dim3(64), 0, s, p);
  return hipGetLastError();
}

}  // namespace mot
