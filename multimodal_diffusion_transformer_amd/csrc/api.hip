// C ABI entry points that validate, then dispatch to the kernels:
// version and status strings, masked attention, region-split projection,
// and the mask / tile-class materialisers used by the tests.
#include <math.h>

#include "common.hpp"
#include "rope_dev.hpp"

namespace mot {
hipError_t attention_bf16_mfma(const mot_attn_args* a, const RopeTable& rt, hipStream_t s);
hipError_t attention_f32_valu(const mot_attn_args* a, const RopeTable& rt, hipStream_t s);
hipError_t region_gemm(const void* x, const void* w_ar, const void* w_dm, void* y, int64_t n_rows,
                       int64_t n_ar, int64_t K, int64_t N, mot_dtype in_dt, mot_dtype out_dt,
                       int epi, const void* res, hipStream_t s);
bool region_gemm_fits(int64_t n_rows, int64_t n_ar, int64_t N, mot_dtype in_dt);

// One dispatch holds at most 2^32 - 1 work-items along a grid dimension.
// True when `units` units of `lanes` work-items each, plus `extra` more,
// stay within that.
static bool fits_dispatch(int64_t units, int64_t lanes, int64_t extra) {
  return units >= 0 && units <= ((int64_t)UINT32_MAX - extra) / lanes;
}

static MaskSpec mask_of(const mot_attn_args* a) {
  MaskSpec m;
  m.mode = a->mask; m.nq = a->nq; m.nk = a->nk; m.q0 = a->q0;
  m.n_ar = a->n_ar; m.n_prefix = a->n_prefix; m.chunk_len = a->chunk_len > 0 ? a->chunk_len : 1;
  return m;
}

static bool mask_args_ok(const mot_attn_args* a) {
  if (a->nq < 1 || a->nk < 1 || a->q0 < 0 || a->q0 > INT64_MAX - a->nq) return false;
  if (a->mask == MOT_AR_CAUSAL_DM_FULL) {
    if (a->n_ar < 0 || a->n_ar > a->nk) return false;
    if (a->nk < a->q0 + a->nq) return false;  // every query sees its diagonal
    return true;
  }
  if (a->mask == MOT_CHUNK_CAUSAL_KV) {
    if (a->chunk_len < 1 || a->n_prefix < 0 || a->n_prefix > a->nk) return false;
    if (a->q0 < a->n_prefix) return false;
    return true;
  }
  return false;
}

__global__ void mask_kernel(MaskSpec m, uint8_t* out) {
  int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= m.nq * m.nk) return;
  int64_t r = e / m.nk, j = e % m.nk;
  out[e] = mask_allowed(m, m.q0 + r, j) ? 1 : 0;
}

__host__ __device__ inline uint8_t classify(const MaskSpec& m, int bm, int bn, int64_t tq, int64_t tk) {
  int64_t ra = tq * bm, rb = ra + bm - 1 < m.nq ? ra + bm - 1 : m.nq - 1;
  int64_t ja = tk * bn, jb = ja + bn - 1 < m.nk ? ja + bn - 1 : m.nk - 1;
  return (uint8_t)tile_class(m, m.q0 + ra, m.q0 + rb, ja, jb);
}

__global__ void tile_kernel(MaskSpec m, int bm, int bn, int64_t ntq, int64_t ntk, uint8_t* out) {
  int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= ntq * ntk) return;
  out[e] = classify(m, bm, bn, e / ntk, e % ntk);
}

}  // namespace mot

using namespace mot;

extern "C" int mot_abi_version(void) { return MOT_ABI_VERSION; }

extern "C" const char* mot_status_string(int32_t s) {
  switch (s) {
    case MOT_OK: return "ok";
    case MOT_ERR_INVALID_ARG: return "invalid argument";
    case MOT_ERR_UNSUPPORTED: return "unsupported combination";
    case MOT_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

extern "C" mot_status mot_attention_fwd(const mot_attn_args* a, void* stream) {
  if (!a) return MOT_ERR_INVALID_ARG;
  if (a->n_heads <= 0 || (a->head_dim != 64 && a->head_dim != 80 && a->head_dim != 128)) return MOT_ERR_INVALID_ARG;
  if (a->dt != MOT_BF16 && a->dt != MOT_FP32) return MOT_ERR_INVALID_ARG;
  // no query rows: a no-op that touches nothing (null pointers allowed), like
  // the other calls' empty inputs
  if (a->nq == 0) return a->nk >= 0 && a->q0 >= 0 ? MOT_OK : MOT_ERR_INVALID_ARG;
  if (!a->q || !a->k || !a->v || !a->o) return MOT_ERR_INVALID_ARG;
  if (!mask_args_ok(a)) return MOT_ERR_INVALID_ARG;
  if (!(a->scale >= 0.f) || !isfinite(a->scale)) return MOT_ERR_INVALID_ARG;
  const int64_t al = a->dt == MOT_BF16 ? 8 : 4;
  const int64_t st[8] = {a->q_ts, a->q_hs, a->k_ts, a->k_hs, a->v_ts, a->v_hs, a->o_ts, a->o_hs};
  for (int i = 0; i < 8; ++i)
    if (st[i] <= 0 || st[i] % al) return MOT_ERR_INVALID_ARG;
  // grouped key/value heads and the batch
  if (a->n_kv_heads < 0 || (a->n_kv_heads > 0 && a->n_heads % a->n_kv_heads)) return MOT_ERR_INVALID_ARG;
  if (a->n_batch < 0 || a->n_batch > 65535) return MOT_ERR_INVALID_ARG;
  if (a->n_batch > 1) {
    const int64_t bs[4] = {a->q_bs, a->k_bs, a->v_bs, a->o_bs};
    for (int i = 0; i < 4; ++i)
      if (bs[i] < 0 || bs[i] % al) return MOT_ERR_INVALID_ARG;
  }
  if (((uintptr_t)a->q | (uintptr_t)a->k | (uintptr_t)a->v | (uintptr_t)a->o) & 15)
    return MOT_ERR_INVALID_ARG;
  if ((uintptr_t)a->lse & 3) return MOT_ERR_INVALID_ARG;
  // the bf16 kernel keeps key indices in 32 bits and addresses a 64-key tile
  // with 32-bit unsigned lane offsets from the tile base
  if (a->dt == MOT_BF16 &&
      (a->nk > INT32_MAX - 64 || a->nq > INT32_MAX || 64 * (a->k_ts > a->v_ts ? a->k_ts : a->v_ts) * 2 >= (1LL << 32)))
    return MOT_ERR_UNSUPPORTED;
  // the bf16 kernel rotates Q on load only; K is rotated beforehand (mrope_apply)
  if (a->dt == MOT_BF16 && a->k_pos) return MOT_ERR_UNSUPPORTED;
  // Dispatch size.  bf16: one workgroup per (row tile, head) with 64 lanes
  // per 32 query rows, so 2 lanes per row and head, the last tile rounded up
  // by fewer than 512 rows, along x; batch items along y.  fp32: 64 query
  // rows of 64 lanes per workgroup along x, heads along y (at most 65535),
  // batch items along z.
  if (a->dt == MOT_BF16 ? !fits_dispatch(a->nq + 512, 2 * (int64_t)a->n_heads, 0)
                        : (!fits_dispatch(a->nq, 1, 63) || a->n_heads > 65535))
    return MOT_ERR_UNSUPPORTED;
  RopeTable rt;
  rt.sec_t = a->sec_t;
  rt.sec_th = a->sec_t + a->sec_h;
  if (a->q_pos || a->k_pos) {
    if (a->sec_t < 0 || a->sec_h < 0 || a->sec_w < 0 ||
        a->sec_t + a->sec_h + a->sec_w != a->head_dim / 2 || !(a->theta > 0.f))
      return MOT_ERR_INVALID_ARG;
    if (((uintptr_t)a->q_pos | (uintptr_t)a->k_pos) & 3) return MOT_ERR_INVALID_ARG;
    for (int k = 0; k < a->head_dim / 2; ++k)
      rt.inv_freq[k] = pow((double)a->theta, -2.0 * k / a->head_dim);
  }
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = a->dt == MOT_BF16 ? attention_bf16_mfma(a, rt, s) : attention_f32_valu(a, rt, s);
  return e == hipSuccess ? MOT_OK : MOT_ERR_HIP;
}

static mot_status region_linear(const void* x, const void* w_ar, const void* w_dm, void* y, int64_t n_rows,
                                int64_t n_ar, int64_t d_in, int64_t d_out, int32_t in_dt, int32_t out_dt,
                                int32_t epilogue, const void* residual, void* stream) {
  if (n_rows < 0 || n_ar < 0 || n_ar > n_rows || d_in <= 0 || d_out <= 0) return MOT_ERR_INVALID_ARG;
  if (n_rows == 0) return MOT_OK;
  if (!x || !y || (n_ar > 0 && !w_ar) || (n_ar < n_rows && !w_dm)) return MOT_ERR_INVALID_ARG;
  if ((in_dt != MOT_BF16 && in_dt != MOT_FP32) || (out_dt != MOT_BF16 && out_dt != MOT_FP32))
    return MOT_ERR_INVALID_ARG;
  if (((uintptr_t)x | (uintptr_t)w_ar | (uintptr_t)w_dm | (uintptr_t)y) & 15) return MOT_ERR_INVALID_ARG;
  if (in_dt == MOT_BF16 && (d_in % 64 || d_out % 64)) return MOT_ERR_UNSUPPORTED;
  if (in_dt == MOT_FP32 && out_dt != MOT_FP32) return MOT_ERR_UNSUPPORTED;
  if (epilogue != MOT_EPI_NONE && epilogue != MOT_EPI_GELU && epilogue != MOT_EPI_ADD)
    return MOT_ERR_INVALID_ARG;
  if ((epilogue == MOT_EPI_ADD) != (residual != nullptr)) return MOT_ERR_INVALID_ARG;
  if ((uintptr_t)residual & 15) return MOT_ERR_INVALID_ARG;
  if (!region_gemm_fits(n_rows, n_ar, d_out, (mot_dtype)in_dt)) return MOT_ERR_UNSUPPORTED;
  hipError_t e = region_gemm(x, w_ar, w_dm, y, n_rows, n_ar, d_in, d_out, (mot_dtype)in_dt,
                             (mot_dtype)out_dt, epilogue, residual, (hipStream_t)stream);
  return e == hipSuccess ? MOT_OK : MOT_ERR_HIP;
}

extern "C" mot_status mot_qkv_project(const void* x, const void* w_ar, const void* w_dm, void* y,
                                      int64_t n_rows, int64_t n_ar, int64_t d_in, int64_t d_out,
                                      int32_t in_dt, int32_t out_dt, void* stream) {
  return region_linear(x, w_ar, w_dm, y, n_rows, n_ar, d_in, d_out, in_dt, out_dt, MOT_EPI_NONE, nullptr,
                       stream);
}

extern "C" mot_status mot_region_linear(const void* x, const void* w_ar, const void* w_dm, void* y,
                                        int64_t n_rows, int64_t n_ar, int64_t d_in, int64_t d_out,
                                        int32_t in_dt, int32_t out_dt, int32_t epilogue,
                                        const void* residual, void* stream) {
  return region_linear(x, w_ar, w_dm, y, n_rows, n_ar, d_in, d_out, in_dt, out_dt, epilogue, residual,
                       stream);
}

extern "C" mot_status mot_mask_materialize(const mot_attn_args* a, uint8_t* mask_dev, int32_t bm,
                                           int32_t bn, uint8_t* tiles_dev, void* stream) {
  if (!a || !mask_args_ok(a)) return MOT_ERR_INVALID_ARG;
  if (tiles_dev && (bm <= 0 || bn <= 0)) return MOT_ERR_INVALID_ARG;
  MaskSpec m = mask_of(a);
  // one lane per mask entry / tile, 256 per workgroup
  if (mask_dev && (m.nq > INT64_MAX / m.nk || !fits_dispatch(m.nq * m.nk, 1, 255)))
    return MOT_ERR_UNSUPPORTED;
  if (tiles_dev) {
    const int64_t ntq = (m.nq + bm - 1) / bm, ntk = (m.nk + bn - 1) / bn;
    if (ntq > INT64_MAX / ntk || !fits_dispatch(ntq * ntk, 1, 255)) return MOT_ERR_UNSUPPORTED;
  }
  hipStream_t s = (hipStream_t)stream;
  if (mask_dev) {
    int64_t n = m.nq * m.nk;
    hipLaunchKernelGGL(mask_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, m, mask_dev);
    MOT_CHECK_LAUNCH();
  }
  if (tiles_dev) {
    int64_t ntq = (m.nq + bm - 1) / bm, ntk = (m.nk + bn - 1) / bn;
    hipLaunchKernelGGL(tile_kernel, dim3((unsigned)((ntq * ntk + 255) / 256)), dim3(256), 0, s, m, bm,
                       bn, ntq, ntk, tiles_dev);
    MOT_CHECK_LAUNCH();
  }
  return MOT_OK;
}

extern "C" mot_status mot_tile_classes_host(const mot_attn_args* a, int32_t bm, int32_t bn,
                                            uint8_t* tiles_host) {
  if (!a || !tiles_host || bm <= 0 || bn <= 0 || !mask_args_ok(a)) return MOT_ERR_INVALID_ARG;
  MaskSpec m = mask_of(a);
  int64_t ntq = (m.nq + bm - 1) / bm, ntk = (m.nk + bn - 1) / bn;
  for (int64_t tq = 0; tq < ntq; ++tq)
    for (int64_t tk = 0; tk < ntk; ++tk) tiles_host[tq * ntk + tk] = classify(m, bm, bn, tq, tk);
  return MOT_OK;
}
