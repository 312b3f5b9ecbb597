// Region-split projection ("Cosmos 3 方法原理全解" §3, §3.2): the AR rows of
// the packed block go through the Reasoner's weights, the DM rows through
// the Generator's:  Y[r] = X[r] @ (r < n_ar ? W_ar : W_dm).
//
// bf16 path: one launch covers both regions as a grouped GEMM (problem 0 =
// rows [0, n_ar) x W_ar, problem 1 = rows [n_ar, n) x W_dm), so no tile ever
// straddles the boundary.  Workgroup tile 128 rows x 128 cols x 64-deep,
// 4 waves each owning 64x64 as 2x2 v_mfma_f32_32x32x16_bf16 blocks.  The
// transposed product Y^T = W^T X^T is formed so that in the accumulator a
// lane owns one output row and 4 consecutive columns per register group
// (8/16-byte stores).  W arrives [d_in][d_out] (d_out contiguous); its tiles
// are transposed while staged into LDS (W^T[n][k], 16-byte chunks XOR
// swizzled), X tiles are stored row-major with a 16-byte pad: both MFMA
// operand reads are conflict-free ds_read_b128.  Two LDS stages overlap the
// next tile's global loads with the current MFMAs.
// fp32 path: a plain LDS-tiled fp32 VALU GEMM.
#include "common.hpp"

namespace mot {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int GM = 128;  // rows per workgroup
constexpr int GN = 128;  // cols per workgroup
constexpr int GK = 64;   // depth per stage
constexpr int XROW = GK + 8;
constexpr int X_ELEMS = GM * XROW;
constexpr int W_ELEMS = GN * GK;
constexpr int G_STAGE = X_ELEMS + W_ELEMS;
constexpr int G_SMEM_BYTES = 2 * G_STAGE * 2;

struct GemmParams {
  const bf16_t* x;
  const bf16_t* w[2];
  void* y;
  int64_t row0[2];     // first row of each problem
  int64_t rows[2];     // rows of each problem
  int tiles_m[2];      // row tiles of each problem
  int tiles_n;
  int64_t K, N;
};

__device__ inline bf16x8_t g_as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }
__device__ inline int w_swz(int n, int ck) { return ck ^ ((n >> 1) & 7); }

__device__ inline uint32_t g_pack_bf16(float a, float b) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  bf2 p = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, p);
}

__device__ inline void gemm_load(const GemmParams& p, const bf16_t* w, int64_t mrow0, int64_t mrows,
                                 int64_t n0, int64_t k0, uint4 (&xr)[4], uint4 (&wr)[4]) {
  const int t = threadIdx.x;
  // X: 128 rows x 64 k -> 8 lanes per row, 4 passes of 32 rows
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    int r = t / 8 + 32 * a, c = t % 8;
    int64_t row = mrow0 + r;
    xr[a] = (r < mrows) ? *reinterpret_cast<const uint4*>(p.x + row * p.K + k0 + 8 * c)
                        : make_uint4(0, 0, 0, 0);
  }
  // W: 64 k x 128 n -> thread owns 4 k-rows x 8 n-cols
  const int kb = t % 16, nb = t / 16;
  const int64_t n = n0 + 8 * nb;
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    int64_t k = k0 + 4 * kb + a;
    wr[a] = (n < p.N) ? *reinterpret_cast<const uint4*>(w + k * p.N + n) : make_uint4(0, 0, 0, 0);
  }
}

__device__ inline void gemm_store_lds(bf16_t* xs, bf16_t* ws, uint4 (&xr)[4], uint4 (&wr)[4]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    int r = t / 8 + 32 * a, c = t % 8;
    *reinterpret_cast<uint4*>(xs + r * XROW + 8 * c) = xr[a];
  }
  const int kb = t % 16, nb = t / 16;
  uint32_t w[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    w[a][0] = wr[a].x; w[a][1] = wr[a].y; w[a][2] = wr[a].z; w[a][3] = wr[a].w;
  }
  const int ck = kb >> 1, half = kb & 1;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int cw = e >> 1;
    uint32_t k01, k23;
    if (e & 1) {
      k01 = __builtin_amdgcn_perm(w[1][cw], w[0][cw], 0x07060302u);
      k23 = __builtin_amdgcn_perm(w[3][cw], w[2][cw], 0x07060302u);
    } else {
      k01 = __builtin_amdgcn_perm(w[1][cw], w[0][cw], 0x05040100u);
      k23 = __builtin_amdgcn_perm(w[3][cw], w[2][cw], 0x05040100u);
    }
    const int n = 8 * nb + e;
    *reinterpret_cast<uint2*>(ws + n * GK + 8 * w_swz(n, ck) + 4 * half) = make_uint2(k01, k23);
  }
}

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void gemm_region_bf16(GemmParams p) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  bf16_t* smem = reinterpret_cast<bf16_t*>(smem_raw);
  int b = blockIdx.x;
  int prob = 0;
  const int per0 = p.tiles_m[0] * p.tiles_n;
  if (b >= per0) { prob = 1; b -= per0; }
  const int tn = b % p.tiles_n;
  const int tm = b / p.tiles_n;
  const int64_t mrow0 = p.row0[prob] + (int64_t)tm * GM;
  int64_t mrows = p.rows[prob] - (int64_t)tm * GM;
  if (mrows > GM) mrows = GM;
  const int64_t n0 = (int64_t)tn * GN;
  const bf16_t* w = p.w[prob];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 5, l32 = lane & 31;
  const int wm = wave & 1, wn = wave >> 1;  // wave's 64x64 sub-tile

  f32x16_t acc[2][2];  // [n block][m block]
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  uint4 xr[4], wr[4];
  const int ksteps = (int)(p.K / GK);
  gemm_load(p, w, mrow0, mrows, n0, 0, xr, wr);
  gemm_store_lds(smem, smem + X_ELEMS, xr, wr);
  __syncthreads();
  for (int kt = 0; kt < ksteps; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < ksteps;
    if (more) gemm_load(p, w, mrow0, mrows, n0, (int64_t)(kt + 1) * GK, xr, wr);
    const bf16_t* xs = smem + buf * G_STAGE;
    const bf16_t* ws = xs + X_ELEMS;
#pragma unroll
    for (int s = 0; s < GK / 16; ++s) {
      bf16x8_t bx[2], aw[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int m = 64 * wm + 32 * j + l32;
        bx[j] = g_as_bf16x8(*reinterpret_cast<const uint4*>(xs + m * XROW + 16 * s + 8 * g));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int n = 64 * wn + 32 * i + l32;
        aw[i] = g_as_bf16x8(*reinterpret_cast<const uint4*>(ws + n * GK + 8 * w_swz(n, 2 * s + g)));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aw[i], bx[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      bf16_t* nx = smem + (buf ^ 1) * G_STAGE;
      gemm_store_lds(nx, nx + X_ELEMS, xr, wr);
    }
    __syncthreads();
  }
  // acc[i][j]: C^T block, lane owns output row m = 64wm+32j+l32 and
  // columns n = 64wn + 32i + 8(r/4) + 4g + r%4
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int mloc = 64 * wm + 32 * j + l32;
    if (mloc >= mrows) continue;
    const int64_t row = mrow0 + mloc;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int64_t n = n0 + 64 * wn + 32 * i + 8 * rr + 4 * g;
        if (n >= p.N) continue;
        if (OUT_BF16) {
          uint2 v;
          v.x = g_pack_bf16(acc[i][j][4 * rr + 0], acc[i][j][4 * rr + 1]);
          v.y = g_pack_bf16(acc[i][j][4 * rr + 2], acc[i][j][4 * rr + 3]);
          *reinterpret_cast<uint2*>(reinterpret_cast<bf16_t*>(p.y) + row * p.N + n) = v;
        } else {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.y) + row * p.N + n) =
              make_float4(acc[i][j][4 * rr + 0], acc[i][j][4 * rr + 1], acc[i][j][4 * rr + 2],
                          acc[i][j][4 * rr + 3]);
        }
      }
  }
}

// ---- fp32 VALU path ----
constexpr int FT = 16;

__global__ __launch_bounds__(256) void gemm_region_f32(const float* x, const float* w_ar,
                                                       const float* w_dm, float* y, int64_t M,
                                                       int64_t n_ar, int64_t K, int64_t N) {
  __shared__ float xs[FT][FT + 1];
  __shared__ float wa[FT][FT + 1];
  __shared__ float wd[FT][FT + 1];
  const int tx = threadIdx.x % FT, ty = threadIdx.x / FT;
  const int64_t row = (int64_t)blockIdx.y * FT + ty;
  const int64_t col = (int64_t)blockIdx.x * FT + tx;
  const int64_t rlo = (int64_t)blockIdx.y * FT;
  const bool need_ar = rlo < n_ar, need_dm = rlo + FT > n_ar;
  float acc = 0.f;
  for (int64_t k0 = 0; k0 < K; k0 += FT) {
    xs[ty][tx] = (row < M && k0 + tx < K) ? x[row * K + k0 + tx] : 0.f;
    if (need_ar) wa[ty][tx] = (k0 + ty < K && col < N) ? w_ar[(k0 + ty) * N + col] : 0.f;
    if (need_dm) wd[ty][tx] = (k0 + ty < K && col < N) ? w_dm[(k0 + ty) * N + col] : 0.f;
    __syncthreads();
    const bool ar = row < n_ar;
#pragma unroll
    for (int e = 0; e < FT; ++e) acc = __builtin_fmaf(xs[ty][e], ar ? wa[e][tx] : wd[e][tx], acc);
    __syncthreads();
  }
  if (row < M && col < N) y[row * N + col] = acc;
}

hipError_t region_gemm(const void* x, const void* w_ar, const void* w_dm, void* y, int64_t n_rows,
                       int64_t n_ar, int64_t K, int64_t N, mot_dtype in_dt, mot_dtype out_dt,
                       hipStream_t s) {
  if (in_dt == MOT_FP32) {
    dim3 grid((unsigned)((N + FT - 1) / FT), (unsigned)((n_rows + FT - 1) / FT));
    hipLaunchKernelGGL(gemm_region_f32, grid, dim3(256), 0, s, (const float*)x,
                       (const float*)w_ar, (const float*)w_dm, (float*)y, n_rows, n_ar, K, N);
    return hipGetLastError();
  }
  GemmParams p;
  p.x = (const bf16_t*)x;
  p.w[0] = (const bf16_t*)w_ar;
  p.w[1] = (const bf16_t*)w_dm;
  p.y = y;
  p.row0[0] = 0; p.rows[0] = n_ar;
  p.row0[1] = n_ar; p.rows[1] = n_rows - n_ar;
  p.tiles_m[0] = (int)((p.rows[0] + GM - 1) / GM);
  p.tiles_m[1] = (int)((p.rows[1] + GM - 1) / GM);
  p.tiles_n = (int)((N + GN - 1) / GN);
  p.K = K; p.N = N;
  const int64_t blocks = (int64_t)(p.tiles_m[0] + p.tiles_m[1]) * p.tiles_n;
  if (blocks == 0) return hipSuccess;
  static bool configured[2] = {false, false};
  const int ob = out_dt == MOT_BF16 ? 1 : 0;
  const void* fn = ob ? (const void*)gemm_region_bf16<true> : (const void*)gemm_region_bf16<false>;
  if (!configured[ob]) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, G_SMEM_BYTES);
    if (e != hipSuccess) return e;
    configured[ob] = true;
  }
  if (ob)
    hipLaunchKernelGGL(gemm_region_bf16<true>, dim3((unsigned)blocks), dim3(256), G_SMEM_BYTES, s, p);
  else
    hipLaunchKernelGGL(gemm_region_bf16<false>, dim3((unsigned)blocks), dim3(256), G_SMEM_BYTES, s, p);
  return hipGetLastError();
}

}  // namespace mot
