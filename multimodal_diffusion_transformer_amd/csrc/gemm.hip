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
//
// Epilogues on the fp32 accumulator, before the store (the rest of the MoT
// layer, §3: each room's MLP and the residual stream): GELU, x Phi(x) in
// its erf form, for the MLP's first matrix; or adding a residual tensor of
// the output's type, read at exactly the offsets the store writes (so it
// may be the output itself), for the output projection and the MLP's
// second matrix.
#include <atomic>
#include <math.h>

#include "common.hpp"
#include "gemm_tiles.hpp"

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

enum Epilogue { EPI_NONE = 0, EPI_GELU = 1, EPI_ADD = 2 };

__device__ __forceinline__ float gelu_erf(float v) { return 0.5f * v * (1.0f + erff(v * 0.70710678118654752f)); }

struct GemmParams {
  const bf16_t* x;
  const bf16_t* w[2];
  void* y;
  const void* res;     // EPI_ADD: residual, the output's type and layout
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

// Applies the epilogue to 4 consecutive outputs at element offset e and
// stores them (the residual, if any, is read at the same offset).
template <bool OUT_BF16, int EPI>
__device__ __forceinline__ void store4(const GemmParams& p, int64_t e, float (&o)[4]) {
  if (EPI == EPI_GELU) {
#pragma unroll
    for (int t = 0; t < 4; ++t) o[t] = gelu_erf(o[t]);
  } else if (EPI == EPI_ADD) {
    if (OUT_BF16) {
      const uint2 r = *reinterpret_cast<const uint2*>(reinterpret_cast<const bf16_t*>(p.res) + e);
      o[0] += __uint_as_float(r.x << 16); o[1] += __uint_as_float(r.x & 0xFFFF0000u);
      o[2] += __uint_as_float(r.y << 16); o[3] += __uint_as_float(r.y & 0xFFFF0000u);
    } else {
      const float4 r = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p.res) + e);
      o[0] += r.x; o[1] += r.y; o[2] += r.z; o[3] += r.w;
    }
  }
  if (OUT_BF16) {
    uint2 v;
    v.x = g_pack_bf16(o[0], o[1]);
    v.y = g_pack_bf16(o[2], o[3]);
    *reinterpret_cast<uint2*>(reinterpret_cast<bf16_t*>(p.y) + e) = v;
  } else {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.y) + e) = make_float4(o[0], o[1], o[2], o[3]);
  }
}

template <bool OUT_BF16, int EPI>
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
        float o[4] = {acc[i][j][4 * rr + 0], acc[i][j][4 * rr + 1], acc[i][j][4 * rr + 2], acc[i][j][4 * rr + 3]};
        store4<OUT_BF16, EPI>(p, row * p.N + n, o);
      }
  }
}

// ---- bf16 path, direct-to-LDS tiles (switched off) ----
//
// Built only with -DMOT_GEMM_DMA=1.  Its first GPU test faulted; the cause
// (a copy reading a base that a VALU wrote with no wait states in between)
// is fixed below, but the fixed kernel has not run on a GPU yet, so the
// library keeps the register-staged kernel above.
#if defined(MOT_GEMM_DMA) && MOT_GEMM_DMA
//
// Workgroup tile 256 rows x 128 cols, 32-deep stages, two LDS stages (48 KB),
// 4 waves each owning 128 rows x 64 cols as 4x2 v_mfma_f32_32x32x16_bf16
// blocks of Y^T = W^T X^T.  Both operands go from HBM straight into LDS with
// global_load_lds_dwordx4 (no staging registers, no VALU):
//  * W tile [32 k][128 n], 256-byte rows, 16-byte chunks XOR-swizzled by
//    4 (k % 4); read transposed (W^T) with ds_read_b64_tr_b16;
//  * X tile [256 m][32 k], 64-byte rows, chunks XOR-swizzled by (m / 4) % 2;
//    read with ds_read_b128.
// Both reads are bank-conflict free.  The next stage's copies are issued at
// the start of a stage and waited for at its end; inside a stage the second
// k-step's operands are read under the first k-step's MFMAs.  The tile
// geometry and every address are GemmTileAddr's (gemm_tiles.hpp).
static_assert(H_SMEM_BYTES <= 65536, "LDS copies stay below 64 KB");

// One wave-wide 16-byte-per-lane copy from global memory (scalar base +
// per-lane unsigned 32-bit offset) into LDS at `lds` + 16 * lane.  Here the
// tile bases are computed on the vector ALUs (block -> tile division) and
// reach the SGPR pair through v_readfirstlane; the hardware needs 5 wait
// states between that VALU write of an SGPR and the copy that reads it, and
// the compiler inserts none in front of inline asm, so the asm provides them.
__device__ __forceinline__ void g_dma16(const void* gbase, uint32_t voff, uint32_t lds) {
  const uint64_t b = (uint64_t)gbase;
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint64_t sb = ((uint64_t)hi << 32) | (uint64_t)lo;
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sb), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ uint32_t g_lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ void g_wait_vmem0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

typedef short g_s16x4_t __attribute__((ext_vector_type(4)));
typedef short g_s16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) g_s16x4_t g_lds_s16x4_t;

// Issue this wave's copies of one stage: W rows [k0, k0+32) x cols [n0, n0+128)
// (2 loads of 4 rows) and X rows [r0, r0+256) of the problem x k [k0, k0+32)
// (4 loads of 16 rows).  Columns past N and rows past the problem re-read
// the last valid ones: never out of range, never stored.
__device__ __forceinline__ void h_issue(const GemmParams& p, const bf16_t* w, int64_t r0, int64_t rows,
                                        int64_t n0, int64_t k0, int wave, int lane, uint32_t lw,
                                        uint32_t lx, unsigned char* dst) {
  using A = GemmTileAddr;
  const int64_t N = p.N, K = p.K;
  const char* wb = reinterpret_cast<const char*>(w) + A::w_tile_el(k0, n0, N) * 2;
  const bool ragged_n = n0 + HN > N;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int i = A::w_load(wave, t);
    if (__builtin_expect(!ragged_n, 1))
      g_dma16(wb + A::w_load_bytes(i, N), lw, g_lds_addr(dst + A::w_lds(i, 0)));
    else
      g_dma16(wb, A::w_ragged_off(i, lane, N, n0), g_lds_addr(dst + A::w_lds(i, 0)));
  }
  const char* xb = reinterpret_cast<const char*>(p.x) + A::x_tile_el(r0, k0, K) * 2;
  const bool ragged_m = rows < HM;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int i = A::x_load(wave, t);
    if (__builtin_expect(!ragged_m, 1))
      g_dma16(xb + A::x_load_bytes(i, K), lx, g_lds_addr(dst + A::x_lds(i, 0)));
    else
      g_dma16(xb, A::x_ragged_off(i, lane, K, rows), g_lds_addr(dst + A::x_lds(i, 0)));
  }
}

template <bool OUT_BF16, int EPI>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_region_mfma(GemmParams p) {
  extern __shared__ __align__(16) unsigned char hsm[];
  int b = blockIdx.x;
  int prob = 0;
  const int per0 = p.tiles_m[0] * p.tiles_n;
  if (b >= per0) { prob = 1; b -= per0; }
  const int tn = b % p.tiles_n;
  const int tm = b / p.tiles_n;
  const int64_t r0 = p.row0[prob] + (int64_t)tm * HM;
  int64_t rows = p.rows[prob] - (int64_t)tm * HM;
  if (rows > HM) rows = HM;
  const int64_t n0 = (int64_t)tn * HN;
  const bf16_t* w = p.w[prob];

  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int g = lane >> 5, l32 = lane & 31;
  const int wm = wave & 1, wn = wave >> 1;  // wave's rows [128 wm, +128), cols [64 wn, +64)

  // loop-invariant lane offsets of the copies (bytes, from the tile base)
  const uint32_t lw = GemmTileAddr::w_lane_off(lane, p.N);
  const uint32_t lx = GemmTileAddr::x_lane_off(lane, p.K);
  // LDS operand offsets within a stage, k-step 0: W^T (transposed reads) for
  // the wave's two 32-col blocks, X for its four 32-row blocks
  uint32_t aoff[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) aoff[nb] = GemmTileAddr::a_read_off(wn, nb, lane);
  const uint32_t boff = GemmTileAddr::b_read_off(wm, lane);

  f32x16_t acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int ksteps = (int)(p.K / HK);
  h_issue(p, w, r0, rows, n0, 0, wave, lane, lw, lx, hsm);
  g_wait_vmem0();
  __syncthreads();
  for (int kt = 0; kt < ksteps; ++kt) {
    unsigned char* cur = hsm + (kt & 1) * H_STAGE;
    if (kt + 1 < ksteps)
      h_issue(p, w, r0, rows, n0, (int64_t)(kt + 1) * HK, wave, lane, lw, lx, hsm + ((kt + 1) & 1) * H_STAGE);
    const unsigned char* wt = cur;
    const unsigned char* xt = cur + H_WB;
    bf16x8_t a[2][2], bx[2][4];  // [k-step][block]
    auto read_a = [&](int s, int nb) {
      const unsigned char* base = wt + aoff[nb] + 16 * s * (HN * 2);
      g_s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((g_lds_s16x4_t*)(base));
      g_s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((g_lds_s16x4_t*)(base + 4 * (HN * 2)));
      g_s16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      a[s][nb] = __builtin_bit_cast(bf16x8_t, v);
    };
    auto read_b = [&](int s, int mb) {
      bx[s][mb] = g_as_bf16x8(*reinterpret_cast<const uint4*>(xt + boff + mb * 32 * (HK * 2) + 32 * s));
    };
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) read_a(0, nb);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) read_b(0, mb);
    __builtin_amdgcn_sched_barrier(0);
    // k-step 0: 8 MFMAs, each followed by one operand read of k-step 1
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int mb = q / 2, nb = q % 2;
      acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0][nb], bx[0][mb], acc[nb][mb], 0, 0, 0);
      if (q < 2) read_a(1, q);
      else if (q < 6) read_b(1, q - 2);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int mb = q / 2, nb = q % 2;
      acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1][nb], bx[1][mb], acc[nb][mb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    g_wait_vmem0();
    __syncthreads();
  }
  // acc[nb][mb]: Y^T block; the lane owns output row m = 128 wm + 32 mb + l32
  // and columns n = 64 wn + 32 nb + 8 (r / 4) + 4 g + r % 4
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int mloc = 128 * wm + 32 * mb + l32;
    if (mloc >= rows) continue;
    const int64_t row = r0 + mloc;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int64_t n = n0 + 64 * wn + 32 * nb + 8 * rr + 4 * g;
        if (n >= p.N) continue;
        float o[4] = {acc[nb][mb][4 * rr + 0], acc[nb][mb][4 * rr + 1], acc[nb][mb][4 * rr + 2],
                      acc[nb][mb][4 * rr + 3]};
        store4<OUT_BF16, EPI>(p, row * p.N + n, o);
      }
  }
}

template <bool OB>
static hipError_t launch_dma_gemm(const GemmParams& p, int epi, int64_t blocks, hipStream_t s) {
  static std::atomic<bool> configured[3] = {{false}, {false}, {false}};
  const void* fn = epi == EPI_GELU ? (const void*)gemm_region_mfma<OB, EPI_GELU>
                   : epi == EPI_ADD ? (const void*)gemm_region_mfma<OB, EPI_ADD>
                                    : (const void*)gemm_region_mfma<OB, EPI_NONE>;
  if (!configured[epi].load(std::memory_order_acquire)) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, H_SMEM_BYTES);
    if (e != hipSuccess) return e;
    configured[epi].store(true, std::memory_order_release);
  }
  const dim3 grid((unsigned)blocks), block(256);
  if (epi == EPI_GELU) hipLaunchKernelGGL((gemm_region_mfma<OB, EPI_GELU>), grid, block, H_SMEM_BYTES, s, p);
  else if (epi == EPI_ADD) hipLaunchKernelGGL((gemm_region_mfma<OB, EPI_ADD>), grid, block, H_SMEM_BYTES, s, p);
  else hipLaunchKernelGGL((gemm_region_mfma<OB, EPI_NONE>), grid, block, H_SMEM_BYTES, s, p);
  return hipGetLastError();
}

#endif  // MOT_GEMM_DMA

// ---- fp32 VALU path ----
constexpr int FT = 16;

template <int EPI>
__global__ __launch_bounds__(256) void gemm_region_f32(const float* x, const float* w_ar,
                                                       const float* w_dm, float* y, int64_t M,
                                                       int64_t n_ar, int64_t K, int64_t N,
                                                       const float* res) {
  __shared__ float xs[FT][FT + 1];
  __shared__ float wa[FT][FT + 1];
  __shared__ float wd[FT][FT + 1];
  const int tx = threadIdx.x % FT, ty = threadIdx.x / FT;
  const int64_t row = (int64_t)blockIdx.y * FT + ty;
  const int64_t col = (int64_t)blockIdx.x * FT + tx;
  // the tile's rows clipped to [0, M): a room's weights are read only when
  // one of the tile's real rows belongs to it (the caller may pass NULL for
  // a room with no rows)
  const int64_t rlo = (int64_t)blockIdx.y * FT;
  const int64_t rhi = rlo + FT < M ? rlo + FT : M;  // exclusive
  const bool need_ar = rlo < n_ar, need_dm = rhi > n_ar;
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
  if (row < M && col < N) {
    if (EPI == EPI_GELU) acc = gelu_erf(acc);
    else if (EPI == EPI_ADD) acc += res[row * N + col];
    y[row * N + col] = acc;
  }
}

// Whether one dispatch (at most 2^32 - 1 work-items along a grid dimension)
// covers the problem: fp32 launches FT x FT output tiles of 256 lanes on a
// 2D grid; bf16 launches one GM x GN tile of 256 lanes per workgroup for
// each room's rows (the direct-to-LDS kernel's tiles are larger).
bool region_gemm_fits(int64_t n_rows, int64_t n_ar, int64_t N, mot_dtype in_dt) {
  const int64_t lim = (int64_t)UINT32_MAX;
  if (in_dt == MOT_FP32) return (N + FT - 1) / FT <= lim / 256 && (n_rows + FT - 1) / FT <= lim;
  const int64_t tiles_m = (n_ar + GM - 1) / GM + (n_rows - n_ar + GM - 1) / GM;
  const int64_t tiles_n = (N + GN - 1) / GN;
  return tiles_n <= lim / 256 && tiles_m <= lim / 256 / tiles_n;
}

template <bool OB>
static hipError_t launch_bf16_gemm(const GemmParams& p, int epi, int64_t blocks, hipStream_t s) {
  // Set the LDS size attribute once per kernel; concurrent first calls may
  // both set it (it is idempotent), and the flag itself is atomic.
  static std::atomic<bool> configured[3] = {{false}, {false}, {false}};
  const void* fn = epi == EPI_GELU ? (const void*)gemm_region_bf16<OB, EPI_GELU>
                   : epi == EPI_ADD ? (const void*)gemm_region_bf16<OB, EPI_ADD>
                                    : (const void*)gemm_region_bf16<OB, EPI_NONE>;
  if (!configured[epi].load(std::memory_order_acquire)) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, G_SMEM_BYTES);
    if (e != hipSuccess) return e;
    configured[epi].store(true, std::memory_order_release);
  }
  const dim3 grid((unsigned)blocks), block(256);
  if (epi == EPI_GELU) hipLaunchKernelGGL((gemm_region_bf16<OB, EPI_GELU>), grid, block, G_SMEM_BYTES, s, p);
  else if (epi == EPI_ADD) hipLaunchKernelGGL((gemm_region_bf16<OB, EPI_ADD>), grid, block, G_SMEM_BYTES, s, p);
  else hipLaunchKernelGGL((gemm_region_bf16<OB, EPI_NONE>), grid, block, G_SMEM_BYTES, s, p);
  return hipGetLastError();
}

hipError_t region_gemm(const void* x, const void* w_ar, const void* w_dm, void* y, int64_t n_rows,
                       int64_t n_ar, int64_t K, int64_t N, mot_dtype in_dt, mot_dtype out_dt,
                       int epi, const void* res, hipStream_t s) {
  if (in_dt == MOT_FP32) {
    dim3 grid((unsigned)((N + FT - 1) / FT), (unsigned)((n_rows + FT - 1) / FT));
    const float *xf = (const float*)x, *wa = (const float*)w_ar, *wd = (const float*)w_dm;
    const float* rf = (const float*)res;
    if (epi == EPI_GELU)
      hipLaunchKernelGGL(gemm_region_f32<EPI_GELU>, grid, dim3(256), 0, s, xf, wa, wd, (float*)y, n_rows, n_ar, K, N, rf);
    else if (epi == EPI_ADD)
      hipLaunchKernelGGL(gemm_region_f32<EPI_ADD>, grid, dim3(256), 0, s, xf, wa, wd, (float*)y, n_rows, n_ar, K, N, rf);
    else
      hipLaunchKernelGGL(gemm_region_f32<EPI_NONE>, grid, dim3(256), 0, s, xf, wa, wd, (float*)y, n_rows, n_ar, K, N, rf);
    return hipGetLastError();
  }
  GemmParams p;
  p.res = res;
  p.x = (const bf16_t*)x;
  p.w[0] = (const bf16_t*)w_ar;
  p.w[1] = (const bf16_t*)w_dm;
  p.y = y;
  p.row0[0] = 0; p.rows[0] = n_ar;
  p.row0[1] = n_ar; p.rows[1] = n_rows - n_ar;
  p.K = K; p.N = N;
#if defined(MOT_GEMM_DMA) && MOT_GEMM_DMA
  if (K % HK == 0 && N % 64 == 0) {  // direct-to-LDS MFMA kernel
    p.tiles_m[0] = (int)((p.rows[0] + HM - 1) / HM);
    p.tiles_m[1] = (int)((p.rows[1] + HM - 1) / HM);
    p.tiles_n = (int)((N + HN - 1) / HN);
    const int64_t blocks = (int64_t)(p.tiles_m[0] + p.tiles_m[1]) * p.tiles_n;
    if (blocks == 0) return hipSuccess;
    return out_dt == MOT_BF16 ? launch_dma_gemm<true>(p, epi, blocks, s) : launch_dma_gemm<false>(p, epi, blocks, s);
  }
#endif
  p.tiles_m[0] = (int)((p.rows[0] + GM - 1) / GM);
  p.tiles_m[1] = (int)((p.rows[1] + GM - 1) / GM);
  p.tiles_n = (int)((N + GN - 1) / GN);
  const int64_t blocks = (int64_t)(p.tiles_m[0] + p.tiles_m[1]) * p.tiles_n;
  if (blocks == 0) return hipSuccess;
  return out_dt == MOT_BF16 ? launch_bf16_gemm<true>(p, epi, blocks, s) : launch_bf16_gemm<false>(p, epi, blocks, s);
}

}  // namespace mot
