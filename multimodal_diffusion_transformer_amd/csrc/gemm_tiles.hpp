// Tile geometry and address arithmetic of the direct-to-LDS region GEMM
// (gemm.hip, built with MOT_GEMM_DMA): where each lane's LDS-DMA copy reads
// X and W and writes LDS, and where the MFMA operands are read back.  Plain
// integer arithmetic on __host__ __device__ functions, so a host program can
// walk the copies and operand reads of any problem shape
// (tests/native/gemm_addr_check.hip).
//
// Workgroup tile HM rows x HN cols, HK-deep stages; 4 waves, wave w owning
// rows [128 (w & 1), +128) and cols [64 (w >> 1), +64) as 4 x 2 blocks of
// v_mfma_f32_32x32x16_bf16 on Y^T = W^T X^T.
//  * W tile [HK k][HN n]: 256-byte rows, 16-byte chunk c of row k stored at
//    chunk c ^ 4 (k % 4); read transposed (W^T) with ds_read_b64_tr_b16.
//  * X tile [HM m][HK k]: 64-byte rows, chunk c of row m stored at chunk
//    c ^ ((m / 4) % 2); read with ds_read_b128.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mot {

constexpr int HM = 256;                    // rows per workgroup
constexpr int HN = 128;                    // cols per workgroup
constexpr int HK = 32;                     // depth per stage
constexpr int H_WB = HK * HN * 2;          // W tile bytes (8 KB)
constexpr int H_XB = HM * HK * 2;          // X tile bytes (16 KB)
constexpr int H_STAGE = H_WB + H_XB;       // 24 KB
constexpr int H_SMEM_BYTES = 2 * H_STAGE;  // 48 KB

struct GemmTileAddr {
  // ---- W copies: copy t of wave w is load i = 2w + t, rows 4i .. 4i+3 ----
  __host__ __device__ __forceinline__ static int w_load(int wave, int t) { return 2 * wave + t; }
  __host__ __device__ __forceinline__ static int w_row(int i, int lane) { return 4 * i + lane / 16; }
  // logical chunk the lane's LDS slot (chunk lane % 16 of its row) holds
  __host__ __device__ __forceinline__ static int w_chunk(int row, int lane) { return (lane % 16) ^ (4 * (row & 3)); }
  // element offset of the stage's W tile from w: W[k0][n0]
  __host__ __device__ __forceinline__ static int64_t w_tile_el(int64_t k0, int64_t n0, int64_t N) {
    return k0 * N + n0;
  }
  // full tile: wave-uniform bytes of load i, plus the loop-invariant lane part
  __host__ __device__ __forceinline__ static int64_t w_load_bytes(int i, int64_t N) { return (int64_t)4 * i * N * 2; }
  __host__ __device__ __forceinline__ static uint32_t w_lane_off(int lane, int64_t N) {
    return (uint32_t)((int64_t)(lane / 16) * N * 2 + 16 * w_chunk(lane / 16, lane));
  }
  // ragged last column tile: the full lane offset from the tile base; chunks
  // past the last valid one re-read it (never stored)
  __host__ __device__ __forceinline__ static uint32_t w_ragged_off(int i, int lane, int64_t N, int64_t n0) {
    const int row = w_row(i, lane);
    int c = w_chunk(row, lane);
    const int last_c = (int)((N - n0) / 8) - 1;
    if (c > last_c) c = last_c;
    return (uint32_t)((int64_t)row * N * 2 + c * 16);
  }
  __host__ __device__ __forceinline__ static int w_lds(int i, int lane) { return i * 1024 + 16 * lane; }

  // ---- X copies: copy t of wave w is load i = 4w + t, rows 16i .. 16i+15 ----
  __host__ __device__ __forceinline__ static int x_load(int wave, int t) { return 4 * wave + t; }
  __host__ __device__ __forceinline__ static int x_row(int i, int lane) { return 16 * i + lane / 4; }
  __host__ __device__ __forceinline__ static int x_chunk(int row, int lane) { return (lane % 4) ^ ((row >> 2) & 1); }
  // element offset of the stage's X tile from x: X[r0][k0]
  __host__ __device__ __forceinline__ static int64_t x_tile_el(int64_t r0, int64_t k0, int64_t K) {
    return r0 * K + k0;
  }
  __host__ __device__ __forceinline__ static int64_t x_load_bytes(int i, int64_t K) { return (int64_t)16 * i * K * 2; }
  __host__ __device__ __forceinline__ static uint32_t x_lane_off(int lane, int64_t K) {
    return (uint32_t)((int64_t)(lane / 4) * K * 2 + 16 * x_chunk(lane / 4, lane));
  }
  // ragged last row tile: rows past the problem re-read its last row
  __host__ __device__ __forceinline__ static uint32_t x_ragged_off(int i, int lane, int64_t K, int64_t rows) {
    int64_t row = x_row(i, lane);
    const int c = x_chunk((int)row, lane);
    if (row > rows - 1) row = rows - 1;
    return (uint32_t)(row * K * 2 + c * 16);
  }
  __host__ __device__ __forceinline__ static int x_lds(int i, int lane) { return H_WB + i * 1024 + 16 * lane; }

  // ---- MFMA operand reads within a stage, k-step 0 (k-step s adds
  // 16 s rows of W, 32 s bytes of X) ----
  // A (W^T) of column block nb of wave column wn: the lane's address for the
  // transposing read of 4 k-rows x 4 cols; the second read of the pair adds
  // 4 rows.  Lane j of a 16-lane group points at k-row 8 g + j / 4, cols
  // 64 wn + 32 nb + 16 q16 + 4 (j % 4), so lane j receives 4 consecutive k
  // of col 64 wn + 32 nb + 16 q16 + j (g = lane / 32, q16 = (lane / 16) % 2).
  __host__ __device__ __forceinline__ static uint32_t a_read_off(int wn, int nb, int lane) {
    const int j = lane & 15, q16 = (lane >> 4) & 1, g = lane >> 5;
    const int row = 8 * g + j / 4;  // + 16 s (+ 4): row % 4 unchanged
    const int c = 8 * wn + 4 * nb + 2 * q16 + (j & 3) / 2;
    return (uint32_t)(row * (HN * 2) + ((c ^ (4 * (row & 3))) * 16) + 8 * (j & 1));
  }
  // B (X) of wave row wm, row block 0: row 128 wm + lane % 32, k 8 (lane / 32)
  // + 0..7; row block mb adds 32 mb rows
  __host__ __device__ __forceinline__ static uint32_t b_read_off(int wm, int lane) {
    const int l32 = lane & 31, g = lane >> 5;
    return (uint32_t)((128 * wm + l32) * (HK * 2) + ((g ^ ((l32 >> 2) & 1)) * 16));
  }
};

}  // namespace mot
