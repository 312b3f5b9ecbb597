// Tile geometry and address arithmetic of the bf16 attention kernel
// (attention.hip): where each lane's LDS-DMA copy reads in global memory
// and writes in LDS, and where each MFMA operand is read back from LDS.
// Everything here is plain integer arithmetic on __host__ __device__
// functions, so a host program can walk every copy and every operand read
// of a launch and check them (tests/native/attn_addr_check.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mot {

constexpr int BN = 64;        // keys per tile
constexpr int NST = BN / 32;  // 32-key MFMA blocks per tile

// Head dimensions the kernel takes: 64, 128, and 80 (hidden 5120 over 64
// query heads).  A tile row is stored with DS = store_dim(D) dims: 80 is
// kept in the 128 geometry (256-byte rows, 16 chunks), whose copies, swizzles
// and transposing reads are the ones already walked; its chunks 10..15 hold
// duplicates of chunks 0..5 of the same row, which no score reads and whose
// outputs (dims 80..95 of the third 32-dim tile) are not stored.
__host__ __device__ constexpr int store_dim(int D) { return D == 80 ? 128 : D; }

template <int D>
struct Lay {
  static constexpr int CH = D / 8;          // 16-byte chunks per row
  static constexpr int ROWB = D * 2;        // bytes per row
  static constexpr int TILE_B = BN * ROWB;  // one K or V tile
  static constexpr int BYTES = 4 * TILE_B;  // K ring (2) + V ring (2)
  static constexpr int RPG = 16 / CH;       // rows per 256-byte bank cycle
  static constexpr int RPI = 64 / CH;       // rows per wave-wide 1 KB load
  static constexpr int NINSTR = BN / RPI;   // 1 KB loads per tile
};

// Chunk swizzles: logical 16-byte chunk c of row r lives at chunk c ^ f(r).
// K rows are read in key_perm order, so one 8-lane group touches rows
// {0..3, 16..19} (+4, +8, ...): the K swizzle gives those eight rows eight
// different chunks (D=128: bits 0-1, 4, 2 of r; D=64: rows are 128 B, so bit
// 0 picks the bank half and bits 1, 2, 4 the chunk).  V is read four rows
// at a time by 16-lane groups; its swizzle separates rows r%4.
template <int D> __host__ __device__ __forceinline__ int swz_k(int r) {
  if constexpr (D == 128) return (r & 3) | (((r >> 4) & 1) << 2) | (((r >> 2) & 1) << 3);
  else return ((r >> 1) & 1) | (((r >> 2) & 1) << 1) | (((r >> 4) & 1) << 2);
}
template <int D> __host__ __device__ __forceinline__ int swz_v(int r) {
  return 4 * ((r / Lay<D>::RPG) % (Lay<D>::CH / 4));
}

// Row of the K tile that feeds MFMA row rho so that lane half g holds keys
// 16g..16g+15 in accumulator registers 0..15.
__host__ __device__ __forceinline__ int key_perm(int rho) { return 16 * ((rho >> 2) & 1) + 4 * (rho >> 3) + (rho & 3); }

// The copies of one tile.  Each wave issues PER_WAVE wave-wide copies; copy
// i of wave w is load n = w * PER_WAVE + i, which fills LDS bytes
// [1024 n, 1024 n + 1024) of the tile, 16 per lane.  The global address is a
// wave-uniform scalar base plus a per-lane unsigned 32-bit offset:
//   scalar base = tensor + 2 * (kbase * ts + head * hs)       (tile_base_el)
//   fast path   : + rows_bytes(n, ts) + lane_off(...)         (all 64 rows valid)
//   ragged tile : + ragged_off(...)                           (rows past the
//                 last key re-read the last key)
template <int D, int W>
struct TileAddr {
  static constexpr int DS = store_dim(D);
  using L = Lay<DS>;
  static constexpr int PER_WAVE = L::NINSTR / W;
  static_assert(PER_WAVE >= 1 && L::NINSTR % W == 0, "loads per wave");
  // With RPI = 64 / CH rows per load, the swizzle bits that vary with the
  // load index are bit 2 of r at D = 128 (so only i & 1 matters) and none at
  // D = 64, or for V: the fast path's lane offset takes NVAR_K values for K
  // and one for V.
  static constexpr int NVAR_K = DS == 128 ? 2 : 1;

  // tile row that lane `lane` of copy i of wave `wave` fills
  __host__ __device__ __forceinline__ static int row_of(int wave, int i, int lane) {
    return (wave * PER_WAVE + i) * L::RPI + lane / L::CH;
  }
  // logical chunk (16 bytes = 8 dims) that lane fills in row r
  template <bool IS_K>
  __host__ __device__ __forceinline__ static int chunk_of(int r, int lane) {
    return (lane % L::CH) ^ (IS_K ? swz_k<DS>(r) : swz_v<DS>(r));
  }
  // chunk of the row in global memory that fills logical chunk c: c itself,
  // or for a stored chunk past the head's D / 8 a duplicate from the start
  // of the same row (in range, finite)
  __host__ __device__ __forceinline__ static int src_chunk(int c) {
    if constexpr (DS == D) return c;
    else return c < D / 8 ? c : c - D / 8;
  }
  // element offset of a tile's base from the tensor pointer
  __host__ __device__ __forceinline__ static int64_t tile_base_el(int64_t kbase, int64_t ts, int head, int64_t hs) {
    return kbase * ts + (int64_t)head * hs;
  }
  // fast path, lane part: rows within the load plus the chunk (loop-invariant)
  template <bool IS_K>
  __host__ __device__ __forceinline__ static uint32_t lane_off(int wave, int i, int lane, int64_t ts) {
    return (uint32_t)((lane / L::CH) * ts * 2 + src_chunk(chunk_of<IS_K>(row_of(wave, i, lane), lane)) * 16);
  }
  // bytes per RPI rows (wave-uniform)
  __host__ __device__ __forceinline__ static uint32_t row_bytes(int64_t ts) { return (uint32_t)(L::RPI * ts * 2); }
  // fast path, wave-uniform part of load n
  __host__ __device__ __forceinline__ static uint32_t rows_bytes(int n, uint32_t row_b) { return (uint32_t)n * row_b; }
  // ragged tile: the full per-lane offset from the tile base; `last` is the
  // tile row of the last key (0 <= last < BN - 1)
  template <bool IS_K>
  __host__ __device__ __forceinline__ static uint32_t ragged_off(int wave, int i, int lane, int64_t ts, int64_t last) {
    const int r = row_of(wave, i, lane);
    const int64_t rr = r > last ? last : r;  // never negative: the lane offset is unsigned
    return (uint32_t)(rr * ts * 2 + src_chunk(chunk_of<IS_K>(r, lane)) * 16);
  }
  // LDS byte offset within the tile that copy n writes for lane
  __host__ __device__ __forceinline__ static int lds_dst(int n, int lane) { return n * 1024 + 16 * lane; }
};

// LDS read offsets of the MFMA operands within one tile, loop-invariant per
// lane.  K (A operand of S^T = K Q^T), k-step s: the lane reads row
// key_perm(lane % 32), logical chunk 2s + lane / 32; score block st adds
// st * 32 rows.
template <int D>
__host__ __device__ __forceinline__ uint32_t k_read_off(int s, int lane) {
  const int row = key_perm(lane & 31);
  return (uint32_t)(row * Lay<D>::ROWB + (((2 * s + (lane >> 5)) ^ swz_k<D>(row)) * 16));
}
// V^T (A operand of O^T += V^T P^T), output tile dt: the lane's address for
// the transposing read of 4 keys x 4 dims; key block st and key half t add
// (32 st + 8 t) rows, the second read of a pair adds 4 rows.  Lane j of a
// 16-lane group points at row 16 g + j / 4, dims 32 dt + 16 q16 + 4 (j % 4),
// so lane j receives 4 consecutive keys of dim 32 dt + 16 q16 + j (g = lane
// / 32, q16 = (lane / 16) % 2).
template <int D>
__host__ __device__ __forceinline__ uint32_t v_read_off(int dt, int lane) {
  const int j = lane & 15, q16 = (lane >> 4) & 1, g = lane >> 5;
  const int rowl = 16 * g + j / 4;  // + 32st + 8t + 4h, all multiples of 4
  const int f = swz_v<D>(rowl);     // so the swizzle is the same for all of them
  const int c = 4 * dt + 2 * q16 + (j & 3) / 2;
  return (uint32_t)(rowl * Lay<D>::ROWB + ((c ^ f) * 16) + 8 * (j & 1));
}

// Head of a workgroup's head slot (blockIdx.x % n_heads).  Workgroups go
// round-robin over the 8 XCDs; with n_heads a multiple of 8, slot hs always
// lands on XCD hs % 8, and XCD x is given heads [x H/8, (x+1) H/8) so that
// the query heads sharing a key/value head (consecutive heads) stay on one
// XCD and its L2.  xcd_heads = H / 8 when H % 8 == 0, else 0 (identity).
__host__ __device__ __forceinline__ int head_of_slot(int hs, int xcd_heads) {
  return xcd_heads ? (hs & 7) * xcd_heads + (hs >> 3) : hs;
}

}  // namespace mot
