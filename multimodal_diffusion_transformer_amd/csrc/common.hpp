// Shared internals of libmotattn: bf16 helpers, the exact mask predicate and
// tile classifier (used by the attention kernels, the mask materialiser and
// the host classifier alike), and launch-status plumbing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/motattn.h"

namespace mot {

typedef uint16_t bf16_t;  // raw bfloat16 bits

__host__ __device__ inline float bf16_to_f32(bf16_t b) {
  union { uint32_t u; float f; } c;
  c.u = (uint32_t)b << 16;
  return c.f;
}

// fp32 -> bf16, round to nearest even (inputs are finite).
__host__ __device__ inline bf16_t f32_to_bf16(float f) {
  union { uint32_t u; float f; } c;
  c.f = f;
  uint32_t bias = ((c.u >> 16) & 1u) + 0x7FFFu;
  return (bf16_t)((c.u + bias) >> 16);
}

// ---------------------------------------------------------------------------
// Masks.  Method page §3 (joint attention): AR queries read AR keys causally,
// DM queries read every key.  Streaming page ("流式生成如何工作"): the cached
// prefix is visible to all; past it, chunk(j) <= chunk(i).  Indices are
// absolute positions in key space.
// ---------------------------------------------------------------------------
struct MaskSpec {
  int32_t mode;
  int64_t nq, nk, q0;
  int64_t n_ar, n_prefix, chunk_len;
};

__host__ __device__ inline int64_t floordiv(int64_t a, int64_t b) {
  int64_t q = a / b;
  return (a % b != 0 && ((a < 0) != (b < 0))) ? q - 1 : q;
}

__host__ __device__ inline bool mask_allowed(const MaskSpec& m, int64_t i, int64_t j) {
  if (m.mode == MOT_AR_CAUSAL_DM_FULL) return (i >= m.n_ar) || (j <= i);
  return (j < m.n_prefix) ||
         (floordiv(j - m.n_prefix, m.chunk_len) <= floordiv(i - m.n_prefix, m.chunk_len));
}

enum TileClass : uint8_t { TILE_EMPTY = 0, TILE_PARTIAL = 1, TILE_FULL = 2 };

// Last key (exclusive) any query in absolute rows [ia, ib] may read.
__host__ __device__ inline int64_t key_end(const MaskSpec& m, int64_t ia, int64_t ib) {
  (void)ia;
  int64_t e;
  if (m.mode == MOT_AR_CAUSAL_DM_FULL) {
    e = (ib >= m.n_ar) ? m.nk : ib + 1;
  } else {
    e = m.n_prefix + (floordiv(ib - m.n_prefix, m.chunk_len) + 1) * m.chunk_len;
  }
  return e < m.nk ? e : m.nk;
}

// Class of the tile of absolute query rows [ia, ib] x keys [ja, jb] (both
// inclusive, already clipped to the valid ranges).  Exact: the predicate is
// monotone in j for every row, so the extreme rows decide.
__host__ __device__ inline TileClass tile_class(const MaskSpec& m, int64_t ia, int64_t ib,
                                                int64_t ja, int64_t jb) {
  if (m.mode == MOT_AR_CAUSAL_DM_FULL) {
    // DM rows allow everything; AR rows allow j <= i.
    bool any_dm = ib >= m.n_ar;
    bool all_dm = ia >= m.n_ar;
    if (all_dm) return TILE_FULL;
    // smallest AR row is ia: full iff jb <= ia
    bool full = jb <= ia;
    if (full) return TILE_FULL;
    if (any_dm) return TILE_PARTIAL;
    // all AR: the largest row ib reads most; empty iff ja > ib
    return (ja > ib) ? TILE_EMPTY : TILE_PARTIAL;
  }
  // chunk mode: row i allows j iff j < n_prefix or chunk(j) <= chunk(i);
  // allowed keys of a row form a prefix [0, key_end(i)).
  int64_t lo = key_end(m, ia, ia);  // fewest keys (smallest row)
  int64_t hi = key_end(m, ib, ib);  // most keys
  if (jb < lo) return TILE_FULL;
  if (ja >= hi) return TILE_EMPTY;
  return TILE_PARTIAL;
}

}  // namespace mot

#define MOT_CHECK_LAUNCH()                                   \
  do {                                                       \
    if (hipGetLastError() != hipSuccess) return MOT_ERR_HIP; \
  } while (0)
