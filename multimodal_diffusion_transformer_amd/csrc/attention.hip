// Masked flash attention on bf16 MFMA for gfx950.
//
// Computes, per head, O = softmax(mask(Q K^T * scale)) V: the joint
// attention of "Cosmos 3 方法原理全解" §3 (AR causal, DM full over [K_AR;K_DM])
// and the chunk-causal streaming attention of "流式生成如何工作".
//
// Design (one workgroup = WAVES waves x 32 query rows of one head, 64-key
// tiles):
//  * The score tile is computed transposed, S^T = K Q^T, on
//    v_mfma_f32_32x32x16_bf16.  In the 32x32 accumulator layout a lane owns
//    one column, so every lane owns ONE query and 16 of its keys per
//    32-key block; row statistics are per-lane scalars and the only
//    cross-lane step (a permlane32 swap) runs on a row's first tile, when a
//    reference max moves, and once at the end for the row sums.
//  * K rows are fed to the MFMA in a permuted order so that lane half g
//    ends up holding keys 16g..16g+15 of each 32-key block in register
//    order.  Those registers, packed to bf16, are exactly the B operand of
//    O^T += V^T P^T for 8 consecutive keys: P never leaves registers.
//  * Software pipeline inside each wave, one fixed schedule per key tile:
//    step j computes the scores of tile j+1 and the PV product of tile j-1
//    on the MFMA while the vector ALUs run the exponentials of tile j.  The
//    three streams are independent inside a step, so score and PV MFMAs
//    alternate, the exponentials are spread evenly between them, each MFMA's
//    LDS operand is read two MFMAs ahead, and a scheduling fence after every
//    MFMA keeps that order.  K runs two tiles ahead of V: K and V have
//    separate two-slot LDS rings, filled straight from HBM with
//    global_load_lds_dwordx4 (no staging registers, no VALU; issued from
//    inline asm with vmcnt managed here, so a copy overlaps the compute
//    before it instead of being drained at the next LDS read).
//  * LDS tiles are row-major with their 16-byte chunks XOR-swizzled per
//    row.  K is read as the A operand with ds_read_b128; V^T is read with
//    ds_read_b64_tr_b16, the gfx950 transposing LDS read (lane i of a
//    16-lane group gets 4 consecutive keys of one column).  The swizzles make
//    both reads bank-conflict free; all LDS addresses are loop-invariant per
//    lane and tile bases are scalar.
//  * Q (rotated by mRoPE on load when positions are given) lives in
//    registers for the whole key loop.  K is used as given (rotated
//    beforehand when positions apply).
//  * Head dims 64 and 128, and 80 (the model table's largest model: hidden
//    5120 over 64 query heads, method page §12.4).  D = 80 tiles are kept
//    in the 128 layout (attn_tiles.hpp); its scores take 5 k-steps, its PV
//    products 3 output tiles of 32 dims, the last one half padding that is
//    never stored, so 10 score and 12 PV MFMAs share a step's schedule.
//  * Softmax in fp32 in the log2 domain (scale*log2(e) folded into one FMA
//    before exp2).  A row's reference is its exact max over its first tile
//    (which always holds key 0); it moves only if a later tile's sum of P
//    passes 2^64, in a rare path that recomputes that tile's scores from K
//    in global memory.  The common tile needs no max, no cross-lane step and
//    no rescale.  Row sums accumulate the bf16-packed P with dot2, so
//    numerator and denominator use the same P.
//  * Both masks give every query a prefix of the keys, [0, key_end(i)).  A
//    per-lane limit decides each pair with one compare, and the limits of a
//    wave's first and last rows classify its tiles exactly: tiles past a
//    wave's last allowed key are skipped, full tiles run unmasked, only
//    partial tiles are masked.
//  * Grid: head is the fastest index, so with H a multiple of 8 every head
//    stays on one XCD (workgroups go round-robin over the 8 XCDs) and shares
//    that XCD's L2; query tiles are issued heaviest first.
#include <atomic>

#include "attn_tiles.hpp"
#include "common.hpp"
#include "rope_dev.hpp"

namespace mot {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

struct AttnParams {
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;
  bf16_t* o;
  float* lse;
  int64_t q_ts, q_hs, k_ts, k_hs, v_ts, v_hs, o_ts, o_hs;
  MaskSpec m;
  int n_heads;
  int kv_group;   // query heads per key/value head
  int xcd_heads;  // heads per XCD when n_heads % 8 == 0, else 0
  int n_qtiles;
  float c_log2;  // scale * log2(e)
  const float* q_pos;
  int64_t q_bs, k_bs, v_bs, o_bs;  // batch strides (elements); grid y is the batch item
  RopeTable rope;
};

constexpr float OVERFLOW_SUM = 18446744073709551616.f;  // 2^64: a lane's tile sum above this moves the reference
// Waves per workgroup (32 query rows each).  Fixed at 4: the only shape
// whose LDS ring, copy count and occupancy have run on the GPU.  An 8-wave
// shape with a 128 KB ring faulted once with no cause found, so no build
// switch selects another count.
constexpr int ATTN_WAVES = 4;

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  bf2 p = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, p);
}

// One wave-wide 16-byte-per-lane copy from global memory (scalar base +
// per-lane offset, which the hardware adds as an unsigned 32-bit value, so it
// must never be "negative") straight into LDS at `lds` + 16 * lane.  Written as
// inline asm so the compiler does not drain every outstanding copy before
// each LDS read (it cannot tell that the copies target another stage); the
// kernel waits on vmcnt itself.  The instruction has no VGPR result.
//
// Hazards: the compiler inserts no wait states in front of inline asm.
//  * A VALU write of an SGPR needs 5 before a vector-memory instruction reads
//    it.  The base must therefore reach the SGPR pair through scalar
//    instructions (as every tile base here does: it is built from kernel
//    arguments and wave-uniform loop counters); a base that only exists in
//    VGPRs, moved over by v_readfirstlane right before the copy, makes the
//    copy read a stale base.
//  * A scalar write of M0 (the LDS destination, set by the "{m0}"
//    constraint just before the asm) needs 1 before an LDS-DMA copy reads
//    it; the asm starts with s_nop 0 for that.
// A host test scans the built library for both patterns.
__device__ __forceinline__ void dma16(const void* gbase, uint32_t voff, uint32_t lds) {
  // the tile base is wave-uniform by construction; make it an SGPR pair
  // (readfirstlane returns int: go through uint32_t so nothing sign-extends)
  const uint64_t b = (uint64_t)gbase;
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint64_t sb = ((uint64_t)hi << 32) | (uint64_t)lo;
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sb), "{m0}"(lds) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

__device__ __forceinline__ void wait_vmem0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Issues the LDS-DMA copies of K and V tiles; the address arithmetic is
// TileAddr's (attn_tiles.hpp), which a host program checks for every copy.
template <int D, int W>
struct TileLoader {
  using A = TileAddr<D, W>;
  static constexpr int PER_WAVE = A::PER_WAVE;
  static constexpr int NVAR_K = A::NVAR_K;
  uint32_t lk[NVAR_K], lv;    // lane parts of the byte offsets
  uint32_t k_row_b, v_row_b;  // bytes per RPI rows (wave-uniform)
  int wave;                   // wave-uniform

  __device__ __forceinline__ void init(int wave_, int lane, int64_t k_ts, int64_t v_ts) {
    wave = wave_;
    k_row_b = A::row_bytes(k_ts);
    v_row_b = A::row_bytes(v_ts);
#pragma unroll
    for (int i = 0; i < NVAR_K; ++i) lk[i] = A::template lane_off<true>(wave, i, lane, k_ts);
    lv = A::template lane_off<false>(wave, 0, lane, v_ts);
  }

  // Issue this wave's share of one tile (K or V) of key/value head `head`
  // of `tensor` (this workgroup's batch item) starting at key kbase into the
  // LDS tile at `dst`.  Rows past the last key re-read the last key (never
  // out of range; those scores are masked and the values finite).
  template <bool IS_K>
  __device__ __forceinline__ void issue(const AttnParams& p, const bf16_t* tensor, int head, int64_t kbase,
                                        unsigned char* dst) const {
    const int64_t ts = IS_K ? p.k_ts : p.v_ts;
    const char* base = reinterpret_cast<const char*>(tensor) +
                       A::tile_base_el(kbase, ts, head, IS_K ? p.k_hs : p.v_hs) * 2;
    const int64_t last = p.m.nk - 1 - kbase;  // last valid tile row
    if (__builtin_expect(last >= BN - 1, 1)) {
#pragma unroll
      for (int i = 0; i < PER_WAVE; ++i) {
        const int n = wave * PER_WAVE + i;
        const uint32_t rows_b = A::rows_bytes(n, IS_K ? k_row_b : v_row_b);  // wave-uniform
        dma16(base + rows_b, IS_K ? lk[i % NVAR_K] : lv, lds_addr(dst + A::lds_dst(n, 0)));
      }
    } else {  // the ragged last tile: full per-lane offsets from the tile base
      const int lane = threadIdx.x & 63;
#pragma unroll
      for (int i = 0; i < PER_WAVE; ++i) {
        const int n = wave * PER_WAVE + i;
        dma16(base, A::template ragged_off<IS_K>(wave, i, lane, ts, last), lds_addr(dst + A::lds_dst(n, 0)));
      }
    }
  }
};

// Rotate one row's chunk pair by mRoPE in registers: lo holds dims
// 16s+8g..+7 and hi the dims D/2 above them, which are their rotate-half
// partners.  pp points at the row's (t, h, w).
template <int D>
__device__ __forceinline__ void rope_chunk_pair(const RopeTable& rt, const float* pp, int s, int g, uint4& lo, uint4& hi) {
  const uint32_t lw[4] = {lo.x, lo.y, lo.z, lo.w};
  const uint32_t hw[4] = {hi.x, hi.y, hi.z, hi.w};
  float y1[8], y2[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int kk = 16 * s + 8 * g + e;
    float cs, sn;
    rope_cs(pp[rope_axis(rt, kk)], rt.inv_freq[kk], cs, sn);
    const float x1 = __uint_as_float((e & 1) ? (lw[e >> 1] & 0xFFFF0000u) : (lw[e >> 1] << 16));
    const float x2 = __uint_as_float((e & 1) ? (hw[e >> 1] & 0xFFFF0000u) : (hw[e >> 1] << 16));
    y1[e] = __builtin_fmaf(x1, cs, -x2 * sn);
    y2[e] = __builtin_fmaf(x1, sn, x2 * cs);
  }
  lo = make_uint4(pack_bf16(y1[0], y1[1]), pack_bf16(y1[2], y1[3]), pack_bf16(y1[4], y1[5]), pack_bf16(y1[6], y1[7]));
  hi = make_uint4(pack_bf16(y2[0], y2[1]), pack_bf16(y2[2], y2[3]), pack_bf16(y2[4], y2[5]), pack_bf16(y2[6], y2[7]));
}

// Rotate one row's chunk by mRoPE when its rotate-half partners, D/2 dims
// away, lie in the other lane half (D = 80: D/2 is not a multiple of 16):
// own holds dims d..d+7, part the dims D/2 above them (d < D/2) or below
// them, loaded by this lane too; only own is rotated, with the same
// arithmetic as rope_chunk_pair.
template <int D>
__device__ __forceinline__ void rope_chunk_half(const RopeTable& rt, const float* pp, int d, uint4& own,
                                                const uint4& part) {
  constexpr int P = D / 2;
  const uint32_t ow[4] = {own.x, own.y, own.z, own.w};
  const uint32_t pw[4] = {part.x, part.y, part.z, part.w};
  const bool first = d < P;
  const int k0 = first ? d : d - P;
  float y[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float cs, sn;
    rope_cs(pp[rope_axis(rt, k0 + e)], rt.inv_freq[k0 + e], cs, sn);
    const float xo = __uint_as_float((e & 1) ? (ow[e >> 1] & 0xFFFF0000u) : (ow[e >> 1] << 16));
    const float xp = __uint_as_float((e & 1) ? (pw[e >> 1] & 0xFFFF0000u) : (pw[e >> 1] << 16));
    y[e] = first ? __builtin_fmaf(xo, cs, -xp * sn) : __builtin_fmaf(xp, sn, xo * cs);
  }
  own = make_uint4(pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3]), pack_bf16(y[4], y[5]), pack_bf16(y[6], y[7]));
}

// Per-wave state of the key loop.
template <int D>
struct WaveState {
  static constexpr int KSTEPS = D / 16;       // MFMA k-steps over the head dim
  static constexpr int DT = (D + 31) / 32;    // 32-wide output tiles (D = 80: the third ends past D)
  static constexpr int NSM = NST * KSTEPS;    // score MFMAs per tile
  static constexpr int NPV = NST * 2 * DT;    // PV MFMAs per tile
  static_assert(D % 32 != 0 || NSM == NPV, "score and PV MFMAs alternate one to one");
  bf16x8_t qreg[KSTEPS];   // B operand of S^T = K Q^T
  uint32_t kaddr[KSTEPS];  // K operand offsets within a K tile
  uint32_t vaddr[DT];      // V^T operand offsets within a V tile
  f32x16_t oacc[DT];
  float m_ref;  // reference maximum (log2 domain): P = exp2(S c - m_ref)
  float l_run;  // this lane's partial row sum
  int lim;      // this lane's key limit
};

// A operand of score MFMA n: 32-key block n / KSTEPS, k-step n % KSTEPS.
template <int D>
__device__ __forceinline__ bf16x8_t k_operand(const WaveState<D>& ws, const unsigned char* ktile, int n) {
  const int st = n / WaveState<D>::KSTEPS, s = n % WaveState<D>::KSTEPS;
  return as_bf16x8(*reinterpret_cast<const uint4*>(ktile + ws.kaddr[s] + st * 32 * Lay<store_dim(D)>::ROWB));
}

// A operand (V^T, 32 dims x 8+8 keys) of PV MFMA n: key block n / (2 DT),
// output tile n % DT, key half (n / DT) % 2.
template <int D>
__device__ __forceinline__ bf16x8_t v_operand(const WaveState<D>& ws, const unsigned char* vtile, int n) {
  constexpr int DT = WaveState<D>::DT;
  const int st = n / (2 * DT), dt = n % DT, t = (n / DT) % 2;
  constexpr int ROWB = Lay<store_dim(D)>::ROWB;
  const unsigned char* base = vtile + ws.vaddr[dt] + (32 * st + 8 * t) * ROWB;
  s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(base));
  s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(base + 4 * ROWB));
  s16x8_t a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8_t, a8);
}

// One step of the key loop, as a fixed instruction schedule.  It runs up to
// three independent streams:
//   DO_S : the score MFMAs of the next tile, nxt = K(j+1) Q^T;
//   DO_PV: the PV MFMAs of the previous tile, O^T += V(j-1)^T P(j-1)^T;
//   DO_E : the exponentials of this tile, P(j) = exp2(cur * c - m_ref)
//          packed to bf16, and their lane sum (c = scale * log2(e)).
// No stream depends on another inside a step, so the schedule alternates
// score and PV MFMAs (with unequal counts, D = 80's 10 and 12, score MFMA
// number floor(m NSM / NM) goes wherever that count steps), spreads the VALU
// operations of the exponentials evenly between them, and reads each MFMA's
// LDS operand PD MFMAs ahead.  A scheduling fence after every MFMA keeps
// that order.
template <int D, bool DO_S, bool DO_E, bool DO_PV>
__device__ __forceinline__ void tile_step(WaveState<D>& ws, const unsigned char* ktile,
                                          const unsigned char* vtile, const f32x16_t (&cur)[NST],
                                          f32x16_t (&nxt)[NST], const bf16x8_t (&pprev)[NST][2],
                                          bf16x8_t (&pcur)[NST][2], float c, float& l_tile) {
  using WS = WaveState<D>;
  constexpr int NM = (DO_S ? WS::NSM : 0) + (DO_PV ? WS::NPV : 0);
  constexpr int OPP = 6;  // per value pair: fma, fma, exp, exp, pack, dot2
  constexpr int NOPS = DO_E ? OPP * NST * 8 : 0;
  const f32x16_t zero16 = {};
  constexpr int PD = 2, NB = PD + 1;
  const bf16x2_t ones2 = {(__bf16)1.0f, (__bf16)1.0f};
  constexpr bool EVEN = WS::NSM == WS::NPV;
  auto s_step = [](int m) { return (m + 1) * WS::NSM / NM != m * WS::NSM / NM; };
  auto is_s = [&](int m) { return DO_S && (!DO_PV || (EVEN ? m % 2 == 0 : s_step(m))); };
  auto idx = [&](int m) {
    if (!(DO_S && DO_PV)) return m;
    if (EVEN) return m / 2;
    return s_step(m) ? m * WS::NSM / NM : m - m * WS::NSM / NM;
  };
  bf16x8_t ops[NB];
#pragma unroll
  for (int m = 0; m < PD && m < NM; ++m)
    ops[m] = is_s(m) ? k_operand<D>(ws, ktile, idx(m)) : v_operand<D>(ws, vtile, idx(m));
  float ex0 = 0.f, ex1 = 0.f;
  uint32_t w[NST][2][4];
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    if (m + PD < NM)
      ops[(m + PD) % NB] = is_s(m + PD) ? k_operand<D>(ws, ktile, idx(m + PD))
                                        : v_operand<D>(ws, vtile, idx(m + PD));
    if (is_s(m)) {
      const int n = idx(m), st = n / WS::KSTEPS, s = n % WS::KSTEPS;
      nxt[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ops[m % NB], ws.qreg[s], s == 0 ? zero16 : nxt[st],
                                                        0, 0, 0);
    } else {
      const int n = idx(m), st = n / (2 * WS::DT), dt = n % WS::DT, t = (n / WS::DT) % 2;
      ws.oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ops[m % NB], pprev[st][t], ws.oacc[dt], 0, 0, 0);
    }
    if (DO_E) {
#pragma unroll
      for (int k = m * NOPS / NM; k < (m + 1) * NOPS / NM; ++k) {
        const int pr = k / OPP, kind = k % OPP;
        const int st = pr / 8, t = (pr % 8) / 4, e = pr % 4, r0 = 8 * t + 2 * e;
        if (kind == 0) {
          ex0 = __builtin_fmaf(cur[st][r0], c, -ws.m_ref);
        } else if (kind == 1) {
          ex1 = __builtin_fmaf(cur[st][r0 + 1], c, -ws.m_ref);
        } else if (kind == 2) {
          ex0 = __builtin_amdgcn_exp2f(ex0);
        } else if (kind == 3) {
          ex1 = __builtin_amdgcn_exp2f(ex1);
        } else if (kind == 4) {
          w[st][t][e] = pack_bf16(ex0, ex1);
          if (e == 3) pcur[st][t] = as_bf16x8(make_uint4(w[st][t][0], w[st][t][1], w[st][t][2], w[st][t][3]));
        } else {
          l_tile = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[st][t][e]), ones2, l_tile, false);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Per-query max of a score tile (both lane halves), NaN-propagating.
__device__ __forceinline__ float query_max(const f32x16_t (&sc)[NST]) {
  float mx = sc[0][0];
#pragma unroll
  for (int st = 0; st < NST; ++st)
#pragma unroll
    for (int r = (st == 0 ? 1 : 0); r < 16; r += 2)
      mx = r + 1 < 16 ? __builtin_elementwise_maximum(__builtin_elementwise_maximum(mx, sc[st][r]), sc[st][r + 1])
                      : __builtin_elementwise_maximum(mx, sc[st][r]);
  auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}

// Masks a score tile for keys at or past this lane's limit.
__device__ __forceinline__ void mask_tile(f32x16_t (&sc)[NST], int lim, int kbase, int g) {
  const int rel = lim - kbase - 16 * g;  // compared with compile-time key offsets
#pragma unroll
  for (int st = 0; st < NST; ++st)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (32 * st + r >= rel) sc[st][r] = -INFINITY;
}

// Scores of one 32-key block of tile kbase, recomputed from K in global
// memory, masked like the tile.
template <int D>
__device__ __forceinline__ f32x16_t block_scores(const AttnParams& p, const WaveState<D>& ws, const bf16_t* kb,
                                                 int kvh, int kbase, int st, bool partial, int lane) {
  constexpr int KSTEPS = WaveState<D>::KSTEPS;
  const int g = lane >> 5;
  int64_t key = (int64_t)kbase + key_perm(lane & 31) + 32 * st;
  if (key > p.m.nk - 1) key = p.m.nk - 1;  // masked below; any valid row will do
  const bf16_t* row = kb + key * p.k_ts + (int64_t)kvh * p.k_hs;
  f32x16_t sc = {};
  // two k-steps at a time (few registers; this path is rare): the fence
  // keeps the loads from being hoisted together
#pragma unroll
  for (int s = 0; s < KSTEPS; s += 2) {
    __builtin_amdgcn_sched_barrier(0);
    const uint4 a0 = *reinterpret_cast<const uint4*>(row + 16 * s + 8 * g);
    if (s + 1 < KSTEPS) {
      const uint4 a1 = *reinterpret_cast<const uint4*>(row + 16 * (s + 1) + 8 * g);
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a0), ws.qreg[s], sc, 0, 0, 0);
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a1), ws.qreg[s + 1], sc, 0, 0, 0);
    } else {  // the last of an odd count (D = 80)
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a0), ws.qreg[s], sc, 0, 0, 0);
    }
  }
  if (partial) {
    const int rel = ws.lim - kbase - 32 * st - 16 * g;
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (r >= rel) sc[r] = -INFINITY;
  }
  return sc;
}

// Rare path, after a step whose tile sum exceeded 2^64 (or overflowed) for
// some lane: the tile's scores are gone from registers and its K slot is
// being refilled, so they are recomputed from K in global memory, one 32-key
// block at a time (twice: for the max, then for P).  The reference moves to
// the tile max where that is higher, O and the running sum (which already
// hold P(j-1)) are rescaled, and P(j) and its sum are redone.
template <int D>
__device__ __forceinline__ void overflow_tile(const AttnParams& p, WaveState<D>& ws, const bf16_t* kb, int kvh,
                                              int kbase, bool partial, int lane, bf16x8_t (&pcur)[NST][2],
                                              float& l_tile) {
  float mx = -INFINITY;
#pragma unroll 1
  for (int st = 0; st < NST; ++st) {
    const f32x16_t sc = block_scores<D>(p, ws, kb, kvh, kbase, st, partial, lane);
#pragma unroll
    for (int r = 0; r < 16; r += 2)
      mx = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mx, sc[r]), sc[r + 1]);
  }
  auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
  mx = __builtin_elementwise_maximum(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  const float m_new = __builtin_elementwise_maximum(ws.m_ref, mx * p.c_log2);
  const float alpha = m_new > ws.m_ref ? __builtin_amdgcn_exp2f(ws.m_ref - m_new) : 1.f;
  ws.l_run *= alpha;
#pragma unroll
  for (int i = 0; i < WaveState<D>::DT; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) ws.oacc[i][r] *= alpha;
  ws.m_ref = m_new;
  const bf16x2_t ones2 = {(__bf16)1.0f, (__bf16)1.0f};
  l_tile = 0.f;
#pragma unroll
  for (int st = 0; st < NST; ++st) {
    const f32x16_t sc = block_scores<D>(p, ws, kb, kvh, kbase, st, partial, lane);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[8 * t + 2 * e], p.c_log2, -ws.m_ref));
        const float b = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[8 * t + 2 * e + 1], p.c_log2, -ws.m_ref));
        w[e] = pack_bf16(a, b);
        l_tile = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[e]), ones2, l_tile, false);
      }
      pcur[st][t] = as_bf16x8(make_uint4(w[0], w[1], w[2], w[3]));
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int D, int W, bool ROPE_Q>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_mfma(AttnParams p) {
  constexpr int DS = store_dim(D);  // dims per stored tile row
  using L = Lay<DS>;
  static_assert(W == 4, "only the 4-wave workgroup shape is built");
  static_assert(L::BYTES <= 65536, "LDS copies stay below 64 KB");
  constexpr int BM = 32 * W;
  constexpr int KSTEPS = D / 16;
  constexpr int DT = (D + 31) / 32;
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* kring = smem;                  // K tiles (ring of 2)
  unsigned char* vring = smem + 2 * L::TILE_B;  // V tiles (ring of 2)

  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int g = lane >> 5;
  const int l32 = lane & 31;
  // Block -> (query tile, head slot, batch item); the slot's head keeps each
  // group of heads that share a key/value head on one XCD (head_of_slot).
  // All indices are block-uniform.
  const int b = blockIdx.y;
  const int hslot = __builtin_amdgcn_readfirstlane((int)(blockIdx.x % (unsigned)p.n_heads));
  const int head = head_of_slot(hslot, p.xcd_heads);
  const int kvh = __builtin_amdgcn_readfirstlane(head / p.kv_group);
  const int qt = p.n_qtiles - 1 - __builtin_amdgcn_readfirstlane((int)(blockIdx.x / (unsigned)p.n_heads));
  const bf16_t* kb = p.k + (int64_t)b * p.k_bs;  // this batch item's K and V
  const bf16_t* vb = p.v + (int64_t)b * p.v_bs;
  const int64_t nq = p.m.nq;
  const int64_t r0 = (int64_t)qt * BM;
  const int64_t rw = r0 + wave * 32;
  const int64_t my_row = rw + l32;
  const bool row_ok = my_row < nq;
  const int64_t i_abs = p.m.q0 + my_row;

  // ---- key range of this workgroup and of this wave ----
  const int64_t ia_wg = p.m.q0 + r0;
  const int64_t ib_wg = p.m.q0 + (r0 + BM - 1 < nq ? r0 + BM - 1 : nq - 1);
  const int64_t kend = key_end(p.m, ia_wg, ib_wg);
  const int ntiles = (int)((kend + BN - 1) / BN);
  const bool wave_live = rw < nq;
  const int64_t ia_w = p.m.q0 + rw;
  const int64_t ib_w = p.m.q0 + (rw + 31 < nq ? rw + 31 : nq - 1);
  // Both masks allow each query a prefix of the keys, [0, key_end(i)), and
  // key_end is non-decreasing in i: a per-lane limit decides every pair and
  // the wave's first and last rows bound its tiles.  The wave computes
  // tiles [0, ntw); past them every pair of its rows is masked.
  const int64_t lim_lo = key_end(p.m, ia_w, ia_w);
  const int64_t lim_hi = key_end(p.m, ib_w, ib_w);
  const int ntw = wave_live ? (int)((lim_hi + BN - 1) / BN) : 0;

  WaveState<D> ws;
  ws.lim = (int)key_end(p.m, i_abs, i_abs);
  TileLoader<D, W> ld;
  ld.init(wave, lane, p.k_ts, p.v_ts);

  // ---- Q into registers (B operand of S^T = K Q^T), rotated on load ----
  {
    uint4 raw[KSTEPS];
    const bf16_t* src = p.q + (int64_t)b * p.q_bs + (row_ok ? my_row : 0) * p.q_ts + (int64_t)head * p.q_hs;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
      raw[s] = row_ok ? *reinterpret_cast<const uint4*>(src + 16 * s + 8 * g) : make_uint4(0, 0, 0, 0);
    if (ROPE_Q && row_ok) {
      if constexpr (D % 32 == 0) {  // a chunk's partners are in the same lane, KSTEPS / 2 chunks up
#pragma unroll
        for (int s = 0; s < KSTEPS / 2; ++s) rope_chunk_pair<D>(p.rope, p.q_pos + 3 * my_row, s, g, raw[s], raw[s + KSTEPS / 2]);
      } else {
        uint4 part[KSTEPS];
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
          const int d = 16 * s + 8 * g;
          part[s] = *reinterpret_cast<const uint4*>(src + (d < D / 2 ? d + D / 2 : d - D / 2));
        }
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) rope_chunk_half<D>(p.rope, p.q_pos + 3 * my_row, 16 * s + 8 * g, raw[s], part[s]);
      }
    }
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) ws.qreg[s] = as_bf16x8(raw[s]);
    // Consume Q here so the compiler's own wait for these loads happens once,
    // before the key loop, instead of at their first use inside it.
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) asm volatile("" ::"v"(ws.qreg[s]));
  }

  // ---- loop-invariant LDS read offsets ----
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) ws.kaddr[s] = k_read_off<DS>(s, lane);
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) ws.vaddr[dt] = v_read_off<DS>(dt, lane);
#pragma unroll
  for (int i = 0; i < DT; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) ws.oacc[i][r] = 0.f;
  ws.m_ref = 0.f;
  ws.l_run = 0.f;

  // ---- prologue: K(0), K(1) resident, V slot 1 zeroed; S(0) computed ----
  ld.template issue<true>(p, kb, kvh, 0, kring);
  for (int i = threadIdx.x; i < L::TILE_B / 16; i += 64 * W)
    reinterpret_cast<uint4*>(vring + L::TILE_B)[i] = make_uint4(0, 0, 0, 0);
  if (ntiles > 1) ld.template issue<true>(p, kb, kvh, BN, kring + L::TILE_B);
  wait_vmem0();
  __syncthreads();
  f32x16_t sa[NST], sb[NST];
  bf16x8_t pa[NST][2], pb[NST][2];
#pragma unroll
  for (int st = 0; st < NST; ++st)
#pragma unroll
    for (int t = 0; t < 2; ++t) pa[st][t] = as_bf16x8(make_uint4(0, 0, 0, 0));
  if (ntw > 0) {
    float unused = 0.f;
    tile_step<D, true, false, false>(ws, kring, vring, sb, sa, pb, pa, p.c_log2, unused);
  }
  __syncthreads();  // every wave has read K(0) before step 0 overwrites its slot

  // Step j: exponentials of tile j, scores of tile j+1, PV of tile j-1.  On
  // entry K(j+1) (K slot (j+1)%2) and V(j-1) (V slot (j+1)%2) are resident;
  // the step starts the copies of K(j+2) into K(j)'s old slot and of V(j)
  // into V(j-2)'s old slot, and waits for both at its end.  Step ntiles only
  // finishes the last PV.
  auto step = [&](int j, f32x16_t (&cur)[NST], f32x16_t (&nxt)[NST], bf16x8_t (&pprev)[NST][2],
                  bf16x8_t (&pcur)[NST][2]) {
    if (j + 2 < ntiles) ld.template issue<true>(p, kb, kvh, (int64_t)(j + 2) * BN, kring + (j & 1) * L::TILE_B);
    if (j < ntiles) ld.template issue<false>(p, vb, kvh, (int64_t)j * BN, vring + (j & 1) * L::TILE_B);
    const unsigned char* kt = kring + ((j + 1) & 1) * L::TILE_B;
    const unsigned char* vt = vring + ((j + 1) & 1) * L::TILE_B;
    const bool do_e = j < ntw;
    const bool do_pv = j >= 1 && j <= ntw;
    float l_tile = 0.f;
    const int64_t kbase = (int64_t)j * BN;
    const bool partial = kbase + BN > lim_lo;  // some key of the tile is masked for some row
    if (do_e) {
      if (partial) mask_tile(cur, ws.lim, (int)kbase, g);
      // The row's reference is its exact max over tile 0 (which holds key 0
      // for every row); later tiles move it only on overflow.
      if (__builtin_expect(j == 0, 0)) {
        const float mq = query_max(cur) * p.c_log2;
        ws.m_ref = mq > -INFINITY && mq < INFINITY ? mq : 0.f;
      }
    }
    // One schedule for every step j <= ntw.  Step 0 multiplies P(-1) = 0
    // into the zero-filled V slot 1; step ntw computes scores and P for a
    // tile past the wave's keys from a stale K slot, and never uses them.
    if (j <= ntw) tile_step<D, true, true, true>(ws, kt, vt, cur, nxt, pprev, pcur, p.c_log2, l_tile);
    if (__builtin_expect(do_e && __builtin_amdgcn_ballot_w64(!(l_tile <= OVERFLOW_SUM)) != 0, 0))
      overflow_tile<D>(p, ws, kb, kvh, (int)kbase, partial, lane, pcur, l_tile);
    if (do_e) ws.l_run += l_tile;
    if (j < ntiles) {
      wait_vmem0();
      __syncthreads();
    }
  };
  for (int j = 0; j <= ntiles; j += 2) {
    step(j, sa, sb, pa, pb);
    if (j + 1 <= ntiles) step(j + 1, sb, sa, pb, pa);
  }

  // ---- epilogue: merge the two lane halves' sums, normalise, store ----
  float l_run = ws.l_run;
  {
    auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
    l_run = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  if (row_ok) {
    const float inv_l = 1.f / l_run;
    bf16_t* dst = p.o + (int64_t)b * p.o_bs + my_row * p.o_ts + (int64_t)head * p.o_hs;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d0 = 32 * dt + 8 * rr + 4 * g;
        if (D % 32 != 0 && d0 >= D) continue;  // the padding dims of the last tile
        uint2 w;
        w.x = pack_bf16(ws.oacc[dt][4 * rr + 0] * inv_l, ws.oacc[dt][4 * rr + 1] * inv_l);
        w.y = pack_bf16(ws.oacc[dt][4 * rr + 2] * inv_l, ws.oacc[dt][4 * rr + 3] * inv_l);
        *reinterpret_cast<uint2*>(dst + d0) = w;
      }
    if (p.lse && g == 0)
      p.lse[((int64_t)b * p.n_heads + head) * nq + my_row] = (ws.m_ref + log2f(l_run)) * 0.69314718055994530942f;
  }
}

template <int D, bool RQ>
static hipError_t launch_attn(const AttnParams& p, int n_batch, hipStream_t s) {
  constexpr int W = ATTN_WAVES;
  constexpr int BYTES = Lay<store_dim(D)>::BYTES;
  // Set the LDS size attribute once; concurrent first calls may both set it
  // (it is idempotent), and the flag itself is atomic.
  static std::atomic<bool> configured{false};
  if (!configured.load(std::memory_order_acquire)) {
    hipError_t e = hipFuncSetAttribute((const void*)attn_fwd_mfma<D, W, RQ>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, BYTES);
    if (e != hipSuccess) return e;
    configured.store(true, std::memory_order_release);
  }
  dim3 grid((unsigned)(p.n_qtiles * p.n_heads), (unsigned)n_batch);
  hipLaunchKernelGGL((attn_fwd_mfma<D, W, RQ>), grid, dim3(64 * W), BYTES, s, p);
  return hipGetLastError();
}

hipError_t attention_bf16_mfma(const mot_attn_args* a, const RopeTable& rt, hipStream_t s) {
  AttnParams p;
  p.q = (const bf16_t*)a->q;
  p.k = (const bf16_t*)a->k;
  p.v = (const bf16_t*)a->v;
  p.o = (bf16_t*)a->o;
  p.lse = a->lse;
  p.q_ts = a->q_ts; p.q_hs = a->q_hs; p.k_ts = a->k_ts; p.k_hs = a->k_hs;
  p.v_ts = a->v_ts; p.v_hs = a->v_hs; p.o_ts = a->o_ts; p.o_hs = a->o_hs;
  p.m.mode = a->mask; p.m.nq = a->nq; p.m.nk = a->nk; p.m.q0 = a->q0;
  p.m.n_ar = a->n_ar; p.m.n_prefix = a->n_prefix; p.m.chunk_len = a->chunk_len > 0 ? a->chunk_len : 1;
  p.n_heads = a->n_heads;
  const int n_kv = a->n_kv_heads > 0 ? a->n_kv_heads : a->n_heads;
  p.kv_group = a->n_heads / n_kv;
  p.xcd_heads = a->n_heads % 8 == 0 ? a->n_heads / 8 : 0;
  const int n_batch = a->n_batch > 1 ? a->n_batch : 1;
  p.q_bs = n_batch > 1 ? a->q_bs : 0;
  p.k_bs = n_batch > 1 ? a->k_bs : 0;
  p.v_bs = n_batch > 1 ? a->v_bs : 0;
  p.o_bs = n_batch > 1 ? a->o_bs : 0;
  p.n_qtiles = (int)((a->nq + 32 * ATTN_WAVES - 1) / (32 * ATTN_WAVES));
  float scale = a->scale != 0.f ? a->scale : 1.f / sqrtf((float)a->head_dim);
  p.c_log2 = scale * 1.4426950408889634f;
  p.q_pos = a->q_pos;
  p.rope = rt;
  // K is used as given (the caller checks that no k_pos was passed)
  const bool rq = a->q_pos != nullptr;
  if (a->head_dim == 128) return rq ? launch_attn<128, true>(p, n_batch, s) : launch_attn<128, false>(p, n_batch, s);
  if (a->head_dim == 80) return rq ? launch_attn<80, true>(p, n_batch, s) : launch_attn<80, false>(p, n_batch, s);
  return rq ? launch_attn<64, true>(p, n_batch, s) : launch_attn<64, false>(p, n_batch, s);
}

}  // namespace mot
