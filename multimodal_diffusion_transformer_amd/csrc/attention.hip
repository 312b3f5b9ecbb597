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
//    cross-lane step (a permlane32 swap) runs when a reference max moves.
//  * K rows are fed to the MFMA in a permuted order so that lane half g
//    ends up holding keys 16g..16g+15 of each 32-key block in register
//    order.  Those registers, packed to bf16, are exactly the B operand of
//    O^T += V^T P^T for 8 consecutive keys: P never leaves registers.
//  * Software pipeline inside each wave: while the softmax of tile j runs on
//    the vector ALUs, the MFMAs of S for tile j+1 are already in flight;
//    then P(j) V(j) follows.  K therefore runs one tile ahead of V: K and V
//    have separate two-stage LDS rings, filled straight from HBM with
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
//    registers for the whole key loop.
//  * Softmax in fp32 in the log2 domain (scale*log2(e) folded into one FMA
//    before exp2), against a reference maximum that only moves when a lane's
//    tile sum exceeds 2^16 (or on a row's first tile): the common tile needs
//    no max, no cross-lane step and no rescale.  Row sums accumulate the
//    bf16-packed P with dot2, so numerator and denominator use the same P.
//  * Both masks give every query a prefix of the keys, [0, key_end(i)).  A
//    per-lane limit decides each pair with one compare, and the limits of a
//    wave's first and last rows classify its tiles exactly: tiles past a
//    wave's last allowed key are skipped, full tiles run unmasked, only
//    partial tiles are masked.
//  * Grid: head is the fastest index, so with H a multiple of 8 every head
//    stays on one XCD (workgroups go round-robin over the 8 XCDs) and shares
//    that XCD's L2; query tiles are issued heaviest first.
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
  int n_qtiles;
  float c_log2;  // scale * log2(e)
  const float* q_pos;
  const float* k_pos;
  RopeTable rope;
};

constexpr int BN = 64;                  // keys per tile
constexpr int NST = BN / 32;            // 32-key MFMA blocks per tile
constexpr float RESCALE_SUM = 65536.f;  // a lane's tile sum above this moves the reference max
#ifndef MOT_ATTN_WAVES
#define MOT_ATTN_WAVES 4
#endif
constexpr int ATTN_WAVES = MOT_ATTN_WAVES;  // waves per workgroup (32 query rows each)

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
template <int D> __device__ inline int swz_k(int r) {
  if constexpr (D == 128) return (r & 3) | (((r >> 4) & 1) << 2) | (((r >> 2) & 1) << 3);
  else return ((r >> 1) & 1) | (((r >> 2) & 1) << 1) | (((r >> 4) & 1) << 2);
}
template <int D> __device__ inline int swz_v(int r) { return 4 * ((r / Lay<D>::RPG) % (Lay<D>::CH / 4)); }

__device__ inline bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

__device__ inline uint32_t pack_bf16(float a, float b) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  bf2 p = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, p);
}

// One wave-wide 16-byte-per-lane copy from global memory (scalar base +
// per-lane offset) straight into LDS at `lds` + 16 * lane.  Written as
// inline asm so the compiler does not drain every outstanding copy before
// each LDS read (it cannot tell that the copies target another stage); the
// kernel waits on vmcnt itself.  The instruction has no VGPR result.
__device__ inline void dma16(const void* gbase, uint32_t voff, uint32_t lds) {
  // the tile base is wave-uniform by construction; make it an SGPR pair
  // (readfirstlane returns int: go through uint32_t so nothing sign-extends)
  const uint64_t b = (uint64_t)gbase;
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint64_t sb = ((uint64_t)hi << 32) | (uint64_t)lo;
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sb), "{m0}"(lds) : "memory");
}

__device__ inline uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

__device__ inline void wait_vmem0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Row of the K tile that feeds MFMA row rho so that lane half g holds keys
// 16g..16g+15 in accumulator registers 0..15.
__device__ inline int key_perm(int rho) { return 16 * ((rho >> 2) & 1) + 4 * (rho >> 3) + (rho & 3); }

template <int D, int W>
struct TileLoader {
  static constexpr int PER_WAVE = Lay<D>::NINSTR / W;
  static_assert(PER_WAVE >= 1 && Lay<D>::NINSTR % W == 0, "loads per wave");
  uint32_t offk[PER_WAVE], offv[PER_WAVE];  // byte offsets of this lane's chunk
  int row[PER_WAVE];                        // tile row this lane loads
  int ck[PER_WAVE], cv[PER_WAVE];           // logical chunks
  int wave;

  __device__ void init(int wave_, int lane, int64_t k_ts, int64_t v_ts) {
    wave = wave_;
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int n = wave * PER_WAVE + i;
      const int r = n * Lay<D>::RPI + lane / Lay<D>::CH;
      const int pc = lane % Lay<D>::CH;
      row[i] = r;
      ck[i] = pc ^ swz_k<D>(r);
      cv[i] = pc ^ swz_v<D>(r);
      offk[i] = (uint32_t)(r * k_ts * 2 + ck[i] * 16);
      offv[i] = (uint32_t)(r * v_ts * 2 + cv[i] * 16);
    }
  }

  // Issue this wave's share of one tile (K or V) starting at key kbase into
  // the LDS tile at `dst`.  Rows past the last key re-read the last key
  // (never out of range; those scores are masked and the values finite).
  template <bool IS_K>
  __device__ void issue(const AttnParams& p, int head, int64_t kbase, unsigned char* dst) const {
    const int64_t ts = IS_K ? p.k_ts : p.v_ts;
    const char* base = reinterpret_cast<const char*>(IS_K ? p.k : p.v) +
                       (kbase * ts + (int64_t)head * (IS_K ? p.k_hs : p.v_hs)) * 2;
    const int64_t last = p.m.nk - 1 - kbase;  // last valid tile row
    const bool ragged = last < BN - 1;
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int n = wave * PER_WAVE + i;
      uint32_t off = IS_K ? offk[i] : offv[i];
      if (ragged && row[i] > last) off = (uint32_t)(last * ts * 2 + (IS_K ? ck[i] : cv[i]) * 16);
      dma16(base, off, lds_addr(dst + n * 1024));
    }
  }
};

// Rotate a K tile in LDS by mRoPE (the optional rotate-on-load path).
template <int D, int W>
__device__ void rope_k_tile(const AttnParams& p, int64_t kbase, unsigned char* tile) {
  constexpr int P = D / 2;
  for (int e = threadIdx.x; e < BN * P; e += 64 * W) {
    const int row = e / P, k = e % P;
    const int64_t key = kbase + row;
    if (key >= p.m.nk) continue;
    float cs, sn;
    rope_cs(p.k_pos[3 * key + rope_axis(p.rope, k)], p.rope.inv_freq[k], cs, sn);
    const int f = swz_k<D>(row);
    bf16_t* a = reinterpret_cast<bf16_t*>(tile + row * Lay<D>::ROWB + (((k / 8) ^ f) * 16) + (k % 8) * 2);
    bf16_t* b = reinterpret_cast<bf16_t*>(tile + row * Lay<D>::ROWB + ((((k + P) / 8) ^ f) * 16) + (k % 8) * 2);
    const float x1 = bf16_to_f32(*a), x2 = bf16_to_f32(*b);
    *a = f32_to_bf16(__builtin_fmaf(x1, cs, -x2 * sn));
    *b = f32_to_bf16(__builtin_fmaf(x1, sn, x2 * cs));
  }
}

// Per-wave state of the key loop.
template <int D>
struct WaveState {
  static constexpr int KSTEPS = D / 16;  // MFMA k-steps over the head dim
  static constexpr int DT = D / 32;      // 32-wide output tiles over the head dim
  bf16x8_t qreg[KSTEPS];
  uint32_t kaddr[KSTEPS];  // K operand offsets within a K tile
  uint32_t vaddr[DT];      // V^T operand offsets within a V tile
  f32x16_t oacc[DT];
  float m_ref;  // reference maximum (log2 domain)
  float l_run;  // this lane's partial row sum
  int64_t lim;  // this lane's key limit
};

// S^T = K Q^T for one tile (NST 32-key blocks).
template <int D>
__device__ inline void scores(const WaveState<D>& ws, const unsigned char* ktile, f32x16_t (&s)[NST]) {
  using L = Lay<D>;
#pragma unroll
  for (int st = 0; st < NST; ++st) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[st][r] = 0.f;
#pragma unroll
    for (int k = 0; k < WaveState<D>::KSTEPS; ++k) {
      const uint4 kv = *reinterpret_cast<const uint4*>(ktile + ws.kaddr[k] + st * 32 * L::ROWB);
      s[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kv), ws.qreg[k], s[st], 0, 0, 0);
    }
  }
}

// P = exp2(s*c - m) packed to bf16; returns the lane's sum of the packed P.
__device__ inline float exps(const f32x16_t (&s)[NST], float c, float m_use, bf16x8_t (&pb)[NST][2]) {
  const bf16x2_t ones2 = {(__bf16)1.0f, (__bf16)1.0f};
  float l = 0.f;
#pragma unroll
  for (int st = 0; st < NST; ++st)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a = __builtin_amdgcn_exp2f(__builtin_fmaf(s[st][8 * t + 2 * e], c, -m_use));
        const float b = __builtin_amdgcn_exp2f(__builtin_fmaf(s[st][8 * t + 2 * e + 1], c, -m_use));
        w[e] = pack_bf16(a, b);
        l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[e]), ones2, l, false);
      }
      pb[st][t] = as_bf16x8(make_uint4(w[0], w[1], w[2], w[3]));
    }
  return l;
}

// Rare path: move the reference max to this tile's max (per lane), rescale
// O and the running sum, and redo the exponentials.
template <int D>
__device__ inline void rescale_and_exps(WaveState<D>& ws, const f32x16_t (&s)[NST], float c,
                                        bf16x8_t (&pb)[NST][2], float& l_tile) {
  float mx = s[0][0];
#pragma unroll
  for (int st = 0; st < NST; ++st)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[st][r]);
  auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
  mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * c;
  const float m_new = fmaxf(ws.m_ref, mx);
  if (m_new > ws.m_ref) {  // only rows whose reference moves
    const float alpha = __builtin_amdgcn_exp2f(ws.m_ref - m_new);
    ws.l_run *= alpha;
#pragma unroll
    for (int i = 0; i < WaveState<D>::DT; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) ws.oacc[i][r] *= alpha;
    ws.m_ref = m_new;
  }
  l_tile = exps(s, c, ws.m_ref == -INFINITY ? 0.f : ws.m_ref, pb);
}

// O^T += V^T P^T for one tile.
template <int D>
__device__ inline void pv(WaveState<D>& ws, const unsigned char* vtile, const bf16x8_t (&pb)[NST][2]) {
  using L = Lay<D>;
#pragma unroll
  for (int dt = 0; dt < WaveState<D>::DT; ++dt)
#pragma unroll
    for (int st = 0; st < NST; ++st)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const unsigned char* base = vtile + ws.vaddr[dt] + (32 * st + 8 * t) * L::ROWB;
        s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(base));
        s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(base + 4 * L::ROWB));
        s16x8_t a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        ws.oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a8), pb[st][t],
                                                              ws.oacc[dt], 0, 0, 0);
      }
}

template <int D, int W, bool ROPE_Q, bool ROPE_K>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_mfma(AttnParams p) {
  using L = Lay<D>;
  static_assert(L::BYTES <= 65536, "LDS copies stay below 64 KB");
  constexpr int BM = 32 * W;
  constexpr int KSTEPS = D / 16;
  constexpr int DT = D / 32;
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* kring = smem;                  // K tiles j+1, j+2 (ring of 2)
  unsigned char* vring = smem + 2 * L::TILE_B;  // V tiles j, j+1 (ring of 2)

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 5;
  const int l32 = lane & 31;
  const int head = blockIdx.x % p.n_heads;
  const int qt = p.n_qtiles - 1 - (int)(blockIdx.x / p.n_heads);
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
  ws.lim = key_end(p.m, i_abs, i_abs);
  TileLoader<D, W> ld;
  ld.init(wave, lane, p.k_ts, p.v_ts);

  // ---- Q into registers (B operand of S^T = K Q^T), rotated on load ----
  {
    uint4 raw[KSTEPS];
    const bf16_t* src = p.q + (row_ok ? my_row : 0) * p.q_ts + (int64_t)head * p.q_hs;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
      raw[s] = row_ok ? *reinterpret_cast<const uint4*>(src + 16 * s + 8 * g) : make_uint4(0, 0, 0, 0);
    if (ROPE_Q && row_ok) {
      const float* pp = p.q_pos + 3 * my_row;
      // dims 16s+8g+e (s < KSTEPS/2) pair with the same slot of s + KSTEPS/2
#pragma unroll
      for (int s = 0; s < KSTEPS / 2; ++s) {
        uint32_t lw[4] = {raw[s].x, raw[s].y, raw[s].z, raw[s].w};
        uint32_t hw[4] = {raw[s + KSTEPS / 2].x, raw[s + KSTEPS / 2].y, raw[s + KSTEPS / 2].z,
                          raw[s + KSTEPS / 2].w};
        float y1[8], y2[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          int kk = 16 * s + 8 * g + e;
          float cs, sn;
          rope_cs(pp[rope_axis(p.rope, kk)], p.rope.inv_freq[kk], cs, sn);
          float x1 = __uint_as_float((e & 1) ? (lw[e >> 1] & 0xFFFF0000u) : (lw[e >> 1] << 16));
          float x2 = __uint_as_float((e & 1) ? (hw[e >> 1] & 0xFFFF0000u) : (hw[e >> 1] << 16));
          y1[e] = __builtin_fmaf(x1, cs, -x2 * sn);
          y2[e] = __builtin_fmaf(x1, sn, x2 * cs);
        }
        raw[s] = make_uint4(pack_bf16(y1[0], y1[1]), pack_bf16(y1[2], y1[3]),
                            pack_bf16(y1[4], y1[5]), pack_bf16(y1[6], y1[7]));
        raw[s + KSTEPS / 2] = make_uint4(pack_bf16(y2[0], y2[1]), pack_bf16(y2[2], y2[3]),
                                         pack_bf16(y2[4], y2[5]), pack_bf16(y2[6], y2[7]));
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
  {
    const int row = key_perm(l32);
    const int f = swz_k<D>(row);
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) ws.kaddr[s] = row * L::ROWB + (((2 * s + g) ^ f) * 16);
  }
  {
    const int j = lane & 15, q16 = (lane >> 4) & 1;
    const int rowl = 16 * g + j / 4;  // + 32st + 8t + 4h, all multiples of 4
    const int f = swz_v<D>(rowl);     // so the swizzle is the same for all of them
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int c = 4 * dt + 2 * q16 + (j & 3) / 2;
      ws.vaddr[dt] = rowl * L::ROWB + ((c ^ f) * 16) + 8 * (j & 1);
    }
  }
#pragma unroll
  for (int i = 0; i < DT; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) ws.oacc[i][r] = 0.f;
  ws.m_ref = -INFINITY;
  ws.l_run = 0.f;

  // ---- prologue: K(0), V(0), K(1) resident; S(0) computed ----
  ld.template issue<true>(p, head, 0, kring);
  ld.template issue<false>(p, head, 0, vring);
  if (ntiles > 1) ld.template issue<true>(p, head, BN, kring + L::TILE_B);
  wait_vmem0();
  __syncthreads();
  if (ROPE_K) {
    rope_k_tile<D, W>(p, 0, kring);
    if (ntiles > 1) rope_k_tile<D, W>(p, BN, kring + L::TILE_B);
    __syncthreads();
  }
  f32x16_t sa[NST], sb[NST];
  if (ntw > 0) scores<D>(ws, kring, sa);
  __syncthreads();  // every wave has read K(0) before step 0 overwrites its slot

  // One pipelined step: tile j's softmax and PV with tile j+1's scores in
  // flight.  On entry V(j) (V slot j%2) and K(j+1) (K slot (j+1)%2) are
  // resident; the step starts the copies of K(j+2) into K(j)'s old slot
  // and of V(j+1) into V(j-1)'s old slot, and waits for both at its end.
  auto step = [&](int j, f32x16_t (&cur)[NST], f32x16_t (&nxt)[NST]) {
    if (j + 2 < ntiles) ld.template issue<true>(p, head, (int64_t)(j + 2) * BN, kring + (j & 1) * L::TILE_B);
    if (j + 1 < ntiles)
      ld.template issue<false>(p, head, (int64_t)(j + 1) * BN, vring + ((j + 1) & 1) * L::TILE_B);
    if (j < ntw) {
      const int64_t kbase = (int64_t)j * BN;
      if (kbase + BN > lim_lo) {  // partial tile: key j is allowed iff j < lim
        const int64_t rel = ws.lim - kbase;
        const int lrel = rel < 0 ? 0 : (rel > BN ? BN : (int)rel);
#pragma unroll
        for (int st = 0; st < NST; ++st)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (32 * st + 16 * g + r >= lrel) cur[st][r] = -INFINITY;
      }
      // One basic block: the MFMAs of S(j+1) interleaved with the
      // exponentials of tile j.  On a wave's last tile the K slot read here
      // holds a stale (valid) tile whose scores are never used.
      bf16x8_t pb[NST][2];
      const float m_use = ws.m_ref == -INFINITY ? 0.f : ws.m_ref;
      scores<D>(ws, kring + ((j + 1) & 1) * L::TILE_B, nxt);
      float l_tile = exps(cur, p.c_log2, m_use, pb);
      // 4 K reads ahead, then per MFMA: 1 MFMA, 1 K read, 6 VALU
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < NST * WaveState<D>::KSTEPS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
      }
      if (__builtin_amdgcn_ballot_w64(ws.m_ref == -INFINITY || !(l_tile <= RESCALE_SUM)) != 0)
        rescale_and_exps<D>(ws, cur, p.c_log2, pb, l_tile);
      ws.l_run += l_tile;
      pv<D>(ws, vring + (j & 1) * L::TILE_B, pb);
      // 8 V^T reads ahead, then per MFMA: 1 MFMA, 2 reads
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 1);
#pragma unroll
      for (int i = 0; i < NST * 2 * WaveState<D>::DT; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
      }
    }
    wait_vmem0();
    __syncthreads();
    if (ROPE_K && j + 2 < ntiles) {
      rope_k_tile<D, W>(p, (int64_t)(j + 2) * BN, kring + (j & 1) * L::TILE_B);
      __syncthreads();
    }
  };
  for (int j = 0; j < ntiles; j += 2) {
    step(j, sa, sb);
    if (j + 1 < ntiles) step(j + 1, sb, sa);
  }

  // ---- epilogue: merge the two lane halves' sums, normalise, store ----
  float l_run = ws.l_run;
  {
    auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
    l_run = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  if (row_ok) {
    const float inv_l = 1.f / l_run;
    bf16_t* dst = p.o + my_row * p.o_ts + (int64_t)head * p.o_hs;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d0 = 32 * dt + 8 * rr + 4 * g;
        uint2 w;
        w.x = pack_bf16(ws.oacc[dt][4 * rr + 0] * inv_l, ws.oacc[dt][4 * rr + 1] * inv_l);
        w.y = pack_bf16(ws.oacc[dt][4 * rr + 2] * inv_l, ws.oacc[dt][4 * rr + 3] * inv_l);
        *reinterpret_cast<uint2*>(dst + d0) = w;
      }
    if (p.lse && g == 0) p.lse[(int64_t)head * nq + my_row] = (ws.m_ref + log2f(l_run)) * 0.69314718055994530942f;
  }
}

template <int D, bool RQ, bool RK>
static hipError_t launch_attn(const AttnParams& p, hipStream_t s) {
  constexpr int W = ATTN_WAVES;
  constexpr int BYTES = Lay<D>::BYTES;
  static bool configured = false;
  if (!configured) {
    hipError_t e = hipFuncSetAttribute((const void*)attn_fwd_mfma<D, W, RQ, RK>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, BYTES);
    if (e != hipSuccess) return e;
    configured = true;
  }
  dim3 grid((unsigned)(p.n_qtiles * p.n_heads));
  hipLaunchKernelGGL((attn_fwd_mfma<D, W, RQ, RK>), grid, dim3(64 * W), BYTES, s, p);
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
  p.n_qtiles = (int)((a->nq + 32 * ATTN_WAVES - 1) / (32 * ATTN_WAVES));
  float scale = a->scale != 0.f ? a->scale : 1.f / sqrtf((float)a->head_dim);
  p.c_log2 = scale * 1.4426950408889634f;
  p.q_pos = a->q_pos;
  p.k_pos = a->k_pos;
  p.rope = rt;
  const bool rq = a->q_pos != nullptr, rk = a->k_pos != nullptr;
  if (a->head_dim == 128) {
    if (rq && rk) return launch_attn<128, true, true>(p, s);
    if (rq) return launch_attn<128, true, false>(p, s);
    if (rk) return launch_attn<128, false, true>(p, s);
    return launch_attn<128, false, false>(p, s);
  }
  if (rq && rk) return launch_attn<64, true, true>(p, s);
  if (rq) return launch_attn<64, true, false>(p, s);
  if (rk) return launch_attn<64, false, true>(p, s);
  return launch_attn<64, false, false>(p, s);
}

}  // namespace mot
