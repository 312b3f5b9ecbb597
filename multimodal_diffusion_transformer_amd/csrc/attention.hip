// Masked flash attention on bf16 MFMA for gfx950.
//
// Computes, per head, O = softmax(mask(Q K^T * scale)) V: the joint
// attention of "Cosmos 3 方法原理全解" §3 (AR causal, DM full over [K_AR;K_DM])
// and the chunk-causal streaming attention of "流式生成如何工作".
//
// Design (one workgroup = 4 waves = 128 query rows of one head):
//  * The score tile is computed transposed, S^T = K Q^T, on
//    v_mfma_f32_32x32x16_bf16.  In the 32x32 accumulator layout a lane owns
//    one column, so every lane owns ONE query and 16 of its keys; the row
//    statistics (max, sum, rescale) are per-lane scalars, and the only
//    cross-lane step is one permlane32 swap to merge the two lane halves.
//  * K rows are fed to the MFMA in a permuted order so that lane half g
//    ends up holding keys 16g..16g+15 of each 32-key block in register
//    order.  Those registers, packed to bf16, are exactly the B operand of
//    O^T += V^T P^T for 8 consecutive keys: P never leaves registers.
//  * Q (rotated by mRoPE on load when positions are given) lives in
//    registers for the whole key loop.  K tiles sit in LDS row-major with a
//    16-byte row pad; V tiles are transposed while staged (V^T[d][key]) with
//    an XOR swizzle of 16-byte chunks, so both MFMA A-operand reads are
//    conflict-free ds_read_b128.  Two LDS stages: the next tile's global
//    loads are in flight while the current one is computed.
//  * Online softmax in fp32 in the log2 domain (scale*log2(e) folded into
//    one FMA before exp2).  The O rescale is skipped when no lane's running
//    maximum moved.
//  * Both masks give every query a prefix of the keys, [0, key_end(i)).  A
//    per-lane limit decides each pair with one compare, and the limits of a
//    wave's first and last rows classify its tiles exactly: empty tiles are
//    skipped, full tiles run unmasked, only partial tiles are masked.
//  * Grid: head is the fastest index, so with H a multiple of 8 every head
//    stays on one XCD (workgroups go round-robin over the 8 XCDs) and shares
//    that XCD's L2; query tiles are issued heaviest first.
#include "common.hpp"
#include "rope_dev.hpp"

namespace mot {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

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

constexpr int BM = 128;  // query rows per workgroup
constexpr int BN = 64;   // keys per tile
constexpr int WAVES = 4;

template <int D>
struct AttnSmem {
  static constexpr int KROW = D + 8;                 // padded K row (elements)
  static constexpr int K_ELEMS = BN * KROW;          // one stage
  static constexpr int V_ELEMS = D * BN;             // one stage (V^T)
  static constexpr int STAGE = K_ELEMS + V_ELEMS;
  static constexpr int BYTES = 2 * STAGE * 2;
};

__device__ inline bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

__device__ inline uint32_t pack_bf16(float a, float b) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  bf2 p = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, p);
}

// Row of the K tile that feeds MFMA row rho so that lane half g holds keys
// 16g..16g+15 in accumulator registers 0..15.
__device__ inline int key_perm(int rho) { return 16 * ((rho >> 2) & 1) + 4 * (rho >> 3) + (rho & 3); }

// Physical 16-byte chunk of logical chunk ck in row d of the V^T tile.
__device__ inline int v_swz(int d, int ck) { return ck ^ ((d >> 1) & 7); }

template <int D, bool ROPE_K>
__device__ inline void load_kv_regs(const AttnParams& p, int head, int64_t kbase, uint4 (&kr)[4],
                                    uint4 (&vr)[4]) {
  const int t = threadIdx.x;
  constexpr int CH = D / 8;  // 16-byte chunks per row
  // K: thread -> (row, chunk c and c + CH/2); rows per pass = 256 / (CH/2)
  constexpr int HALF = CH / 2;
  constexpr int RPP = 256 / HALF;
  constexpr int KPASS = BN / RPP;
  static_assert(KPASS * 2 <= 4, "K staging registers");
#pragma unroll
  for (int a = 0; a < KPASS; ++a) {
    int row = t / HALF + a * RPP;
    int c = t % HALF;
    int64_t key = kbase + row;
    if (key < p.m.nk) {
      const bf16_t* src = p.k + key * p.k_ts + (int64_t)head * p.k_hs;
      kr[2 * a] = *reinterpret_cast<const uint4*>(src + 8 * c);
      kr[2 * a + 1] = *reinterpret_cast<const uint4*>(src + 8 * (c + HALF));
    } else {
      kr[2 * a] = make_uint4(0, 0, 0, 0);
      kr[2 * a + 1] = make_uint4(0, 0, 0, 0);
    }
  }
  // V: thread -> (key block kb of 4 keys, d chunk db); D=128: 16 x 16.
  constexpr int KB = BN / 4;
  const int kb = t % KB;
  const int db = t / KB;
  if (db < CH) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      int64_t key = kbase + 4 * kb + a;
      if (key < p.m.nk) {
        const bf16_t* src = p.v + key * p.v_ts + (int64_t)head * p.v_hs;
        vr[a] = *reinterpret_cast<const uint4*>(src + 8 * db);
      } else {
        vr[a] = make_uint4(0, 0, 0, 0);
      }
    }
  }
}

template <int D, bool ROPE_K>
__device__ inline void store_kv_lds(const AttnParams& p, int64_t kbase, bf16_t* ks, bf16_t* vs,
                                    uint4 (&kr)[4], uint4 (&vr)[4]) {
  using S = AttnSmem<D>;
  const int t = threadIdx.x;
  constexpr int CH = D / 8;
  constexpr int HALF = CH / 2;
  constexpr int RPP = 256 / HALF;
  constexpr int KPASS = BN / RPP;
#pragma unroll
  for (int a = 0; a < KPASS; ++a) {
    int row = t / HALF + a * RPP;
    int c = t % HALF;
    uint4 lo = kr[2 * a], hi = kr[2 * a + 1];
    if (ROPE_K) {
      int64_t key = kbase + row;
      if (key < p.m.nk) {
        const float* pp = p.k_pos + 3 * key;
        uint32_t lw[4] = {lo.x, lo.y, lo.z, lo.w}, hw[4] = {hi.x, hi.y, hi.z, hi.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          int kk = 8 * c + e;
          float cs, sn;
          rope_cs(pp[rope_axis(p.rope, kk)], p.rope.inv_freq[kk], cs, sn);
          float x1 = bf16_to_f32((bf16_t)((e & 1) ? (lw[e >> 1] >> 16) : (lw[e >> 1] & 0xFFFF)));
          float x2 = bf16_to_f32((bf16_t)((e & 1) ? (hw[e >> 1] >> 16) : (hw[e >> 1] & 0xFFFF)));
          uint32_t y1 = f32_to_bf16(__builtin_fmaf(x1, cs, -x2 * sn));
          uint32_t y2 = f32_to_bf16(__builtin_fmaf(x1, sn, x2 * cs));
          if (e & 1) {
            lw[e >> 1] = (lw[e >> 1] & 0xFFFFu) | (y1 << 16);
            hw[e >> 1] = (hw[e >> 1] & 0xFFFFu) | (y2 << 16);
          } else {
            lw[e >> 1] = (lw[e >> 1] & 0xFFFF0000u) | y1;
            hw[e >> 1] = (hw[e >> 1] & 0xFFFF0000u) | y2;
          }
        }
        lo = make_uint4(lw[0], lw[1], lw[2], lw[3]);
        hi = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      }
    }
    *reinterpret_cast<uint4*>(ks + row * S::KROW + 8 * c) = lo;
    *reinterpret_cast<uint4*>(ks + row * S::KROW + 8 * (c + HALF)) = hi;
  }
  constexpr int KB = BN / 4;
  const int kb = t % KB;
  const int db = t / KB;
  if (db < CH) {
    // transpose 4 keys x 8 dims into 8 rows of V^T, 4 keys (8 bytes) each
    uint32_t w[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      w[a][0] = vr[a].x; w[a][1] = vr[a].y; w[a][2] = vr[a].z; w[a][3] = vr[a].w;
    }
    const int ck = kb >> 1;   // logical 16-byte chunk (8 keys)
    const int half = kb & 1;  // which 8-byte half of it
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int cw = e >> 1;
      uint32_t k01, k23;
      if (e & 1) {  // high halves
        k01 = __builtin_amdgcn_perm(w[1][cw], w[0][cw], 0x07060302u);
        k23 = __builtin_amdgcn_perm(w[3][cw], w[2][cw], 0x07060302u);
      } else {      // low halves
        k01 = __builtin_amdgcn_perm(w[1][cw], w[0][cw], 0x05040100u);
        k23 = __builtin_amdgcn_perm(w[3][cw], w[2][cw], 0x05040100u);
      }
      const int d = 8 * db + e;
      bf16_t* dst = vs + d * BN + 8 * v_swz(d, ck) + 4 * half;
      *reinterpret_cast<uint2*>(dst) = make_uint2(k01, k23);
    }
  }
}

template <int D, bool ROPE_Q, bool ROPE_K>
__global__ __launch_bounds__(256) void attn_fwd_mfma(AttnParams p) {
  using S = AttnSmem<D>;
  constexpr int KSTEPS = D / 16;  // MFMA k-steps over the head dim
  constexpr int DT = D / 32;      // 32-wide output tiles over the head dim
  extern __shared__ __align__(16) unsigned char smem_raw[];
  bf16_t* smem = reinterpret_cast<bf16_t*>(smem_raw);

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

  // ---- Q into registers (B operand of S^T = K Q^T) ----
  bf16x8_t qreg[KSTEPS];
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
    for (int s = 0; s < KSTEPS; ++s) qreg[s] = as_bf16x8(raw[s]);
  }

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
  // the wave's first and last rows bound its tiles.
  const int64_t lim = key_end(p.m, i_abs, i_abs);
  const int64_t lim_lo = key_end(p.m, ia_w, ia_w);
  const int64_t lim_hi = key_end(p.m, ib_w, ib_w);

  f32x16_t oacc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;
  float m_run = -INFINITY;  // running max, log2 domain
  float l_run = 0.f;        // this lane's partial row sum

  uint4 kr[4], vr[4];
  load_kv_regs<D, ROPE_K>(p, head, 0, kr, vr);
  store_kv_lds<D, ROPE_K>(p, 0, smem, smem + S::K_ELEMS, kr, vr);
  __syncthreads();

  const int krow = key_perm(l32);
  for (int kt = 0; kt < ntiles; ++kt) {
    const int buf = kt & 1;
    const int64_t kbase = (int64_t)kt * BN;
    const bool more = kt + 1 < ntiles;
    if (more) load_kv_regs<D, ROPE_K>(p, head, kbase + BN, kr, vr);

    const bf16_t* ks = smem + buf * S::STAGE;
    const bf16_t* vs = ks + S::K_ELEMS;
    // exact per-wave class from the wave's smallest / largest key limit
    int cls = TILE_EMPTY;
    if (wave_live) {
      if (kbase + BN <= lim_lo) cls = TILE_FULL;
      else if (kbase < lim_hi) cls = TILE_PARTIAL;
    }
    if (cls != TILE_EMPTY) {
      // ---- S^T = K Q^T for two 32-key blocks ----
      f32x16_t sacc[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[st][r] = 0.f;
        const bf16_t* krp = ks + (32 * st + krow) * S::KROW + 8 * g;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
          bf16x8_t a = as_bf16x8(*reinterpret_cast<const uint4*>(krp + 16 * s));
          sacc[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[s], sacc[st], 0, 0, 0);
        }
      }
      // ---- mask (partial tiles only): key j is allowed iff j < lim ----
      if (cls == TILE_PARTIAL) {
        const int64_t rel = lim - kbase;
        const int lrel = rel < 0 ? 0 : (rel > BN ? BN : (int)rel);
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (32 * st + 16 * g + r >= lrel) sacc[st][r] = -INFINITY;
      }
      // ---- online softmax ----
      float mx = sacc[0][0];
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[st][r]);
      {
        auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      }
      const float m_new = fmaxf(m_run, mx * p.c_log2);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      if (__builtin_amdgcn_ballot_w64(m_new > m_run) != 0) {
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < DT; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
      }
      m_run = m_new;
      bf16x8_t pb[2][2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        float pv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          pv[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[st][r], p.c_log2, -m_use));
          l_run += pv[r];
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          uint4 u = make_uint4(pack_bf16(pv[8 * t + 0], pv[8 * t + 1]), pack_bf16(pv[8 * t + 2], pv[8 * t + 3]),
                               pack_bf16(pv[8 * t + 4], pv[8 * t + 5]), pack_bf16(pv[8 * t + 6], pv[8 * t + 7]));
          pb[st][t] = as_bf16x8(u);
        }
      }
      // ---- O^T += V^T P^T ----
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int d = 32 * dt + l32;
        const bf16_t* vrow = vs + d * BN;
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int ck = 4 * st + 2 * g + t;
            bf16x8_t a = as_bf16x8(*reinterpret_cast<const uint4*>(vrow + 8 * v_swz(d, ck)));
            oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[st][t], oacc[dt], 0, 0, 0);
          }
      }
    }
    if (more) {
      bf16_t* nks = smem + (buf ^ 1) * S::STAGE;
      store_kv_lds<D, ROPE_K>(p, kbase + BN, nks, nks + S::K_ELEMS, kr, vr);
    }
    __syncthreads();
  }

  // ---- epilogue: merge the two lane halves' sums, normalise, store ----
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
        w.x = pack_bf16(oacc[dt][4 * rr + 0] * inv_l, oacc[dt][4 * rr + 1] * inv_l);
        w.y = pack_bf16(oacc[dt][4 * rr + 2] * inv_l, oacc[dt][4 * rr + 3] * inv_l);
        *reinterpret_cast<uint2*>(dst + d0) = w;
      }
    if (p.lse && g == 0) p.lse[(int64_t)head * nq + my_row] = (m_run + log2f(l_run)) * 0.69314718055994530942f;
  }
}

template <int D, bool RQ, bool RK>
static hipError_t launch_attn(const AttnParams& p, hipStream_t s) {
  using S = AttnSmem<D>;
  static bool configured = false;
  if (!configured) {
    hipError_t e = hipFuncSetAttribute((const void*)attn_fwd_mfma<D, RQ, RK>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, S::BYTES);
    if (e != hipSuccess) return e;
    configured = true;
  }
  dim3 grid((unsigned)(p.n_qtiles * p.n_heads));
  hipLaunchKernelGGL((attn_fwd_mfma<D, RQ, RK>), grid, dim3(256), S::BYTES, s, p);
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
  p.n_qtiles = (int)((a->nq + BM - 1) / BM);
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
