// Host walk of the direct-to-LDS region GEMM's addresses (gemm_tiles.hpp):
// for a problem of `rows` rows starting at row r0 of X [M][K], weights
// W [K][N], every LDS-DMA copy of the chosen tiles and stages (X and W), and
// every MFMA operand read back from LDS.  Checks, for each lane:
//  * the copy's per-lane offset is the unsigned 32-bit value the kernel
//    passes (no wrap), and base + offset is exactly the 8-element run of X
//    or W the tile row and chunk need, inside the matrix (rows past the
//    problem and chunks past N re-read the last valid ones);
//  * LDS slots are written once, at the swizzled chunk;
//  * the B operand (X, ds_read_b128) gives lane l row m = 128 wm + 32 mb +
//    l % 32 and k = 16 s + 8 (l / 32) + 0..7, and the A operand (W^T, the
//    transposing reads) gives col n = 64 wn + 32 nb + l % 32 and the same k,
//    wherever the output they feed is stored (m < rows, n < N).
// Prints "ok <copies> <reads>" or the first mismatches; exit status 1 on any.
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "gemm_tiles.hpp"

using namespace mot;
using A = GemmTileAddr;

static long errors = 0, copies = 0, reads = 0;
#define CHECK(c, ...)                               \
  do {                                              \
    if (!(c)) {                                     \
      if (errors < 10) {                            \
        printf("FAIL %s:%d: ", __FILE__, __LINE__); \
        printf(__VA_ARGS__);                        \
        printf("\n");                               \
      }                                             \
      ++errors;                                     \
    }                                               \
  } while (0)

struct Slot { int mat; int64_t r, c; };  // mat 0: X (row, k), 1: W (k, n)

static void stage(int64_t M, int64_t K, int64_t N, int64_t r0, int64_t rows, int64_t n0, int64_t k0) {
  std::vector<Slot> lds(H_STAGE / 16, Slot{-1, -1, -1});
  const int64_t last_c = (N - n0) / 8 - 1;
  const bool ragged_n = n0 + HN > N, ragged_m = rows < HM;
  for (int wave = 0; wave < 4; ++wave)
    for (int lane = 0; lane < 64; ++lane) {
      for (int t = 0; t < 2; ++t) {  // W
        const int i = A::w_load(wave, t);
        const int row = A::w_row(i, lane);
        int c = A::w_chunk(row, lane);
        int64_t off;
        if (!ragged_n) {
          const uint32_t lo = A::w_lane_off(lane, N);
          CHECK((int64_t)lo == (int64_t)(lane / 16) * N * 2 + 16 * c, "W lane offset wraps");
          off = A::w_tile_el(k0, n0, N) * 2 + A::w_load_bytes(i, N) + lo;
        } else {
          if (c > last_c) c = (int)last_c;
          const uint32_t ro = A::w_ragged_off(i, lane, N, n0);
          CHECK((int64_t)ro == (int64_t)row * N * 2 + 16 * c, "W ragged offset wraps");
          off = A::w_tile_el(k0, n0, N) * 2 + ro;
        }
        const int64_t k = k0 + row, n = n0 + 8 * c;
        CHECK(off == 2 * (k * N + n), "W address (k %lld n %lld)", (long long)k, (long long)n);
        CHECK(k < K && n >= 0 && n + 8 <= N, "W run outside the matrix (k %lld n %lld)", (long long)k, (long long)n);
        const int dst = A::w_lds(i, lane);
        CHECK(dst >= 0 && dst + 16 <= H_WB, "W lds");
        const int srow = dst / (HN * 2), phys = (dst % (HN * 2)) / 16;
        // the slot holds logical chunk w_chunk at physical chunk w_chunk ^ 4 (row % 4)
        CHECK(srow == row && phys == (A::w_chunk(row, lane) ^ (4 * (row & 3))), "W slot");
        CHECK(lds[dst / 16].mat == -1, "W slot written twice");
        lds[dst / 16] = Slot{1, k, n};
        ++copies;
      }
      for (int t = 0; t < 4; ++t) {  // X
        const int i = A::x_load(wave, t);
        const int row = A::x_row(i, lane);
        const int c = A::x_chunk(row, lane);
        int64_t off, rr = row;
        if (!ragged_m) {
          const uint32_t lo = A::x_lane_off(lane, K);
          CHECK((int64_t)lo == (int64_t)(lane / 4) * K * 2 + 16 * c, "X lane offset wraps");
          off = A::x_tile_el(r0, k0, K) * 2 + A::x_load_bytes(i, K) + lo;
        } else {
          if (rr > rows - 1) rr = rows - 1;
          const uint32_t ro = A::x_ragged_off(i, lane, K, rows);
          CHECK((int64_t)ro == rr * K * 2 + 16 * c, "X ragged offset wraps");
          off = A::x_tile_el(r0, k0, K) * 2 + ro;
        }
        const int64_t m = r0 + rr, k = k0 + 8 * c;
        CHECK(off == 2 * (m * K + k), "X address (m %lld k %lld)", (long long)m, (long long)k);
        CHECK(m >= 0 && m < M && k + 8 <= K, "X run outside the matrix (m %lld k %lld)", (long long)m, (long long)k);
        const int dst = A::x_lds(i, lane);
        CHECK(dst >= H_WB && dst + 16 <= H_STAGE, "X lds");
        const int srow = (dst - H_WB) / (HK * 2), phys = ((dst - H_WB) % (HK * 2)) / 16;
        CHECK(srow == row && phys == (c ^ ((row >> 2) & 1)), "X slot");
        CHECK(lds[dst / 16].mat == -1, "X slot written twice");
        lds[dst / 16] = Slot{0, m, k};
        ++copies;
      }
    }
  for (size_t s = 0; s < lds.size(); ++s) CHECK(lds[s].mat != -1, "slot %zu never written", s);
  // operand reads
  for (int wave = 0; wave < 4; ++wave) {
    const int wm = wave & 1, wn = wave >> 1;
    for (int s = 0; s < HK / 16; ++s) {
      for (int mb = 0; mb < 4; ++mb)
        for (int lane = 0; lane < 64; ++lane) {
          const uint32_t a = H_WB + A::b_read_off(wm, lane) + mb * 32 * (HK * 2) + 32 * s;
          CHECK(a % 16 == 0 && a + 16 <= (uint32_t)H_STAGE, "X read %u", a);
          const Slot& sl = lds[a / 16];
          const int64_t m = 128 * wm + 32 * mb + (lane & 31);
          if (m < rows) {
            CHECK(sl.mat == 0 && sl.r == r0 + m && sl.c == k0 + 16 * s + 8 * (lane >> 5),
                  "B operand (wave %d s %d mb %d lane %d)", wave, s, mb, lane);
          }
          ++reads;
        }
      for (int nb = 0; nb < 2; ++nb)
        for (int hh = 0; hh < 2; ++hh) {
          Slot seg[64];
          int segc[64];
          for (int lane = 0; lane < 64; ++lane) {
            const uint32_t a = A::a_read_off(wn, nb, lane) + (16 * s + 4 * hh) * (HN * 2);
            CHECK(a % 8 == 0 && a + 8 <= (uint32_t)H_WB, "W read %u", a);
            seg[lane] = lds[a / 16];
            segc[lane] = 4 * ((a % 16) / 8);
          }
          for (int lane = 0; lane < 64; ++lane) {
            const int grp = lane & ~15, i = lane & 15;
            for (int k = 0; k < 4; ++k) {
              const int src = grp + i / 4 + 4 * k;
              const int64_t n = 64 * wn + 32 * nb + (lane & 31);
              if (n0 + n < N) {
                CHECK(seg[src].mat == 1 && seg[src].c + segc[src] + i % 4 == n0 + n &&
                          seg[src].r == k0 + 16 * s + 8 * (lane >> 5) + 4 * hh + k,
                      "A operand (wave %d s %d nb %d lane %d)", wave, s, nb, lane);
              }
              ++reads;
            }
          }
        }
    }
  }
}

int main(int argc, char** argv) {
  // argv: M K N r0 rows, repeated: problem rows [r0, r0 + rows) of X [M][K]
  for (int a = 1; a + 4 < argc; a += 5) {
    const int64_t M = atoll(argv[a]), K = atoll(argv[a + 1]), N = atoll(argv[a + 2]);
    const int64_t r0 = atoll(argv[a + 3]), rows = atoll(argv[a + 4]);
    const int64_t tm = (rows + HM - 1) / HM, tn = (N + HN - 1) / HN, ks = K / HK;
    // every tile and stage for small problems; the corners otherwise (the
    // addresses are affine in the tile and stage indices)
    auto pick = [](int64_t n) {
      std::vector<int64_t> v;
      for (int64_t i = 0; i < n; ++i)
        if (n <= 6 || i < 2 || i >= n - 2) v.push_back(i);
      return v;
    };
    for (int64_t im : pick(tm))
      for (int64_t in : pick(tn))
        for (int64_t kt : pick(ks)) {
          const int64_t rr = rows - im * HM < HM ? rows - im * HM : HM;
          stage(M, K, N, r0 + im * HM, rr, in * HN, kt * HK);
        }
  }
  if (errors) {
    printf("FAIL %ld errors\n", errors);
    return 1;
  }
  printf("ok %ld %ld\n", copies, reads);
  return 0;
}
