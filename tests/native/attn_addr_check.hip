// Host walk of the bf16 attention kernel's tile addresses (attn_tiles.hpp):
// every LDS-DMA copy of every K and V tile of every key/value head of every
// batch item, and every MFMA operand read back from LDS, for a K/V view
// [nb][nk][H][D] with batch, token and head strides bs, ts, hs (elements)
// inside a buffer of `extent` elements.  Checks, for each lane:
//  * the copy's per-lane offset is the unsigned 32-bit value the kernel
//    passes (no wrap), and scalar base + offset is exactly the element run
//    (key, head, 8 dims) of its batch item that the tile row needs, with
//    key < nk (rows past the last key re-read the last key), inside the
//    buffer;
//  * the copy's LDS destination is the row's swizzled chunk, each 16-byte
//    slot of the tile written once;
//  * the K operand reads give MFMA row rho key key_perm(rho) and k-step s
//    dims 16 s + 8 (lane / 32) + 0..7, and key_perm puts keys 16 g + r in
//    accumulator register r of lane half g;
//  * the transposing V reads give lane l dim 32 dt + l % 32 and keys
//    16 (l / 32) + 8 t + 0..7 of block st, the keys the P operand holds.
// D = 80 is stored in the 128 geometry: a stored chunk c past the row's 10
// is copied from chunk c - 10 of the same row, so it stays inside the
// row; score reads never reach it, and the V reads of dims 80..95 get
// dims 0..15 of the same key.
// Prints "ok <copies> <reads>" or the first mismatches; exit status 1 on any.
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "attn_tiles.hpp"

using namespace mot;

static long errors = 0;
#define CHECK(c, ...)                                   \
  do {                                                  \
    if (!(c)) {                                         \
      if (errors < 10) {                                \
        printf("FAIL %s:%d: ", __FILE__, __LINE__);     \
        printf(__VA_ARGS__);                            \
        printf("\n");                                   \
      }                                                 \
      ++errors;                                         \
    }                                                   \
  } while (0)

struct View { int64_t nk, ts, hs; int h; int nb; int64_t bs, extent; };

template <int D>
struct Walk {
  static constexpr int DS = store_dim(D);
  using A = TileAddr<D, 4>;
  using L = Lay<DS>;
  long copies = 0, reads = 0;
  std::vector<int64_t> key;  // per 16-byte LDS slot: the key it holds
  std::vector<int> dim;      // ... and its first dim

  template <bool IS_K>
  void copy_tile(const View& v, int b, int head, int64_t kbase) {
    key.assign(L::TILE_B / 16, -1);
    dim.assign(L::TILE_B / 16, -1);
    // the kernel offsets the tensor pointer by the batch item, then takes
    // the tile base from it
    const int64_t base_el = (int64_t)b * v.bs + A::tile_base_el(kbase, v.ts, head, v.hs);
    const int64_t last = v.nk - 1 - kbase;
    const uint32_t row_b = A::row_bytes(v.ts);
    CHECK((int64_t)row_b == (int64_t)L::RPI * v.ts * 2, "row bytes wrap ts=%lld", (long long)v.ts);
    for (int wave = 0; wave < 4; ++wave)
      for (int i = 0; i < A::PER_WAVE; ++i)
        for (int lane = 0; lane < 64; ++lane) {
          const int n = wave * A::PER_WAVE + i;
          const int r = A::row_of(wave, i, lane);
          const int c = A::template chunk_of<IS_K>(r, lane);
          const int src = c < D / 8 ? c : c - D / 8;  // the row's chunk the slot holds
          CHECK(src == A::src_chunk(c), "source chunk");
          uint64_t off;  // bytes from the tensor pointer
          int64_t exact;
          if (last >= BN - 1) {
            const uint32_t rb = A::rows_bytes(n, row_b);
            const uint32_t lo = IS_K ? A::template lane_off<true>(wave, i % A::NVAR_K, lane, v.ts)
                                     : A::template lane_off<false>(wave, 0, lane, v.ts);
            CHECK((int64_t)rb == (int64_t)n * L::RPI * v.ts * 2, "rows bytes wrap");
            exact = (int64_t)(lane / L::CH) * v.ts * 2 + (int64_t)src * 16;
            CHECK((int64_t)lo == exact, "lane offset wrap or load-index aliasing lane %d i %d", lane, i);
            off = (uint64_t)(base_el * 2) + rb + lo;
          } else {
            const uint32_t ro = A::template ragged_off<IS_K>(wave, i, lane, v.ts, last);
            exact = (int64_t)(r > last ? last : r) * v.ts * 2 + (int64_t)src * 16;
            CHECK((int64_t)ro == exact && exact >= 0, "ragged offset wrap");
            off = (uint64_t)(base_el * 2) + ro;
          }
          const int64_t k = kbase + (r > last ? last : r);
          CHECK(k >= 0 && k < v.nk, "key %lld out of range", (long long)k);
          CHECK(c >= 0 && 8 * c + 8 <= DS && src >= 0 && 8 * src + 8 <= D, "chunk %d", c);
          const int64_t want = 2 * ((int64_t)b * v.bs + k * v.ts + (int64_t)head * v.hs + 8 * src);
          CHECK((int64_t)off == want, "address %llu != %lld (head %d kbase %lld lane %d)",
                (unsigned long long)off, (long long)want, head, (long long)kbase, lane);
          CHECK(want >= 0 && want / 2 + 8 <= v.extent, "outside the buffer: element %lld of %lld",
                (long long)(want / 2), (long long)v.extent);
          const int dst = A::lds_dst(n, lane);
          CHECK(dst >= 0 && dst + 16 <= L::TILE_B, "lds dst %d", dst);
          const int srow = dst / L::ROWB, phys = (dst % L::ROWB) / 16;
          CHECK(srow == r, "lds row %d != %d", srow, r);
          CHECK(phys == (c ^ (IS_K ? swz_k<DS>(r) : swz_v<DS>(r))), "swizzle");
          const int slot = dst / 16;
          CHECK(key[slot] == -1, "slot written twice");
          key[slot] = k;
          dim[slot] = 8 * src;
          ++copies;
        }
    for (size_t s = 0; s < key.size(); ++s) CHECK(key[s] != -1, "slot %zu never written", s);
  }

  void read_k(int64_t kbase, int64_t last) {
    // the score MFMA writes row rho = 8 (r / 4) + 4 (lane / 32) + r % 4 of
    // its 32x32 accumulator to register r of lane; fed in key_perm order,
    // lane half g must hold keys 16 g + r (the order the P operand uses)
    for (int lane = 0; lane < 64; ++lane)
      for (int r = 0; r < 16; ++r) {
        const int rho = 8 * (r / 4) + 4 * (lane >> 5) + r % 4;
        CHECK(key_perm(rho) == 16 * (lane >> 5) + r, "score register %d of lane %d", r, lane);
      }
    for (int lane = 0; lane < 64; ++lane)
      for (int st = 0; st < NST; ++st)
        for (int s = 0; s < D / 16; ++s) {
          const uint32_t a = k_read_off<DS>(s, lane) + st * 32 * L::ROWB;
          CHECK(a % 16 == 0 && a + 16 <= (uint32_t)L::TILE_B, "k read %u", a);
          const int rho = lane & 31;
          const int r = 32 * st + key_perm(rho);
          CHECK(key[a / 16] == kbase + (r > last ? last : r), "K operand key (lane %d st %d s %d)", lane, st, s);
          CHECK(dim[a / 16] == 16 * s + 8 * (lane >> 5), "K operand dims");
          ++reads;
        }
  }

  void read_v(int64_t kbase, int64_t last) {
    for (int dt = 0; dt < (D + 31) / 32; ++dt)
      for (int st = 0; st < NST; ++st)
        for (int t = 0; t < 2; ++t)
          for (int hh = 0; hh < 2; ++hh) {
            // each lane's 8-byte segment: 4 bf16 of one key, dims d0..d0+3
            int64_t seg_key[64];
            int seg_dim[64];
            for (int lane = 0; lane < 64; ++lane) {
              const uint32_t a = v_read_off<DS>(dt, lane) + (32 * st + 8 * t + 4 * hh) * L::ROWB;
              CHECK(a % 8 == 0 && a + 8 <= (uint32_t)L::TILE_B, "v read %u", a);
              seg_key[lane] = key[a / 16];
              seg_dim[lane] = dim[a / 16] + 4 * ((a % 16) / 8);
            }
            // transposing read: lane i of a 16-lane group receives element
            // i % 4 of the segments of lanes i/4, i/4 + 4, i/4 + 8, i/4 + 12
            for (int lane = 0; lane < 64; ++lane) {
              const int grp = lane & ~15, i = lane & 15;
              for (int k = 0; k < 4; ++k) {
                const int src = grp + i / 4 + 4 * k;
                const int64_t got_key = seg_key[src];
                const int got_dim = seg_dim[src] + i % 4;
                const int r = 32 * st + 16 * (lane >> 5) + 8 * t + 4 * hh + k;
                CHECK(got_key == kbase + (r > last ? last : r), "V operand key (lane %d dt %d)", lane, dt);
                const int want_dim = 32 * dt + (lane & 31);  // past D: a duplicate of dim - D
                CHECK(got_dim == (want_dim < D ? want_dim : want_dim - D), "V operand dim (lane %d dt %d)", lane, dt);
                ++reads;
              }
            }
          }
  }

  void run(const View& v) {
    const int64_t ntiles = (v.nk + BN - 1) / BN;
    for (int b = 0; b < v.nb; ++b)
      for (int head = 0; head < v.h; ++head)
        for (int64_t j = 0; j < ntiles; ++j) {
          const int64_t kbase = j * BN, last = v.nk - 1 - kbase;
          copy_tile<true>(v, b, head, kbase);
          read_k(kbase, last);
          copy_tile<false>(v, b, head, kbase);
          read_v(kbase, last);
        }
  }
};

// Head slot -> head map: a bijection of the heads, and with H % 8 == 0 and
// kv_group dividing H / 8 every group of kv_group consecutive heads (the
// query heads of one key/value head) on a single XCD.
static void head_map(int n_heads, int kv_group) {
  const int xh = n_heads % 8 == 0 ? n_heads / 8 : 0;
  std::vector<int> seen(n_heads, 0), xcd_of_kv(n_heads / kv_group, -1);
  for (int hs = 0; hs < n_heads; ++hs) {
    const int h = head_of_slot(hs, xh);
    CHECK(h >= 0 && h < n_heads && !seen[h], "head map not a bijection (H %d)", n_heads);
    if (h < 0 || h >= n_heads) continue;
    seen[h] = 1;
    if (xh && xh % kv_group == 0) {  // a group fits in one XCD's heads
      int& x = xcd_of_kv[h / kv_group];
      CHECK(x == -1 || x == hs % 8, "key/value head %d spread over XCDs", h / kv_group);
      x = hs % 8;
    }
  }
}

int main(int argc, char** argv) {
  // argv: "map" H kv_group | D nk ts hs H nb bs extent, repeated
  long copies = 0, reads = 0;
  int a = 1;
  while (a + 2 < argc && argv[a][0] == 'm') {
    head_map(atoi(argv[a + 1]), atoi(argv[a + 2]));
    a += 3;
  }
  for (; a + 7 < argc; a += 8) {
    const int d = atoi(argv[a]);
    View v{atoll(argv[a + 1]), atoll(argv[a + 2]), atoll(argv[a + 3]), atoi(argv[a + 4]),
           atoi(argv[a + 5]), atoll(argv[a + 6]), atoll(argv[a + 7])};
    if (d == 128) {
      Walk<128> w;
      w.run(v);
      copies += w.copies;
      reads += w.reads;
    } else if (d == 64) {
      Walk<64> w;
      w.run(v);
      copies += w.copies;
      reads += w.reads;
    } else if (d == 80) {
      Walk<80> w;
      w.run(v);
      copies += w.copies;
      reads += w.reads;
    } else {
      printf("FAIL unknown head dim %d\n", d);
      return 1;
    }
  }
  if (errors) {
    printf("FAIL %ld errors\n", errors);
    return 1;
  }
  printf("ok %ld %ld\n", copies, reads);
  return 0;
}
