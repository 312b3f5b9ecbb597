// Host-side code of libmotattn under AddressSanitizer and
// UndefinedBehaviorSanitizer: the packed-sequence layout, the noise
// schedule, the host tile classifier and the argument checks of every
// device entry point (each call here is rejected before any launch, so no
// GPU is touched).  Built with the sanitizers on the host side only, from
// the library's own sources.  Prints "ok <calls>" on success; a sanitizer
// report aborts the program.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "motattn.h"

static long calls = 0;
static int failures = 0;

#define EXPECT(cond, what)                           \
  do {                                               \
    ++calls;                                         \
    if (!(cond)) {                                   \
      printf("FAIL %s (line %d)\n", what, __LINE__); \
      ++failures;                                    \
    }                                                \
  } while (0)

static mot_segment seg(int region, int kind, int64_t n_tokens, int64_t frames = 0, int64_t views = 1,
                       int64_t gh = 0, int64_t gw = 0, double rate = 0.0, int64_t frame0 = -1,
                       int64_t step0 = 0) {
  mot_segment s;
  memset(&s, 0, sizeof(s));
  s.region = region; s.kind = kind; s.n_tokens = n_tokens; s.n_frames = frames; s.n_views = views;
  s.grid_h = gh; s.grid_w = gw; s.rate = rate; s.frame0 = frame0; s.step0 = step0;
  return s;
}

// Sizes the layout, then builds it into buffers of exactly that size.
static mot_status layout(const std::vector<mot_segment>& s, int64_t* n_out) {
  int64_t n = 0, n_ar = 0;
  mot_status st = mot_build_layout(s.data(), (int32_t)s.size(), 0, &n, &n_ar, NULL, NULL);
  *n_out = n;
  if (n == 0) return st;
  std::vector<float> pos((size_t)(3 * n));
  std::vector<uint8_t> reg((size_t)n);
  st = mot_build_layout(s.data(), (int32_t)s.size(), n, &n, &n_ar, pos.data(), reg.data());
  for (int64_t i = 0; st == MOT_OK && i < n; ++i)
    if (!isfinite(pos[3 * i]) || reg[i] > 2) return MOT_ERR_HIP;  // never a valid outcome
  return st;
}

static void layouts() {
  const int AR = MOT_REGION_AR, CL = MOT_REGION_DM_CLEAN, NO = MOT_REGION_DM_NOISY;
  const int TEXT = MOT_KIND_TEXT, SP = MOT_KIND_SPECIAL, VID = MOT_KIND_VIDEO, AUD = MOT_KIND_AUDIO,
            ACT = MOT_KIND_ACTION, PRO = MOT_KIND_PROPRIO;
  int64_t n;
  // the five workloads' shapes
  EXPECT(layout({seg(AR, TEXT, 32), seg(AR, SP, 1), seg(AR, SP, 1), seg(CL, VID, 0, 1, 1, 4, 6, 24),
                 seg(NO, VID, 0, 2, 1, 4, 6, 24), seg(NO, ACT, 8, 0, 1, 0, 0, 15)}, &n) == MOT_OK &&
             n == 114, "tiny");
  EXPECT(layout({seg(AR, TEXT, 256), seg(AR, SP, 1), seg(AR, SP, 1), seg(CL, VID, 0, 1, 3, 12, 20, 24),
                 seg(CL, PRO, 1), seg(NO, VID, 0, 2, 3, 12, 20, 24), seg(NO, ACT, 32, 0, 1, 0, 0, 15)},
                &n) == MOT_OK && n == 2451, "policy");
  EXPECT(layout({seg(AR, TEXT, 512), seg(AR, SP, 2), seg(NO, VID, 0, 16, 1, 30, 52, 24)}, &n) == MOT_OK &&
             n == 25474, "480p");
  EXPECT(layout({seg(AR, TEXT, 256), seg(AR, SP, 2), seg(CL, VID, 0, 8, 6, 12, 20, 24, 0),
                 seg(NO, VID, 0, 1, 6, 12, 20, 24, 8)}, &n) == MOT_OK && n == 13218, "stream");
  EXPECT(layout({seg(AR, TEXT, 512), seg(AR, SP, 2), seg(CL, VID, 0, 1, 1, 30, 52, 24),
                 seg(NO, VID, 0, 48, 1, 30, 52, 24)}, &n) == MOT_OK && n == 76954, "long 480p");
  EXPECT(layout({seg(AR, TEXT, 3), seg(NO, AUD, 40, 0, 1, 0, 0, 25, -1, 7)}, &n) == MOT_OK && n == 43, "audio");
  // rejected shapes: every one returns before writing anything
  EXPECT(layout({seg(NO, VID, 0, 1, 1, 2, 2, 24), seg(AR, TEXT, 3)}, &n) == MOT_ERR_INVALID_ARG, "AR after DM");
  EXPECT(layout({seg(NO, ACT, 3, 0, 1, 0, 0, 15), seg(NO, VID, 0, 1, 1, 2, 2, 24)}, &n) ==
             MOT_ERR_INVALID_ARG, "vision after action");
  EXPECT(layout({seg(AR, 9, 3)}, &n) == MOT_ERR_INVALID_ARG, "bad kind");
  EXPECT(layout({seg(7, TEXT, 3)}, &n) == MOT_ERR_INVALID_ARG, "bad region");
  EXPECT(layout({seg(AR, TEXT, 0)}, &n) == MOT_ERR_INVALID_ARG, "empty segment");
  EXPECT(layout({seg(AR, TEXT, -5)}, &n) == MOT_ERR_INVALID_ARG, "negative count");
  EXPECT(layout({seg(NO, VID, 0, 1, 1, 2, 2, 0.0)}, &n) == MOT_ERR_INVALID_ARG, "zero fps");
  EXPECT(layout({seg(NO, VID, 0, 1, 1, 2, 2, NAN)}, &n) == MOT_ERR_INVALID_ARG, "nan fps");
  EXPECT(layout({seg(NO, ACT, 2, 0, 1, 0, 0, -1.0)}, &n) == MOT_ERR_INVALID_ARG, "negative rate");
  // counts past int64
  EXPECT(layout({seg(NO, VID, 0, INT64_MAX / 2, 3, 1, 1, 24)}, &n) == MOT_ERR_INVALID_ARG, "video count overflow");
  EXPECT(layout({seg(AR, TEXT, INT64_MAX), seg(AR, TEXT, 1)}, &n) == MOT_ERR_INVALID_ARG, "total overflow");
  EXPECT(layout({seg(NO, VID, 0, 4, 1, 1, 1, 24, INT64_MAX - 2)}, &n) == MOT_ERR_INVALID_ARG, "frame index overflow");
  EXPECT(layout({seg(NO, ACT, 4, 0, 1, 0, 0, 15, -1, INT64_MAX - 2)}, &n) == MOT_ERR_INVALID_ARG, "step overflow");
  // a continuing video segment whose running frame count passes int64
  EXPECT(layout({seg(NO, VID, 0, 1, 1, 1, 1, 24, INT64_MAX - 1), seg(NO, VID, 0, 2, 1, 1, 1, 24)}, &n) ==
             MOT_ERR_INVALID_ARG, "running frame count overflow");
  EXPECT(layout({seg(NO, VID, 0, 1, 1, 1, 1, 24, INT64_MAX - 2), seg(NO, VID, 0, 1, 1, 1, 1, 24)}, &n) ==
             MOT_OK && n == 2, "running frame count at the int64 limit");
  // capacity and null checks
  int64_t nn = 0, na = 0;
  mot_segment one = seg(AR, TEXT, 4);
  float pos[6];
  uint8_t reg[2];
  EXPECT(mot_build_layout(&one, 1, 2, &nn, &na, pos, reg) == MOT_ERR_INVALID_ARG && nn == 4, "capacity");
  EXPECT(mot_build_layout(NULL, 1, 0, &nn, &na, NULL, NULL) == MOT_ERR_INVALID_ARG, "null segs");
  EXPECT(mot_build_layout(&one, 0, 0, &nn, &na, NULL, NULL) == MOT_ERR_INVALID_ARG, "no segs");
  EXPECT(mot_build_layout(&one, 1, 4, &nn, &na, NULL, reg) == MOT_ERR_INVALID_ARG, "null pos");
  EXPECT(mot_build_layout(&one, 1, -1, &nn, &na, NULL, NULL) == MOT_ERR_INVALID_ARG, "negative capacity");
}

static void schedules() {
  std::vector<float> s(1001);
  const double shifts[] = {1.0, 5.0, 10.0, 0.5, 0x1p-20, 0x1p20, 3e-6, 9e5};
  for (double sh : shifts)
    for (int n = 1; n <= 1000; n = n < 60 ? n + 1 : n * 2) {
      EXPECT(mot_sigma_schedule(n, sh, s.data()) == MOT_OK, "schedule");
      EXPECT(s[0] == 1.0f && s[n] == 0.0f, "schedule end points");
    }
  EXPECT(mot_sigma_schedule(0, 1.0, s.data()) == MOT_ERR_INVALID_ARG, "zero steps");
  EXPECT(mot_sigma_schedule(4, 0.0, s.data()) == MOT_ERR_INVALID_ARG, "zero shift");
  EXPECT(mot_sigma_schedule(4, -2.0, s.data()) == MOT_ERR_INVALID_ARG, "negative shift");
  EXPECT(mot_sigma_schedule(4, INFINITY, s.data()) == MOT_ERR_INVALID_ARG, "inf shift");
  EXPECT(mot_sigma_schedule(4, 1e-300, s.data()) == MOT_ERR_INVALID_ARG, "shift below the range");
  EXPECT(mot_sigma_schedule(4, 0x1p-21, s.data()) == MOT_ERR_INVALID_ARG, "shift just below the range");
  EXPECT(mot_sigma_schedule(4, 0x1p21, s.data()) == MOT_ERR_INVALID_ARG, "shift above the range");
  EXPECT(mot_sigma_schedule(4, NAN, s.data()) == MOT_ERR_INVALID_ARG, "nan shift");
  EXPECT(mot_sigma_schedule(4, 1.0, NULL) == MOT_ERR_INVALID_ARG, "null buffer");
  EXPECT(mot_sigma_schedule(INT32_MIN, 1.0, s.data()) == MOT_ERR_INVALID_ARG, "int32 min steps");
}

static mot_attn_args args(int64_t nq, int64_t nk, int64_t q0, int mask, int64_t n_ar, int64_t n_prefix,
                          int64_t chunk_len) {
  mot_attn_args a;
  memset(&a, 0, sizeof(a));
  a.mask = mask; a.nq = nq; a.nk = nk; a.q0 = q0; a.n_ar = n_ar; a.n_prefix = n_prefix;
  a.chunk_len = chunk_len;
  return a;
}

static void tile_classes() {
  struct { int64_t nq, nk, q0; int mask; int64_t n_ar, n_prefix, chunk; int bm, bn; } cases[] = {
      {1030, 1030, 0, 0, 514, 0, 0, 128, 64},   {333, 1111, 700, 0, 514, 0, 0, 128, 64},
      {304, 562, 258, 1, 0, 258, 97, 128, 64},  {1, 5, 4, 0, 2, 0, 0, 1, 1},
      {25474, 25474, 0, 0, 514, 0, 0, 128, 64}, {1440, 13218, 11778, 1, 0, 258, 1440, 128, 64},
      {7, 7, 0, 1, 0, 0, 3, 1, 1},              {50, 60, 10, 0, 60, 0, 0, 7, 13}};
  for (auto& c : cases) {
    mot_attn_args a = args(c.nq, c.nk, c.q0, c.mask, c.n_ar, c.n_prefix, c.chunk);
    std::vector<uint8_t> t((size_t)(((c.nq + c.bm - 1) / c.bm) * ((c.nk + c.bn - 1) / c.bn)));
    EXPECT(mot_tile_classes_host(&a, c.bm, c.bn, t.data()) == MOT_OK, "tile classes");
    for (uint8_t v : t) EXPECT(v <= 2, "tile class value");
  }
  mot_attn_args a = args(10, 10, 0, 0, 3, 0, 0);
  uint8_t t[4];
  EXPECT(mot_tile_classes_host(&a, 0, 4, t) == MOT_ERR_INVALID_ARG, "bm 0");
  EXPECT(mot_tile_classes_host(&a, 4, 4, NULL) == MOT_ERR_INVALID_ARG, "null tiles");
  a = args(10, 5, 0, 0, 3, 0, 0);
  EXPECT(mot_tile_classes_host(&a, 4, 4, t) == MOT_ERR_INVALID_ARG, "AR mode nk < q0 + nq");
  a = args(INT64_MAX, 10, 5, 0, 3, 0, 0);
  EXPECT(mot_tile_classes_host(&a, 4, 4, t) == MOT_ERR_INVALID_ARG, "q0 + nq past int64");
  a = args(10, 20, 0, 1, 0, 5, 3);
  EXPECT(mot_tile_classes_host(&a, 4, 4, t) == MOT_ERR_INVALID_ARG, "chunk mode q0 < n_prefix");
  a = args(10, 20, 5, 1, 0, 5, 0);
  EXPECT(mot_tile_classes_host(&a, 4, 4, t) == MOT_ERR_INVALID_ARG, "chunk_len 0");
}

// Fake device pointers: every call below is rejected by its argument
// checks, which run before any launch, so these are never dereferenced.
static void* const P16 = (void*)(uintptr_t)0x10000;
static void* const P16B = (void*)(uintptr_t)0x20000;
static void* const P_ODD = (void*)(uintptr_t)0x10008;

static mot_attn_args attn(int dt, int hd) {
  mot_attn_args a = args(100, 100, 0, 0, 10, 0, 0);
  a.q = P16; a.k = P16; a.v = P16; a.o = P16B;
  a.dt = dt; a.n_heads = 2; a.head_dim = hd;
  a.q_ts = a.k_ts = a.v_ts = a.o_ts = 2 * hd;
  a.q_hs = a.k_hs = a.v_hs = a.o_hs = hd;
  return a;
}

static void device_argument_checks() {
  mot_attn_args a;
  EXPECT(mot_attention_fwd(NULL, NULL) == MOT_ERR_INVALID_ARG, "null args");
  a = attn(MOT_BF16, 96);
  EXPECT(mot_attention_fwd(&a, NULL) == MOT_ERR_INVALID_ARG, "head_dim 96");
  a = attn(MOT_BF16, 128); a.q = NULL;
  EXPECT(mot_attention_fwd(&a, NULL) == MOT_ERR_INVALID_ARG, "null q");
  a = attn(MOT_BF16, 128); a.k = P_ODD;
  EXPECT(mot_attention_fwd(&a, NULL) == MOT_ERR_INVALID_ARG, "misaligned k");
  a = attn(MOT_BF16, 128); a.k_ts = 130;
  EXPECT(mot_attention_fwd(&a, NULL) == MOT_ERR_INVALID_ARG, "stride not a multiple of 8");
  a = attn(MOT_BF16, 128); a.v_hs = 0;
  EXPECT(mot_attention_fwd(&a, NULL) == MOT_ERR_INVALID_ARG, "zero stride");
  a = attn(MOT_BF16, 128); a.dt = 7;
  EXPECT(mot_attention_fwd(&a, NULL) == MOT_ERR_INVALID_ARG, "bad dtype");
  a = attn(MOT_BF16, 128); a.scale = -1.0f;
  EXPECT(mot_attention_fwd(&a, NULL) == MOT_ERR_INVALID_ARG, "negative scale");
  a = attn(MOT_BF16, 128); a.scale = NAN;
  EXPECT(mot_attention_fwd(&a, NULL) == MOT_ERR_INVALID_ARG, "nan scale");
  a = attn(MOT_BF16, 128); a.k_pos = (const float*)P16;
  EXPECT(mot_attention_fwd(&a, NULL) == MOT_ERR_UNSUPPORTED, "bf16 k_pos");
  a = attn(MOT_BF16, 128); a.nk = (int64_t)INT32_MAX; a.n_ar = 0;
  EXPECT(mot_attention_fwd(&a, NULL) == MOT_ERR_UNSUPPORTED, "nk past int32");
  a = attn(MOT_BF16, 128); a.k_ts = (int64_t)1 << 25;
  EXPECT(mot_attention_fwd(&a, NULL) == MOT_ERR_UNSUPPORTED, "64-row tile past 4 GiB");
  a = attn(MOT_BF16, 128); a.nq = (int64_t)1 << 40; a.nk = (int64_t)1 << 41;
  EXPECT(mot_attention_fwd(&a, NULL) == MOT_ERR_UNSUPPORTED, "dispatch past 2^32 work-items");
  a = attn(MOT_FP32, 64); a.q_pos = (const float*)P16; a.sec_t = 8; a.sec_h = 12; a.sec_w = 11;
  EXPECT(mot_attention_fwd(&a, NULL) == MOT_ERR_INVALID_ARG, "sections off by one");
  a = attn(MOT_FP32, 64); a.q_pos = (const float*)P16; a.sec_t = 8; a.sec_h = 12; a.sec_w = 12;
  a.theta = 0.0f;
  EXPECT(mot_attention_fwd(&a, NULL) == MOT_ERR_INVALID_ARG, "theta 0");
  a = attn(MOT_FP32, 64); a.mask = 5;
  EXPECT(mot_attention_fwd(&a, NULL) == MOT_ERR_INVALID_ARG, "bad mask");
  a = attn(MOT_FP32, 64); a.q0 = INT64_MAX;
  EXPECT(mot_attention_fwd(&a, NULL) == MOT_ERR_INVALID_ARG, "q0 overflow");
  a = attn(MOT_BF16, 128); a.n_kv_heads = 3;
  EXPECT(mot_attention_fwd(&a, NULL) == MOT_ERR_INVALID_ARG, "kv heads not dividing");
  a = attn(MOT_BF16, 128); a.n_batch = 70000;
  EXPECT(mot_attention_fwd(&a, NULL) == MOT_ERR_INVALID_ARG, "batch past grid y");
  a = attn(MOT_BF16, 128); a.n_batch = 2; a.k_bs = -256;
  EXPECT(mot_attention_fwd(&a, NULL) == MOT_ERR_INVALID_ARG, "negative batch stride");
  a = attn(MOT_FP32, 64); a.n_heads = 70000;
  a.q_hs = a.k_hs = a.v_hs = a.o_hs = 64; a.q_ts = a.k_ts = a.v_ts = a.o_ts = 64 * 70000;
  EXPECT(mot_attention_fwd(&a, NULL) == MOT_ERR_UNSUPPORTED, "fp32 heads past grid y");

  EXPECT(mot_qkv_project(P16, P16, P16, P16B, 10, 11, 64, 64, MOT_BF16, MOT_BF16, NULL) ==
             MOT_ERR_INVALID_ARG, "n_ar > n_rows");
  EXPECT(mot_qkv_project(P16, P16, P16, P16B, 0, 0, 64, 64, MOT_BF16, MOT_BF16, NULL) == MOT_OK,
         "empty projection is a no-op");
  EXPECT(mot_qkv_project(P16, NULL, P16, P16B, 10, 5, 64, 64, MOT_BF16, MOT_BF16, NULL) ==
             MOT_ERR_INVALID_ARG, "null weights of a room with rows");
  EXPECT(mot_qkv_project(P16, P16, P16, P16B, 10, 5, 60, 64, MOT_BF16, MOT_BF16, NULL) ==
             MOT_ERR_UNSUPPORTED, "d_in not a multiple of 64");
  EXPECT(mot_qkv_project(P16, P16, P16, P16B, 10, 5, 64, 64, MOT_FP32, MOT_BF16, NULL) ==
             MOT_ERR_UNSUPPORTED, "fp32 in, bf16 out");
  EXPECT(mot_qkv_project(P_ODD, P16, P16, P16B, 10, 5, 64, 64, MOT_BF16, MOT_BF16, NULL) ==
             MOT_ERR_INVALID_ARG, "misaligned x");
  EXPECT(mot_qkv_project(P16, P16, P16, P16B, (int64_t)1 << 40, 5, 64, 1 << 20, MOT_BF16, MOT_BF16,
                         NULL) == MOT_ERR_UNSUPPORTED, "projection dispatch too large");

  EXPECT(mrope_apply(P16, MOT_BF16, 10, 2, 128, 256, 128, (const float*)P16B, 16, 24, 23, 1e4f, NULL) ==
             MOT_ERR_INVALID_ARG, "mrope sections");
  EXPECT(mrope_apply(P16, MOT_BF16, 0, 2, 128, 256, 128, (const float*)P16B, 16, 24, 24, 1e4f, NULL) ==
             MOT_OK, "mrope empty is a no-op");
  EXPECT(mrope_apply(P16, MOT_BF16, (int64_t)1 << 40, 2, 128, 256, 128, (const float*)P16B, 16, 24, 24,
                     1e4f, NULL) == MOT_ERR_UNSUPPORTED, "mrope dispatch too large");
  EXPECT(mrope_apply(P16, MOT_BF16, 10, 2, 128, 250, 128, (const float*)P16B, 16, 24, 24, 1e4f, NULL) ==
             MOT_ERR_INVALID_ARG, "mrope stride");

  EXPECT(flow_euler_step((float*)P16, P16B, MOT_BF16, -1, 1.0f, 0.5f, NULL, NULL) == MOT_ERR_INVALID_ARG,
         "euler negative n");
  EXPECT(flow_euler_step((float*)P16, P16B, MOT_BF16, 0, 1.0f, 0.5f, NULL, NULL) == MOT_OK,
         "euler empty is a no-op");
  EXPECT(flow_euler_step((float*)P_ODD, P16B, MOT_BF16, 8, 1.0f, 0.5f, NULL, NULL) == MOT_ERR_INVALID_ARG,
         "euler misaligned");
  EXPECT(flow_euler_step((float*)P16, P16B, 9, 8, 1.0f, 0.5f, NULL, NULL) == MOT_ERR_INVALID_ARG,
         "euler bad dtype");
  EXPECT(flow_cfg_euler_step((float*)P16, P16B, NULL, MOT_BF16, 8, 3.0f, 1.0f, 0.5f, NULL, NULL) ==
             MOT_ERR_INVALID_ARG, "guided euler null base");
  EXPECT(flow_cfg_euler_step((float*)P16, P16B, P16B, MOT_BF16, 8, NAN, 1.0f, 0.5f, NULL, NULL) ==
             MOT_ERR_INVALID_ARG, "guided euler nan guidance");
  EXPECT(flow_cfg_euler_step((float*)P16, P16B, P_ODD, MOT_BF16, 8, 3.0f, 1.0f, 0.5f, NULL, NULL) ==
             MOT_ERR_INVALID_ARG, "guided euler misaligned");
  EXPECT(flow_cfg_euler_step((float*)P16, P16B, P16B, 9, 8, 3.0f, 1.0f, 0.5f, NULL, NULL) ==
             MOT_ERR_INVALID_ARG, "guided euler bad dtype");

  EXPECT(mot_region_linear(P16, P16, P16, P16B, 10, 5, 64, 64, MOT_BF16, MOT_BF16, 7, NULL, NULL) ==
             MOT_ERR_INVALID_ARG, "unknown epilogue");
  EXPECT(mot_region_linear(P16, P16, P16, P16B, 10, 5, 64, 64, MOT_BF16, MOT_BF16, MOT_EPI_ADD, NULL, NULL) ==
             MOT_ERR_INVALID_ARG, "add without residual");
  EXPECT(mot_region_linear(P16, P16, P16, P16B, 10, 5, 64, 64, MOT_BF16, MOT_BF16, MOT_EPI_GELU, P16, NULL) ==
             MOT_ERR_INVALID_ARG, "residual without add");
  EXPECT(mot_layernorm_region(P16, P16B, 10, 4, 100, (const float*)P16, (const float*)P16,
                              (const float*)P16, (const float*)P16, 1e-6f, MOT_BF16, MOT_BF16, NULL) ==
             MOT_ERR_INVALID_ARG, "layernorm hidden");
  EXPECT(mot_layernorm_region(P16, P16B, 10, 4, 64, (const float*)P16, (const float*)P16, NULL, NULL, 1e-6f,
                              MOT_BF16, MOT_BF16, NULL) == MOT_ERR_INVALID_ARG, "layernorm DM rows, no params");
  EXPECT(mot_layernorm_region(P16, P16B, 10, 4, 64, (const float*)P16, (const float*)P16, (const float*)P16,
                              (const float*)P16, -1.0f, MOT_BF16, MOT_BF16, NULL) == MOT_ERR_INVALID_ARG,
         "layernorm eps");
  EXPECT(mot_layernorm_region(P16, P16B, (int64_t)1 << 40, 4, 64, (const float*)P16, (const float*)P16,
                              (const float*)P16, (const float*)P16, 1e-6f, MOT_BF16, MOT_BF16, NULL) ==
             MOT_ERR_UNSUPPORTED, "layernorm dispatch too large");
  EXPECT(mot_attention_merge(P16, (const float*)P16, 0, 0, 10, 2, 128, 256, 128, P16B, 256, 128, NULL,
                             MOT_BF16, NULL) == MOT_ERR_INVALID_ARG, "merge no parts");
  EXPECT(mot_attention_merge(P16, (const float*)P16, 2, 4, 10, 2, 128, 256, 128, P16B, 256, 128, NULL,
                             MOT_BF16, NULL) == MOT_ERR_INVALID_ARG, "merge part stride");
  EXPECT(mot_attention_merge(P16, (const float*)P16, 2, 0, (int64_t)1 << 40, 2, 128, 256, 128, P16B, 256, 128,
                             NULL, MOT_BF16, NULL) == MOT_ERR_UNSUPPORTED, "merge dispatch too large");
  a = args(10, 5, 0, 0, 3, 0, 0);
  EXPECT(mot_mask_materialize(&a, (uint8_t*)P16, 128, 64, NULL, NULL) == MOT_ERR_INVALID_ARG,
         "mask invalid args");
  a = args((int64_t)1 << 33, (int64_t)1 << 34, 0, 0, 0, 0, 0);
  EXPECT(mot_mask_materialize(&a, (uint8_t*)P16, 128, 64, NULL, NULL) == MOT_ERR_UNSUPPORTED,
         "mask dispatch too large");
  EXPECT(strcmp(mot_status_string((mot_status)42), "unknown status") == 0, "status string");
}

int main() {
  layouts();
  schedules();
  tile_classes();
  device_argument_checks();
  if (failures) {
    printf("FAIL %d of %ld checks\n", failures, calls);
    return 1;
  }
  printf("ok %ld\n", calls);
  return 0;
}
