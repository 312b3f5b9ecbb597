// Packed-sequence layout: region tags and (t, h, w) mRoPE coordinates.
//
// "Cosmos 3 方法原理全解" §2: [AR text, EOS, BOG | DM clean | DM noisy], with
// vision, audio, action inside each DM group.  §5: text t = h = w (1D RoPE);
// video t = time, (h, w) = latent grid; audio/action t only, h = w = 0;
// TPS_video = FPS/4, Δt = 6/TPS; the DM time axis starts 15000 after AR.
// §4.1/§5: clean prefix and noisy future share one frame count.
//
// Built with -ffp-contract=off: every position is one double expression
// rounded once to float, so the result is bit-reproducible.
#include <stdint.h>
#include <string.h>

#include "../../include/motattn.h"

namespace {

const double kArDmTimeGap = 15000.0;

int dm_class(int32_t kind) {
  switch (kind) {
    case MOT_KIND_VIDEO: return 0;
    case MOT_KIND_AUDIO: return 1;
    case MOT_KIND_ACTION:
    case MOT_KIND_PROPRIO: return 2;
    default: return -1;
  }
}

// Tokens of a segment, or -1 when the count does not fit in int64.
int64_t seg_count(const mot_segment& s) {
  if (s.kind != MOT_KIND_VIDEO) return s.n_tokens;
  int64_t c = s.n_frames;
  if (__builtin_mul_overflow(c, s.n_views, &c) || __builtin_mul_overflow(c, s.grid_h, &c) ||
      __builtin_mul_overflow(c, s.grid_w, &c))
    return -1;
  return c;
}

bool seg_valid(const mot_segment& s) {
  if (s.region < MOT_REGION_AR || s.region > MOT_REGION_DM_NOISY) return false;
  if (s.kind < MOT_KIND_TEXT || s.kind > MOT_KIND_PROPRIO) return false;
  if (s.kind == MOT_KIND_VIDEO) {
    if (s.n_frames <= 0 || s.n_views <= 0 || s.grid_h <= 0 || s.grid_w <= 0) return false;
    if (!(s.rate > 0.0)) return false;
    if (s.frame0 > INT64_MAX - s.n_frames) return false;  // frame indices stay in int64
  } else {
    if (s.n_tokens <= 0) return false;
    if ((s.kind == MOT_KIND_AUDIO || s.kind == MOT_KIND_ACTION) && !(s.rate > 0.0)) return false;
    if (s.kind == MOT_KIND_AUDIO || s.kind == MOT_KIND_ACTION) {
      if (s.step0 < 0 || s.step0 > INT64_MAX - s.n_tokens) return false;
    }
  }
  if (s.region == MOT_REGION_AR) return s.kind == MOT_KIND_TEXT || s.kind == MOT_KIND_SPECIAL;
  return dm_class(s.kind) >= 0;
}

// Time of token k on a ladder of `tps` tokens per second (§5).
inline float ladder_time(double t0, int64_t k, double tps) {
  double num = 6.0 * (double)k;
  double dt = num / tps;
  double t = t0 + dt;
  return (float)t;
}

}  // namespace

extern "C" mot_status mot_build_layout(const mot_segment* segs, int32_t n_segs,
                                       int64_t capacity, int64_t* n_tok_out,
                                       int64_t* n_ar_out, float* pos, uint8_t* region) {
  if (!segs || n_segs <= 0 || !n_tok_out || !n_ar_out || capacity < 0) return MOT_ERR_INVALID_ARG;
  if (capacity > 0 && (!pos || !region)) return MOT_ERR_INVALID_ARG;
  *n_tok_out = 0;
  *n_ar_out = 0;
  // Validate and count; enforce the §2 order.
  int64_t n = 0, n_ar = 0;
  int64_t frames = 0;  // running latent-frame count (a video segment with frame0 < 0 continues it)
  bool seen_dm = false;
  int32_t last_region = MOT_REGION_AR;
  int last_class = -1;
  for (int32_t a = 0; a < n_segs; ++a) {
    const mot_segment& s = segs[a];
    if (!seg_valid(s)) return MOT_ERR_INVALID_ARG;
    const int64_t c = seg_count(s);
    if (c < 0 || c > INT64_MAX - n) return MOT_ERR_INVALID_ARG;  // count past int64
    if (s.kind == MOT_KIND_VIDEO) {
      const int64_t f0 = s.frame0 >= 0 ? s.frame0 : frames;
      if (f0 > INT64_MAX - s.n_frames) return MOT_ERR_INVALID_ARG;  // frame index past int64
      frames = f0 + s.n_frames;
    }
    if (s.region == MOT_REGION_AR) {
      if (seen_dm) return MOT_ERR_INVALID_ARG;
      n_ar += c;
    } else {
      seen_dm = true;
      if (s.region < last_region) return MOT_ERR_INVALID_ARG;
      if (s.region != last_region) last_class = -1;
      int cl = dm_class(s.kind);
      if (cl < last_class) return MOT_ERR_INVALID_ARG;
      last_region = s.region;
      last_class = cl;
    }
    n += c;
  }
  *n_tok_out = n;
  *n_ar_out = n_ar;
  if (n > capacity) return MOT_ERR_INVALID_ARG;

  const double t0 = (double)n_ar + kArDmTimeGap;
  int64_t i = 0, i_ar = 0, frames_seen = 0;
  for (int32_t a = 0; a < n_segs; ++a) {
    const mot_segment& s = segs[a];
    if (s.region == MOT_REGION_AR) {
      for (int64_t k = 0; k < s.n_tokens; ++k, ++i, ++i_ar) {
        float p = (float)i_ar;
        pos[3 * i + 0] = p;
        pos[3 * i + 1] = p;
        pos[3 * i + 2] = p;
        region[i] = (uint8_t)s.region;
      }
      continue;
    }
    if (s.kind == MOT_KIND_VIDEO) {
      int64_t f0 = s.frame0 >= 0 ? s.frame0 : frames_seen;
      double tps = s.rate / 4.0;
      for (int64_t f = 0; f < s.n_frames; ++f) {
        float t = ladder_time(t0, f0 + f, tps);
        for (int64_t v = 0; v < s.n_views; ++v)
          for (int64_t r = 0; r < s.grid_h; ++r)
            for (int64_t c = 0; c < s.grid_w; ++c, ++i) {
              pos[3 * i + 0] = t;
              pos[3 * i + 1] = (float)r;
              pos[3 * i + 2] = (float)(v * s.grid_w + c);
              region[i] = (uint8_t)s.region;
            }
      }
      frames_seen = f0 + s.n_frames;
    } else if (s.kind == MOT_KIND_AUDIO || s.kind == MOT_KIND_ACTION) {
      for (int64_t k = 0; k < s.n_tokens; ++k, ++i) {
        pos[3 * i + 0] = ladder_time(t0, s.step0 + k, s.rate);
        pos[3 * i + 1] = 0.0f;
        pos[3 * i + 2] = 0.0f;
        region[i] = (uint8_t)s.region;
      }
    } else {  // proprio: the current observation time
      for (int64_t k = 0; k < s.n_tokens; ++k, ++i) {
        pos[3 * i + 0] = (float)t0;
        pos[3 * i + 1] = 0.0f;
        pos[3 * i + 2] = 0.0f;
        region[i] = (uint8_t)s.region;
      }
    }
  }
  return MOT_OK;
}
