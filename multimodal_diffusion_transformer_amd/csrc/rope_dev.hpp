// Device-side mRoPE helpers shared by the kernels that rotate on load.
#pragma once

#include "common.hpp"

namespace mot {

struct RopeTable {
  double inv_freq[64];  // theta^(-2k/D) for pair k < D/2
  int sec_t;            // pairs [0, sec_t) read t
  int sec_th;           // pairs [sec_t, sec_th) read h, the rest w
};

// cos/sin of a = pos * inv_freq ("Cosmos 3 方法原理全解" §5 coordinates).
// The angle and its reduction to [-pi, pi] are done in fp64 (DM times sit
// near 1.5e4 rad, where fp32 has ~1e-3 rad of spacing); the reduced angle is
// then evaluated with fp32 sincosf.
__device__ inline void rope_cs(float pos, double inv_freq, float& c, float& s) {
  const double two_pi = 6.283185307179586476925286766559;
  const double inv_two_pi = 0.15915494309189533576888376337251;
  double a = (double)pos * inv_freq;
  double n = rint(a * inv_two_pi);
  double r = fma(-n, two_pi, a);
  sincosf((float)r, &s, &c);
}

__device__ inline int rope_axis(const RopeTable& rt, int k) {
  return k < rt.sec_t ? 0 : (k < rt.sec_th ? 1 : 2);
}

}  // namespace mot
