// Sampler noise levels with the flow shift, host only.
//
// "Cosmos 3 方法原理全解" §6.3: with t̄ = 1 - t the shifted noise level is
// σ = s·t̄ / (1 + (s - 1)·t̄); §7.2: the sampler walks σ from 1 to 0;
// §12.1: steps and shift per model and mode.  The n-step grid is t = k/n.
//
// Built with -ffp-contract=off: each σ is one double expression, evaluated
// left to right and rounded once to float, so the result is reproducible
// bit for bit.
#include <math.h>
#include <stdint.h>

#include "../../include/motattn.h"

extern "C" mot_status mot_sigma_schedule(int32_t n_steps, double shift, float* sigmas_host) {
  if (n_steps < 1 || !sigmas_host) return MOT_ERR_INVALID_ARG;
  // A shift in [2^-20, 2^20]: the pages use 1 to 10.  Below the range the
  // denominator 1 + (s - 1) loses s to cancellation (sigma_0 would not be 1).
  if (!(shift >= 0x1p-20 && shift <= 0x1p20)) return MOT_ERR_INVALID_ARG;
  const double n = (double)n_steps;
  for (int32_t k = 0; k <= n_steps; ++k) {
    const double t_bar = (double)(n_steps - k) / n;
    const double sigma = shift * t_bar / (1.0 + (shift - 1.0) * t_bar);
    sigmas_host[k] = (float)sigma;
  }
  return MOT_OK;
}
