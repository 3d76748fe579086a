// The analytic speedup model of speculative decoding, evaluated on the host
// from measured step times to choose the speculation length.
//
// MagicDec (summary on jarxiv.com; deep notes on papercache.org, §3.1 and
// §4.1): one round drafts gamma tokens and verifies them in one batched
// target pass; with a per-token acceptance rate alpha it yields Omega(gamma,
// alpha) tokens on average, and the speedup over plain decoding is
// T_T * Omega / (T_select + gamma * T_D + T_V(gamma)), the selection term
// being the cost of choosing the draft's compressed cache. A static selection
// is charged once (a fixed share per round), a dynamic one at every draft
// step (gamma searches per round).
#include <math.h>

#include "sd.h"

namespace {

bool time_ok(double t) { return t >= 0.0 && t < HUGE_VAL; }

}  // namespace

extern "C" double sd_expected_tokens(int32_t gamma, double alpha) {
  if (gamma < 0 || !(alpha >= 0.0 && alpha <= 1.0)) return NAN;
  // at least i drafts are accepted with probability alpha^i, i = 0..gamma
  double sum = 0.0, p = 1.0;
  for (int32_t i = 0; i <= gamma; ++i) {
    sum += p;
    p *= alpha;
  }
  return sum;
}

extern "C" double sd_speedup(double t_target, double t_draft, double t_verify, int32_t gamma, double alpha,
                             double t_select_fixed, double t_select_step) {
  if (!(t_target > 0.0) || !time_ok(t_target) || !time_ok(t_draft) || !time_ok(t_verify) ||
      !time_ok(t_select_fixed) || !time_ok(t_select_step))
    return NAN;
  const double omega = sd_expected_tokens(gamma, alpha);
  const double round = t_select_fixed + gamma * t_select_step + gamma * t_draft + t_verify;
  if (omega != omega || !(round > 0.0)) return NAN;
  return t_target * omega / round;
}

extern "C" sd_status sd_best_gamma(double t_target, double t_draft, const double *t_verify, int32_t max_gamma,
                                   double alpha, double t_select_fixed, double t_select_step,
                                   int32_t *gamma_out, double *speedup_out) {
  if (t_verify == nullptr || gamma_out == nullptr || speedup_out == nullptr || max_gamma < 1)
    return SD_ERR_INVALID_ARG;
  int32_t best = 0;
  double best_time = HUGE_VAL;  // expected time per token
  for (int32_t g = 1; g <= max_gamma; ++g) {
    if (sd_speedup(t_target, t_draft, t_verify[g - 1], g, alpha, t_select_fixed, t_select_step) !=
        sd_speedup(t_target, t_draft, t_verify[g - 1], g, alpha, t_select_fixed, t_select_step))
      return SD_ERR_INVALID_ARG;  // NaN: a bad time or alpha
    const double round = t_select_fixed + g * t_select_step + g * t_draft + t_verify[g - 1];
    const double per_token = round / sd_expected_tokens(g, alpha);
    if (per_token < best_time) {  // ties keep the smaller gamma
      best_time = per_token;
      best = g;
    }
  }
  *gamma_out = best;
  *speedup_out = t_target / best_time;
  return SD_OK;
}
