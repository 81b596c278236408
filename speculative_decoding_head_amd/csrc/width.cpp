// Adaptive verify width, host side (lucebox-hub PR "feat(qwen4exp): MTP speculative
// decoding", section "What": by default the width adapts, up to seven drafts, from the
// acceptance seen at each draft depth and a per-request fit of the cycle's cost).
//
// The controller is a plain struct the caller owns, one per request stream; it is fed
// the acceptance outputs of each cycle (copied to the host) and the cycle's measured
// time, and it proposes the next width.  Arithmetic in double, in a fixed order.
//
// Exploration: a depth decided too rarely to be current (recency weight below 1/2) is
// estimated by the depth before it.  Acceptance seldom rises with depth, so depths the
// current width never reaches get an optimistic estimate, and a rise in acceptance at the
// shallow depths makes the controller try deeper drafts, which then measure their own rate.
#include <cmath>

#include "../../include/mtp.h"

extern "C" {

int mtp_width_init(mtp_width_ctl* c, int32_t k_max, double decay, double alpha0, double slope_prior) {
  if (!c) return MTP_ERR_NULL;
  if (k_max < 1 || k_max > 7) return MTP_ERR_SHAPE;
  if (!(decay > 0.0 && decay <= 1.0) || !(alpha0 >= 0.0 && alpha0 <= 1.0) || !(slope_prior >= 0.0) ||
      !std::isfinite(slope_prior))
    return MTP_ERR_RANGE;
  *c = mtp_width_ctl{};
  c->k_max = k_max;
  c->decay = decay;
  c->slope_prior = slope_prior;
  for (double& a : c->alpha) a = alpha0;
  for (double& w : c->weight) w = 0.0;
  return MTP_OK;
}

int mtp_width_observe(mtp_width_ctl* c, int32_t k, int32_t B, const int32_t* n_accept, const uint32_t* flags,
                      double seconds) {
  if (!c || !n_accept || !flags) return MTP_ERR_NULL;
  if (k < 1 || k > 7 || B < 1) return MTP_ERR_SHAPE;
  for (int b = 0; b < B; ++b)
    if (n_accept[b] < 0 || n_accept[b] > k) return MTP_ERR_RANGE;
  c->verifier_passes += 1;
  const double lam = c->decay;
  for (int b = 0; b < B; ++b) {
    const int a = n_accept[b];
    const uint32_t f = flags[b];
    c->cycles += 1;
    c->drafted += (uint64_t)k;
    c->accepted += (uint64_t)a;
    c->depth_hist[a] += 1;
    for (double& w : c->weight) w = (1.0 - lam) * w;
    // an accepted EOS draft is draft a+1, accepted
    const int accepted = (a < k && (f & MTP_ACC_EOS_DRAFT)) ? a + 1 : a;
    for (int j = 0; j < accepted; ++j) {   // drafts 1..accepted
      c->alpha[j] += lam * (1.0 - c->alpha[j]);
      c->weight[j] += 1.0;
    }
    // a rejection at draft a+1 (an EOS correction included); an unusable target row or a
    // full accept say nothing about it
    if (accepted == a && a < k && !(f & (MTP_ACC_ROW_INVALID | MTP_ACC_ALL_ACCEPTED))) {
      c->alpha[a] += lam * (0.0 - c->alpha[a]);
      c->weight[a] += 1.0;
    }
  }
  if (seconds > 0.0 && std::isfinite(seconds)) {
    const double g = 1.0 - lam;
    c->sw = g * c->sw + 1.0;
    c->sk = g * c->sk + k;
    c->skk = g * c->skk + (double)k * k;
    c->st = g * c->st + seconds;
    c->skt = g * c->skt + k * seconds;
  }
  return MTP_OK;
}

static void cost_params(const mtp_width_ctl* c, double* c0, double* c1) {
  if (c->sw <= 0.0) {
    *c0 = 1.0;
    *c1 = c->slope_prior;
    return;
  }
  const double den = c->sw * c->skk - c->sk * c->sk;
  if (den > 1e-9 * c->sw * c->sw) {
    double s = (c->sw * c->skt - c->sk * c->st) / den;
    if (s < 0.0) s = 0.0;
    *c1 = s;
    *c0 = (c->st - s * c->sk) / c->sw;
  } else {
    const double kbar = c->sk / c->sw;
    *c0 = (c->st / c->sw) / (1.0 + c->slope_prior * kbar);
    *c1 = c->slope_prior * *c0;
  }
}

double mtp_width_cost(const mtp_width_ctl* c, int32_t k) {
  if (!c) return NAN;
  double c0, c1;
  cost_params(c, &c0, &c1);
  return c0 + c1 * k;
}

double mtp_width_expected_tokens(const mtp_width_ctl* c, int32_t k) {
  if (!c || k < 0 || k > 7) return NAN;
  constexpr double kStaleWeight = 0.5;
  double e = 1.0, run = 1.0, est = c->alpha[0];
  for (int j = 0; j < k; ++j) {
    if (j > 0 && c->weight[j] >= kStaleWeight) est = c->alpha[j];   // else: depth j-1's estimate
    run *= est;
    e += run;
  }
  return e;
}

int32_t mtp_width_choose(const mtp_width_ctl* c) {
  if (!c || c->k_max < 1 || c->k_max > 7) return 1;
  double best = -INFINITY;
  int32_t best_k = 1;
  for (int k = 1; k <= c->k_max; ++k) {
    const double cost = mtp_width_cost(c, k);
    if (!(cost > 0.0)) continue;
    const double v = mtp_width_expected_tokens(c, k) / cost;
    if (v > best) {
      best = v;
      best_k = k;
    }
  }
  return best_k;
}

}  // extern "C"
