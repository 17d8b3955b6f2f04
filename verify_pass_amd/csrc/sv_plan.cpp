// Draft-length planning (host only, fp64).
//
// BUDGET follows "Speculative Decoding and Batching Compete for the Same
// Compute Slack on RDNA4", sections "The budget is fixed, and the batch is
// inside it" and "What the budget says to build": a decode step hides a fixed
// number of tokens of compute under its weight stream (decode floor divided by
// per-token compute time); each live sequence commits one of them, and what is
// left is split over the sequences.
//
// SPEEDUP follows "Speculative Decoding at High Batch Size: Where the 3x
// Speedup Turns Into a Tax", sections "What does one speculative iteration
// actually cost?" (speedup = expected tokens x plain step time over verify
// plus draft time; expected tokens (1 - a^(g+1)) / (1 - a)), "How does the
// roofline model work?" (step time = max of weight-plus-KV read time and
// compute time; crossover B* = t_w / ((g + 1) c - k)) and "Why should you not
// trust an independent-acceptance model for long drafts?" (acceptance given
// per position, as conditional rates).
#include <cmath>
#include <limits>

#include "../../include/sv.h"

namespace {

double expected_tokens(const sv_plan_params &p, int g) {
  if (p.n_alpha == 1) {
    const double a = p.alpha[0];
    if (a == 1.0) return g + 1.0;
    return (1.0 - std::pow(a, g + 1)) / (1.0 - a);
  }
  double e = 1.0, run = 1.0;
  for (int k = 0; k < g; ++k) {
    run *= p.alpha[k < p.n_alpha ? k : p.n_alpha - 1];
    e += run;
  }
  return e;
}

// The roofline step model: a pass over b sequences of n tokens each, through
// a model `size` times the target's, costs the larger of its reads (weights
// scaled by size, every sequence's KV not) and its arithmetic.
struct StepModel {
  double t_w, k, c;
  double pass(double b, double n, double size) const {
    const double reads = size * t_w + b * k, arithmetic = size * c * b * n;
    return reads >= arithmetic ? reads : arithmetic;
  }
  // target verifies g + 1 tokens per sequence, drafter of size f proposes g
  double iteration(double b, int g, double f) const { return pass(b, g + 1.0, 1.0) + pass(b, g, f); }
};

// Throughput relative to plain decoding at the same batch (g = 0: exactly 1).
double speedup(double b, int g, const sv_plan_params &p) {
  if (g == 0) return 1.0;
  const StepModel m{p.t_w_ms, p.k_ms, p.c_ms};
  return expected_tokens(p, g) * m.pass(b, 1.0, 1.0) / m.iteration(b, g, p.draft_frac);
}

double crossover(int g, const sv_plan_params &p) {
  if (!(p.t_w_ms > 0) || !(p.c_ms > 0)) return std::numeric_limits<double>::infinity();
  const double den = (g + 1) * p.c_ms - p.k_ms;
  return den <= 0 ? std::numeric_limits<double>::infinity() : p.t_w_ms / den;
}

}  // namespace

extern "C" sv_status sv_plan_gamma(const sv_plan_params *prm, int32_t B_live, int32_t *gamma_out,
                                   double *bstar_out) {
  if (!prm || B_live < 0 || prm->gamma_max < 0) return SV_ERR_INVALID_ARG;
  if (B_live > 0 && !gamma_out) return SV_ERR_INVALID_ARG;
  const sv_plan_params &p = *prm;
  int gbig = 0;
  if (p.mode == SV_PLAN_BUDGET) {
    long long n = p.budget_tokens;
    if (n <= 0) {
      if (!(p.t_floor_ms > 0) || !(p.c_ms > 0)) return SV_ERR_INVALID_ARG;
      n = (long long)std::floor(p.t_floor_ms / p.c_ms);
    }
    if (B_live >= n) {
      for (int i = 0; i < B_live; ++i) gamma_out[i] = 0;
    } else if (B_live > 0) {
      const long long freet = n - B_live;
      const long long base = freet / B_live, rem = freet % B_live;
      for (int i = 0; i < B_live; ++i) {
        long long g = base + ((p.fill_remainder && i < rem) ? 1 : 0);
        if (g > p.gamma_max) g = p.gamma_max;
        gamma_out[i] = (int32_t)g;
        if (g > gbig) gbig = (int)g;
      }
    }
  } else if (p.mode == SV_PLAN_SPEEDUP) {
    if (p.n_alpha < 1 || !p.alpha) return SV_ERR_INVALID_ARG;
    for (int i = 0; i < p.n_alpha; ++i)
      if (!(p.alpha[i] >= 0.0 && p.alpha[i] <= 1.0)) return SV_ERR_INVALID_ARG;
    if (!(p.t_w_ms > 0) || !(p.c_ms > 0) || !(p.k_ms >= 0) || !(p.draft_frac >= 0))
      return SV_ERR_INVALID_ARG;
    int best = 0;
    double best_s = 1.0;
    for (int g = 1; g <= p.gamma_max; ++g) {
      const double s = speedup((double)B_live, g, p);
      if (s > best_s) {
        best_s = s;
        best = g;
      }
    }
    for (int i = 0; i < B_live; ++i) gamma_out[i] = best;
    gbig = B_live > 0 ? best : 0;
  } else {
    return SV_ERR_INVALID_ARG;
  }
  if (bstar_out) *bstar_out = crossover(gbig, p);
  return SV_OK;
}
