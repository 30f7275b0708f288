// Host-side policy of the staggering scheduler: how long a group drafts before
// its next verification.
//
// [VC Key System Innovations P2: high acceptance of same-model compressed
//  drafting lets the system verify less often; P1: while one request group
//  drafts (HBM), another loads its full KV and verifies]  The pages give the
// principle, not a rule.  The rule here: each draft of a round matches with a
// probability a (estimated from the group's history) until the first
// mismatch, so a round of draft length k emits 1 + a + ... + a^k tokens on
// average; a round costs max(k t_draft, t_overlap) + t_rest, where t_overlap
// is the other group's work that the drafting runs beside (drafting shorter
// than it is not faster) and t_rest the part of the cycle that does not depend
// on k.  The next k maximises tokens per unit of time.
//
// Plain fp64, no contraction: the arithmetic is a handful of operations per
// candidate k, evaluated in a fixed order.
#include <cmath>

#include "vc_common.h"

#pragma clang fp contract(off)

extern "C" double vc_sched_accept_rate(long long accepted, long long rejections) {
  if (accepted < 0 || rejections < 0) return NAN;
  return ((double)accepted + 1.0) / ((double)accepted + (double)rejections + 2.0);
}

extern "C" double vc_sched_expected_tokens(double a, int k) {
  if (!(a >= 0.0 && a <= 1.0) || k < 0) return NAN;
  double s = 1.0, p = 1.0;
  for (int i = 1; i <= k; ++i) {
    p = p * a;
    s = s + p;
  }
  return s;
}

extern "C" int vc_sched_choose_k(long long accepted, long long rejections, double t_draft, double t_overlap,
                                 double t_rest, int k_min, int k_max) {
  VC_CHECK(accepted >= 0 && rejections >= 0, "vc_sched_choose_k: negative history (%lld, %lld)", accepted,
           rejections);
  VC_CHECK(k_min >= 1 && k_max >= k_min && k_max <= 64, "vc_sched_choose_k: need 1 <= k_min <= k_max <= 64 (%d, %d)",
           k_min, k_max);
  VC_CHECK(std::isfinite(t_draft) && t_draft > 0.0 && std::isfinite(t_overlap) && t_overlap >= 0.0 &&
               std::isfinite(t_rest) && t_rest >= 0.0,
           "vc_sched_choose_k: times must be finite, t_draft > 0, the others >= 0");
  const double a = vc_sched_accept_rate(accepted, rejections);
  int best = k_min;
  double best_rate = -1.0;
  double s = 1.0, p = 1.0;  // expected tokens, built up k by k in the same order as above
  for (int k = 1; k <= k_max; ++k) {
    p = p * a;
    s = s + p;
    if (k < k_min) continue;
    const double d = (double)k * t_draft;
    const double t = (d > t_overlap ? d : t_overlap) + t_rest;
    const double rate = s / t;
    if (rate > best_rate) {  // strict: ties keep the shorter round
      best_rate = rate;
      best = k;
    }
  }
  return best;
}
