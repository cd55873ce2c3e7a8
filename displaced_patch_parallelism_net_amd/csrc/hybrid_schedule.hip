// Hybridiff adaptive parallelism switching (Hybridiff technical summary,
// section 2B): the denoising discrepancy (rel-MAE between the conditional and
// unconditional noise predictions, dpp_cfg_combine_relmae) splits the
// denoising steps into a warm-up stage (T -> tau1, branches run serially), a
// parallel stage (tau1 -> tau2, the two branches on two devices) and a
// fully-connecting stage (tau2 -> 0).  tau1 is where the discrepancy's decline
// slows and tau2 where it starts to rise; the pages give no thresholds, so the
// rule below is a reading with two parameters (rho, eps).  Host code only.
#include <math.h>
#include <stdint.h>

#include "../../include/dpp.h"

extern "C" int dpp_hybrid_schedule(const float* relmae, int64_t T, float rho, float eps, int64_t min_warmup,
                                   int32_t* stage, int64_t* tau1, int64_t* tau2) {
  if (!relmae || !stage || !tau1 || !tau2) return DPP_ERR_NULL;
  if (T <= 0 || min_warmup < 1 || !(rho >= 0.f && rho <= 1.f) || !(eps >= 0.f)) return DPP_ERR_SHAPE;
  int64_t t1 = T, t2 = T;
  float max_drop = 0.f;   // fastest decline d[i-1] - d[i] seen so far (NaN steps ignored)
  float run_min = 0.f;    // minimum discrepancy since tau1
  for (int64_t i = 0; i < T; ++i) {
    const float d = relmae[i];
    if (t1 == T) {
      if (i >= 1) {
        const float drop = relmae[i - 1] - d;
        if (drop > max_drop) max_drop = drop;
        // decline slowed to at most rho of its fastest rate
        if (i >= min_warmup && max_drop > 0.f && drop <= rho * max_drop) {
          t1 = i;
          run_min = d;
        }
      }
    } else if (t2 == T) {
      if (d > (1.f + eps) * run_min) t2 = i;  // rose above the parallel stage's minimum
      else if (d < run_min) run_min = d;
    }
    stage[i] = i < t1 ? 0 : (i < t2 ? 1 : 2);
  }
  *tau1 = t1;
  *tau2 = t2;
  return DPP_OK;
}
