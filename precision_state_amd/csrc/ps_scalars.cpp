// ps_scalars.cpp - step-dependent fp32 scalars of the (N)AdamW update,
// computed in double and rounded to fp32 once [NADAM opening post: AdamW,
// Nesterov momentum].
//
// Adam bias corrections: A = lr / (1 - beta1^t), RS2 = 1 / sqrt(1 - beta2^t).
// NAdam (Dozat) with the momentum schedule mu_i = beta1 (1 - 0.5 * 0.96^(i psi)):
//   AG = lr (1 - mu_t) / (1 - P_t),  AM = lr mu_{t+1} / (1 - P_t mu_{t+1}),
//   P_t = mu_1 * ... * mu_t.
// Decoupled weight decay: CWD = lr * wd.
#include <cmath>

#include "ps_internal.h"

namespace ps {

namespace {
double nadam_mu(double beta1, double psi, int64_t i) { return beta1 * (1.0 - 0.5 * std::pow(0.96, (double)i * psi)); }
}  // namespace

void step_scalars(const ps_hparams& hp, int64_t t, StepScalars* o) {
  const double lr = hp.lr, b1 = hp.beta1, b2 = hp.beta2, psi = hp.momentum_decay;
  o->B1 = (float)b1;
  o->C1 = (float)(1.0 - b1);
  o->B2 = (float)b2;
  o->C2 = (float)(1.0 - b2);
  o->EPS = (float)hp.eps;
  o->A = (float)(lr / (1.0 - std::pow(b1, (double)t)));
  o->RS2 = (float)(1.0 / std::sqrt(1.0 - std::pow(b2, (double)t)));
  // Once P < 2^-60, both 1 - P and 1 - P*mu round to exactly 1.0 in double,
  // so the remaining factors cannot change AG or AM.
  double prod = 1.0;
  for (int64_t i = 1; i <= t && prod >= 0x1p-60; ++i) prod *= nadam_mu(b1, psi, i);
  const double mu_t = nadam_mu(b1, psi, t);
  const double mu_next = nadam_mu(b1, psi, t + 1);
  o->AG = (float)(lr * (1.0 - mu_t) / (1.0 - prod));
  o->AM = (float)(lr * mu_next / (1.0 - prod * mu_next));
  o->CWD = (float)(lr * hp.weight_decay);
  o->sr_step = (uint32_t)t;
  o->pad = 0;
  o->sr_seed = hp.split_mode == PS_SPLIT_STOCHASTIC ? hp.seed : 0;
}

}  // namespace ps
