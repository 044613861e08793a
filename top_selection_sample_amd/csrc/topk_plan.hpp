// Host-side parameter arithmetic (Prof-K Algorithm 1, Lemma 1, Theorem 3).
#pragma once

#include <stdint.h>

#include "topk_launch.hpp"

namespace tk {

struct Alg1 {
  double z = 0, s_star = 0;
  int64_t S = 0, t = 0, M = 0;
};

struct TailParams {
  int64_t t = 0, M = 0;
};

struct ParamIn {
  double eps = 1e-3;
  int64_t s_min = 32768, s_max = 131072;
  double cost_ratio = 1.0;
  int policy = 2;      // 0 exact tail, 1 Algorithm 1, 2 tuned sample size
  int force_path = 0;  // 0 auto, 1 filter, 2 exact
  int64_t S = 0, t = 0, M = 0;
  int64_t cus = 256;   // compute units of the device the call runs on
  // tau_B / tau_A measured for this engine (calibrated on MI355X over the
  // sample-size grid): k <= KSMALL refines in one workgroup, larger k runs
  // the bucket sort, whose cost per candidate is lower relative to sampling
  double tuned_ratio = 0.13;
  int64_t tuned_s_min = 1024;  // least sample size the tuned policy considers
  double tuned_ratio_large = 0.01;
  // k <= KSMALL in calls of at least tuned_batch_rows rows: the rows'
  // samples are gathered together, so sampling costs bandwidth, while the
  // rows are refined side by side (about one workgroup each)
  double tuned_ratio_batched = 0.03;
  int64_t tuned_batch_rows = 32;
  // recall target (relaxed-recall mode below 1): parameters for
  // ceil(recall * k), and rows with at least that many survivors keep them
  double recall = 1.0;
  bool force_tau = false;   // the caller gives the threshold key (sampled route, no sampler)
};

double normal_quantile(double p);
Alg1 algorithm1(int64_t N, int64_t k, double eps, int64_t s_min, int64_t s_max, double ratio);
double hyper_cdf(int64_t N, int64_t K, int64_t S, int64_t t, bool fast);
double hyper_sf(int64_t N, int64_t K, int64_t S, int64_t t);
TailParams exact_tail(int64_t N, int64_t k, int64_t S, double eps);
int64_t tuned_sample_size(int64_t N, int64_t k, double eps, int64_t s_lo, int64_t s_hi,
                          double ratio);
void sample_params(int64_t N, int64_t k, const ParamIn& in, int64_t* S, int64_t* t, int64_t* M,
                   double* p_recall, double* p_overflow);
int make_plan(int64_t n, int64_t rows, int64_t k, int dtype, const ParamIn& in, Plan* out);

}  // namespace tk
