// The SLO-constrained, EC-aware scheduler (SPEAR page, abstract: a scheduler
// that decides under a latency objective where the error compensators run),
// for one batch: keep the ECs whose total weight is largest among the sets
// whose predicted batch latency (the planner's cost model) fits the SLO.
// Pure host arithmetic on plans; nothing touches the device beyond the CU
// count the planner may read.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

#include "internal.h"

namespace {

constexpr int kMaxSchedLayers = 4096;
constexpr int kSlackSteps = 65536;   // grid of the knapsack's capacity, up to kFullGridLayers layers
constexpr int kFullGridLayers = 256;

// Grid steps for n layers: 65536 up to 256 layers, fewer beyond (65536 x 256
// / n, at least 256), so a call stays near 2^24 cell updates.
int slack_steps(int n) { return n <= kFullGridLayers ? kSlackSteps : std::max(256, kSlackSteps * kFullGridLayers / n); }

}  // namespace

extern "C" spear_status_t spear_schedule_ec_costs(const double* extra_us, const float* weight, int32_t n,
                                                  double slack_us, uint8_t* ec_on, double* added_us) {
  if (n < 0 || n > kMaxSchedLayers) return SPEAR_ERR_INVALID_SHAPE;
  if (n > 0 && (!extra_us || !weight || !ec_on)) return SPEAR_ERR_NULL_POINTER;
  if (!std::isfinite(slack_us)) return SPEAR_ERR_INVALID_ARGUMENT;
  for (int i = 0; i < n; ++i) {
    if (!std::isfinite(weight[i]) || weight[i] < 0.0f || !std::isfinite(extra_us[i])) return SPEAR_ERR_INVALID_ARGUMENT;
    ec_on[i] = 0;
  }
  if (added_us) *added_us = 0.0;
  if (slack_us < 0.0 || n == 0) return SPEAR_OK;
  // 0/1 knapsack over a grid of the slack: costs rounded up (a chosen set's
  // true extra time never exceeds the slack).  best[c]: the largest weight
  // (summed in layer order) of a set of cost <= c, ties to the least cost;
  // layers with a negative extra (no EC) or no weight are never taken.
  const int steps = slack_steps(n);
  const double unit = std::max(slack_us / steps, 1e-9);
  const int cap = (int)std::min<double>(steps, std::floor(slack_us / unit));
  std::vector<int> cost((size_t)n, 0);
  std::vector<int> items;
  for (int i = 0; i < n; ++i) {
    if (extra_us[i] < 0.0 || weight[i] <= 0.0f) continue;
    const double cu = std::ceil(extra_us[i] / unit - 1e-9);
    if (cu > cap) continue;
    cost[i] = (int)std::max(0.0, cu);
    items.push_back(i);
  }
  struct Cell { double w; int c; };
  std::vector<Cell> best((size_t)cap + 1, Cell{0.0, 0});
  // take[t]: bit c set when item t improved best[c] (one bit per cell).
  const size_t words = ((size_t)cap + 64) / 64;
  std::vector<uint64_t> take(items.size() * words, 0);
  for (size_t t = 0; t < items.size(); ++t) {
    const int i = items[t], ci = cost[i];
    const double wi = weight[i];
    for (int c = cap; c >= ci; --c) {
      const Cell cand{best[(size_t)(c - ci)].w + wi, best[(size_t)(c - ci)].c + ci};
      const Cell cur = best[(size_t)c];
      if (cand.w > cur.w || (cand.w == cur.w && cand.c < cur.c)) {
        best[(size_t)c] = cand;
        take[t * words + (size_t)c / 64] |= (uint64_t)1 << (c % 64);
      }
    }
  }
  double added = 0.0;
  int c = cap;
  for (size_t t = items.size(); t-- > 0;) {
    if ((take[t * words + (size_t)c / 64] >> (c % 64)) & 1u) {
      const int i = items[t];
      ec_on[i] = 1;
      added += extra_us[i];
      c -= cost[i];
    }
  }
  if (added_us) *added_us = added;
  return SPEAR_OK;
}

extern "C" spear_status_t spear_schedule_ec(const spear_sched_layer_t* layers, int32_t n_layers, int32_t M,
                                            double slo_us, int32_t device_cus, uint8_t* ec_on,
                                            double* predicted_us) {
  if (n_layers < 0 || n_layers > kMaxSchedLayers || M < 1) return SPEAR_ERR_INVALID_SHAPE;
  if (n_layers > 0 && (!layers || !ec_on)) return SPEAR_ERR_NULL_POINTER;
  if (!std::isfinite(slo_us)) return SPEAR_ERR_INVALID_ARGUMENT;
  // Per layer: time with the EC off, and the extra time of turning it on
  // (negative: the layer has no EC).
  std::vector<double> extra((size_t)n_layers, -1.0);
  std::vector<float> weight((size_t)n_layers, 0.0f);
  double base = 0.0;
  for (int i = 0; i < n_layers; ++i) {
    const spear_sched_layer_t& l = layers[i];
    if (!std::isfinite(l.weight) || l.weight < 0.0f) return SPEAR_ERR_INVALID_ARGUMENT;
    spear_linear_desc_t d;
    std::memset(&d, 0, sizeof(d));
    d.M = M; d.K = l.K; d.N = l.N; d.rank = l.rank;
    d.variant = SPEAR_VARIANT_AUTO; d.device_cus = device_cus; d.group_size = l.group_size;
    spear_plan_t p;
    const spear_status_t st = spear_dispatch_plan(&d, &p);
    if (st != SPEAR_OK) return st;
    base += p.predicted_no_ec_us;
    if (l.rank > 0) extra[i] = std::max(0.0, (double)p.predicted_us - (double)p.predicted_no_ec_us);
    weight[i] = l.weight;
  }
  double added = 0.0;
  const spear_status_t st = spear_schedule_ec_costs(extra.data(), weight.data(), n_layers, slo_us - base, ec_on, &added);
  if (st != SPEAR_OK) return st;
  if (predicted_us) *predicted_us = base + added;
  return SPEAR_OK;
}
