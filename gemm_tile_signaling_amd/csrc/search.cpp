// Predictive search for the wave-group partition (host code).
//
// Method: deep-dive page "FlashOverlap: 信号驱动计算通信重叠论文详解",
//   四、实时调优: 预测搜索方法 › 在线阶段: 预测搜索算法 and its Algorithm 1
//   (Grouping Tuning Algorithm): every candidate partition of the T waves is
//   scored by a latency model instead of being run -- per group, computation
//   takes the GEMM's duration / T per wave and communication a latency read
//   off a sampled latency-versus-size curve; a group's communication starts
//   once both its own computation and the previous group's communication are
//   done.  The smallest predicted end of the last communication wins.
//
// Readings taken where the pages leave a step open: the first group has no
// communication before it; the last group's communication takes the same
// max as the others; the curve is interpolated linearly between samples,
// held at the first sample's latency below it and extended at the last
// sample's bandwidth beyond it; a group's size is its span in bytes;
// candidates are visited in cut-mask order (bit i set: a group ends after
// wave i+1); among equal predictions the one with more groups wins (it
// starts communicating sooner and spreads the communication over more of
// the computation, which the model does not price), then the first.
//
// Cost: 2^(T-1) candidates of O(T) each; T <= 24 keeps a search well under a
// second on one core.  The waves come from the plan; its own composition is
// not used.
#include <cmath>
#include <vector>

#include "fo_internal.h"

namespace {

struct Curve {
  const double *x;  // bytes, strictly increasing
  const double *y;  // seconds
  int n;
  double latency(double size) const {
    if (size <= 0.0) return 0.0;
    if (size <= x[0]) return y[0];
    if (size >= x[n - 1]) return y[n - 1] * (size / x[n - 1]);
    int lo = 0, hi = n - 1;  // x[lo] < size < x[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) / 2;
      (x[mid] <= size ? lo : hi) = mid;
    }
    return y[lo] + (y[hi] - y[lo]) * (size - x[lo]) / (x[hi] - x[lo]);
  }
};

}  // namespace

extern "C" int fo_plan_search(const fo_plan *p, double gemm_seconds, const double *curve_bytes,
                              const double *curve_seconds, int32_t points, int32_t *best_comp,
                              int32_t *best_num_groups, double *best_seconds, double *all_seconds) {
  if (!p || !curve_bytes || !curve_seconds || points < 1 || !best_num_groups || !best_seconds)
    return FO_ERR_INVALID;
  if (!std::isfinite(gemm_seconds) || gemm_seconds < 0.0) return FO_ERR_INVALID;
  for (int k = 0; k < points; ++k) {
    if (!std::isfinite(curve_bytes[k]) || !std::isfinite(curve_seconds[k]) || curve_seconds[k] < 0.0 ||
        curve_bytes[k] <= 0.0)
      return FO_ERR_INVALID;
    if (k > 0 && !(curve_bytes[k] > curve_bytes[k - 1])) return FO_ERR_INVALID;
  }
  const int T = p->T;
  if (T > 24) return FO_ERR_UNSUPPORTED;
  if (T > 0 && !best_comp) return FO_ERR_INVALID;
  if (T == 0) {
    *best_num_groups = 0;
    *best_seconds = 0.0;
    return FO_OK;
  }
  // bytes of output each wave produces (16-bit elements)
  std::vector<double> wave_bytes(T, 0.0);
  {
    std::vector<int64_t> acc(T, 0);
    for (int32_t b = 0; b < p->NT; ++b) acc[b / p->W] += (int64_t)p->slots[b].rows * p->slots[b].cols * 2;
    for (int w = 0; w < T; ++w) wave_bytes[w] = (double)acc[w];
  }
  const Curve curve{curve_bytes, curve_seconds, points};
  const double per_wave = gemm_seconds / T;
  const uint32_t candidates = 1u << (T - 1);
  double best = 0.0;
  uint32_t best_mask = 0;
  int best_groups = 0;
  for (uint32_t mask = 0; mask < candidates; ++mask) {
    // comm_end(i) = max(compute_end(i), comm_end(i-1)) + latency(bytes of group i), comm_end(-1) = 0
    double comm_end = 0.0, bytes = 0.0;
    int waves_done = 0;
    for (int w = 0; w < T; ++w) {
      bytes += wave_bytes[w];
      ++waves_done;
      if (w == T - 1 || ((mask >> w) & 1u)) {  // a group ends after wave w+1
        const double compute_end = per_wave * waves_done;
        comm_end = std::max(compute_end, comm_end) + curve.latency(bytes);
        bytes = 0.0;
      }
    }
    if (all_seconds) all_seconds[mask] = comm_end;
    const int groups = 1 + __builtin_popcount(mask);
    if (mask == 0 || comm_end < best || (comm_end == best && groups > best_groups)) {
      best = comm_end;
      best_mask = mask;
      best_groups = groups;
    }
  }
  int P = 0, run = 0;
  for (int w = 0; w < T; ++w) {
    ++run;
    if (w == T - 1 || ((best_mask >> w) & 1u)) {
      best_comp[P++] = run;
      run = 0;
    }
  }
  *best_num_groups = P;
  *best_seconds = best;
  return FO_OK;
}
