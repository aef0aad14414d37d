// Static plans of the distributed step (host only).
//
// DP static partition: which whole parameters each data-parallel rank owns.
// This is the planner in front of the step: a rank's share of the parameters
// becomes the batch it hands to muon_plan.
//
// Canzona analysis page (paper-graph-ui), section 3.4:
// - "Paradigm 3: Static Partitioning": a parameter belongs to the rank whose
//   geometric slice (width S = |B| / R) holds its first element
//   (muon_dp_partition_static);
// - "The DP Load-Balance Optimization Problem" and "The alpha-Balanced Greedy
//   LPT Algorithm (Algorithm 1)": buckets in descending load order; per bucket
//   the deficits against the mean, the alpha-blend of the even and fill
//   shares, and cuts at the parameter boundaries closest to the cumulative
//   targets (muon_dp_partition).
//
// TP micro groups (same section, "The TP Hierarchical Partitioning and
// Scheduling"): tensors sorted by (cost, ID) descending, packed greedily into
// groups with a rollback when the min-heap LPT assignment of the tentative
// group to the host ranks exceeds C_max (muon_tp_micro_groups).
//
// Cuts are parameter indices within a bucket, non-decreasing, with the tie in
// "closest" going to the earlier boundary. The sums are formed in the order
// the algorithm states them, and without contraction into fused multiply-adds,
// so the result does not depend on the compiler.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <functional>
#include <numeric>
#include <queue>
#include <string>
#include <utility>
#include <vector>

#include "muon.h"

#pragma clang fp contract(off)

// Defined in muon_api.cpp: sets this thread's error message, returns st.
__attribute__((visibility("hidden"))) muon_status muon_fail_message(muon_status st, const char* msg);

namespace {

muon_status check_buckets(const int64_t* sizes, const double* loads, const int32_t* bucket_len,
                          int32_t n_buckets, int32_t ranks, int32_t* cuts, int64_t* total_params) {
  if (!sizes || !bucket_len || !cuts) return muon_fail_message(MUON_ERR_INVALID_ARG, "sizes, bucket_len or cuts is NULL");
  if (n_buckets < 1) return muon_fail_message(MUON_ERR_INVALID_ARG, "n_buckets must be >= 1");
  if (ranks < 1 || ranks > (1 << 20)) return muon_fail_message(MUON_ERR_INVALID_ARG, "ranks must be in [1, 2^20]");
  int64_t n = 0;
  for (int32_t i = 0; i < n_buckets; ++i) {
    if (bucket_len[i] < 1) return muon_fail_message(MUON_ERR_INVALID_ARG, "every bucket must hold >= 1 parameter");
    n += bucket_len[i];
  }
  for (int64_t j = 0; j < n; ++j) {
    if (sizes[j] < 1 || sizes[j] > (int64_t(1) << 40))
      return muon_fail_message(MUON_ERR_INVALID_ARG, "parameter sizes must be in [1, 2^40]");
    if (loads && !(std::isfinite(loads[j]) && loads[j] >= 0.0))
      return muon_fail_message(MUON_ERR_INVALID_ARG, "loads must be finite and >= 0");
  }
  *total_params = n;
  return MUON_OK;
}

// Load of every rank over all buckets, from the cuts.
void sum_rank_loads(const std::vector<std::vector<double>>& w, const int32_t* cuts, int32_t ranks, double* out) {
  std::fill(out, out + ranks, 0.0);
  for (size_t i = 0; i < w.size(); ++i) {
    const int32_t* c = cuts + i * size_t(ranks + 1);
    for (int32_t r = 0; r < ranks; ++r)
      for (int32_t j = c[r]; j < c[r + 1]; ++j) out[r] += w[i][j];
  }
}

std::vector<std::vector<double>> bucket_loads(const int64_t* sizes, const double* loads, const int32_t* bucket_len,
                                              int32_t n_buckets) {
  std::vector<std::vector<double>> w(n_buckets);
  int64_t o = 0;
  for (int32_t i = 0; i < n_buckets; ++i) {
    w[i].resize(bucket_len[i]);
    for (int32_t j = 0; j < bucket_len[i]; ++j, ++o) w[i][j] = loads ? loads[o] : double(sizes[o]);
  }
  return w;
}

}  // namespace

extern "C" {

muon_status muon_dp_partition_static(const int64_t* sizes, const double* loads, const int32_t* bucket_len,
                                     int32_t n_buckets, int32_t ranks, int32_t* cuts, double* rank_loads) {
  int64_t n = 0;
  muon_status st = check_buckets(sizes, loads, bucket_len, n_buckets, ranks, cuts, &n);
  if (st != MUON_OK) return st;
  int64_t o = 0;
  for (int32_t i = 0; i < n_buckets; ++i) {
    int64_t total = 0;
    for (int32_t j = 0; j < bucket_len[i]; ++j) total += sizes[o + j];
    // Rank of parameter j: floor(start * R / |B|), exactly, in integers
    // (r S <= start < (r + 1) S with S = |B| / R). Owners are non-decreasing,
    // so cut r is the number of parameters owned by ranks below r.
    int32_t* c = cuts + size_t(i) * (ranks + 1);
    std::fill(c, c + ranks + 1, bucket_len[i]);
    c[0] = 0;
    int64_t start = 0;
    int32_t next = 1;  // the next cut not yet placed
    for (int32_t j = 0; j < bucket_len[i]; ++j) {
      const int64_t owner = int64_t((__int128)start * ranks / total);
      while (next <= owner) c[next++] = j;
      start += sizes[o + j];
    }
    o += bucket_len[i];
  }
  if (rank_loads) sum_rank_loads(bucket_loads(sizes, loads, bucket_len, n_buckets), cuts, ranks, rank_loads);
  return MUON_OK;
}

muon_status muon_dp_partition(const int64_t* sizes, const double* loads, const int32_t* bucket_len,
                              int32_t n_buckets, int32_t ranks, double alpha, int32_t* cuts, double* rank_loads) {
  int64_t n = 0;
  muon_status st = check_buckets(sizes, loads, bucket_len, n_buckets, ranks, cuts, &n);
  if (st != MUON_OK) return st;
  if (!(alpha >= 0.0 && alpha <= 1.0)) return muon_fail_message(MUON_ERR_INVALID_ARG, "alpha must be in [0, 1]");
  const std::vector<std::vector<double>> w = bucket_loads(sizes, loads, bucket_len, n_buckets);
  std::vector<double> total(n_buckets, 0.0);
  double all = 0.0;
  for (int32_t i = 0; i < n_buckets; ++i) {
    for (double x : w[i]) total[i] = total[i] + x;
    all = all + total[i];
  }
  const double mu = all / ranks;
  // Decision order: heaviest bucket first; equal loads keep index order.
  std::vector<int32_t> order(n_buckets);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return total[a] > total[b]; });
  std::vector<double> L(ranks, 0.0), d(ranks), v(ranks), phi;
  for (int32_t k : order) {
    const int32_t m = bucket_len[k];
    phi.assign(m + 1, 0.0);
    for (int32_t j = 0; j < m; ++j) phi[j + 1] = phi[j] + w[k][j];
    double D = 0.0;
    for (int32_t r = 0; r < ranks; ++r) {
      d[r] = std::max(0.0, mu - L[r]);
      D = D + d[r];
    }
    for (int32_t r = 0; r < ranks; ++r)
      v[r] = D > 0.0 ? (1.0 - alpha) * (1.0 / ranks) + alpha * (d[r] / D) : 1.0 / ranks;
    int32_t* c = cuts + size_t(k) * (ranks + 1);
    c[0] = 0;
    double C = 0.0;
    for (int32_t r = 0; r + 1 < ranks; ++r) {
      C = C + total[k] * v[r];
      // The boundary u >= c[r] with the smallest |phi[u] - C|, the earliest on
      // a tie. phi is non-decreasing: the candidates are the first u with
      // phi[u] >= C and the earliest u whose phi equals the last value below C.
      const auto first = phi.begin() + c[r];
      const int32_t hi = int32_t(std::lower_bound(first, phi.end(), C) - phi.begin());
      int32_t best = hi;
      if (hi > c[r]) {
        const int32_t lo = int32_t(std::lower_bound(first, phi.begin() + hi, phi[hi - 1]) - phi.begin());
        if (hi > m || C - phi[lo] <= phi[hi] - C) best = lo;
      }
      c[r + 1] = best;
      L[r] += phi[c[r + 1]] - phi[c[r]];
    }
    c[ranks] = m;
    L[ranks - 1] += phi[m] - phi[c[ranks - 1]];
  }
  if (rank_loads) sum_rank_loads(w, cuts, ranks, rank_loads);
  return MUON_OK;
}

namespace {

// LPT of the items (tensor IDs, in the order they joined the group) on R host
// ranks: by cost, descending (stable), each to the least-loaded rank (lowest
// index on a tie). Writes the host of each item into host_of (by ID) when it
// is not null, and returns the largest load.
double min_heap_solve(const std::vector<int32_t>& items, const double* cost, int32_t ranks, int32_t* host_of,
                      std::vector<int32_t>& tmp) {
  tmp = items;
  std::stable_sort(tmp.begin(), tmp.end(), [&](int32_t a, int32_t b) { return cost[a] > cost[b]; });
  using Slot = std::pair<double, int32_t>;
  std::priority_queue<Slot, std::vector<Slot>, std::greater<Slot>> pq;
  for (int32_t r = 0; r < ranks; ++r) pq.push({0.0, r});
  double worst = 0.0;
  for (int32_t id : tmp) {
    Slot s = pq.top();
    pq.pop();
    if (host_of) host_of[id] = s.second;
    s.first = s.first + cost[id];
    worst = std::max(worst, s.first);
    pq.push(s);
  }
  return worst;
}

}  // namespace

muon_status muon_tp_micro_groups(const double* cost, int32_t n, int32_t ranks, double c_max, int32_t* order,
                                 int32_t* group_of, int32_t* host_of, int32_t* n_groups) {
  if (!cost || !order || !group_of || !host_of || !n_groups)
    return muon_fail_message(MUON_ERR_INVALID_ARG, "a pointer argument is NULL");
  if (n < 1) return muon_fail_message(MUON_ERR_INVALID_ARG, "n must be >= 1");
  if (ranks < 1 || ranks > (1 << 20)) return muon_fail_message(MUON_ERR_INVALID_ARG, "ranks must be in [1, 2^20]");
  if (!(std::isfinite(c_max) && c_max > 0.0)) return muon_fail_message(MUON_ERR_INVALID_ARG, "c_max must be finite and > 0");
  for (int32_t i = 0; i < n; ++i)
    if (!(std::isfinite(cost[i]) && cost[i] >= 0.0))
      return muon_fail_message(MUON_ERR_INVALID_ARG, "costs must be finite and >= 0");
  // Phase 1: (cost, ID) descending.
  std::iota(order, order + n, 0);
  std::sort(order, order + n, [&](int32_t a, int32_t b) { return cost[a] > cost[b] || (cost[a] == cost[b] && a > b); });
  // Phase 2: greedy packing with rollback.
  std::vector<int32_t> curr, tmp;
  int32_t g = 0;
  auto close = [&]() {
    min_heap_solve(curr, cost, ranks, host_of, tmp);
    for (int32_t id : curr) group_of[id] = g;
    ++g;
  };
  for (int32_t j = 0; j < n; ++j) {
    const int32_t p = order[j];
    curr.push_back(p);
    if (curr.size() == 1) continue;  // a group's first tensor is always taken
    if (min_heap_solve(curr, cost, ranks, nullptr, tmp) > c_max) {
      curr.pop_back();
      close();
      curr.assign(1, p);
    }
  }
  close();
  *n_groups = g;
  return MUON_OK;
}

}  // extern "C"
