// launch_plan.cpp - host-side launch planning of the decode step (see launch_plan.h).
#include "launch_plan.h"

#include <algorithm>
#include <queue>
#include <utility>

namespace hsa {

int64_t balance_wgs(const std::vector<AttnPart*>& parts, int64_t slots) {
  using Item = std::pair<double, std::pair<int, int>>;
  std::priority_queue<Item> pq;
  int64_t used = 0;
  auto can_split = [](int64_t keys, int64_t w) { return keys >= kMinKeys * (w + 1); };
  for (int p = 0; p < (int)parts.size(); ++p) {
    AttnPart& a = *parts[p];
    a.wgs.assign(a.keys->size(), 0);
    for (int i = 0; i < (int)a.keys->size(); ++i) {
      const int64_t k = (*a.keys)[i];
      a.wgs[i] = std::max<int64_t>(k > 0 ? 1 : 0, a.min_wgs);
      used += a.wgs[i];
      if (a.wgs[i] > 0 && can_split(k, a.wgs[i])) pq.push({a.lat + (double)k / a.wgs[i], {p, i}});
    }
  }
  while (used < slots && !pq.empty()) {
    const auto pi = pq.top().second;
    pq.pop();
    AttnPart& a = *parts[pi.first];
    const int64_t k = (*a.keys)[pi.second];
    const int64_t w = ++a.wgs[pi.second];
    ++used;
    if (can_split(k, w)) pq.push({a.lat + (double)k / w, pi});
  }
  return used;
}

void plan_slices(const int64_t* n, int n_rows, int32_t k, int32_t slice_override, int32_t default_slice,
                 int32_t* first, int32_t* gmax, int32_t* slice, int32_t* k1) {
  *k1 = (k + 3) & ~3;
  *slice = slice_override > 0 ? slice_override : std::max(default_slice, 16 * *k1);
  int32_t total = 0, g_max = 1;
  for (int i = 0; i < n_rows; ++i) {
    const bool sliced = n[i] > *slice && n[i] > *k1;
    const int32_t g = sliced ? (int32_t)((n[i] + *slice - 1) / *slice) : 1;
    first[i] = total;
    total += g;
    g_max = std::max(g_max, g);
  }
  first[n_rows] = total;
  *gmax = g_max;
}

}  // namespace hsa
