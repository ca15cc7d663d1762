// launch_plan.cpp - host-side launch planning of the decode step (see launch_plan.h).
#include "launch_plan.h"

#include <algorithm>
#include <cmath>
#include <queue>
#include <utility>

namespace hsa {

int64_t balance_wgs(const std::vector<AttnPart*>& parts, int64_t slots) {
  // Every (part, request) with keys starts at its floor w0; one that can be split
  // may grow up to cap = max(w0, keys / kMinKeys) (no workgroup under kMinKeys keys).
  struct Item {
    double lat;
    int64_t keys, w0, cap, w;
    int64_t* out;
  };
  std::vector<Item> items;
  int64_t used = 0;
  for (AttnPart* a : parts) {
    a->wgs.assign(a->keys->size(), 0);
    for (size_t i = 0; i < a->keys->size(); ++i) {
      const int64_t k = (*a->keys)[i];
      const int64_t w0 = std::max<int64_t>(k > 0 ? 1 : 0, a->min_wgs);
      a->wgs[i] = w0;
      used += w0;
      if (w0 > 0 && k >= kMinKeys * (w0 + 1))
        items.push_back(Item{(double)a->lat, k, w0, std::max(w0, k / kMinKeys), w0, &a->wgs[i]});
    }
  }
  if (used >= slots || items.empty()) return used;
  // The greedy hand-out (one slot at a time to the largest estimate lat + keys / w)
  // ends at the smallest largest estimate E the slots allow, where every item holds
  // at least need(E), the fewest w with lat + keys / w <= E (within [w0, cap]). So
  // start every item at need(T) for some feasible T >= E, found from the
  // proportional share (the estimate with every workgroup equally loaded) in a few
  // tries, and hand out the rest greedily.
  auto need = [](const Item& t, double T) -> int64_t {
    if (T <= t.lat) return t.cap;
    const double w = std::ceil((double)t.keys / (T - t.lat) * (1.0 - 1e-12));
    return std::min(t.cap, std::max(t.w0, (int64_t)w));
  };
  double ksum = 0.0, tmin = 0.0, lmax = 0.0;
  int64_t wsum = 0;
  for (const Item& t : items) {
    ksum += (double)t.keys;
    wsum += t.w0;
    lmax = std::max(lmax, t.lat);
    tmin = std::max(tmin, t.lat + (double)t.keys / (double)t.cap);
  }
  double T = 1.02 * std::max(tmin, lmax + ksum / (double)(slots - used + wsum));
  int64_t sum = 0;
  for (;;) {
    sum = used;
    for (const Item& t : items) sum += need(t, T) - t.w0;
    if (sum <= slots) break;
    T *= 1.25;
  }
  for (Item& t : items) t.w = need(t, T);
  used = sum;
  // the slots left over go one at a time to the largest estimate, as the greedy
  // hand-out would give them
  using Entry = std::pair<double, int>;
  std::priority_queue<Entry> pq;
  for (int j = 0; j < (int)items.size(); ++j)
    if (items[j].w < items[j].cap) pq.push({items[j].lat + (double)items[j].keys / items[j].w, j});
  while (used < slots && !pq.empty()) {
    const int j = pq.top().second;
    pq.pop();
    Item& t = items[j];
    ++t.w;
    ++used;
    if (t.w < t.cap) pq.push({t.lat + (double)t.keys / t.w, j});
  }
  for (const Item& t : items) *t.out = t.w;
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
