// launch_plan.h - host-side launch planning of the decode step (no device code):
// how many attention workgroups each request gets, and how long score rows are cut
// into slices for a two-round top-k. Linked into the product library and into the
// CPU-only host library, where the tests check it.
#pragma once

#include <cstdint>
#include <vector>

namespace hsa {

// No attention workgroup is left with fewer keys than this (unless its request has
// fewer).
constexpr int64_t kMinKeys = 16;

// One part of an attention launch: per request, the keys it streams (`keys`), the
// work it does before its first key in units of keys (`lat`), and the fewest
// workgroups it gets (`min_wgs`, 0 or 1). balance_wgs fills `wgs`.
struct AttnPart {
  const std::vector<int64_t>* keys;
  int64_t lat;
  int32_t min_wgs;
  std::vector<int64_t> wgs;
};

// A request gets one workgroup per part it has keys in (and at least min_wgs); the
// launch's remaining slots go one at a time to the (part, request) whose workgroups
// are estimated to finish last, the estimate being lat + keys / workgroups. This
// greedy choice minimises the largest estimate for the slots it hands out. A
// (part, request) stops receiving workgroups once another would leave one with
// fewer than kMinKeys keys. Returns the workgroups handed out.
int64_t balance_wgs(const std::vector<AttnPart*>& parts, int64_t slots);

// Slices of score rows for the top-k: row i (n[i] scores) is cut into slices of
// `slice` scores when it is longer than both the slice and k1 = k rounded up to a
// multiple of 4 (its slices then keep at least k real candidates); otherwise it is
// one workgroup. slice_override > 0 fixes the slice length, else it is
// max(default_slice, 16 k1), so that the second round selects over at most 1/16 of
// the row. Writes first[0..n] (workgroup prefix), returns the longest slice count
// of a row in *gmax, the slice length in *slice and k1 in *k1.
void plan_slices(const int64_t* n, int n_rows, int32_t k, int32_t slice_override, int32_t default_slice,
                 int32_t* first, int32_t* gmax, int32_t* slice, int32_t* k1);

}  // namespace hsa
