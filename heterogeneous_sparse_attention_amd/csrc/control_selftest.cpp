// control_selftest.cpp - randomized self-consistency test of the control plane,
// built with AddressSanitizer and UBSan (host code only). After every operation:
// each block's refcount equals the number of tables that hold it, a block is free
// exactly when its refcount is 0, each table has floor(L/128) blocks (one fewer
// while a deferred seal is pending), and a failed call changed nothing.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <string>
#include <vector>

#include "control.h"

using namespace hsa;

static int check(const Control& c, const std::vector<int32_t>& live) {
  std::vector<int32_t> rc(c.max_blocks(), 0);
  for (int32_t s : live) {
    const int64_t L = c.len(s), nb = c.n_blocks(s);
    const int64_t expect = L / kBlockTokens - ((c.pending(s) && L % kBlockTokens == 0) ? 1 : 0);
    if (nb != expect) return 1;
    for (int32_t b : c.table(s)) rc[b]++;
  }
  int64_t nfree = 0;
  for (int64_t b = 0; b < c.max_blocks(); ++b) {
    if (rc[b] != c.refcount(b)) return 2;
    nfree += rc[b] == 0;
  }
  if (nfree != c.free_blocks()) return 3;
  return 0;
}

int main() {
  std::mt19937_64 rng(12345);
  for (int trial = 0; trial < 200; ++trial) {
    Control c(256, 8, 40, 0 + 40);
    std::vector<int32_t> live;
    for (int op = 0; op < 300; ++op) {
      const int kind = rng() % 6;
      std::string why;
      if (kind == 0) {
        int32_t s;
        if (c.state_alloc(&s) == kOk) live.push_back(s);
      } else if (kind == 1 && !live.empty()) {
        const size_t i = rng() % live.size();
        if (c.state_free(live[i]) != kOk) return 10;
        live.erase(live.begin() + i);
      } else if ((kind == 2 || kind == 3) && !live.empty()) {
        std::vector<int32_t> st;
        std::vector<int64_t> cu{0};
        for (int32_t s : live)
          if (rng() % 2) {
            st.push_back(s);
            cu.push_back(cu.back() + (int64_t)(rng() % 300));
          }
        const bool defer = kind == 3;
        std::vector<int64_t> before;
        for (int32_t s : live) before.push_back(c.len(s));
        AppendPlan plan;
        int r = c.plan_append((int32_t)st.size(), st.data(), cu.data(), defer, &plan, &why);
        if (r == kOk) {
          c.commit(&plan);
        } else {
          for (size_t i = 0; i < live.size(); ++i)
            if (c.len(live[i]) != before[i]) return 11;
        }
      } else if (kind == 4 && !live.empty()) {
        AppendPlan plan;
        if (c.plan_flush((int32_t)live.size(), live.data(), &plan, &why) == kOk) c.commit(&plan);
      } else if (kind == 5 && live.size() >= 2) {
        const int32_t a = live[rng() % live.size()], b = live[rng() % live.size()];
        if (c.check_share(a, b, &why) == kOk) c.commit_share(a, b);
      }
      const int e = check(c, live);
      if (e) {
        std::printf("inconsistent state %d at trial %d op %d\n", e, trial, op);
        return 20 + e;
      }
    }
  }
  std::printf("control selftest ok\n");
  return 0;
}
