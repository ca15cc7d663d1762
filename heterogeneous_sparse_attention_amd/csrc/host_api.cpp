// host_api.cpp - C entry points over the host control plane alone, built with g++
// into a CPU-only library so the integer logic (State slots, block ids, tables,
// refcounts, seal planning) can be checked against the oracle without a GPU. The
// product library links the same control.cpp.
#include <cstdint>
#include <string>
#include <vector>

#include "control.h"
#include "launch_plan.h"

using hsa::AppendPlan;
using hsa::Control;

extern "C" {

void* hsah_create(int32_t n_win, int32_t max_states, int64_t max_blocks, int64_t max_bps) {
  return new Control(n_win, max_states, max_blocks, max_bps ? max_bps : max_blocks);
}

void hsah_destroy(void* c) { delete static_cast<Control*>(c); }

int32_t hsah_state_alloc(void* c, int32_t* out) { return static_cast<Control*>(c)->state_alloc(out); }

int32_t hsah_state_free(void* c, int32_t s) { return static_cast<Control*>(c)->state_free(s); }

// Append (flags bit 0 = defer seal). On success writes the sealed blocks as
// (state, logical block, id) triples to `seals` (capacity `cap` triples).
int32_t hsah_append(void* c_, int32_t n_req, const int32_t* states, const int64_t* cu,
                    uint32_t flags, int64_t* seals, int64_t cap, int64_t* n_seals) {
  Control* c = static_cast<Control*>(c_);
  AppendPlan plan;
  std::string why;
  int st = c->plan_append(n_req, states, cu, (flags & 1u) != 0, &plan, &why);
  if (st) return st;
  c->commit(&plan);
  *n_seals = (int64_t)plan.seals.size();
  for (int64_t i = 0; i < *n_seals && i < cap; ++i) {
    seals[3 * i] = plan.seals[i].state;
    seals[3 * i + 1] = plan.seals[i].lblock;
    seals[3 * i + 2] = plan.seals[i].id;
  }
  return 0;
}

int32_t hsah_flush(void* c_, int32_t n_req, const int32_t* states, int64_t* n_seals) {
  Control* c = static_cast<Control*>(c_);
  AppendPlan plan;
  std::string why;
  int st = c->plan_flush(n_req, states, &plan, &why);
  if (st) return st;
  c->commit(&plan);
  *n_seals = (int64_t)plan.seals.size();
  return 0;
}

int32_t hsah_share(void* c_, int32_t src, int32_t dst) {
  Control* c = static_cast<Control*>(c_);
  std::string why;
  int st = c->check_share(src, dst, &why);
  if (st) return st;
  c->commit_share(src, dst);
  return 0;
}

int32_t hsah_block_ref(void* c_, const int32_t* blocks, int64_t n, int32_t delta) {
  Control* c = static_cast<Control*>(c_);
  std::string why;
  int st = c->check_block_ref(blocks, n, delta, &why);
  if (st) return st;
  c->commit_block_ref(blocks, n, delta);
  return 0;
}

int32_t hsah_attach(void* c_, int32_t dst, const int32_t* blocks, int64_t len) {
  Control* c = static_cast<Control*>(c_);
  std::string why;
  int st = c->check_attach(dst, blocks, len, &why);
  if (st) return st;
  c->commit_attach(dst, blocks, len);
  return 0;
}

int32_t hsah_query(void* c_, int32_t s, int64_t* len, int64_t* nb, int32_t* pending) {
  Control* c = static_cast<Control*>(c_);
  if (!c->valid_state(s)) return hsa::kInvalid;
  *len = c->len(s);
  *nb = c->n_blocks(s);
  *pending = c->pending(s) ? 1 : 0;
  return 0;
}

int32_t hsah_table(void* c_, int32_t s, int32_t* ids, int64_t cap, int64_t* n) {
  Control* c = static_cast<Control*>(c_);
  if (!c->valid_state(s)) return hsa::kInvalid;
  const auto& t = c->table(s);
  *n = (int64_t)t.size();
  for (int64_t i = 0; i < *n && i < cap; ++i) ids[i] = t[i];
  return 0;
}

int32_t hsah_refcount(void* c_, int64_t b) { return static_cast<Control*>(c_)->refcount(b); }

int64_t hsah_free_blocks(void* c_) { return static_cast<Control*>(c_)->free_blocks(); }

// Workgroup planning (launch_plan.h) for up to two parts of n requests: keys_a /
// keys_b [n] (keys_b NULL for one part), lat and min_wgs per part; writes wgs_a /
// wgs_b [n] and returns the workgroups handed out.
int64_t hsah_balance(int32_t n, const int64_t* keys_a, int64_t lat_a, int32_t min_a, const int64_t* keys_b,
                     int64_t lat_b, int32_t min_b, int64_t slots, int64_t* wgs_a, int64_t* wgs_b) {
  std::vector<int64_t> ka(keys_a, keys_a + n), kb;
  hsa::AttnPart pa{&ka, lat_a, min_a, {}}, pb{&kb, lat_b, min_b, {}};
  std::vector<hsa::AttnPart*> parts{&pa};
  if (keys_b) {
    kb.assign(keys_b, keys_b + n);
    parts.push_back(&pb);
  }
  const int64_t used = hsa::balance_wgs(parts, slots);
  for (int i = 0; i < n; ++i) {
    wgs_a[i] = pa.wgs[i];
    if (keys_b) wgs_b[i] = pb.wgs[i];
  }
  return used;
}

// Slices of n score rows (launch_plan.h); first has n + 1 entries; out = {gmax,
// slice, k1}.
void hsah_slices(int32_t n, const int64_t* scores, int32_t k, int32_t slice_override, int32_t default_slice,
                 int32_t* first, int32_t* out) {
  hsa::plan_slices(scores, n, k, slice_override, default_slice, first, &out[0], &out[1], &out[2]);
}

}  // extern "C"
