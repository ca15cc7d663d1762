// control.cpp - host control plane (see control.h).
#include "control.h"

#include <algorithm>

namespace hsa {

// ------------------------------------------------------------------ IdPool

IdPool::IdPool(int64_t n) : n_(n), nfree_(n) {
  const int64_t nw = (n + 63) / 64;
  words_.assign(nw, ~0ull);
  if (n % 64) words_[nw - 1] = (1ull << (n % 64)) - 1;
  summary_.assign((nw + 63) / 64, 0ull);
  for (int64_t w = 0; w < nw; ++w)
    if (words_[w]) summary_[w / 64] |= 1ull << (w % 64);
}

bool IdPool::is_free(int64_t id) const {
  return id >= 0 && id < n_ && ((words_[id / 64] >> (id % 64)) & 1ull);
}

int64_t IdPool::take_lowest() {
  for (size_t s = 0; s < summary_.size(); ++s) {
    if (!summary_[s]) continue;
    const int64_t w = static_cast<int64_t>(s) * 64 + __builtin_ctzll(summary_[s]);
    const int64_t bit = __builtin_ctzll(words_[w]);
    words_[w] &= words_[w] - 1;
    if (!words_[w]) summary_[s] &= ~(1ull << (w % 64));
    --nfree_;
    return w * 64 + bit;
  }
  return -1;
}

void IdPool::give(int64_t id) {
  const int64_t w = id / 64;
  words_[w] |= 1ull << (id % 64);
  summary_[w / 64] |= 1ull << (w % 64);
  ++nfree_;
}

// ------------------------------------------------------------------ Control

Control::Control(int32_t n_win, int32_t max_states, int64_t max_blocks, int64_t max_bps)
    : n_win_(n_win), max_states_(max_states), max_blocks_(max_blocks), max_bps_(max_bps),
      states_(max_states), blocks_(max_blocks), used_(max_states, 0), len_(max_states, 0),
      table_(max_states), refcount_(max_blocks, 0) {}

bool Control::valid_state(int32_t s) const {
  return s >= 0 && s < max_states_ && used_[s];
}

int Control::state_alloc(int32_t* out) {
  const int64_t s = states_.take_lowest();
  if (s < 0) return kOomStates;
  used_[s] = 1;
  len_[s] = 0;
  table_[s].clear();
  *out = static_cast<int32_t>(s);
  return kOk;
}

int Control::state_free(int32_t s) {
  if (!valid_state(s)) return kInvalid;
  for (int32_t b : table_[s]) {
    if (--refcount_[b] == 0) blocks_.give(b);
  }
  table_[s].clear();
  table_[s].shrink_to_fit();
  len_[s] = 0;
  used_[s] = 0;
  states_.give(s);
  return kOk;
}

int Control::check_states(int32_t n_req, const int32_t* states, bool distinct, bool nonempty,
                          std::string* why) const {
  if (n_req < 0 || (n_req > 0 && !states)) {
    *why = "bad request list";
    return kInvalid;
  }
  std::vector<uint8_t> seen;
  if (distinct) seen.assign(max_states_, 0);
  for (int32_t i = 0; i < n_req; ++i) {
    const int32_t s = states[i];
    if (!valid_state(s)) {
      *why = "state " + std::to_string(s) + " is not allocated";
      return kInvalid;
    }
    if (distinct) {
      if (seen[s]) {
        *why = "state " + std::to_string(s) + " listed twice";
        return kInvalid;
      }
      seen[s] = 1;
    }
    if (nonempty && len_[s] == 0) {
      *why = "state " + std::to_string(s) + " holds no token";
      return kInvalid;
    }
  }
  return kOk;
}

int Control::plan_append(int32_t n_req, const int32_t* states, const int64_t* cu, bool defer,
                         AppendPlan* plan, std::string* why) const {
  plan->reqs.clear();
  plan->seals.clear();
  plan->new_blocks = 0;
  int st = check_states(n_req, states, true, false, why);
  if (st) return st;
  if (n_req > 0 && !cu) {
    *why = "cu_tokens is NULL";
    return kInvalid;
  }
  if (n_req > 0 && cu[0] != 0) {
    *why = "cu_tokens[0] must be 0";
    return kInvalid;
  }
  // lifecycle checks first (request order), capacity checks after
  for (int32_t i = 0; i < n_req; ++i) {
    const int64_t n = cu[i + 1] - cu[i];
    if (n < 0) {
      *why = "cu_tokens must be nondecreasing";
      return kInvalid;
    }
    const int32_t s = states[i];
    const int64_t nb = n_blocks(s);
    const int64_t tail = len_[s] - kBlockTokens * nb;
    if (n > 0 && tail == kBlockTokens) {
      *why = "state " + std::to_string(s) + " has a full deferred tail; flush it first";
      return kState;
    }
    if (defer && tail + n > kBlockTokens) {
      *why = "deferred append would pass one block";
      return kState;
    }
    const int64_t add = defer ? 0 : (tail + n) / kBlockTokens;
    plan->reqs.push_back(AppendReq{s, len_[s], len_[s] + n, nb, nb + add, cu[i]});
  }
  int64_t need = 0;
  for (const AppendReq& r : plan->reqs) {
    if (r.nb_new > max_bps_ || r.len_new >= (int64_t(1) << 31)) {
      *why = "state " + std::to_string(r.state) + " would exceed its block table";
      plan->reqs.clear();
      return kOomBlocks;
    }
    need += r.nb_new - r.nb_old;
  }
  if (need > blocks_.free_count()) {
    *why = "Block Cache full: need " + std::to_string(need) + " blocks, " +
           std::to_string(blocks_.free_count()) + " free";
    plan->reqs.clear();
    return kOomBlocks;
  }
  plan->new_blocks = need;
  return kOk;
}

int Control::plan_flush(int32_t n_req, const int32_t* states, AppendPlan* plan,
                        std::string* why) const {
  plan->reqs.clear();
  plan->seals.clear();
  plan->new_blocks = 0;
  int st = check_states(n_req, states, true, false, why);
  if (st) return st;
  int64_t need = 0;
  for (int32_t i = 0; i < n_req; ++i) {
    const int32_t s = states[i];
    const int64_t nb = n_blocks(s);
    const int64_t add = pending(s) ? 1 : 0;
    if (nb + add > max_bps_) {
      *why = "block table full";
      return kOomBlocks;
    }
    need += add;
    // row0 < 0: every token of a flushed block is already resident in the State.
    plan->reqs.push_back(AppendReq{s, len_[s], len_[s], nb, nb + add, -1});
  }
  if (need > blocks_.free_count()) {
    *why = "Block Cache full";
    return kOomBlocks;
  }
  plan->new_blocks = need;
  return kOk;
}

void Control::commit(AppendPlan* plan) {
  plan->seals.clear();
  for (size_t i = 0; i < plan->reqs.size(); ++i) {
    const AppendReq& r = plan->reqs[i];
    for (int64_t lb = r.nb_old; lb < r.nb_new; ++lb) {
      const int32_t id = static_cast<int32_t>(blocks_.take_lowest());
      refcount_[id] = 1;
      table_[r.state].push_back(id);
      plan->seals.push_back(SealItem{static_cast<int32_t>(i), r.state, lb, id, r.len_old, r.row0});
    }
    len_[r.state] = r.len_new;
  }
}

int Control::check_share(int32_t src, int32_t dst, std::string* why) const {
  if (!valid_state(src) || !valid_state(dst)) {
    *why = "share: state not allocated";
    return kInvalid;
  }
  if (src == dst) {
    *why = "share: src == dst";
    return kInvalid;
  }
  if (len_[dst] != 0 || !table_[dst].empty()) {
    *why = "share: dst is not empty";
    return kState;
  }
  if (pending(src)) {
    *why = "share: src has a pending seal";
    return kState;
  }
  return kOk;
}

void Control::commit_share(int32_t src, int32_t dst) {
  for (int32_t b : table_[src]) ++refcount_[b];
  table_[dst] = table_[src];
  len_[dst] = len_[src];
}

int Control::check_block_ref(const int32_t* blocks, int64_t n, int32_t delta, std::string* why) const {
  if (delta != 1 && delta != -1) {
    *why = "block_ref: delta must be +1 or -1";
    return kInvalid;
  }
  if (n < 0 || (n > 0 && !blocks)) {
    *why = "block_ref: bad block list";
    return kInvalid;
  }
  std::vector<int32_t> sorted(blocks, blocks + n);
  std::sort(sorted.begin(), sorted.end());
  for (int64_t i = 0; i < n;) {
    int64_t j = i;
    while (j < n && sorted[j] == sorted[i]) ++j;
    const int32_t b = sorted[i];
    if (!valid_block(b) || refcount_[b] <= 0) {
      *why = "block_ref: block not in use";
      return kInvalid;
    }
    if (delta < 0 && j - i > refcount_[b]) {
      *why = "block_ref: block released more times than it is held";
      return kInvalid;
    }
    i = j;
  }
  return kOk;
}

void Control::commit_block_ref(const int32_t* blocks, int64_t n, int32_t delta) {
  for (int64_t i = 0; i < n; ++i) {
    refcount_[blocks[i]] += delta;
    if (refcount_[blocks[i]] == 0) blocks_.give(blocks[i]);
  }
}

int Control::check_attach(int32_t dst, const int32_t* blocks, int64_t len, std::string* why) const {
  if (!valid_state(dst)) {
    *why = "attach: state not allocated";
    return kInvalid;
  }
  if (len_[dst] != 0 || !table_[dst].empty()) {
    *why = "attach: dst is not empty";
    return kState;
  }
  const int64_t nb = len / kBlockTokens;
  if (len < 0 || nb > max_bps_ || (nb > 0 && !blocks)) {
    *why = "attach: bad length or block list";
    return kInvalid;
  }
  for (int64_t i = 0; i < nb; ++i)
    if (!valid_block(blocks[i]) || refcount_[blocks[i]] <= 0) {
      *why = "attach: block not in use";
      return kInvalid;
    }
  return kOk;
}

void Control::commit_attach(int32_t dst, const int32_t* blocks, int64_t len) {
  const int64_t nb = len / kBlockTokens;
  for (int64_t i = 0; i < nb; ++i) ++refcount_[blocks[i]];
  table_[dst].assign(blocks, blocks + nb);
  len_[dst] = len;
}

int Control::check_attach_batch(int32_t n_req, const int32_t* states, const int64_t* len,
                                const int32_t* blocks, int64_t n_blocks, const int64_t* off,
                                std::string* why) const {
  int st = check_states(n_req, states, true, false, why);
  if (st) return st;
  if (n_req > 0 && (!len || !off) ) {
    *why = "attach: NULL lengths or offsets";
    return kInvalid;
  }
  for (int32_t i = 0; i < n_req; ++i) {
    const int64_t nb = len[i] >= 0 ? len[i] / kBlockTokens : 0;
    if (len[i] < 0 || off[i] < 0 || off[i] + nb > n_blocks) {
      *why = "attach: length or block offset out of range";
      return kInvalid;
    }
    st = check_attach(states[i], nb > 0 ? blocks + off[i] : nullptr, len[i], why);
    if (st) return st;
  }
  return kOk;
}

int Control::check_state_write(int32_t n_req, const int32_t* states, const int64_t* cu,
                               const int64_t* pos0, std::string* why) const {
  int st = check_states(n_req, states, true, false, why);
  if (st) return st;
  if (n_req == 0) return kOk;
  if (!cu || !pos0 || cu[0] != 0) {
    *why = "state_write: bad cu_tokens or pos0";
    return kInvalid;
  }
  for (int32_t i = 0; i < n_req; ++i) {
    const int64_t n = cu[i + 1] - cu[i];
    if (n < 0) {
      *why = "state_write: cu_tokens must be nondecreasing";
      return kInvalid;
    }
    if (n > 0 && (pos0[i] < 0 || pos0[i] + n > len_[states[i]])) {
      *why = "state_write: positions outside [0, L)";
      return kInvalid;
    }
  }
  return kOk;
}

}  // namespace hsa
