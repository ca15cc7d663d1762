// control.h - host control plane of the heterogeneous KV cache (pure C++, no HIP).
//
// Holds the host mirror of everything integer: State slots, per-state length and
// block table, block refcounts and the free-block set. Every mutating operation
// is split into a check/plan step that changes nothing and a commit step that
// cannot fail, so a call that returns an error leaves the cache unchanged.
//
// Pages: [Q&A] "V4 为何要分池？块对齐与尾缓冲怎么配合？"; [Ch12] "Ch 12 · 推理框架 —
// KV 的异构调度".
#pragma once

#include <cstdint>
#include <string>
#include <vector>

namespace hsa {

enum Status : int {
  kOk = 0,
  kInvalid = -1,
  kOomBlocks = -2,
  kOomStates = -3,
  kState = -4,
  kDevice = -5,
};

constexpr int64_t kBlockTokens = 128;  // lcm(4, 128) ([Q&A] §2.2)
constexpr int kC4PerBlock = 32;        // 128 / 4 ([Ch12] §2.2)

// Lowest-free id set over [0, n): a two-level bitset (bit = 1 means free).
class IdPool {
 public:
  IdPool() = default;
  explicit IdPool(int64_t n);
  int64_t size() const { return n_; }
  int64_t free_count() const { return nfree_; }
  bool is_free(int64_t id) const;
  int64_t take_lowest();  // -1 when empty
  void give(int64_t id);

 private:
  int64_t n_ = 0, nfree_ = 0;
  std::vector<uint64_t> words_;
  std::vector<uint64_t> summary_;  // bit w set <=> words_[w] != 0
};

// One request's part of an append call, planned before anything changes.
struct AppendReq {
  int32_t state;
  int64_t len_old, len_new;   // tokens before / after the call
  int64_t nb_old, nb_new;     // sealed blocks before / after
  int64_t row0;               // packed input row of position len_old
};

// One block sealed by a call: logical block `lblock` of `state`, physical `id`.
struct SealItem {
  int32_t req;       // index in the call's request list
  int32_t state;
  int64_t lblock;
  int32_t id;
  int64_t len_old;   // the state's length before the call
  int64_t row0;      // packed input row of position len_old (tokens >= len_old)
};

struct AppendPlan {
  std::vector<AppendReq> reqs;
  std::vector<SealItem> seals;  // filled by commit, in id-allocation order
  int64_t new_blocks = 0;
};

class Control {
 public:
  Control(int32_t n_win, int32_t max_states, int64_t max_blocks, int64_t max_bps);

  int32_t n_win() const { return n_win_; }
  int32_t max_states() const { return max_states_; }
  int64_t max_blocks() const { return max_blocks_; }
  int64_t max_blocks_per_state() const { return max_bps_; }

  // State pool ([Ch12] §2.1).
  int state_alloc(int32_t* out);
  int state_free(int32_t s);  // refcount-- on its blocks; zero -> free

  // Append of cu[i+1]-cu[i] tokens to states[i] ([Q&A] §3.1, §4).
  int plan_append(int32_t n_req, const int32_t* states, const int64_t* cu, bool defer,
                  AppendPlan* plan, std::string* why) const;
  // Flush of deferred full tails ([Q&A] §3.1).
  int plan_flush(int32_t n_req, const int32_t* states, AppendPlan* plan, std::string* why) const;
  // Allocates block ids (lowest free; requests in order, blocks in token order),
  // updates lengths and tables, fills plan->seals. Cannot fail after a plan_*.
  void commit(AppendPlan* plan);

  // Prefix fork ([Ch12] §2.2).
  int check_share(int32_t src, int32_t dst, std::string* why) const;
  void commit_share(int32_t src, int32_t dst);

  // Prefix hits ([Ch12] §3.1; [Disk] SWA policies): block references held by a
  // prefix entry (delta +1 / -1; a block at 0 is freed), and a fresh state taking
  // a prefix's first len / 128 blocks and length len (its window is filled later).
  int check_block_ref(const int32_t* blocks, int64_t n, int32_t delta, std::string* why) const;
  void commit_block_ref(const int32_t* blocks, int64_t n, int32_t delta);
  int check_attach(int32_t dst, const int32_t* blocks, int64_t len, std::string* why) const;
  void commit_attach(int32_t dst, const int32_t* blocks, int64_t len);
  // A batch: states[i] (distinct) takes blocks[off[i] .. off[i] + len[i] / 128) of a
  // list of n_blocks ids (lists may overlap) and length len[i].
  int check_attach_batch(int32_t n_req, const int32_t* states, const int64_t* len, const int32_t* blocks,
                         int64_t n_blocks, const int64_t* off, std::string* why) const;
  // Replay of raw tokens into states: distinct states, cu[0] = 0 and nondecreasing,
  // positions [pos0[i], pos0[i] + n_i) inside [0, L) of states[i].
  int check_state_write(int32_t n_req, const int32_t* states, const int64_t* cu, const int64_t* pos0,
                        std::string* why) const;
  // Read-side validation: allocated states; optionally distinct / non-empty.
  int check_states(int32_t n_req, const int32_t* states, bool distinct, bool nonempty,
                   std::string* why) const;

  bool valid_state(int32_t s) const;
  bool valid_block(int64_t b) const { return b >= 0 && b < max_blocks_; }
  int64_t len(int32_t s) const { return len_[s]; }
  int64_t n_blocks(int32_t s) const { return static_cast<int64_t>(table_[s].size()); }
  bool pending(int32_t s) const { return len_[s] - kBlockTokens * n_blocks(s) == kBlockTokens; }
  const std::vector<int32_t>& table(int32_t s) const { return table_[s]; }
  int32_t refcount(int64_t b) const { return refcount_[b]; }
  int64_t free_blocks() const { return blocks_.free_count(); }

 private:
  int32_t n_win_, max_states_;
  int64_t max_blocks_, max_bps_;
  IdPool states_, blocks_;
  std::vector<uint8_t> used_;
  std::vector<int64_t> len_;
  std::vector<std::vector<int32_t>> table_;
  std::vector<int32_t> refcount_;
};

}  // namespace hsa
