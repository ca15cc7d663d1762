// hsa.cpp - the C ABI (include/hsa.h): validation, host control plane, pool and
// scratch management, and kernel launches on the caller's stream.
#include "../../include/hsa.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "control.h"
#include "device.h"
#include "kernels.h"
#include "launch_plan.h"
#include "noalloc.h"

using namespace hsa;

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& why) {
  g_err = why;
  return code;
}

#define HIP_TRY(expr)                                                               \
  do {                                                                              \
    hipError_t e_ = (expr);                                                         \
    if (e_ != hipSuccess) return fail(kDevice, std::string(#expr) + ": " + hipGetErrorString(e_)); \
  } while (0)

}  // namespace

struct hsa_ctx {
  int device = 0;
  bool poison = false;        // HSA_CREATE_POISON: fill every allocation with 0xFF bytes
  Control ctl;
  Pools P{};
  std::vector<void*> allocs;

  // scratch (device, grown on demand)
  float* scores = nullptr;
  size_t scores_cap = 0;
  float* part_acc = nullptr;   // [chunks][16][128] unnormalised attention partials
  size_t part_acc_cap = 0;     // in chunks
  float* part_ml = nullptr;    // [chunks][2][16] running max and sum
  size_t part_ml_cap = 0;
  float* seal_part = nullptr;  // kMaxReq * kSealSplit HCA partials of decode-time seals

  // bulk-plan staging: pinned host -> device
  void* plan_host = nullptr;
  void* plan_dev = nullptr;
  size_t plan_cap = 0;
  hipEvent_t plan_ev = nullptr;
  bool plan_busy = false;

  // timing
  uint32_t tmask = 0;
  std::vector<hipEvent_t> ev_free;
  struct Rec {
    int kid;
    hipEvent_t a, b;
  };
  std::vector<Rec> recs;

  int32_t attend_wgs = 512;   // attention workgroups per launch to aim for (one round)
  int32_t step_slots = 256;   // decode step: attention workgroups one launch holds at once
                              // (one per CU at the step kernels' register use)
  int32_t select_slice = 0;   // top-k: longer score rows are selected in two rounds (0: by k)
  int32_t step_fused = 1;     // decode step in three launches when every row fits the LDS cache
  // three-launch form: part-A keys a mixed workgroup takes (the rest go to part-A
  // workgroups in the same launch; negative: all), and the selection's cost in keys
  // of one workgroup for the balance
  int32_t mixed_a = 8;
  int32_t sel_lat = 16;
  int32_t mx_unit = 0;        // MXFP4 keys: blocks per scoring workgroup (0: by batch size)
  // layers: the pools of each (P is the current layer's); an append made at layer 0
  // and not yet repeated on every layer is kept in `seq` for the later layers
  std::vector<Pools> layers;
  int32_t cur_layer = 0;
  struct Seq {
    int kind = 0;                 // 1 append, 2 flush, 3 decode step
    std::vector<int32_t> states;
    std::vector<int64_t> cu;
    uint32_t flags = 0;
    AppendPlan plan;
    int32_t next = 0;             // the layer whose turn it is
  } seq;
  bool seq_open = false;
  void* fixed = nullptr;      // this device's fixed scratch buffer (hsa_decode_step_noalloc)
  int32_t* rows = nullptr;    // decode step: physical C4 rows of the selected entries
  size_t rows_cap = 0;
  int32_t* cand_ord = nullptr;  // top-k of sliced rows: per-slice candidates (ordinals, scores)
  size_t cand_ord_cap = 0;
  float* cand_score = nullptr;
  size_t cand_score_cap = 0;

  hsa_ctx(int32_t n_win, int32_t ms, int64_t mb, int64_t bps) : ctl(n_win, ms, mb, bps) {
    // launch-shape targets; the environment can override them for tuning sweeps
    if (const char* e = std::getenv("HSA_ATTEND_WGS")) attend_wgs = std::max(16, std::atoi(e));
    if (const char* e = std::getenv("HSA_STEP_SLOTS")) step_slots = std::max(16, std::min(1 << 16, std::atoi(e)));
    if (const char* e = std::getenv("HSA_STEP_FUSED")) step_fused = std::atoi(e) != 0;
    if (const char* e = std::getenv("HSA_MIXED_A")) mixed_a = std::atoi(e);
    if (const char* e = std::getenv("HSA_SEL_LAT")) sel_lat = std::max(0, std::atoi(e));
    if (const char* e = std::getenv("HSA_MX_UNIT")) mx_unit = std::max(1, std::min(kMxUnitMax, std::atoi(e)));
    if (const char* e = std::getenv("HSA_SELECT_SLICE"))   // a multiple of 32, at least 32
      select_slice = std::max(32, std::min(1 << 24, std::atoi(e)) / 32 * 32);
  }
};

namespace {

int dev_alloc(hsa_ctx* c, void** p, size_t bytes) {
  HIP_TRY(hipMalloc(p, bytes ? bytes : 16));
  c->allocs.push_back(*p);
  if (c->poison) {   // a debugging aid: never on a hot path (allocations are not)
    HIP_TRY(hipMemset(*p, 0xff, bytes ? bytes : 16));
    HIP_TRY(hipDeviceSynchronize());
  }
  return kOk;
}

int grow(hsa_ctx* c, void** p, size_t* cap, size_t need, size_t elem) {
  if (need <= *cap) return kOk;
  size_t n = std::max(need + need / 4, *cap + *cap / 2);   // headroom: growing synchronises the device
  HIP_TRY(hipDeviceSynchronize());
  if (*p) {
    c->allocs.erase(std::remove(c->allocs.begin(), c->allocs.end(), *p), c->allocs.end());
    HIP_TRY(hipFree(*p));
    *p = nullptr;
  }
  int st = dev_alloc(c, p, n * elem);
  if (st) return st;
  *cap = n;
  return kOk;
}

// Timing of one launch of kernel `kid`: the launch takes ev() and the dispatch
// records the pair; the record is kept only if the kernel was launched.
struct Timed {
  hsa_ctx* c;
  int kid;
  hipEvent_t a = nullptr, b = nullptr;
  bool fired = false;
  Timed(hsa_ctx* c_, int kid_, hipStream_t) : c(c_), kid(kid_) {
    if (!(c->tmask & (1u << kid))) return;
    for (hipEvent_t* e : {&a, &b}) {
      if (!c->ev_free.empty()) {
        *e = c->ev_free.back();
        c->ev_free.pop_back();
      } else if (hipEventCreateWithFlags(e, hipEventDisableSystemFence) != hipSuccess) {
        // timing only: no system-scope cache writeback / invalidate around the kernel
        *e = nullptr;
      }
    }
  }
  LaunchEv ev() {
    LaunchEv e;
    if (a && b) {
      e.a = a;
      e.b = b;
      e.fired = &fired;
    }
    return e;
  }
  ~Timed() {
    if (a && b && fired) {
      c->recs.push_back({kid, a, b});
    } else {
      if (a) c->ev_free.push_back(a);
      if (b) c->ev_free.push_back(b);
    }
  }
};

int set_device(hsa_ctx* c) {
  HIP_TRY(hipSetDevice(c->device));
  return kOk;
}

// Stage a bulk plan (seal and write descriptors) and copy it to the device.
int upload_plan(hsa_ctx* c, const void* data, size_t bytes, hipStream_t st) {
  if (c->plan_busy) {
    HIP_TRY(hipEventSynchronize(c->plan_ev));
    c->plan_busy = false;
  }
  if (bytes > c->plan_cap) {
    size_t n = std::max(bytes, c->plan_cap * 2);
    HIP_TRY(hipDeviceSynchronize());
    if (c->plan_host) HIP_TRY(hipHostFree(c->plan_host));
    if (c->plan_dev) {
      c->allocs.erase(std::remove(c->allocs.begin(), c->allocs.end(), c->plan_dev), c->allocs.end());
      HIP_TRY(hipFree(c->plan_dev));
    }
    c->plan_host = nullptr;
    c->plan_dev = nullptr;
    c->plan_cap = 0;
    HIP_TRY(hipHostMalloc(&c->plan_host, n, hipHostMallocDefault));
    int s = dev_alloc(c, &c->plan_dev, n);
    if (s) return s;
    c->plan_cap = n;
  }
  std::memcpy(c->plan_host, data, bytes);
  HIP_TRY(hipMemcpyAsync(c->plan_dev, c->plan_host, bytes, hipMemcpyHostToDevice, st));
  HIP_TRY(hipEventRecord(c->plan_ev, st));
  c->plan_busy = true;
  return kOk;
}

// Enqueue the seals and ring/tail writes of a committed bulk plan.
int run_bulk(hsa_ctx* c, const AppendPlan& plan, const void* k, const void* v, const float* ik,
             hipStream_t st) {
  std::vector<SealDesc> seals;
  seals.reserve(plan.seals.size());
  if (c->P.c4 || c->P.hca)   // an SWA layer keeps nothing in the Block Cache
    for (const SealItem& s : plan.seals)
      seals.push_back(SealDesc{s.state, s.id, s.lblock * kBlk, s.len_old, s.row0});
  std::vector<WriteDesc> writes;
  int64_t total = 0;
  for (const AppendReq& r : plan.reqs) {
    if (r.len_new == r.len_old) continue;
    const int64_t w0 = std::max(r.len_old, r.len_new - (int64_t)c->P.n_win);
    writes.push_back(WriteDesc{r.state, (int32_t)r.nb_new, r.len_old, r.len_new, w0, r.row0, total});
    total += r.len_new - w0;
  }
  if (seals.empty() && writes.empty()) return kOk;
  const size_t sb = seals.size() * sizeof(SealDesc), wb = writes.size() * sizeof(WriteDesc);
  std::vector<char> buf(sb + wb);
  if (sb) std::memcpy(buf.data(), seals.data(), sb);
  if (wb) std::memcpy(buf.data() + sb, writes.data(), wb);
  int s = upload_plan(c, buf.data(), buf.size(), st);
  if (s) return s;
  const SealDesc* dseal = reinterpret_cast<const SealDesc*>(c->plan_dev);
  const WriteDesc* dwrite = reinterpret_cast<const WriteDesc*>(static_cast<char*>(c->plan_dev) + sb);
  {
    Timed t(c, HSA_KERNEL_SEAL, st);
    HIP_TRY(launch_bulk_seal(c->P, dseal, (int64_t)seals.size(), k, v, ik, st, t.ev()));
  }
  {
    Timed t(c, HSA_KERNEL_WRITE, st);
    HIP_TRY(launch_bulk_write(c->P, dwrite, (int32_t)writes.size(), total, k, v, ik, st, t.ev()));
  }
  return kOk;
}

// Enqueue a committed one-token-per-request append (decode), in batches of kMaxReq.
int run_decode_append(hsa_ctx* c, const AppendPlan& plan, const void* k, const void* v,
                      const float* ik, hipStream_t st) {
  std::vector<int32_t> new_id(plan.reqs.size(), -1);
  for (const SealItem& s : plan.seals) new_id[s.req] = s.id;
  const size_t n = plan.reqs.size();
  for (size_t b0 = 0; b0 < n; b0 += kMaxReq) {
    ReqBatch B{};
    B.n = (int32_t)std::min<size_t>(kMaxReq, n - b0);
    for (int i = 0; i < B.n; ++i) {
      const AppendReq& r = plan.reqs[b0 + i];
      B.r[i] = Req{r.state, (int32_t)r.len_new, (int32_t)r.nb_new, new_id[b0 + i]};
      if (new_id[b0 + i] >= 0 && (c->P.c4 || c->P.hca)) B.seal_req[B.n_seal++] = (int8_t)i;
    }
    {
      Timed t(c, HSA_KERNEL_APPEND, st);
      HIP_TRY(launch_decode_append(c->P, B, static_cast<const uint16_t*>(k) + b0 * kRow,
                                   static_cast<const uint16_t*>(v) + b0 * kRow, ik + b0 * kIRow,
                                   c->seal_part, st, t.ev()));
    }
    if (B.n_seal && c->P.hca) {
      Timed t(c, HSA_KERNEL_SEAL, st);
      HIP_TRY(launch_seal_merge(c->P, B, c->seal_part, st, t.ev()));
    }
  }
  return kOk;
}

// Eager C4, host side: complete groups of the open block, top-k candidates and
// score-row length of a request of length len with nb sealed blocks (as open_groups,
// c4_cands and c4_rowlen on the device).
int64_t h_open(const Pools& P, int64_t len, int64_t nb) { return P.eager ? (len - kBlk * nb) / 4 : 0; }
int64_t h_cands(const Pools& P, int64_t len, int64_t nb) { return P.c4 ? kC4 * nb + h_open(P, len, nb) : 0; }
int64_t h_rowlen(const Pools& P, int64_t len, int64_t nb) {
  return P.c4 ? kC4 * (nb + (h_open(P, len, nb) > 0 ? 1 : 0)) : 0;
}

// Eager C4: recompute every open-block entry of the listed states from their rings
// (after a bulk append, a fork, a replay or a restore). No-op otherwise.
int recompute_open(hsa_ctx* c, const int32_t* states, int32_t n, hipStream_t st) {
  if (!c->P.eager) return kOk;
  std::vector<OpenDesc> d;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t s = states[i];
    const int64_t nb = c->ctl.n_blocks(s), g = h_open(c->P, c->ctl.len(s), nb);
    for (int64_t gi = 0; gi < g; ++gi) d.push_back(OpenDesc{s, (int32_t)nb, (int32_t)gi, 0});
  }
  if (d.empty()) return kOk;
  int s = upload_plan(c, d.data(), d.size() * sizeof(OpenDesc), st);
  if (s) return s;
  HIP_TRY(launch_open_c4(c->P, static_cast<const OpenDesc*>(c->plan_dev), (int32_t)d.size(), st));
  return kOk;
}

// Top-k workgroups of a batch (plan_slices). On the 4 x 2^20-token workload (k 2048),
// 32768-score slices measured 736 us per step, against 759 us for 16384 and 764 us
// for 65536. The candidates of sliced rows need n * gmax * k1 entries of scratch.
void plan_select_host(hsa_ctx* c, const ReqBatch& B, int32_t k, SelPlan& SP) {
  SP = SelPlan{};
  int64_t n[kMaxReq];
  for (int i = 0; i < B.n; ++i) n[i] = h_rowlen(c->P, B.r[i].len, B.r[i].nb);
  SP.eager = c->P.eager;
  plan_slices(n, B.n, k, c->select_slice, kSliceN, SP.first, &SP.gmax, &SP.slice, &SP.k1);
  SP.n_wgs = SP.first[B.n];
}
size_t sel_cand_need(const ReqBatch& B, const SelPlan& SP) {
  return SP.gmax > 1 ? (size_t)B.n * SP.gmax * SP.k1 : 0;
}

// plan_select_host, with the candidates in the context's scratch.
int plan_select(hsa_ctx* c, const ReqBatch& B, int32_t k, SelPlan& SP) {
  plan_select_host(c, B, k, SP);
  const size_t need = sel_cand_need(B, SP);
  if (need) {
    int s = grow(c, reinterpret_cast<void**>(&c->cand_ord), &c->cand_ord_cap, need, sizeof(int32_t));
    if (s) return s;
    s = grow(c, reinterpret_cast<void**>(&c->cand_score), &c->cand_score_cap, need, sizeof(float));
    if (s) return s;
    SP.cand_ord = c->cand_ord;
    SP.cand_score = c->cand_score;
  }
  return kOk;
}

ReqBatch read_batch(hsa_ctx* c, const int32_t* states, int32_t b0, int32_t n) {
  ReqBatch B{};
  B.n = n;
  for (int i = 0; i < n; ++i) {
    const int32_t s = states[b0 + i];
    B.r[i] = Req{s, (int32_t)c->ctl.len(s), (int32_t)c->ctl.n_blocks(s), 0};
  }
  return B;
}

int run_topk(hsa_ctx* c, int32_t n_req, const int32_t* states, const float* q_idx, int32_t k,
             uint32_t flags, int32_t* idx_out, float* score_out, hipStream_t st) {
  for (int32_t b0 = 0; b0 < n_req; b0 += kMaxReq) {
    const int32_t n = std::min<int32_t>(kMaxReq, n_req - b0);
    ReqBatch B = read_batch(c, states, b0, n);
    if (!c->P.c4)   // no C4 entries in this layer: every row is padding
      for (int i = 0; i < n; ++i) B.r[i].nb = 0;
    int64_t total = 0, maxnb = 0;   // scored blocks (eager C4: the open block too)
    for (int i = 0; i < n; ++i) {
      const int64_t bl = h_rowlen(c->P, B.r[i].len, B.r[i].nb) / kC4;
      total += bl;
      maxnb = std::max<int64_t>(maxnb, bl);
    }
    const int64_t ld = std::max<int64_t>(kC4 * maxnb, 1);
    int s = grow(c, reinterpret_cast<void**>(&c->scores), &c->scores_cap, (size_t)(ld * n), sizeof(float));
    if (s) return s;
    {
      Timed t(c, HSA_KERNEL_SCORE, st);
      HIP_TRY(launch_score(c->P, B, total, q_idx + (int64_t)b0 * kIRow, c->scores, ld, st, t.ev()));
    }
    SelPlan SP;
    s = plan_select(c, B, k, SP);
    if (s) return s;
    {
      Timed t(c, HSA_KERNEL_SELECT, st);
      HIP_TRY(launch_select(B, SP, k, (flags & HSA_TOPK_SORTED) ? 1 : 0, c->scores, ld,
                            idx_out + (int64_t)b0 * k, score_out ? score_out + (int64_t)b0 * k : nullptr,
                            st, t.ev()));
    }
  }
  return kOk;
}

// Keys per attention chunk: a multiple of 16 such that the launch has about
// attend_wgs workgroups, i.e. fills the GPU once.
int32_t attend_chunk(int64_t total_keys, int32_t n, int32_t target) {
  const int64_t slots = std::max<int64_t>(64, target - n);
  int64_t chunk = (total_keys + slots - 1) / slots;
  chunk = std::max<int64_t>(16, (chunk + 15) / 16 * 16);
  return (int32_t)std::min<int64_t>(chunk, 1 << 20);
}

int run_attend(hsa_ctx* c, int32_t n_req, const int32_t* states, const void* q,
               const int32_t* topk, int32_t k, float* out, hipStream_t st) {
  for (int32_t b0 = 0; b0 < n_req; b0 += kMaxReq) {
    const int32_t n = std::min<int32_t>(kMaxReq, n_req - b0);
    ReqBatch B = read_batch(c, states, b0, n);
    std::vector<int64_t> nk(n);
    int64_t keys = 0;
    for (int i = 0; i < n; ++i) {
      const int64_t swa = std::min<int64_t>(B.r[i].len, c->P.n_win);
      nk[i] = swa + (c->P.hca ? B.r[i].nb : 0) + std::min<int64_t>(k, h_cands(c->P, B.r[i].len, B.r[i].nb));
      keys += nk[i];
    }
    const int32_t chunk = attend_chunk(keys, n, c->attend_wgs);
    int64_t total = 0;
    for (int i = 0; i < n; ++i) total += (nk[i] + chunk - 1) / chunk;
    int s = grow(c, reinterpret_cast<void**>(&c->part_acc), &c->part_acc_cap, (size_t)total,
                 kRow * sizeof(float));
    if (s) return s;
    s = grow(c, reinterpret_cast<void**>(&c->part_ml), &c->part_ml_cap, (size_t)total,
             2 * kH * sizeof(float));
    if (s) return s;
    const void* qb = static_cast<const uint16_t*>(q) + (int64_t)b0 * kRow;
    const int32_t* tk = topk ? topk + (int64_t)b0 * k : nullptr;
    {
      Timed t(c, HSA_KERNEL_ATTEND, st);
      HIP_TRY(launch_attend(c->P, B, total, chunk, qb, tk, k, c->part_acc, c->part_ml,
                            out + (int64_t)b0 * kRow, st, t.ev()));
    }
    if (total > n) {   // some request spans two or more chunks
      Timed t(c, HSA_KERNEL_MERGE, st);
      HIP_TRY(launch_merge(c->P, B, chunk, k, c->part_acc, c->part_ml, out + (int64_t)b0 * kRow, st, t.ev()));
    }
  }
  return kOk;
}

// One batch (at most kMaxReq requests) of a decode step: the launch descriptors and
// the scratch they need, in elements.
struct StepBatch {
  ReqBatch B;
  StepArgs S;
  size_t n_scores = 0;   // floats: score rows (+16: the three-launch selection reads one
                         // float4 at the start of every row)
  size_t n_chunks = 0;   // attention partials (kRow + 2 kH floats each)
  size_t n_rows = 0;     // int32: physical C4 rows of the selected entries
  size_t n_cand = 0;     // top-k candidates of sliced rows (an int32 and a float each)
  size_t n_seal = 0;     // floats: HCA partials of the blocks sealed in this step
};

// Host plan of the batch of requests b0 .. b0 + kMaxReq - 1 of a one-token-per-request
// append plan (committed or not): form, workgroups, and scratch sizes. No device work.
void plan_step_batch(hsa_ctx* c, const AppendPlan& plan, const std::vector<int32_t>& new_id, int32_t b0,
                     int32_t k, uint32_t flags, StepBatch& sb) {
  const int32_t n = std::min<int32_t>(kMaxReq, (int32_t)plan.reqs.size() - b0);
  ReqBatch& B = sb.B;
  StepArgs& S = sb.S;
  B = ReqBatch{};
  S = StepArgs{};
  B.n = n;
  // three launches when every score row fits the selection's LDS cache (and the
  // top-k is wanted in ordinal order): every attention workgroup then selects for
  // itself and the new HCA key joins the merge
  // A layer without C4 entries needs no selection and no part B: part A only, the
  // new HCA key in the merge, padding top-k rows, and no S1 when nothing seals.
  const bool c4 = c->P.c4 != 0, hca = c->P.hca != 0;
  const bool a_only = !c4;
  bool fused = !a_only && c->step_fused != 0 && !(flags & HSA_TOPK_SORTED);
  for (int i = 0; i < n; ++i)
    fused = fused && h_rowlen(c->P, plan.reqs[b0 + i].len_new, plan.reqs[b0 + i].nb_new) <= kCacheN;
  std::vector<int64_t> na(n), nb(n);
  int64_t maxnb = 0, n_score = 0;
  // MXFP4 keys: one scoring pass per workgroup (kMxPass blocks, whose loads a
  // workgroup issues together); units of two passes or of a partial pass measured
  // slower on both small and large batches
  const int mx_unit = !c->P.mx4 ? 0 : c->mx_unit ? c->mx_unit : kMxPass;
  for (int i = 0; i < n; ++i) {
    const AppendReq& r = plan.reqs[b0 + i];
    const int32_t id = new_id[b0 + i];
    B.r[i] = Req{r.state, (int32_t)r.len_new, (int32_t)r.nb_new, id};
    if (id >= 0 && (c4 || hca)) B.seal_req[B.n_seal++] = (int8_t)i;   // an SWA layer seals nothing
    const int64_t sealed = id >= 0 ? 1 : 0;
    na[i] = std::min<int64_t>(r.len_new, c->P.n_win) + (hca ? r.nb_new - sealed : 0);
    nb[i] = (fused || !hca || a_only ? 0 : sealed) + std::min<int64_t>(k, h_cands(c->P, r.len_new, r.nb_new));
    maxnb = std::max<int64_t>(maxnb, h_rowlen(c->P, r.len_new, r.nb_new) / kC4);
    // eager C4: the open block is scored too, and a completed group gets its entry
    const bool open = h_open(c->P, r.len_new, r.nb_new) > 0;
    if (c4) n_score += score_units(r.nb_new, mx_unit, id >= 0) + (open ? kScoreSplit : 0);
    if (c->P.eager && r.len_new % 4 == 0 && r.len_new % kBlk != 0) B.open_req[B.n_open++] = (int8_t)i;
  }
  S.ld = std::max<int64_t>(kC4 * maxnb, 1);
  S.k = k;
  S.sorted = (flags & HSA_TOPK_SORTED) ? 1 : 0;
  S.fused = fused ? 1 : 0;
  S.mx_unit = mx_unit;
  S.a_only = a_only ? 1 : 0;
  // (with FP8 KV the part-A read of the newest token must see its stored value, so
  // the append stays in S1)
  S.s2_append = a_only && B.n_seal == 0 && !c->P.kv8 ? 1 : 0;
  S.n_score = (int32_t)n_score;
  if (!fused && !a_only) plan_select_host(c, B, k, S.sel);
  // workgroups: three-launch form, S2 holds mixed workgroups (at least one per
  // request: the first writes the top-k padding), each with a share of part B and
  // of part A, and part-A workgroups beside them; four-launch form, part A shares
  // S2 with the selections, part B has S3
  std::vector<int64_t> nab(n);
  for (int i = 0; i < n; ++i) nab[i] = na[i] + nb[i];
  AttnPart pa{&na, 0, 0, {}}, pb{fused ? &nab : &nb, 0, fused ? 1 : 0, {}};
  for (int i = 0; i < n; ++i) S.a_split[i] = (int32_t)na[i];
  if (fused && c->mixed_a >= 0) {
    // Every mixed workgroup (selection, then part B) runs the selection before its
    // part-B keys are known; it takes mixed_a part-A keys, whose loads are in flight
    // meanwhile. Part-A workgroups take the other part-A keys and stream them while
    // the mixed ones select. The balance counts a selection as sel_lat keys.
    std::vector<int64_t> ka = na, kb = nb;
    AttnPart pm{&kb, c->sel_lat, 1, {}}, px{&ka, 0, 0, {}};
    for (int it = 0; it < 2; ++it) {
      balance_wgs({&pm, &px}, c->step_slots - B.n_seal);
      for (int i = 0; i < n; ++i) {
        const int64_t am = px.wgs[i] == 0 ? na[i] : std::min<int64_t>(na[i], (int64_t)c->mixed_a * pm.wgs[i]);
        ka[i] = na[i] - am;
        kb[i] = nb[i] + am;
      }
    }
    for (int i = 0; i < n; ++i) {
      if (ka[i] == 0) px.wgs[i] = 0;
      S.a_split[i] = (int32_t)ka[i];
    }
    pa.wgs = px.wgs;
    pb.wgs = pm.wgs;
  } else if (fused) {
    balance_wgs({&pb}, c->step_slots - B.n_seal);
    pa.wgs.assign(n, 0);
    for (int i = 0; i < n; ++i) S.a_split[i] = 0;
  } else if (a_only) {
    balance_wgs({&pa}, c->step_slots - B.n_seal - (S.s2_append ? n : 0));
    pb.wgs.assign(n, 0);
  } else {
    balance_wgs({&pa}, c->step_slots - S.sel.n_wgs - B.n_seal);
    balance_wgs({&pb}, c->step_slots);
  }
  int64_t ta = 0, tb = 0, ts = 0;
  for (int i = 0; i < n; ++i) {
    S.first_a[i] = (int32_t)ta;
    S.first_b[i] = (int32_t)tb;
    S.first_s[i] = (int32_t)ts;
    ta += pa.wgs[i];
    tb += pb.wgs[i];
    ts += c4 ? score_units(B.r[i].nb, mx_unit, B.r[i].aux >= 0) +
                   (h_open(c->P, B.r[i].len, B.r[i].nb) > 0 ? kScoreSplit : 0)
             : 0;
  }
  S.first_a[n] = (int32_t)ta;
  S.first_b[n] = (int32_t)tb;
  S.first_s[n] = (int32_t)ts;
  S.n_a = (int32_t)ta;
  S.n_b = (int32_t)tb;
  sb.n_scores = (size_t)(S.ld * n + 16);
  sb.n_chunks = (size_t)(ta + tb + n);
  sb.n_rows = (size_t)n * k;
  sb.n_cand = sel_cand_need(B, S.sel);
  sb.n_seal = (size_t)B.n_seal * kSealSplit * kPartFloats;
}

// The batch's input and output pointers (rows b0 .. of the caller's arrays).
void bind_step_io(StepBatch& sb, int32_t b0, const void* k_new, const void* v_new, const float* idx_new,
                  const void* q, const float* q_idx, int32_t* topk_out, float* score_out, float* out) {
  StepArgs& S = sb.S;
  S.kin = static_cast<const uint16_t*>(k_new) + (int64_t)b0 * kRow;
  S.vin = static_cast<const uint16_t*>(v_new) + (int64_t)b0 * kRow;
  S.iin = idx_new + (int64_t)b0 * kIRow;
  S.q = static_cast<const uint16_t*>(q) + (int64_t)b0 * kRow;
  S.qi = q_idx + (int64_t)b0 * kIRow;
  S.topk = topk_out + (int64_t)b0 * S.k;
  S.score_out = score_out ? score_out + (int64_t)b0 * S.k : nullptr;
  S.out = out + (int64_t)b0 * kRow;
}

// The batch's scratch in the context's buffers (grown when too small).
int bind_ctx_scratch(hsa_ctx* c, StepBatch& sb) {
  StepArgs& S = sb.S;
  int s = grow(c, reinterpret_cast<void**>(&c->scores), &c->scores_cap, sb.n_scores, sizeof(float));
  if (!s) s = grow(c, reinterpret_cast<void**>(&c->part_acc), &c->part_acc_cap, sb.n_chunks, kRow * sizeof(float));
  if (!s) s = grow(c, reinterpret_cast<void**>(&c->part_ml), &c->part_ml_cap, sb.n_chunks, 2 * kH * sizeof(float));
  if (!s) s = grow(c, reinterpret_cast<void**>(&c->rows), &c->rows_cap, sb.n_rows, sizeof(int32_t));
  if (!s && sb.n_cand) {
    s = grow(c, reinterpret_cast<void**>(&c->cand_ord), &c->cand_ord_cap, sb.n_cand, sizeof(int32_t));
    if (!s) s = grow(c, reinterpret_cast<void**>(&c->cand_score), &c->cand_score_cap, sb.n_cand, sizeof(float));
    S.sel.cand_ord = c->cand_ord;
    S.sel.cand_score = c->cand_score;
  }
  if (s) return s;
  S.scores = c->scores;
  S.part_acc = c->part_acc;
  S.part_ml = c->part_ml;
  S.rows = c->rows;
  S.seal_part = c->seal_part;
  return kOk;
}

// Fixed-buffer layout of a batch's scratch: each segment at a 256-byte boundary.
size_t seg_bytes(size_t n, size_t elem) { return (n * elem + 255) / 256 * 256; }
size_t fixed_scratch_bytes(const StepBatch& sb) {
  return seg_bytes(sb.n_scores, 4) + seg_bytes(sb.n_chunks, kRow * 4) + seg_bytes(sb.n_chunks, 2 * kH * 4) +
         seg_bytes(sb.n_rows, 4) + 2 * seg_bytes(sb.n_cand, 4) + seg_bytes(sb.n_seal, 4);
}
void bind_fixed_scratch(char* base, StepBatch& sb) {
  StepArgs& S = sb.S;
  auto take = [&](size_t n, size_t elem) {
    char* p = base;
    base += seg_bytes(n, elem);
    return p;
  };
  S.scores = reinterpret_cast<float*>(take(sb.n_scores, 4));
  S.part_acc = reinterpret_cast<float*>(take(sb.n_chunks, kRow * 4));
  S.part_ml = reinterpret_cast<float*>(take(sb.n_chunks, 2 * kH * 4));
  S.rows = reinterpret_cast<int32_t*>(take(sb.n_rows, 4));
  S.sel.cand_ord = reinterpret_cast<int32_t*>(take(sb.n_cand, 4));
  S.sel.cand_score = reinterpret_cast<float*>(take(sb.n_cand, 4));
  S.seal_part = reinterpret_cast<float*>(take(sb.n_seal, 4));
}

// Enqueue the three or four launches of a planned and bound batch.
int launch_step_batch(hsa_ctx* c, const StepBatch& sb, hipStream_t st) {
  const ReqBatch& B = sb.B;
  const StepArgs& S = sb.S;
  if (!S.s2_append) {
    Timed t(c, HSA_KERNEL_STEP1, st);
    HIP_TRY(launch_step1(c->P, B, S, st, t.ev()));
  }
  {
    Timed t(c, HSA_KERNEL_STEP2, st);
    HIP_TRY(launch_step2(c->P, B, S, st, t.ev()));
  }
  if (!S.fused && S.sel.gmax > 1) {
    Timed t(c, HSA_KERNEL_STEP2B, st);
    HIP_TRY(launch_step2b(c->P, B, S, st, t.ev()));
  }
  {
    Timed t(c, HSA_KERNEL_STEP3, st);
    HIP_TRY(launch_step3(c->P, B, S, st, t.ev()));
  }
  {
    Timed t(c, HSA_KERNEL_STEP4, st);
    HIP_TRY(launch_step4(c->P, B, S, st, t.ev()));
  }
  return kOk;
}

std::vector<int32_t> sealed_ids(const AppendPlan& plan) {
  std::vector<int32_t> new_id(plan.reqs.size(), -1);
  for (const SealItem& s : plan.seals) new_id[s.req] = s.id;
  return new_id;
}

// Largest fixed-buffer scratch of any batch of a decode step over `plan`.
size_t step_fixed_need(hsa_ctx* c, const AppendPlan& plan, int32_t k, uint32_t flags) {
  const std::vector<int32_t> new_id = sealed_ids(plan);
  size_t need = 0;
  StepBatch sb;
  for (int32_t b0 = 0; b0 < (int32_t)plan.reqs.size(); b0 += kMaxReq) {
    plan_step_batch(c, plan, new_id, b0, k, flags, sb);
    need = std::max(need, fixed_scratch_bytes(sb));
  }
  return need;
}

// The decode step (committed one-token append + top-k + attention) in three or four
// launches per batch of kMaxReq requests. Scratch: the context's buffers, or, with
// `fixed` (at least step_fixed_need bytes of device memory), that buffer, reused by
// every batch in stream order.
int run_decode_step(hsa_ctx* c, const AppendPlan& plan, const void* k_new, const void* v_new,
                    const float* idx_new, const void* q, const float* q_idx, int32_t k,
                    uint32_t flags, int32_t* topk_out, float* score_out, float* out,
                    hipStream_t st, char* fixed = nullptr) {
  const std::vector<int32_t> new_id = sealed_ids(plan);
  StepBatch sb;
  for (int32_t b0 = 0; b0 < (int32_t)plan.reqs.size(); b0 += kMaxReq) {
    plan_step_batch(c, plan, new_id, b0, k, flags, sb);
    bind_step_io(sb, b0, k_new, v_new, idx_new, q, q_idx, topk_out, score_out, out);
    if (fixed) {
      bind_fixed_scratch(fixed, sb);
    } else {
      const int s = bind_ctx_scratch(c, sb);
      if (s) return s;
    }
    const int s = launch_step_batch(c, sb, st);
    if (s) return s;
  }
  return kOk;
}

// ---- layers: an append made at layer 0 is repeated at layers 1 .. n-1 ----

enum SeqKind { kSeqAppend = 1, kSeqFlush = 2, kSeqStep = 3 };

// Gate of an appending call at the current layer. Layer 0 (or a one-layer context)
// plans and commits it (*replay = false). A later layer must repeat, in layer order,
// the call made at layer 0 (same kind, states, token counts and flags), whose
// committed plan it runs on its own pools (*replay = true).
int layer_gate(hsa_ctx* c, int kind, int32_t n_req, const int32_t* states, const int64_t* cu,
               uint32_t flags, bool* replay) {
  *replay = false;
  if (c->layers.size() <= 1) return kOk;
  if (c->cur_layer == 0) {
    if (c->seq_open)
      return fail(kState, "layer " + std::to_string(c->seq.next) + " of the previous append is pending");
    return kOk;
  }
  if (!c->seq_open || c->seq.next != c->cur_layer)
    return fail(kState, "an append is made at layer 0, then at each later layer in order");
  const hsa_ctx::Seq& q = c->seq;
  bool same = q.kind == kind && n_req >= 0 && (size_t)n_req == q.states.size() && q.flags == flags &&
              (n_req == 0 || states);
  for (int32_t i = 0; same && i < n_req; ++i) same = states[i] == q.states[i];
  if (same && kind == kSeqAppend) {
    same = cu != nullptr || n_req == 0;
    for (int32_t i = 0; same && i <= n_req && n_req > 0; ++i) same = cu[i] == q.cu[i];
  }
  if (!same) return fail(kInvalid, "the call differs from the one made at layer 0");
  *replay = true;
  return kOk;
}

void layer_record(hsa_ctx* c, int kind, int32_t n_req, const int32_t* states, const int64_t* cu,
                  uint32_t flags, const AppendPlan& plan) {
  if (c->layers.size() <= 1) return;
  hsa_ctx::Seq& q = c->seq;
  q.kind = kind;
  q.states.assign(states, states + std::max(n_req, 0));
  q.cu.assign(cu && n_req > 0 ? cu : nullptr, cu && n_req > 0 ? cu + n_req + 1 : nullptr);
  q.flags = flags;
  q.plan = plan;
  q.next = 1;
  c->seq_open = true;
}

void layer_advance(hsa_ctx* c) {
  if (++c->seq.next >= (int32_t)c->layers.size()) c->seq_open = false;
}

// Calls that change states or blocks wait until every layer has taken the last append.
int no_open_seq(hsa_ctx* c) {
  return c->seq_open ? fail(kState, "layer " + std::to_string(c->seq.next) + " of the last append is pending")
                     : kOk;
}

// The SWA ring of a layer as two byte arrays of one row per slot (slot g = state *
// n_win + p % n_win): the bf16 K and V rows, or with FP8 KV the code rows (K codes,
// V codes) and the scale rows. A checkpoint holds n_win rows of each, then the tail.
struct RingPart {
  char* base;
  size_t row;
};
void ring_parts(const Pools& P, RingPart out[2]) {
  if (P.kv8) {
    out[0] = RingPart{reinterpret_cast<char*>(P.swq), (size_t)kC4Bytes};
    out[1] = RingPart{reinterpret_cast<char*>(P.sws), (size_t)kC4Scales * 4};
  } else {
    out[0] = RingPart{reinterpret_cast<char*>(P.swa_k), (size_t)kRow * 2};
    out[1] = RingPart{reinterpret_cast<char*>(P.swa_v), (size_t)kRow * 2};
  }
}

int check_config(const hsa_config* cfg) {
  if (!cfg) return fail(kInvalid, "config is NULL");
  if (cfg->n_heads != kH || cfg->head_dim != kD)
    return fail(kInvalid, "only 16 heads x 128 dims are supported");
  if (cfg->m_csa != 4 || cfg->m_hca != kBlk) return fail(kInvalid, "m_csa must be 4 and m_hca 128");
  if (cfg->idx_heads != kHi || cfg->idx_dim != kDi)
    return fail(kInvalid, "indexer must be 4 heads x 64 dims");
  if (cfg->n_win < kBlk || cfg->n_win % kBlk) return fail(kInvalid, "n_win must be a positive multiple of 128");
  if (cfg->max_states < 1 || cfg->max_blocks < 1) return fail(kInvalid, "pool sizes must be positive");
  if (cfg->max_blocks > INT32_MAX) return fail(kInvalid, "max_blocks must fit int32 ids");
  const int64_t bps = cfg->max_blocks_per_state ? cfg->max_blocks_per_state : cfg->max_blocks;
  if (bps < 1 || bps > (int64_t(1) << 24)) return fail(kInvalid, "max_blocks_per_state out of range");
  if (!cfg->gate_csa || !cfg->gate_hca) return fail(kInvalid, "gate weights are NULL");
  if (cfg->entry_format != HSA_ENTRY_BF16 && cfg->entry_format != HSA_ENTRY_FP8)
    return fail(kInvalid, "entry_format must be HSA_ENTRY_BF16 or HSA_ENTRY_FP8");
  if (cfg->index_format != HSA_INDEX_F32 && cfg->index_format != HSA_INDEX_MXFP4)
    return fail(kInvalid, "index_format must be HSA_INDEX_F32 or HSA_INDEX_MXFP4");
  if (cfg->n_layers < 0 || cfg->n_layers > 1024) return fail(kInvalid, "n_layers must be in [0, 1024]");
  if (cfg->create_flags & ~HSA_CREATE_POISON) return fail(kInvalid, "unknown create_flags");
  if (cfg->c4_mode != HSA_C4_SEALED && cfg->c4_mode != HSA_C4_EAGER)
    return fail(kInvalid, "c4_mode must be HSA_C4_SEALED or HSA_C4_EAGER");
  if (cfg->kv_format != HSA_KV_BF16 && cfg->kv_format != HSA_KV_FP8)
    return fail(kInvalid, "kv_format must be HSA_KV_BF16 or HSA_KV_FP8");
  if (cfg->c4_mode == HSA_C4_EAGER &&
      (cfg->entry_format != HSA_ENTRY_BF16 || cfg->index_format != HSA_INDEX_F32 || cfg->kv_format != HSA_KV_BF16))
    return fail(kInvalid, "eager C4 takes bf16 entries, bf16 KV and fp32 indexer keys");
  if (cfg->layer_types)
    for (int l = 0; l < std::max(1, cfg->n_layers); ++l)
      if (cfg->layer_types[l] < HSA_LAYER_MIXED || cfg->layer_types[l] > HSA_LAYER_HCA)
        return fail(kInvalid, "layer_types must be HSA_LAYER_MIXED, _SWA, _CSA or _HCA");
  return kOk;
}

}  // namespace

extern "C" {

hsa_status hsa_create(const hsa_config* cfg, int device, hsa_ctx** out) {
  if (!out) return fail(kInvalid, "out is NULL");
  *out = nullptr;
  int st = check_config(cfg);
  if (st) return st;
  int ndev = 0;
  HIP_TRY(hipGetDeviceCount(&ndev));
  if (device < 0 || device >= ndev) return fail(kInvalid, "no such device");
  HIP_TRY(hipSetDevice(device));
  void* fixed = nullptr;   // the fixed scratch buffer's address on this device
  HIP_TRY(noalloc_scratch(device, &fixed));
  const int64_t bps = cfg->max_blocks_per_state ? cfg->max_blocks_per_state : cfg->max_blocks;
  hsa_ctx* c = new hsa_ctx(cfg->n_win, cfg->max_states, cfg->max_blocks, bps);
  c->device = device;
  c->poison = (cfg->create_flags & HSA_CREATE_POISON) != 0;
  c->fixed = fixed;
  if (!std::getenv("HSA_STEP_SLOTS")) {   // one step-kernel workgroup per CU
    int n_cu = 0;
    if (hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, device) == hipSuccess && n_cu > 0)
      c->step_slots = n_cu;
  }
  const size_t S = (size_t)cfg->max_states, NB = (size_t)cfg->max_blocks, W = (size_t)cfg->n_win;
  const bool fp8 = cfg->entry_format == HSA_ENTRY_FP8;
  const bool mx4 = cfg->index_format == HSA_INDEX_MXFP4;
  const int n_layers = cfg->n_layers > 0 ? cfg->n_layers : 1;
  const bool eager = cfg->c4_mode == HSA_C4_EAGER;
  const bool kv8 = cfg->kv_format == HSA_KV_FP8;
  // eager C4: each state's open block is C4 block id max_blocks + state, and its table
  // row has one more entry (the open block's)
  const size_t NB4 = NB + (eager ? S : 0), stride = (size_t)bps + (eager ? 1 : 0);
  // shared by the layers: block tables, seal partials, every layer's gates
  void* sh[3] = {};
  const size_t sh_bytes[3] = {S * stride * 4, (size_t)kMaxReq * kSealSplit * kPartFloats * 4,
                              (size_t)n_layers * 2 * kRow * 4};
  for (int i = 0; i < 3; ++i) {
    st = dev_alloc(c, &sh[i], sh_bytes[i]);
    if (st) {
      hsa_destroy(c);
      return st;
    }
  }
  int32_t* table = static_cast<int32_t*>(sh[0]);
  c->seal_part = static_cast<float*>(sh[1]);
  float* gates = static_cast<float*>(sh[2]);
  c->layers.resize(n_layers);
  for (int l = 0; l < n_layers; ++l) {
    const int type = cfg->layer_types ? cfg->layer_types[l] : HSA_LAYER_MIXED;
    const bool c4 = type == HSA_LAYER_MIXED || type == HSA_LAYER_CSA;
    const bool hca = type == HSA_LAYER_MIXED || type == HSA_LAYER_HCA;
    // per layer, by type: the SWA ring always; C4 entries, indexer keys and the
    // indexer tail for C4 layers; HCA entries for HCA layers
    constexpr int kPools = 16;
    void* p[kPools] = {};
    const size_t bytes[kPools] = {
        kv8 ? 0 : S * W * kRow * 2, kv8 ? 0 : S * W * kRow * 2,                // swa_k, swa_v
        c4 ? S * kBlk * kIRow * 4 : 0,                                          // idx_tail
        c4 && !fp8 ? NB4 * kC4 * kRow * 2 : 0, c4 && !fp8 ? NB4 * kC4 * kRow * 2 : 0,   // csa (bf16)
        hca && !kv8 ? NB * kRow * 2 : 0, hca && !kv8 ? NB * kRow * 2 : 0,       // hca
        c4 && !mx4 ? NB * kBlk * kIRow * 4 : 0,                                 // idx_k (fp32 keys)
        c4 && fp8 ? NB * kC4 * kC4Bytes : 0, c4 && fp8 ? NB * kC4 * kC4Scales * 4 : 0,   // FP8 C4
        c4 && mx4 ? NB * kBlk * kIRowQ : 0, c4 && mx4 ? NB * kBlk * kIRowE : 0,        // MXFP4 keys
        kv8 ? S * W * kC4Bytes : 0, kv8 ? S * W * kC4Scales * 4 : 0,            // FP8 ring
        kv8 && hca ? NB * kC4Bytes : 0, kv8 && hca ? NB * kC4Scales * 4 : 0};   // FP8 HCA
    for (int i = 0; i < kPools; ++i) {
      st = dev_alloc(c, &p[i], bytes[i]);
      if (st) {
        hsa_destroy(c);
        return st;
      }
    }
    Pools& P = c->layers[l];
    P.swa_k = static_cast<uint16_t*>(p[0]);
    P.swa_v = static_cast<uint16_t*>(p[1]);
    P.idx_tail = static_cast<float*>(p[2]);
    P.csa_k = static_cast<uint16_t*>(p[3]);
    P.csa_v = static_cast<uint16_t*>(p[4]);
    P.hca_k = static_cast<uint16_t*>(p[5]);
    P.hca_v = static_cast<uint16_t*>(p[6]);
    P.idx_k = static_cast<float*>(p[7]);
    P.c4q = static_cast<uint8_t*>(p[8]);
    P.c4s = static_cast<float*>(p[9]);
    P.idx_q = static_cast<uint8_t*>(p[10]);
    P.idx_e = static_cast<uint8_t*>(p[11]);
    P.swq = static_cast<uint8_t*>(p[12]);
    P.sws = static_cast<float*>(p[13]);
    P.hcq = static_cast<uint8_t*>(p[14]);
    P.hcs = static_cast<float*>(p[15]);
    P.kv8 = kv8 ? 1 : 0;
    P.table = table;
    P.table_stride = (int64_t)stride;
    P.gate_csa = gates + (size_t)l * 2 * kRow;
    P.gate_hca = gates + (size_t)l * 2 * kRow + kRow;
    P.n_win = cfg->n_win;
    P.max_blocks = (int32_t)cfg->max_blocks;
    P.fp8 = fp8 ? 1 : 0;
    P.mx4 = mx4 ? 1 : 0;
    P.c4 = c4 ? 1 : 0;
    P.hca = hca ? 1 : 0;
    P.eager = eager && c4 ? 1 : 0;
    P.c4_ids = (int32_t)(c4 ? NB4 : NB);
  }
  c->P = c->layers[0];
  // attention partials: a decode step has at most max(slots, requests) workgroups per
  // part, and hsa_decode_attend at most max(64, target - n) + n <= target + 64, so
  // these never grow (no device synchronisation in a decode loop)
  {
    const size_t chunks = std::max<size_t>(2 * ((size_t)c->step_slots + kMaxReq),
                                           (size_t)c->attend_wgs + kMaxReq);
    st = grow(c, reinterpret_cast<void**>(&c->part_acc), &c->part_acc_cap, chunks, kRow * sizeof(float));
    if (st == kOk)
      st = grow(c, reinterpret_cast<void**>(&c->part_ml), &c->part_ml_cap, chunks, 2 * kH * sizeof(float));
    if (st) {
      hsa_destroy(c);
      return st;
    }
  }
  hipError_t e = hipSuccess;
  for (int l = 0; l < n_layers && e == hipSuccess; ++l) {
    e = hipMemcpy(gates + (size_t)l * 2 * kRow, cfg->gate_csa + (size_t)l * kRow, kRow * 4, hipMemcpyHostToDevice);
    if (e == hipSuccess)
      e = hipMemcpy(gates + (size_t)l * 2 * kRow + kRow, cfg->gate_hca + (size_t)l * kRow, kRow * 4,
                    hipMemcpyHostToDevice);
  }
  if (e == hipSuccess) e = hipMemset(table, 0xff, sh_bytes[0]);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&c->plan_ev, hipEventDisableTiming);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    hsa_destroy(c);
    return fail(kDevice, std::string("hsa_create: ") + hipGetErrorString(e));
  }
  *out = c;
  return kOk;
}

hsa_status hsa_destroy(hsa_ctx* c) {
  if (!c) return kOk;
  // teardown releases what it can: an error here leaves nothing to undo
  (void)hipSetDevice(c->device);
  (void)hipDeviceSynchronize();
  for (void* p : c->allocs) (void)hipFree(p);
  if (c->plan_host) (void)hipHostFree(c->plan_host);
  if (c->plan_ev) (void)hipEventDestroy(c->plan_ev);
  for (auto& r : c->recs) {
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  for (hipEvent_t e : c->ev_free) (void)hipEventDestroy(e);
  delete c;
  return kOk;
}

hsa_status hsa_state_alloc(hsa_ctx* c, int32_t* out) {
  if (!c || !out) return fail(kInvalid, "NULL argument");
  int st = c->ctl.state_alloc(out);
  return st ? fail(st, "no free State slot") : kOk;
}

hsa_status hsa_state_free(hsa_ctx* c, int32_t s) {
  if (!c) return fail(kInvalid, "NULL context");
  int st = no_open_seq(c);
  if (st) return st;
  st = c->ctl.state_free(s);
  return st ? fail(st, "state " + std::to_string(s) + " is not allocated") : kOk;
}

hsa_status hsa_append_kv(hsa_ctx* c, int32_t n_req, const int32_t* states, const int64_t* cu,
                         const void* k, const void* v, const float* idx_k, uint32_t flags,
                         void* stream) {
  if (!c) return fail(kInvalid, "NULL context");
  if (flags & ~HSA_APPEND_DEFER_SEAL) return fail(kInvalid, "unknown flags");
  bool replay = false;
  int st = layer_gate(c, kSeqAppend, n_req, states, cu, flags, &replay);
  if (st) return st;
  std::string why;
  AppendPlan fresh;
  if (!replay) {
    st = c->ctl.plan_append(n_req, states, cu, (flags & HSA_APPEND_DEFER_SEAL) != 0, &fresh, &why);
    if (st) return fail(st, why);
  }
  const AppendPlan& plan = replay ? c->seq.plan : fresh;
  const int64_t T = n_req > 0 ? cu[n_req] : 0;
  if (T > 0 && (!k || !v || (!idx_k && c->P.c4))) return fail(kInvalid, "input pointer is NULL");
  if ((st = set_device(c))) return st;
  bool one_each = n_req > 0;
  for (const AppendReq& r : plan.reqs) one_each = one_each && (r.len_new - r.len_old == 1);
  if (replay) {
    layer_advance(c);
  } else {
    c->ctl.commit(&fresh);
    layer_record(c, kSeqAppend, n_req, states, cu, flags, fresh);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = one_each ? run_decode_append(c, plan, k, v, idx_k, s) : run_bulk(c, plan, k, v, idx_k, s);
  if (st) return st;
  return recompute_open(c, states, n_req, s);   // eager C4: the open blocks' entries
}

hsa_status hsa_compress_flush(hsa_ctx* c, int32_t n_req, const int32_t* states, void* stream) {
  if (!c) return fail(kInvalid, "NULL context");
  bool replay = false;
  int st = layer_gate(c, kSeqFlush, n_req, states, nullptr, 0, &replay);
  if (st) return st;
  if (replay) {
    layer_advance(c);
    if (c->seq.plan.new_blocks == 0) return kOk;
    if ((st = set_device(c))) return st;
    return run_bulk(c, c->seq.plan, nullptr, nullptr, nullptr, static_cast<hipStream_t>(stream));
  }
  std::string why;
  AppendPlan plan;
  st = c->ctl.plan_flush(n_req, states, &plan, &why);
  if (st) return fail(st, why);
  if ((st = set_device(c))) return st;
  c->ctl.commit(&plan);
  layer_record(c, kSeqFlush, n_req, states, nullptr, 0, plan);
  if (plan.new_blocks == 0) return kOk;
  return run_bulk(c, plan, nullptr, nullptr, nullptr, static_cast<hipStream_t>(stream));
}

hsa_status hsa_block_table_share(hsa_ctx* c, int32_t src, int32_t dst, void* stream) {
  if (!c) return fail(kInvalid, "NULL context");
  std::string why;
  int st = no_open_seq(c);
  if (st) return st;
  st = c->ctl.check_share(src, dst, &why);
  if (st) return fail(st, why);
  if ((st = set_device(c))) return st;
  c->ctl.commit_share(src, dst);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t L = c->ctl.len(dst), nb = c->ctl.n_blocks(dst), W = c->P.n_win;
  const size_t stride = (size_t)c->P.table_stride;
  if (nb > 0)
    HIP_TRY(hipMemcpyAsync(c->P.table + dst * stride, c->P.table + src * stride, nb * 4,
                           hipMemcpyDeviceToDevice, s));
  const int64_t slots = std::min(L, W), tail = L - kBlk * nb;
  for (const Pools& P : c->layers) {   // the State of every layer
    RingPart rp[2];
    ring_parts(P, rp);
    if (slots > 0)
      for (const RingPart& q : rp)
        HIP_TRY(hipMemcpyAsync(q.base + (size_t)dst * W * q.row, q.base + (size_t)src * W * q.row,
                               (size_t)slots * q.row, hipMemcpyDeviceToDevice, s));
    if (tail > 0 && P.c4)
      HIP_TRY(hipMemcpyAsync(P.idx_tail + (size_t)dst * kBlk * kIRow, P.idx_tail + (size_t)src * kBlk * kIRow,
                             (size_t)tail * kIRow * 4, hipMemcpyDeviceToDevice, s));
  }
  // eager C4: dst's own open-block entries, from its copied ring, in every layer
  const Pools cur = c->P;
  for (const Pools& P : c->layers) {
    c->P = P;
    st = recompute_open(c, &dst, 1, s);
    if (st) break;
  }
  c->P = cur;
  return st;
}

// ---- prefix hits: block references, attach, replay, checkpoints -------------------

hsa_status hsa_block_ref(hsa_ctx* c, const int32_t* blocks, int64_t n, int32_t delta) {
  if (!c) return fail(kInvalid, "NULL context");
  std::string why;
  int st = no_open_seq(c);
  if (st) return st;
  st = c->ctl.check_block_ref(blocks, n, delta, &why);
  if (st) return fail(st, why);
  c->ctl.commit_block_ref(blocks, n, delta);
  return kOk;
}

hsa_status hsa_prefix_attach(hsa_ctx* c, int32_t n_req, const int32_t* states, const int64_t* len,
                             const int32_t* blocks, int64_t n_blocks, const int64_t* block_off,
                             void* stream) {
  if (!c) return fail(kInvalid, "NULL context");
  std::string why;
  if (n_blocks < 0 || (n_blocks > 0 && !blocks)) return fail(kInvalid, "bad block list");
  int st = no_open_seq(c);
  if (st) return st;
  st = c->ctl.check_attach_batch(n_req, states, len, blocks, n_blocks, block_off, &why);
  if (st) return fail(st, why);
  if ((st = set_device(c))) return st;
  std::vector<AttachDesc> d;
  int64_t used = 0;   // ids needed: the list up to the furthest one referenced
  for (int32_t i = 0; i < n_req; ++i) {
    const int64_t nb = len[i] / kBlk;
    c->ctl.commit_attach(states[i], blocks + block_off[i], len[i]);
    if (nb == 0) continue;
    d.push_back(AttachDesc{states[i], 0, nb, block_off[i]});
    used = std::max(used, block_off[i] + nb);
  }
  if (d.empty()) return kOk;
  // descriptors, then the ids, staged in one upload; one launch writes every row
  const size_t db = d.size() * sizeof(AttachDesc);
  std::vector<char> buf(db + (size_t)used * 4);
  std::memcpy(buf.data(), d.data(), db);
  std::memcpy(buf.data() + db, blocks, (size_t)used * 4);
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = upload_plan(c, buf.data(), buf.size(), s);
  if (st) return st;
  const char* dev = static_cast<const char*>(c->plan_dev);
  HIP_TRY(launch_attach_rows(c->P, reinterpret_cast<const AttachDesc*>(dev), (int32_t)d.size(),
                             reinterpret_cast<const int32_t*>(dev + db), s));
  return kOk;
}

hsa_status hsa_state_write(hsa_ctx* c, int32_t n_req, const int32_t* states, const int64_t* cu_tokens,
                           const int64_t* pos0, const void* k, const void* v, const float* idx,
                           void* stream) {
  if (!c) return fail(kInvalid, "NULL context");
  std::string why;
  int st = c->ctl.check_state_write(n_req, states, cu_tokens, pos0, &why);
  if (st) return fail(st, why);
  if (n_req == 0 || cu_tokens[n_req] == 0) return kOk;
  if (!k || !v || (!idx && c->P.c4)) return fail(kInvalid, "input pointer is NULL");
  if ((st = set_device(c))) return st;
  std::vector<WriteDesc> writes;
  int64_t total = 0;
  for (int32_t i = 0; i < n_req; ++i) {
    const int64_t n = cu_tokens[i + 1] - cu_tokens[i];
    const int32_t s = states[i];
    const int64_t L = c->ctl.len(s);
    const int64_t w0 = std::max(pos0[i], L - (int64_t)c->P.n_win);   // older positions are dropped
    if (n == 0 || w0 >= pos0[i] + n) continue;
    writes.push_back(WriteDesc{s, (int32_t)c->ctl.n_blocks(s), pos0[i], pos0[i] + n, w0, cu_tokens[i], total});
    total += pos0[i] + n - w0;
  }
  if (writes.empty()) return kOk;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  st = upload_plan(c, writes.data(), writes.size() * sizeof(WriteDesc), hs);
  if (st) return st;
  Timed t(c, HSA_KERNEL_WRITE, hs);
  HIP_TRY(launch_bulk_write(c->P, static_cast<const WriteDesc*>(c->plan_dev), (int32_t)writes.size(), total,
                            k, v, idx, hs, t.ev()));
  return recompute_open(c, states, n_req, hs);   // eager C4: entries of the replayed groups
}

hsa_status hsa_checkpoint_bytes(hsa_ctx* c, int64_t* bytes) {
  if (!c || !bytes) return fail(kInvalid, "NULL argument");
  RingPart rp[2];
  ring_parts(c->P, rp);
  *bytes = (int64_t)c->P.n_win * (int64_t)(rp[0].row + rp[1].row) + (int64_t)kBlk * kIRow * 4;
  return kOk;
}

hsa_status hsa_state_checkpoint(hsa_ctx* c, int32_t s_, void* buf, int64_t* len_out, void* stream) {
  if (!c) return fail(kInvalid, "NULL context");
  if (!c->ctl.valid_state(s_)) return fail(kInvalid, "state not allocated");
  if (!buf || !len_out) return fail(kInvalid, "NULL argument");
  if (c->ctl.pending(s_)) return fail(kState, "the state has a pending seal");
  int st = set_device(c);
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t L = c->ctl.len(s_), W = c->P.n_win, tail = L - kBlk * c->ctl.n_blocks(s_);
  const int64_t slots = std::min(L, W);
  char* b = static_cast<char*>(buf);
  const size_t S = (size_t)s_;
  RingPart rp[2];
  ring_parts(c->P, rp);
  size_t at = 0;   // the parts' rows, n_win of each, then the tail
  for (const RingPart& q : rp) {
    if (slots > 0)
      HIP_TRY(hipMemcpyAsync(b + at, q.base + S * W * q.row, (size_t)slots * q.row, hipMemcpyDefault, s));
    at += (size_t)W * q.row;
  }
  if (tail > 0 && c->P.c4)
    HIP_TRY(hipMemcpyAsync(b + at, c->P.idx_tail + S * kBlk * kIRow, (size_t)tail * kIRow * 4,
                           hipMemcpyDefault, s));
  *len_out = L;
  return kOk;
}

hsa_status hsa_state_restore(hsa_ctx* c, int32_t s_, const void* buf, int64_t ckpt_len, void* stream) {
  if (!c) return fail(kInvalid, "NULL context");
  if (!c->ctl.valid_state(s_)) return fail(kInvalid, "state not allocated");
  if (!buf) return fail(kInvalid, "NULL buffer");
  if (ckpt_len < 0 || ckpt_len > c->ctl.len(s_)) return fail(kInvalid, "checkpoint is past the state's length");
  int st = set_device(c);
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t W = c->P.n_win, slots = std::min(ckpt_len, W), tail = ckpt_len % kBlk;
  const char* b = static_cast<const char*>(buf);
  const size_t S = (size_t)s_;
  RingPart rp[2];
  ring_parts(c->P, rp);
  size_t at = 0;
  for (const RingPart& q : rp) {
    if (slots > 0)
      HIP_TRY(hipMemcpyAsync(q.base + S * W * q.row, b + at, (size_t)slots * q.row, hipMemcpyDefault, s));
    at += (size_t)W * q.row;
  }
  if (tail > 0 && c->P.c4)
    HIP_TRY(hipMemcpyAsync(c->P.idx_tail + S * kBlk * kIRow, b + at, (size_t)tail * kIRow * 4,
                           hipMemcpyDefault, s));
  return recompute_open(c, &s_, 1, s);   // eager C4: the open block's entries
}

hsa_status hsa_state_restore_batch(hsa_ctx* c, int32_t n, const int32_t* states, const void* const* bufs,
                                   const int64_t* ckpt_lens, void* stream) {
  if (!c) return fail(kInvalid, "NULL context");
  if (n < 0) return fail(kInvalid, "n must be >= 0");
  if (n == 0) return kOk;
  if (!states || !bufs || !ckpt_lens) return fail(kInvalid, "NULL argument");
  int st = set_device(c);
  if (st) return st;
  std::vector<int32_t> seen(states, states + n);
  std::sort(seen.begin(), seen.end());
  if (std::adjacent_find(seen.begin(), seen.end()) != seen.end()) return fail(kInvalid, "a state appears twice");
  const int64_t W = c->P.n_win;
  RingPart rp[2];
  ring_parts(c->P, rp);
  std::vector<CopySeg> segs;
  int64_t total = 0;
  auto add = [&](const char* src, void* dst, size_t bytes) {
    if (bytes == 0) return;
    const int64_t n16 = (int64_t)(bytes / 16);
    segs.push_back(CopySeg{reinterpret_cast<const uint4*>(src), static_cast<uint4*>(dst), n16, total});
    total += (n16 + kCopyChunk16 - 1) / kCopyChunk16;
  };
  for (int32_t i = 0; i < n; ++i) {
    const int32_t s_ = states[i];
    if (!c->ctl.valid_state(s_)) return fail(kInvalid, "state not allocated");
    if (ckpt_lens[i] < 0 || ckpt_lens[i] > c->ctl.len(s_))
      return fail(kInvalid, "checkpoint is past the state's length");
    if (!bufs[i] || reinterpret_cast<uintptr_t>(bufs[i]) % 16 != 0)
      return fail(kInvalid, "checkpoint buffer is NULL or not 16-byte aligned");
    // the kernel reads the buffer: device memory, or pinned host memory through its
    // device address
    hipPointerAttribute_t a{};
    if (hipPointerGetAttributes(&a, bufs[i]) != hipSuccess) {
      (void)hipGetLastError();
      return fail(kInvalid, "checkpoint buffer is not device or pinned host memory");
    }
    const char* b = nullptr;
    if (a.type == hipMemoryTypeDevice || a.type == hipMemoryTypeManaged) b = static_cast<const char*>(bufs[i]);
    else if (a.type == hipMemoryTypeHost && a.devicePointer)
      b = static_cast<const char*>(a.devicePointer) +
          (static_cast<const char*>(bufs[i]) - static_cast<const char*>(a.hostPointer));
    if (!b) return fail(kInvalid, "checkpoint buffer is not device or pinned host memory");
    const int64_t slots = std::min<int64_t>(ckpt_lens[i], W), tail = ckpt_lens[i] % kBlk;
    const size_t S = (size_t)s_;
    size_t at = 0;
    for (const RingPart& q : rp) {
      add(b + at, q.base + S * W * q.row, (size_t)slots * q.row);
      at += (size_t)W * q.row;
    }
    if (tail > 0 && c->P.c4) add(b + at, c->P.idx_tail + S * kBlk * kIRow, (size_t)tail * kIRow * 4);
  }
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (!segs.empty()) {
    if (segs.size() > (size_t)INT32_MAX) return fail(kInvalid, "too many states");
    st = upload_plan(c, segs.data(), segs.size() * sizeof(CopySeg), hs);
    if (st) return st;
    HIP_TRY(launch_copy_segs(static_cast<const CopySeg*>(c->plan_dev), (int32_t)segs.size(), total, hs));
  }
  return recompute_open(c, states, n, hs);   // eager C4: the open blocks' entries
}

hsa_status hsa_indexer_topk(hsa_ctx* c, int32_t n_req, const int32_t* states, const float* q_idx,
                            int32_t k, uint32_t flags, int32_t* idx_out, float* score_out,
                            void* stream) {
  if (!c) return fail(kInvalid, "NULL context");
  std::string why;
  int st = c->ctl.check_states(n_req, states, false, false, &why);
  if (st) return fail(st, why);
  if (k < 1 || k > HSA_MAX_TOPK) return fail(kInvalid, "k must be in [1, 4096]");
  if (flags & ~HSA_TOPK_SORTED) return fail(kInvalid, "unknown flags");
  if (n_req > 0 && (!q_idx || !idx_out)) return fail(kInvalid, "NULL device pointer");
  if (n_req == 0) return kOk;
  if ((st = set_device(c))) return st;
  return run_topk(c, n_req, states, q_idx, k, flags, idx_out, score_out,
                  static_cast<hipStream_t>(stream));
}

hsa_status hsa_decode_attend(hsa_ctx* c, int32_t n_req, const int32_t* states, const void* q,
                             const int32_t* topk, int32_t k, float* out, void* stream) {
  if (!c) return fail(kInvalid, "NULL context");
  std::string why;
  int st = c->ctl.check_states(n_req, states, false, true, &why);
  if (st) return fail(st, why);
  if (k < 0 || k > HSA_MAX_TOPK) return fail(kInvalid, "k must be in [0, 4096]");
  if (k > 0 && !topk) return fail(kInvalid, "topk is NULL with k > 0");
  if (n_req > 0 && (!q || !out)) return fail(kInvalid, "NULL device pointer");
  if (n_req == 0) return kOk;
  if ((st = set_device(c))) return st;
  return run_attend(c, n_req, states, q, k > 0 ? topk : nullptr, k, out,
                    static_cast<hipStream_t>(stream));
}

namespace {

// hsa_decode_step and hsa_decode_step_noalloc: with `noalloc`, every kernel's scratch
// comes from the fixed buffer, which must hold the step's largest batch (checked
// before anything changes), and no device memory is allocated.
int decode_step_impl(hsa_ctx* c, int32_t n_req, const int32_t* states, const void* k_new,
                     const void* v_new, const float* idx_new, const void* q, const float* q_idx,
                     int32_t k, uint32_t flags, int32_t* topk_out, float* score_out, float* out,
                     void* stream, bool noalloc) {
  if (!c) return fail(kInvalid, "NULL context");
  if (n_req < 0) return fail(kInvalid, "n_req < 0");
  if (n_req == 0) return kOk;
  if (k < 1 || k > HSA_MAX_TOPK) return fail(kInvalid, "k must be in [1, 4096]");
  if (flags & ~HSA_TOPK_SORTED) return fail(kInvalid, "unknown flags");
  if (!k_new || !v_new || (c->P.c4 && (!idx_new || !q_idx)) || !q || !topk_out || !out)
    return fail(kInvalid, "NULL device pointer");
  if (noalloc && !c->fixed) return fail(kDevice, "the fixed scratch buffer was not found");
  bool replay = false;
  int st = layer_gate(c, kSeqStep, n_req, states, nullptr, 0, &replay);
  if (st) return st;
  AppendPlan fresh;
  if (!replay) {
    std::vector<int64_t> cu(n_req + 1);
    for (int32_t i = 0; i <= n_req; ++i) cu[i] = i;
    std::string why;
    st = c->ctl.plan_append(n_req, states, cu.data(), false, &fresh, &why);
    if (st) return fail(st, why);
  }
  const AppendPlan& plan = replay ? c->seq.plan : fresh;
  if (noalloc) {
    const size_t need = step_fixed_need(c, plan, k, flags);
    if (need > kNoAllocScratchBytes)
      return fail(kInvalid, "the step needs " + std::to_string(need) + " bytes of scratch; the fixed buffer holds " +
                                std::to_string(kNoAllocScratchBytes));
  }
  if ((st = set_device(c))) return st;
  if (replay) {
    layer_advance(c);
  } else {
    c->ctl.commit(&fresh);
    layer_record(c, kSeqStep, n_req, states, nullptr, 0, fresh);
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (!noalloc)
    return run_decode_step(c, plan, k_new, v_new, idx_new, q, q_idx, k, flags, topk_out, score_out, out, s);
  const uint32_t tmask = c->tmask;   // no timing events either
  c->tmask = 0;
  st = run_decode_step(c, plan, k_new, v_new, idx_new, q, q_idx, k, flags, topk_out, score_out, out, s,
                       static_cast<char*>(c->fixed));
  c->tmask = tmask;
  return st;
}

}  // namespace

hsa_status hsa_decode_step(hsa_ctx* c, int32_t n_req, const int32_t* states, const void* k_new,
                           const void* v_new, const float* idx_new, const void* q,
                           const float* q_idx, int32_t k, uint32_t flags, int32_t* topk_out,
                           float* score_out, float* out, void* stream) {
  return decode_step_impl(c, n_req, states, k_new, v_new, idx_new, q, q_idx, k, flags, topk_out,
                          score_out, out, stream, false);
}

hsa_status hsa_decode_step_noalloc(hsa_ctx* c, int32_t n_req, const int32_t* states,
                                   const void* k_new, const void* v_new, const float* idx_new,
                                   const void* q, const float* q_idx, int32_t k, uint32_t flags,
                                   int32_t* topk_out, float* score_out, float* out, void* stream) {
  return decode_step_impl(c, n_req, states, k_new, v_new, idx_new, q, q_idx, k, flags, topk_out,
                          score_out, out, stream, true);
}

hsa_status hsa_noalloc_scratch_bytes(int64_t* bytes) {
  if (!bytes) return fail(kInvalid, "NULL argument");
  *bytes = (int64_t)kNoAllocScratchBytes;
  return kOk;
}

hsa_status hsa_set_layer(hsa_ctx* c, int32_t layer) {
  if (!c) return fail(kInvalid, "NULL context");
  if (layer < 0 || layer >= (int32_t)c->layers.size()) return fail(kInvalid, "no such layer");
  c->cur_layer = layer;
  c->P = c->layers[layer];
  return kOk;
}

hsa_status hsa_state_query(hsa_ctx* c, int32_t s, hsa_state_info* out) {
  if (!c || !out) return fail(kInvalid, "NULL argument");
  if (!c->ctl.valid_state(s)) return fail(kInvalid, "state not allocated");
  const int64_t L = c->ctl.len(s), nb = c->ctl.n_blocks(s);
  out->len = L;
  out->n_blocks = nb;
  out->csa_tail = (int32_t)(L % 4);
  out->hca_tail = (int32_t)(L - kBlk * nb);
  out->swa_len = (int32_t)std::min<int64_t>(L, c->P.n_win);
  out->pending_seal = c->ctl.pending(s) ? 1 : 0;
  return kOk;
}

hsa_status hsa_block_table_get(hsa_ctx* c, int32_t s, int32_t* ids, int64_t cap, int64_t* n) {
  if (!c || !n) return fail(kInvalid, "NULL argument");
  if (!c->ctl.valid_state(s)) return fail(kInvalid, "state not allocated");
  const auto& t = c->ctl.table(s);
  *n = (int64_t)t.size();
  if (ids) std::copy(t.begin(), t.begin() + std::min<int64_t>(cap, *n), ids);
  return kOk;
}

hsa_status hsa_block_refcount(hsa_ctx* c, int32_t b, int32_t* rc) {
  if (!c || !rc) return fail(kInvalid, "NULL argument");
  if (!c->ctl.valid_block(b)) return fail(kInvalid, "no such block");
  *rc = c->ctl.refcount(b);
  return kOk;
}

hsa_status hsa_export_block(hsa_ctx* c, int32_t b, void* csa_k, void* csa_v, void* hca_k,
                            void* hca_v, float* idx_k, void* stream) {
  if (!c) return fail(kInvalid, "NULL context");
  if (!c->ctl.valid_block(b) || c->ctl.refcount(b) == 0) return fail(kInvalid, "block not in use");
  int st = set_device(c);
  if (st) return st;
  if (c->P.fp8 && (csa_k || csa_v)) return fail(kInvalid, "FP8 entries: export them with hsa_export_c4_fp8");
  if (c->P.mx4 && idx_k) return fail(kInvalid, "MXFP4 indexer keys: export them with hsa_export_idx_mxfp4");
  if (!c->P.c4 && (csa_k || csa_v || idx_k)) return fail(kInvalid, "this layer keeps no C4 entries or indexer keys");
  if (!c->P.hca && (hca_k || hca_v)) return fail(kInvalid, "this layer keeps no HCA entries");
  if (c->P.kv8 && (hca_k || hca_v)) return fail(kInvalid, "HCA entries are FP8: use hsa_export_hca_fp8");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t B = (size_t)b;
  if (csa_k) HIP_TRY(hipMemcpyAsync(csa_k, c->P.csa_k + B * kC4 * kRow, kC4 * kRow * 2, hipMemcpyDeviceToHost, s));
  if (csa_v) HIP_TRY(hipMemcpyAsync(csa_v, c->P.csa_v + B * kC4 * kRow, kC4 * kRow * 2, hipMemcpyDeviceToHost, s));
  if (hca_k) HIP_TRY(hipMemcpyAsync(hca_k, c->P.hca_k + B * kRow, kRow * 2, hipMemcpyDeviceToHost, s));
  if (hca_v) HIP_TRY(hipMemcpyAsync(hca_v, c->P.hca_v + B * kRow, kRow * 2, hipMemcpyDeviceToHost, s));
  if (idx_k) HIP_TRY(hipMemcpyAsync(idx_k, c->P.idx_k + B * kBlk * kIRow, kBlk * kIRow * 4, hipMemcpyDeviceToHost, s));
  HIP_TRY(hipStreamSynchronize(s));
  return kOk;
}

hsa_status hsa_export_c4_fp8(hsa_ctx* c, int32_t b, uint8_t* codes_k, uint8_t* codes_v,
                             float* scale_k, float* scale_v, void* stream) {
  if (!c) return fail(kInvalid, "NULL context");
  if (!c->P.fp8) return fail(kInvalid, "the context stores bf16 entries");
  if (!c->P.c4) return fail(kInvalid, "this layer keeps no C4 entries");
  if (!c->ctl.valid_block(b) || c->ctl.refcount(b) == 0) return fail(kInvalid, "block not in use");
  int st = set_device(c);
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint8_t* q = c->P.c4q + (size_t)b * kC4 * kC4Bytes;
  if (codes_k) HIP_TRY(hipMemcpy2DAsync(codes_k, kRow, q, kC4Bytes, kRow, kC4, hipMemcpyDeviceToHost, s));
  if (codes_v) HIP_TRY(hipMemcpy2DAsync(codes_v, kRow, q + kRow, kC4Bytes, kRow, kC4, hipMemcpyDeviceToHost, s));
  std::vector<float> sc((size_t)kC4 * kC4Scales);
  HIP_TRY(hipMemcpyAsync(sc.data(), c->P.c4s + (size_t)b * kC4 * kC4Scales, sc.size() * 4,
                         hipMemcpyDeviceToHost, s));
  HIP_TRY(hipStreamSynchronize(s));
  for (int e = 0; e < kC4; ++e)
    for (int h = 0; h < kH; ++h) {   // stored at 4 (h % 4) + h / 4 (the attention lane order)
      const int hp = 4 * (h % 4) + h / 4;
      if (scale_k) scale_k[e * kH + h] = sc[(size_t)e * kC4Scales + hp];
      if (scale_v) scale_v[e * kH + h] = sc[(size_t)e * kC4Scales + kH + hp];
    }
  return kOk;
}

hsa_status hsa_export_idx_mxfp4(hsa_ctx* c, int32_t b, uint8_t* codes, uint8_t* scales, void* stream) {
  if (!c) return fail(kInvalid, "NULL context");
  if (!c->P.mx4) return fail(kInvalid, "the context stores fp32 indexer keys");
  if (!c->P.c4) return fail(kInvalid, "this layer keeps no indexer keys");
  if (!c->ctl.valid_block(b) || c->ctl.refcount(b) == 0) return fail(kInvalid, "block not in use");
  int st = set_device(c);
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t R = (size_t)b * kBlk;
  if (codes) HIP_TRY(hipMemcpyAsync(codes, c->P.idx_q + R * kIRowQ, kBlk * kIRowQ, hipMemcpyDeviceToHost, s));
  if (scales) HIP_TRY(hipMemcpyAsync(scales, c->P.idx_e + R * kIRowE, kBlk * kIRowE, hipMemcpyDeviceToHost, s));
  HIP_TRY(hipStreamSynchronize(s));
  return kOk;
}

hsa_status hsa_mxfp4_quantize_rows(const float* x, int64_t n_rows, uint8_t* codes, uint8_t* scales,
                                   void* stream) {
  if (n_rows < 0 || n_rows > (int64_t(1) << 32)) return fail(kInvalid, "n_rows out of range");
  if (n_rows == 0) return kOk;
  if (!x || !codes || !scales) return fail(kInvalid, "NULL buffer");
  HIP_TRY(launch_mx4_rows(x, n_rows, codes, scales, static_cast<hipStream_t>(stream)));
  return kOk;
}

hsa_status hsa_fp8_quantize_rows(const float* x, int64_t n_rows, uint8_t* codes, float* scales,
                                 void* stream) {
  if (n_rows < 0 || n_rows > (int64_t(1) << 34)) return fail(kInvalid, "n_rows out of range");
  if (n_rows == 0) return kOk;
  if (!x || !codes || !scales) return fail(kInvalid, "NULL buffer");
  HIP_TRY(launch_fp8_rows(x, n_rows, codes, scales, static_cast<hipStream_t>(stream)));
  return kOk;
}

hsa_status hsa_export_state(hsa_ctx* c, int32_t s_, void* swa_k, void* swa_v, float* idx_tail,
                            void* stream) {
  if (!c) return fail(kInvalid, "NULL context");
  if (!c->ctl.valid_state(s_)) return fail(kInvalid, "state not allocated");
  if (idx_tail && !c->P.c4) return fail(kInvalid, "this layer keeps no indexer tail");
  int st = set_device(c);
  if (st) return st;
  if (c->P.kv8 && (swa_k || swa_v)) return fail(kInvalid, "the ring is FP8: use hsa_export_state_fp8");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t W = (size_t)c->P.n_win, S = (size_t)s_;
  if (swa_k) HIP_TRY(hipMemcpyAsync(swa_k, c->P.swa_k + S * W * kRow, W * kRow * 2, hipMemcpyDeviceToHost, s));
  if (swa_v) HIP_TRY(hipMemcpyAsync(swa_v, c->P.swa_v + S * W * kRow, W * kRow * 2, hipMemcpyDeviceToHost, s));
  if (idx_tail)
    HIP_TRY(hipMemcpyAsync(idx_tail, c->P.idx_tail + S * kBlk * kIRow, kBlk * kIRow * 4, hipMemcpyDeviceToHost, s));
  HIP_TRY(hipStreamSynchronize(s));
  return kOk;
}

namespace {
// n rows of FP8 scales as stored (head h at 4 (h % 4) + h / 4, K then V) to head order.
void scales_to_heads(const float* in, int64_t n, float* out) {
  for (int64_t r = 0; r < n; ++r)
    for (int h = 0; h < kH; ++h) {
      const int hp = 4 * (h % 4) + h / 4;
      out[r * kC4Scales + h] = in[r * kC4Scales + hp];
      out[r * kC4Scales + kH + h] = in[r * kC4Scales + kH + hp];
    }
}
}  // namespace

hsa_status hsa_export_state_fp8(hsa_ctx* c, int32_t s_, uint8_t* codes, float* scales, void* stream) {
  if (!c) return fail(kInvalid, "NULL context");
  if (!c->P.kv8) return fail(kInvalid, "the ring is bf16");
  if (!c->ctl.valid_state(s_)) return fail(kInvalid, "state not allocated");
  int st = set_device(c);
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t W = (size_t)c->P.n_win, g0 = (size_t)s_ * W;
  if (codes) HIP_TRY(hipMemcpyAsync(codes, c->P.swq + g0 * kC4Bytes, W * kC4Bytes, hipMemcpyDeviceToHost, s));
  std::vector<float> sc(W * kC4Scales);
  if (scales)
    HIP_TRY(hipMemcpyAsync(sc.data(), c->P.sws + g0 * kC4Scales, sc.size() * 4, hipMemcpyDeviceToHost, s));
  HIP_TRY(hipStreamSynchronize(s));
  if (scales) scales_to_heads(sc.data(), (int64_t)W, scales);
  return kOk;
}

hsa_status hsa_export_hca_fp8(hsa_ctx* c, int32_t b, uint8_t* codes, float* scales, void* stream) {
  if (!c) return fail(kInvalid, "NULL context");
  if (!c->P.kv8) return fail(kInvalid, "HCA entries are bf16");
  if (!c->P.hca) return fail(kInvalid, "this layer keeps no HCA entries");
  if (!c->ctl.valid_block(b) || c->ctl.refcount(b) == 0) return fail(kInvalid, "block not in use");
  int st = set_device(c);
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (codes) HIP_TRY(hipMemcpyAsync(codes, c->P.hcq + (size_t)b * kC4Bytes, kC4Bytes, hipMemcpyDeviceToHost, s));
  float sc[kC4Scales];
  if (scales) HIP_TRY(hipMemcpyAsync(sc, c->P.hcs + (size_t)b * kC4Scales, sizeof(sc), hipMemcpyDeviceToHost, s));
  HIP_TRY(hipStreamSynchronize(s));
  if (scales) scales_to_heads(sc, 1, scales);
  return kOk;
}

hsa_status hsa_timing_enable(hsa_ctx* c, uint32_t mask) {
  if (!c) return fail(kInvalid, "NULL context");
  c->tmask = mask;
  return kOk;
}

hsa_status hsa_timing_read(hsa_ctx* c, double* ms, int64_t* launches) {
  if (!c) return fail(kInvalid, "NULL context");
  for (int i = 0; i < HSA_KERNEL_COUNT; ++i) {
    if (ms) ms[i] = 0.0;
    if (launches) launches[i] = 0;
  }
  for (auto& r : c->recs) {
    HIP_TRY(hipEventSynchronize(r.b));
    float t = 0.f;
    HIP_TRY(hipEventElapsedTime(&t, r.a, r.b));
    if (ms) ms[r.kid] += t;
    if (launches) launches[r.kid] += 1;
    c->ev_free.push_back(r.a);
    c->ev_free.push_back(r.b);
  }
  c->recs.clear();
  return kOk;
}

const char* hsa_status_str(hsa_status s) {
  switch (s) {
    case HSA_OK: return "ok";
    case HSA_ERR_INVALID: return "invalid argument";
    case HSA_ERR_OOM_BLOCKS: return "Block Cache full";
    case HSA_ERR_OOM_STATES: return "no free State slot";
    case HSA_ERR_STATE: return "lifecycle error";
    case HSA_ERR_DEVICE: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* hsa_last_error(void) { return g_err.c_str(); }

}  // extern "C"
