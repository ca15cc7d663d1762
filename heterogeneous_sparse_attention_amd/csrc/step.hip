// step.hip - the decode step of the heterogeneous KV cache (hsa_decode_step) in
// three or four launches.
//
// Pages: [Q&A] "V4 为何要分池？块对齐与尾缓冲怎么配合？" §4: a new token goes to the
// tail, a full block is compressed into the Classical pool, the SWA slides, and
// attention reads the compressed entries plus the exact State. The work of one
// step, for every request of the batch:
//
//   S1  append the token (ring + indexer tail), seal a full block (C4 entries,
//       indexer keys, sixteen HCA partials) and indexer scores of every sealed
//       block. Nothing read in S1 is written in S1: the new token is read from
//       the input wherever it is needed (last indexer key of a block sealed now,
//       last token of the seal).
//   S2  the HCA merge of blocks sealed in S1, the top-k over the scores, and
//       attention. Part A of the keys (the SWA tokens and the HCA entries of
//       blocks sealed before this step) needs no top-k; part B (the selected C4
//       entries, and the HCA entry of the block sealed now) does.
//   S4  log-sum-exp merge of every request's attention partials.
//
// Three-launch form (every score row fits the selection's LDS cache, top-k in
// ordinal order): each mixed S2 workgroup takes a share of part B of one request
// and the part-A keys its waves can prefetch (the last of the request's part-A
// list); it loads the request's score row, starts loading those part-A keys, runs
// the top-k itself from LDS and then streams its keys. Part-A workgroups in the
// same launch stream the rest of the part-A keys meanwhile. S4 also takes the HCA
// entry of the block sealed now as one more key.
// Four-launch form (long rows, or sorted top-k output): S2 runs the selections
// (one workgroup per row, or per slice of a long row with a second round in
// S2b) beside part A; S3 attends part B through the physical C4 rows S2 wrote.
//
// Key order differs from hsa_decode_attend only in the order of the softmax sum.
#include <algorithm>

#include "attn_dev.h"
#include "device.h"
#include "kernels.h"
#include "score_dev.h"
#include "seal_dev.h"

namespace hsa {

namespace {

__device__ __forceinline__ int sealed_now(const Req& r) { return r.aux >= 0 ? 1 : 0; }
// Part-A keys: the SWA tokens and, in layers with HCA entries, the HCA entries of
// blocks sealed before this step.
__device__ __forceinline__ int keys_a(const Pools& P, const Req& r) {
  return (r.len < P.n_win ? r.len : P.n_win) + (P.hca ? r.nb - sealed_now(r) : 0);
}
// Part-B keys: the selected C4 entries (layers with C4 entries), and in the
// four-launch form the HCA entry of the block sealed now (layers with HCA entries;
// the three-launch form takes that key in the merge).
__device__ __forceinline__ int keys_b(const Pools& P, const Req& r, int32_t k, int32_t fused) {
  const int nc = c4_cands(P.c4, P.eager, r);
  return (fused || !P.hca ? 0 : sealed_now(r)) + (k < nc ? k : nc);
}

// Eager C4: the open block's unit (lb == R.nb): keys from the indexer tail, the
// newest token's from the input; entries past the block's complete groups score -inf.
__device__ __forceinline__ void score_open_unit(const Pools& P, const ReqBatch& B, const StepArgs& S,
                                                int r, int t0) {
  const Req R = B.r[r];
  float* out = S.scores + (int64_t)r * S.ld + (int64_t)kC4 * R.nb + t0 / 4;
  const float* tail = P.idx_tail + (int64_t)R.state * kBlk * kIRow;
  const float* inrow = S.iin + (int64_t)r * kIRow;
  const int newest = R.len - 1 - kBlk * R.nb;   // the input token's slot in the block
  score_block<8 / kScoreSplit>([&](int t) { return t0 + t == newest ? inrow : tail + (t0 + t) * kIRow; },
                               S.qi + (int64_t)r * kIRow, out, open_groups(1, R) - t0 / 4);
}

// Indexer scores of scoring unit `unit` (fp32 keys): 128 / kScoreSplit tokens of one
// sealed block.
__device__ __forceinline__ void score_unit(const Pools& P, const ReqBatch& B, const StepArgs& S,
                                           int unit) {
  constexpr int kTok = kBlk / kScoreSplit;   // tokens per scoring unit
  const int r = owner_of(S.first_s, B.n, unit);
  const int u = unit - S.first_s[r];
  const int lb = u / kScoreSplit;
  const int t0 = kTok * (u % kScoreSplit);
  const Req R = B.r[r];
  if (lb == R.nb) {   // eager C4: the open block
    score_open_unit(P, B, S, r, t0);
    return;
  }
  float* out = S.scores + (int64_t)r * S.ld + (int64_t)kC4 * lb + t0 / 4;
  const float* qrow = S.qi + (int64_t)r * kIRow;
  if (R.aux >= 0 && lb == R.nb - 1) {
    // the block sealed in this step: keys from the indexer tail, the newest from
    // the input (its tail slot is being written in this launch)
    const float* tail = P.idx_tail + (int64_t)R.state * kBlk * kIRow;
    const float* inrow = S.iin + (int64_t)r * kIRow;
    score_block<8 / kScoreSplit>(
        [&](int t) { return t0 + t == kBlk - 1 ? inrow : tail + (t0 + t) * kIRow; }, qrow, out);
  } else {
    const int32_t id = P.table[(int64_t)R.state * P.table_stride + lb];
    if (id < 0 || id >= P.max_blocks) {   // never taken: tables are written before use
      if (threadIdx.x < kTok / 4) out[threadIdx.x] = -INFINITY;
      return;
    }
    const float* blk = P.idx_k + ((int64_t)id * kBlk + t0) * kIRow;
    score_block<8 / kScoreSplit>([&](int t) { return blk + t * kIRow; }, qrow, out);
  }
}


// Indexer scores of scoring unit `unit` with MXFP4 keys: stored blocks
// [u G, u G + G) of one request (G = S.mx_unit), kMxPass blocks' loads in flight at
// a time. A block sealed in this step (the request's last) has kMxRawSplit units of
// its own after them, each scoring 32 of its tokens from the fp32 tail and the input,
// quantised as the seal stores them.
__device__ __forceinline__ void score_unit_mx(const Pools& P, const ReqBatch& B, const StepArgs& S,
                                              int unit) {
  const int r = owner_of(S.first_s, B.n, unit);
  const Req R = B.r[r];
  const int nst = R.aux >= 0 ? R.nb - 1 : R.nb;   // stored blocks
  const int u = unit - S.first_s[r];
  const int nsu = (nst + S.mx_unit - 1) / S.mx_unit;
  const float* qrow = S.qi + (int64_t)r * kIRow;
  if (u >= nsu) {
    constexpr int kTok = kBlk / kMxRawSplit;
    const int t0 = (u - nsu) * kTok;
    const float* tail = P.idx_tail + (int64_t)R.state * kBlk * kIRow;
    const float* inrow = S.iin + (int64_t)r * kIRow;
    score_block_mx_raw<kTok / 32>(
        [&](int t) { return t0 + t == kBlk - 1 ? inrow : tail + (int64_t)(t0 + t) * kIRow; }, qrow,
        S.scores + (int64_t)r * S.ld + (int64_t)kC4 * nst + t0 / 4);
    return;
  }
  const int lb0 = u * S.mx_unit;
  const int lbs = min(lb0 + S.mx_unit, nst);   // stored blocks [lb0, lbs) of this unit
  float* out = S.scores + (int64_t)r * S.ld + (int64_t)kC4 * lb0;
  const int32_t* tab = P.table + (int64_t)R.state * P.table_stride;
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int b = lane & 7;
#pragma unroll 1
  for (int p = 0; lb0 + p < lbs; p += kMxPass) {
    uint4 w[kMxPass][4];
    int e[kMxPass][4];
    bool ok[kMxPass];
    // Every load is unconditional: a slot past the stored blocks reads the pass's
    // last stored block again, an invalid id (never written) block 0. A load inside
    // a branch makes the compiler wait for every load in flight where the branch
    // joins, which would serialise the pass into one round trip per load.
    int32_t ids[kMxPass];   // all of the pass's ids first: one round trip, not one per block
#pragma unroll
    for (int j = 0; j < kMxPass; ++j) ids[j] = tab[min(lb0 + p + j, lbs - 1)];
#pragma unroll
    for (int j = 0; j < kMxPass; ++j) {
      const int lb = lb0 + p + j;
      const int32_t id = ids[j];
      const bool valid = id >= 0 && id < P.max_blocks;
      ok[j] = lb < lbs && valid;
      const int64_t kr = (int64_t)(valid ? id : 0) * kBlk;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t t = kr + (wave * 4 + g) * 8 + (lane >> 3);
        w[j][g] = load_stream(reinterpret_cast<const uint4*>(P.idx_q + t * kIRowQ) + b);
        e[j][g] = (int)P.idx_e[t * kIRowE + b];
      }
    }
    // the query after the keys (read again each pass), so its round trip overlaps theirs
    float q[32];
    mx_load_q(qrow, b, q);
#pragma unroll
    for (int j = 0; j < kMxPass; ++j) {
      const int lb = lb0 + p + j;
      if (lb >= lbs) continue;
      float* o = out + kC4 * (p + j);
      if (!ok[j]) {
        if (threadIdx.x < kC4) o[threadIdx.x] = -INFINITY;
        continue;
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) mx_write_pair(mx_dot(w[j][g], e[j][g] - 127, q), o + 2 * (wave * 4 + g));
    }
  }
}

// FP8 entries: the seal's quantisation needs more registers than 4 workgroups per
// CU leave, so that instance runs 3 per CU; the bf16 instance keeps 4.
// (C4 false: a layer without C4 entries, whose seal keeps only the HCA partial)
// (KV8: FP8 KV, whose seal reads codes and scales from the ring)
template <bool FP8, bool C4, bool KV8>
__global__ __launch_bounds__(256, FP8 || KV8 ? 3 : 4) void k_step1(Pools P, ReqBatch B, StepArgs S) {
  int bid = blockIdx.x;
  // -- seal pieces (first, so the longest single workgroups start early)
  if (bid < kSealSplit * B.n_seal) {
    const int item = bid / kSealSplit;
    const int ri = B.seal_req[item];
    seal_piece<FP8, C4, KV8>(P, B.r[ri], ri, item, bid % kSealSplit, S.kin, S.vin, S.iin, S.seal_part);
    return;
  }
  bid -= kSealSplit * B.n_seal;
  // -- append
  if (bid < B.n) {
    append_token<C4>(P, B.r[bid], bid, S.kin, S.vin, S.iin);
    return;
  }
  bid -= B.n;
  // -- eager C4: the entry of the open block's group this token completes
  if (bid < B.n_open) {
    const int ri = B.open_req[bid];
    const Req R = B.r[ri];
    open_entry(P, R.state, R.nb, open_groups(1, R) - 1, R.len - 1, S.kin + (int64_t)ri * kRow,
               S.vin + (int64_t)ri * kRow);
    return;
  }
  bid -= B.n_open;
  // -- indexer scores, one workgroup per unit (a 1/kScoreSplit block of fp32 keys,
  //    or S.mx_unit blocks of MXFP4 keys); a layer without C4 entries scores nothing
  if constexpr (C4) {
    if (bid < S.n_score) {
      if (P.mx4)
        score_unit_mx(P, B, S, bid);
      else
        score_unit(P, B, S, bid);
    }
  }
}


// Attention part A (SWA tokens + HCA of blocks sealed before this step) of chunk
// `bid`, over the request's part-A keys [0, a_split): it needs no top-k, so it runs
// beside the selection.
template <int WAVES, bool KV8, int RING = ring_depth<WAVES>()>
__device__ __forceinline__ void part_a(const Pools& P, const ReqBatch& B, const StepArgs& S, int bid,
                                       AttnSharedT<WAVES>& sh) {
  const int r = owner_of(S.first_a, B.n, bid);
  const int w = bid - S.first_a[r];
  const int nch = S.first_a[r + 1] - S.first_a[r];
  const Req R = B.r[r];
  const int swa = R.len < P.n_win ? R.len : P.n_win;
  int x0, x1;
  chunk_range(S.a_split[r], nch, w, x0, x1);
  const int64_t g0 = (int64_t)R.state * P.n_win;   // the state's first ring slot
  const int32_t* tab = P.table + (int64_t)R.state * P.table_stride;
  const int64_t p0 = (int64_t)R.len - swa;   // oldest SWA position; the ring holds all (S1 wrote the newest)
  auto key_a = [&](int x) {
    KeyAddr a;
    a.k = a.v = nullptr;
    if (x < swa) {
      if (S.s2_append && p0 + x == R.len - 1) {   // being appended in this launch: from the input
        a.k = S.kin + (int64_t)r * kRow;          // (bf16 KV only: FP8 KV appends in S1)
        a.v = S.vin + (int64_t)r * kRow;
        return a;
      }
      const C4Addr c = ring_addr(P, g0 + (p0 + x) % P.n_win);
      a.k = c.k;
      a.v = c.v;
      return a;
    }
    const int32_t id = tab[x - swa];
    if (id < 0 || id >= P.max_blocks) return a;
    const C4Addr c = hca_addr(P, id);
    a.k = c.k;
    a.v = c.v;
    return a;
  };
  const C4Addr dm = dummy_rows(P, R.state);
  float M, L, A8[8];
  attend_keys<WAVES, RING, KV8, KV8>(key_a, x0, x1, S.q + (int64_t)r * kRow, dm.k, dm.v, sh, M, L, A8);
  if (threadIdx.x < 256) store_partial(S.part_acc, S.part_ml, bid, M, L, A8);
}

// Ring of the three-launch form's part-A workgroups, which stream while the mixed
// workgroups select: 3 keys (2 in flight per wave) measured faster than 2, 4 or 5 on
// the b32 workload.
#ifndef HSA_SPLIT_A_RING
#define HSA_SPLIT_A_RING 3
#endif
constexpr int kSplitARing = HSA_SPLIT_A_RING;

constexpr int kStep2Threads = 512;   // 8 waves: 256 VGPRs per wave for the attention role
constexpr int kStep2Waves = kStep2Threads / 64;

struct Step2Shared {
  union {
    SelShared sel;
    AttnSharedT<kStep2Waves> attn;
  };
  int32_t rows[kCacheN];   // three-launch part B: physical C4 rows of the workgroup's share
};

// Three-launch form, mixed workgroup `bid` of request r (w of nch): it attends its
// share of both of the request's key lists, part A (SWA tokens and HCA entries of
// earlier blocks: share chunk w of nch of the keys [a_split, keys_a), the rest being
// the part-A workgroups') and part B (the selected C4 entries, same share of the
// selection), in one online softmax. It first loads the request's scores (at
// most kCacheN, into registers) and issues its first part-A key loads, then runs the
// top-k itself from LDS while those loads are in flight: it keeps in LDS the
// physical C4 rows of its share [b0, b1) of the selection and writes the same share
// of the top-k output (workgroup 0 also the padding). Every workgroup of a request
// selects from the same scores, so the shares agree.
template <int WAVES, bool KV8, bool F8>
__device__ __forceinline__ void part_mixed(const Pools& P, const ReqBatch& B, const StepArgs& S, int bid,
                                           Step2Shared& sh) {
  constexpr int NT = WAVES * 64;
  const int r = owner_of(S.first_b, B.n, bid);
  const int w = bid - S.first_b[r];
  const int nch = S.first_b[r + 1] - S.first_b[r];
  const Req R = B.r[r];
  const int N = c4_rowlen(P.c4, P.eager, R);     // score-row length
  const int nc = c4_cands(P.c4, P.eager, R);     // candidates
  const int kk = min(S.k, nc);
  int a0, a1, b0, b1;
  const int as = S.a_split[r];   // part-A keys [as, keys_a) are the mixed workgroups'
  chunk_range(keys_a(P, R) - as, nch, w, a0, a1);
  a0 += as;
  a1 += as;
  chunk_range(kk, nch, w, b0, b1);
  const int32_t* tab = P.table + (int64_t)R.state * P.table_stride;
  SelPre<NT> pre;
  sel_preload<NT>(N, S.scores + (int64_t)r * S.ld, tab, N / kC4, pre);
  __builtin_amdgcn_sched_barrier(0);   // the row's loads go out ahead of the key prefetch

  const int64_t g0 = (int64_t)R.state * P.n_win;   // the state's first ring slot
  const int swa = R.len < P.n_win ? R.len : P.n_win;
  const int64_t p0 = (int64_t)R.len - swa;
  auto key_a = [&](int x) {
    KeyAddr a;
    a.k = a.v = nullptr;
    if (x < swa) {
      const C4Addr c = ring_addr(P, g0 + (p0 + x) % P.n_win);
      a.k = c.k;
      a.v = c.v;
      return a;
    }
    const int32_t id = load_global(tab + (x - swa));
    if (id < 0 || id >= P.max_blocks) return a;   // never taken
    const C4Addr c = hca_addr(P, id);
    a.k = c.k;
    a.v = c.v;
    return a;
  };
  const int64_t max_row = (int64_t)P.c4_ids * kC4;   // blocks and (eager) open blocks
  auto key_b = [&](int x) {
    KeyAddr a;
    a.k = a.v = nullptr;
    const int64_t row = sh.rows[x - b0];
    if (row < 0 || row >= max_row) return a;   // never taken
    const C4Addr c = c4_addr(P, row);
    a.k = c.k;
    a.v = c.v;
    return a;
  };
  const int64_t k = S.k;
  // the row is staged in LDS (waiting for its loads) before the key prefetch goes
  // out, so the prefetch does not queue ahead of it
  auto stage = [&]() { select_stage<NT>(pre, sh.sel); };
  auto select = [&]() {
    select_lds<NT>(N, S.k, S.topk + r * k, S.score_out ? S.score_out + r * k : nullptr, sh.sel, sh.rows,
                   SelWin{b0, b1, w == 0}, nc);
    __syncthreads();   // rows in LDS complete; the selection's LDS is free for attention
  };
  const C4Addr dm = dummy_rows(P, R.state);
  float M, L, A8[8];
  attend_two<WAVES, kMixedRing, KV8, F8>(key_a, a0, a1, key_b, b0, b1, stage, select,
                                          S.q + (int64_t)r * kRow, dm.k, dm.v, sh.attn, M, L, A8);
  if (threadIdx.x < 256) store_partial(S.part_acc, S.part_ml, (int64_t)S.n_a + bid, M, L, A8);
}

// KV8: FP8 SWA ring and HCA entries; F8: FP8 C4 entries (the attention's key formats)
template <bool KV8, bool F8>
__global__ __launch_bounds__(kStep2Threads) void k_step2(Pools P, ReqBatch B, StepArgs S) {
  __shared__ Step2Shared sh;
  int bid = blockIdx.x;
  if (S.fused) {
    if (bid < S.n_b) {
      part_mixed<kStep2Waves, KV8, F8>(P, B, S, bid, sh);
      return;
    }
    bid -= S.n_b;
  } else {
    // a layer without C4 entries whose step seals nothing skips S1: its appends
    // come first. The slot a token is written to holds a position outside every
    // window of this step (or none), so part A's reads do not race with it.
    if (S.s2_append) {
      if (bid < B.n) {
        if (threadIdx.x < 256) append_token<false>(P, B.r[bid], bid, S.kin, S.vin, S.iin);
        return;
      }
      bid -= B.n;
    }
    if (bid < S.sel.n_wgs) {
      select_round1<kStep2Threads>(bid, B.n, B.r, S.sel, S.k, S.sorted, S.scores, S.ld, S.topk,
                                   S.score_out, sh.sel, P.table, P.table_stride, S.rows);
      return;
    }
    bid -= S.sel.n_wgs;
  }
  if (bid < B.n_seal) {   // the HCA entries of blocks sealed in S1
    if (P.hca) seal_merge(P, B.r[B.seal_req[bid]].aux, S.seal_part, bid);
    return;
  }
  bid -= B.n_seal;
  if (S.fused)
    part_a<kStep2Waves, KV8, kSplitARing>(P, B, S, bid, sh.attn);
  else
    part_a<kStep2Waves, KV8>(P, B, S, bid, sh.attn);
}

// Round 2 of the top-k of rows sliced in k_step2 (launched only when some are).
__global__ __launch_bounds__(kSelThreads) void k_step2b(Pools P, ReqBatch B, StepArgs S) {
  __shared__ SelShared sh;
  select_round2<kSelThreads>(blockIdx.x, B.r, S.sel, S.k, S.sorted, S.topk, S.score_out, sh, P.table,
                             P.table_stride, S.rows);
}

#ifndef HSA_STEP3_WAVES
#define HSA_STEP3_WAVES 4
#endif
constexpr int kStep3Waves = HSA_STEP3_WAVES;

template <bool KV8, bool F8>
__global__ __launch_bounds__(kStep3Waves * 64) void k_step3(Pools P, ReqBatch B, StepArgs S) {
  __shared__ AttnSharedT<kStep3Waves> sh;
  const int bid = blockIdx.x;
  const int r = owner_of(S.first_b, B.n, bid);
  const int w = bid - S.first_b[r];
  const int nch = S.first_b[r + 1] - S.first_b[r];
  const Req R = B.r[r];
  int x0, x1;
  chunk_range(keys_b(P, R, S.k, 0), nch, w, x0, x1);
  const int sn = P.hca ? sealed_now(R) : 0;
  const int32_t* rows = S.rows + (int64_t)r * S.k;
  const int64_t max_row = (int64_t)P.c4_ids * kC4;   // blocks and (eager) open blocks
  auto key_b = [&](int x) {
    KeyAddr a;
    a.k = a.v = nullptr;
    if (x < sn) {
      const C4Addr c = hca_addr(P, R.aux);
      a.k = c.k;
      a.v = c.v;
      return a;
    }
    const int64_t row = rows[x - sn];   // C4 row of a selected entry, from S2
    if (row < 0 || row >= max_row) return a;   // never taken
    const C4Addr c = c4_addr(P, row);
    a.k = c.k;
    a.v = c.v;
    return a;
  };
  const C4Addr dm = dummy_rows(P, R.state);   // valid rows (L >= 1)
  float M, L, A8[8];
  // the HCA entry of the block sealed now (key 0 when sn) is in the KV format
  attend_keys<kStep3Waves, ring_depth<kStep3Waves>(), KV8, F8>(key_b, x0, x1, S.q + (int64_t)r * kRow, dm.k,
                                                               dm.v, sh, M, L, A8, sn);
  if (threadIdx.x < 256) store_partial(S.part_acc, S.part_ml, (int64_t)S.n_a + bid, M, L, A8);
}

// S4: the log-sum-exp merge of each request's partials, one 512-thread workgroup per
// request, so that every head of the request costs one memory round trip when it has
// at most 32 partials (merge_partials_wg; four workgroups of one head per wave
// measured 0.2 us slower per b32 step). The HCA entry of a block sealed in this step
// joins as one more key.
__global__ __launch_bounds__(512) void k_step4(Pools P, ReqBatch B, StepArgs S) {
  const int r = blockIdx.x;
  const int fa = S.first_a[r], ca = S.first_a[r + 1] - fa;
  const int fb = S.first_b[r], cb = S.first_b[r + 1] - fb;
  const Req R = B.r[r];
  ExtraKey xk{nullptr, nullptr, nullptr, false};
  if (S.a_only)   // no C4 entries: the top-k row is padding
    for (int i = threadIdx.x; i < S.k; i += 512) {
      S.topk[(int64_t)r * S.k + i] = -1;
      if (S.score_out) S.score_out[(int64_t)r * S.k + i] = -INFINITY;
    }
  if ((S.fused || S.a_only) && R.aux >= 0 && P.hca) {   // the HCA entry of the block sealed now, merged in S2
    const C4Addr c = hca_addr(P, R.aux);
    xk = ExtraKey{c.k, c.v, S.q + (int64_t)r * kRow, P.kv8 != 0};
  }
  merge_partials_wg([&](int j) { return (int64_t)(j < ca ? fa + j : S.n_a + fb + (j - ca)); }, ca + cb,
                    S.part_acc, S.part_ml, S.out + (int64_t)r * kRow, xk);
}

// S4 when some request has more than 32 partials (few long requests over the whole
// GPU): one 8-wave workgroup per (request, head), each wave merging every eighth
// partial (32 in one memory round trip), the waves' states combined in LDS.
__global__ __launch_bounds__(512) void k_step4_heads(Pools P, ReqBatch B, StepArgs S) {
  __shared__ MergeShared<8> sh;
  const int r = blockIdx.x >> 4;
  const int h = blockIdx.x & (kH - 1);
  const int fa = S.first_a[r], ca = S.first_a[r + 1] - fa;
  const int fb = S.first_b[r], cb = S.first_b[r + 1] - fb;
  const Req R = B.r[r];
  ExtraKey xk{nullptr, nullptr, nullptr, false};
  if (S.a_only && h == 0)   // no C4 entries: the top-k row is padding
    for (int i = threadIdx.x; i < S.k; i += 512) {
      S.topk[(int64_t)r * S.k + i] = -1;
      if (S.score_out) S.score_out[(int64_t)r * S.k + i] = -INFINITY;
    }
  if ((S.fused || S.a_only) && R.aux >= 0 && P.hca) {   // the HCA entry of the block sealed now, merged in S2
    const C4Addr c = hca_addr(P, R.aux);
    xk = ExtraKey{c.k, c.v, S.q + (int64_t)r * kRow, P.kv8 != 0};
  }
  merge_partials_split<8>([&](int j) { return (int64_t)(j < ca ? fa + j : S.n_a + fb + (j - ca)); }, ca + cb,
                          h, S.part_acc, S.part_ml, S.out + (int64_t)r * kRow, xk, sh);
}

}  // namespace

hipError_t launch_step1(const Pools& P, const ReqBatch& B, const StepArgs& S, hipStream_t st,
                 const LaunchEv& ev) {
  const int grid = kSealSplit * B.n_seal + B.n + B.n_open + S.n_score;
  if (grid == 0) return hipSuccess;
  const dim3 g(grid), t(kAttnWaves * 64);
  if (P.kv8) {
    if (!P.c4) return launch_k(k_step1<false, false, true>, g, t, st, ev, P, B, S);
    if (P.fp8) return launch_k(k_step1<true, true, true>, g, t, st, ev, P, B, S);
    return launch_k(k_step1<false, true, true>, g, t, st, ev, P, B, S);
  }
  if (!P.c4) return launch_k(k_step1<false, false, false>, g, t, st, ev, P, B, S);
  if (P.fp8) return launch_k(k_step1<true, true, false>, g, t, st, ev, P, B, S);
  return launch_k(k_step1<false, true, false>, g, t, st, ev, P, B, S);
}

hipError_t launch_step2(const Pools& P, const ReqBatch& B, const StepArgs& S, hipStream_t st,
                 const LaunchEv& ev) {
  const int grid = (S.fused ? S.n_b : S.sel.n_wgs) + B.n_seal + S.n_a + (S.s2_append ? B.n : 0);
  if (grid == 0) return hipSuccess;
  const dim3 g(grid), t(kStep2Threads);
  if (P.kv8) return P.fp8 ? launch_k(k_step2<true, true>, g, t, st, ev, P, B, S)
                          : launch_k(k_step2<true, false>, g, t, st, ev, P, B, S);
  return P.fp8 ? launch_k(k_step2<false, true>, g, t, st, ev, P, B, S)
               : launch_k(k_step2<false, false>, g, t, st, ev, P, B, S);
}

hipError_t launch_step2b(const Pools& P, const ReqBatch& B, const StepArgs& S, hipStream_t st,
                         const LaunchEv& ev) {
  if (B.n == 0 || S.fused || S.sel.gmax <= 1) return hipSuccess;
  return launch_k(k_step2b, dim3(B.n), dim3(kSelThreads), st, ev, P, B, S);
}

hipError_t launch_step3(const Pools& P, const ReqBatch& B, const StepArgs& S, hipStream_t st,
                 const LaunchEv& ev) {
  if (S.n_b == 0 || S.fused) return hipSuccess;
  const dim3 g(S.n_b), t(kStep3Waves * 64);
  if (P.kv8) return P.fp8 ? launch_k(k_step3<true, true>, g, t, st, ev, P, B, S)
                          : launch_k(k_step3<true, false>, g, t, st, ev, P, B, S);
  return P.fp8 ? launch_k(k_step3<false, true>, g, t, st, ev, P, B, S)
               : launch_k(k_step3<false, false>, g, t, st, ev, P, B, S);
}

hipError_t launch_step4(const Pools& P, const ReqBatch& B, const StepArgs& S, hipStream_t st,
                 const LaunchEv& ev) {
  if (B.n == 0) return hipSuccess;
  int parts = 0;   // the most partials of one request
  for (int i = 0; i < B.n; ++i)
    parts = std::max(parts, S.first_a[i + 1] - S.first_a[i] + S.first_b[i + 1] - S.first_b[i]);
  if (parts > 32) return launch_k(k_step4_heads, dim3(kH * B.n), dim3(512), st, ev, P, B, S);
  return launch_k(k_step4, dim3(B.n), dim3(512), st, ev, P, B, S);
}

}  // namespace hsa
