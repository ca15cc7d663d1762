// indexer_topk.hip - indexer scores over sealed blocks and top-k selection
// (hsa_indexer_topk). The arithmetic and its readings are in score_dev.h.
#include "attn_dev.h"
#include "device.h"
#include "kernels.h"
#include "score_dev.h"

namespace hsa {

namespace {

// One workgroup per sealed block of the batch's requests (128 KiB of fp32 keys, or
// 17 KiB of MXFP4 keys).
__global__ __launch_bounds__(256, 4) void k_score(Pools P, ReqBatch B, const float* q_idx,
                                                  float* scores, int64_t ld) {
  int r, w, first;
  find_item(B.n, blockIdx.x, [&](int i) { return c4_rowlen(P.c4, P.eager, B.r[i]) / kC4; }, r, w, first);
  const Req R = B.r[r];
  if (w == R.nb) {   // eager C4: the open block, its keys in the indexer tail
    const float* tail = P.idx_tail + (int64_t)R.state * kBlk * kIRow;
    score_block([&](int t) { return tail + t * kIRow; }, q_idx + (int64_t)r * kIRow,
                scores + (int64_t)r * ld + (int64_t)kC4 * w, open_groups(P.eager, R));
    return;
  }
  const int32_t id = P.table[(int64_t)R.state * P.table_stride + w];
  float* out = scores + (int64_t)r * ld + (int64_t)kC4 * w;
  if (id < 0 || id >= P.max_blocks) {          // never taken: tables are written before use
    if (threadIdx.x < kC4) out[threadIdx.x] = -INFINITY;
    return;
  }
  const int64_t kr = (int64_t)id * kBlk;
  if (P.mx4) {
    score_block_mx<kBlk / 32>(P.idx_q + kr * kIRowQ, P.idx_e + kr * kIRowE, q_idx + (int64_t)r * kIRow, out);
  } else {
    const float* blk = P.idx_k + kr * kIRow;
    score_block([&](int t) { return blk + t * kIRow; }, q_idx + (int64_t)r * kIRow, out);
  }
}

__global__ __launch_bounds__(kSelThreads) void k_select(ReqBatch B, SelPlan SP, int32_t k,
                                                        int32_t sorted, const float* scores, int64_t ld,
                                                        int32_t* idx_out, float* score_out) {
  __shared__ SelShared sh;
  select_round1<kSelThreads>(blockIdx.x, B.n, B.r, SP, k, sorted, scores, ld, idx_out, score_out, sh,
                             nullptr, 0, nullptr);
}

__global__ __launch_bounds__(kSelThreads) void k_select2(ReqBatch B, SelPlan SP, int32_t k,
                                                         int32_t sorted, int32_t* idx_out,
                                                         float* score_out) {
  __shared__ SelShared sh;
  select_round2<kSelThreads>(blockIdx.x, B.r, SP, k, sorted, idx_out, score_out, sh, nullptr, 0,
                             nullptr);
}

}  // namespace

hipError_t launch_score(const Pools& P, const ReqBatch& B, int64_t total_blocks, const float* q_idx,
                        float* scores, int64_t ld, hipStream_t st,
                 const LaunchEv& ev) {
  if (total_blocks == 0) return hipSuccess;
  return launch_k(k_score, dim3((unsigned)total_blocks), dim3(256), st, ev, P, B, q_idx, scores, ld);
}

hipError_t launch_select(const ReqBatch& B, const SelPlan& SP, int32_t k, int32_t sorted,
                         const float* scores, int64_t ld, int32_t* idx_out, float* score_out,
                         hipStream_t st, const LaunchEv& ev) {
  if (B.n == 0) return hipSuccess;
  hipError_t e = launch_k(k_select, dim3(SP.n_wgs), dim3(kSelThreads), st, ev, B, SP, k, sorted, scores,
                          ld, idx_out, score_out);
  if (e != hipSuccess || SP.gmax <= 1) return e;
  return launch_k(k_select2, dim3(B.n), dim3(kSelThreads), st, LaunchEv{}, B, SP, k, sorted, idx_out,
                  score_out);
}

}  // namespace hsa
