// step.hip - the decode step of the heterogeneous KV cache (hsa_decode_step) as four
// launches.
//
// Pages: [Q&A] "V4 为何要分池？块对齐与尾缓冲怎么配合？" §4: a new token goes to the
// tail, a full block is compressed into the Classical pool, the SWA slides, and
// attention reads the compressed entries plus the exact State. The work of one
// step, for every request of the batch:
//
//   S1  append the token (ring + indexer tail), seal a full block (C4 entries,
//       indexer keys, eight HCA partials), indexer scores of every sealed block,
//       and attention part A: the SWA tokens and the HCA entries of blocks sealed
//       before this step. Nothing read in S1 is written in S1: the new token is
//       read from the input wherever it is needed (SWA key, last indexer key of a
//       block sealed now, last token of the seal).
//   S2  top-k selection over the scores; the HCA merge of blocks sealed in S1.
//   S3  attention part B: the HCA entry of the block sealed now and the selected
//       C4 entries.
//   S4  log-sum-exp merge of every request's part A and part B partials.
//
// Part A does not depend on the top-k, so it streams alongside the indexer scan in
// S1 and leaves only the C4 gather after the selection. Key order differs from
// hsa_decode_attend only in the order of the softmax sum.
#include "attn_dev.h"
#include "device.h"
#include "kernels.h"
#include "score_dev.h"
#include "seal_dev.h"

namespace hsa {

namespace {

__device__ __forceinline__ int sealed_now(const Req& r) { return r.aux >= 0 ? 1 : 0; }
__device__ __forceinline__ int keys_a(const Pools& P, const Req& r) {
  return (r.len < P.n_win ? r.len : P.n_win) + r.nb - sealed_now(r);
}
__device__ __forceinline__ int keys_b(const Req& r, int32_t k) {
  const int nc = kC4 * r.nb;
  return sealed_now(r) + (k < nc ? k : nc);
}
__device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }

__global__ __launch_bounds__(kAttnWaves * 64) void k_step1(Pools P, ReqBatch B, StepArgs S) {
  __shared__ AttnShared sh;
  int bid = blockIdx.x;
  // -- seal eighths (first, so the longest single workgroups start early)
  if (bid < kSealSplit * B.n_seal) {
    const int item = bid / kSealSplit;
    const int ri = B.seal_req[item];
    seal_eighth(P, B.r[ri], ri, item, bid % kSealSplit, S.kin, S.vin, S.iin, S.seal_part);
    return;
  }
  bid -= kSealSplit * B.n_seal;
  // -- append
  if (bid < B.n) {
    append_token(P, B.r[bid], bid, S.kin, S.vin, S.iin);
    return;
  }
  bid -= B.n;
  // -- indexer scores, one workgroup per sealed block
  if (bid < S.n_score) {
    int r, lb, first;
    find_item(B.n, bid, [&](int i) { return B.r[i].nb; }, r, lb, first);
    const Req R = B.r[r];
    float* out = S.scores + (int64_t)r * S.ld + (int64_t)kC4 * lb;
    const float* qrow = S.qi + (int64_t)r * kIRow;
    if (R.aux >= 0 && lb == R.nb - 1) {
      // the block sealed in this step: keys from the indexer tail, the newest from
      // the input (its tail slot is being written in this launch)
      const float* tail = P.idx_tail + (int64_t)R.state * kBlk * kIRow;
      const float* inrow = S.iin + (int64_t)r * kIRow;
      score_block([&](int t) { return t == kBlk - 1 ? inrow : tail + t * kIRow; }, qrow, out);
    } else {
      const int32_t id = P.table[(int64_t)R.state * P.table_stride + lb];
      if (id < 0 || id >= P.max_blocks) {   // never taken: tables are written before use
        if (threadIdx.x < kC4) out[threadIdx.x] = -INFINITY;
        return;
      }
      const float* blk = P.idx_k + (int64_t)id * kBlk * kIRow;
      score_block([&](int t) { return blk + t * kIRow; }, qrow, out);
    }
    return;
  }
  bid -= S.n_score;
  // -- attention part A: SWA tokens + HCA of blocks sealed before this step
  int r, w, first;
  find_item(B.n, bid, [&](int i) { return cdiv(keys_a(P, B.r[i]), S.chunk_a); }, r, w, first);
  const Req R = B.r[r];
  const int swa = R.len < P.n_win ? R.len : P.n_win;
  const int na = keys_a(P, R);
  const uint16_t* ring_k = P.swa_k + (int64_t)R.state * P.n_win * kRow;
  const uint16_t* ring_v = P.swa_v + (int64_t)R.state * P.n_win * kRow;
  const int32_t* tab = P.table + (int64_t)R.state * P.table_stride;
  const int64_t newest = (int64_t)R.len - 1;
  auto key_a = [&](int x) {
    KeyAddr a;
    a.k = a.v = nullptr;
    if (x < swa) {
      const int64_t p = newest + 1 - swa + x;
      if (p == newest) {
        a.k = S.kin + (int64_t)r * kRow;
        a.v = S.vin + (int64_t)r * kRow;
      } else {
        a.k = ring_k + (p % P.n_win) * kRow;
        a.v = ring_v + (p % P.n_win) * kRow;
      }
      return a;
    }
    const int32_t id = tab[x - swa];
    if (id < 0 || id >= P.max_blocks) return a;
    a.k = P.hca_k + (int64_t)id * kRow;
    a.v = P.hca_v + (int64_t)id * kRow;
    return a;
  };
  float M, L, A8[8];
  attend_keys(key_a, w * S.chunk_a, min(na, (w + 1) * S.chunk_a), S.q + (int64_t)r * kRow,
              S.kin + (int64_t)r * kRow, S.vin + (int64_t)r * kRow, sh, M, L, A8);
  store_partial(S.part_acc, S.part_ml, bid, M, L, A8);
}

__global__ __launch_bounds__(kSelThreads) void k_step2(Pools P, ReqBatch B, StepArgs S) {
  __shared__ SelShared sh;
  const int bid = blockIdx.x;
  if (bid < B.n) {
    const int64_t k = S.k;
    select_run(kC4 * B.r[bid].nb, S.k, S.sorted, S.scores + (int64_t)bid * S.ld,
               S.topk + bid * k, S.score_out ? S.score_out + bid * k : nullptr, sh);
    return;
  }
  const int item = bid - B.n;
  seal_merge(P, B.r[B.seal_req[item]].aux, S.seal_part, item);
}

__global__ __launch_bounds__(kAttnWaves * 64) void k_step3(Pools P, ReqBatch B, StepArgs S) {
  __shared__ AttnShared sh;
  int r, w, first;
  find_item(B.n, blockIdx.x, [&](int i) { return cdiv(keys_b(B.r[i], S.k), S.chunk_b); }, r, w,
            first);
  const Req R = B.r[r];
  const int nbk = keys_b(R, S.k);
  const int sn = sealed_now(R);
  const int32_t* tab = P.table + (int64_t)R.state * P.table_stride;
  const int32_t* sel = S.topk + (int64_t)r * S.k;
  auto key_b = [&](int x) {
    KeyAddr a;
    a.k = a.v = nullptr;
    if (x < sn) {
      a.k = P.hca_k + (int64_t)R.aux * kRow;
      a.v = P.hca_v + (int64_t)R.aux * kRow;
      return a;
    }
    const int32_t j = sel[x - sn];
    if (j < 0 || j >= kC4 * R.nb) return a;
    const int32_t id = tab[j / kC4];
    if (id < 0 || id >= P.max_blocks) return a;
    const int64_t off = ((int64_t)id * kC4 + j % kC4) * kRow;
    a.k = P.csa_k + off;
    a.v = P.csa_v + off;
    return a;
  };
  const uint16_t* dk = P.swa_k + (int64_t)R.state * P.n_win * kRow;   // valid row (L >= 1)
  const uint16_t* dv = P.swa_v + (int64_t)R.state * P.n_win * kRow;
  float M, L, A8[8];
  attend_keys(key_b, w * S.chunk_b, min(nbk, (w + 1) * S.chunk_b), S.q + (int64_t)r * kRow, dk, dv,
              sh, M, L, A8);
  store_partial(S.part_acc, S.part_ml, (int64_t)S.n_a + blockIdx.x, M, L, A8);
}

__global__ __launch_bounds__(256) void k_step4(Pools P, ReqBatch B, StepArgs S) {
  const int r = blockIdx.x >> 2;
  int fa, ca, fb, cb;
  prefix_of(B.n, r, [&](int i) { return cdiv(keys_a(P, B.r[i]), S.chunk_a); }, fa, ca);
  prefix_of(B.n, r, [&](int i) { return cdiv(keys_b(B.r[i], S.k), S.chunk_b); }, fb, cb);
  const int h = 4 * (blockIdx.x & 3) + (threadIdx.x >> 6);
  merge_partials([&](int j) { return (int64_t)(j < ca ? fa + j : S.n_a + fb + (j - ca)); }, ca + cb,
                 h, S.part_acc, S.part_ml, S.out + (int64_t)r * kRow);
}

}  // namespace

hipError_t launch_step1(const Pools& P, const ReqBatch& B, const StepArgs& S, hipStream_t st) {
  const int grid = kSealSplit * B.n_seal + B.n + S.n_score + S.n_a;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(k_step1, dim3(grid), dim3(kAttnWaves * 64), 0, st, P, B, S);
  return hipGetLastError();
}

hipError_t launch_step2(const Pools& P, const ReqBatch& B, const StepArgs& S, hipStream_t st) {
  const int grid = B.n + B.n_seal;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(k_step2, dim3(grid), dim3(kSelThreads), 0, st, P, B, S);
  return hipGetLastError();
}

hipError_t launch_step3(const Pools& P, const ReqBatch& B, const StepArgs& S, hipStream_t st) {
  if (S.n_b == 0) return hipSuccess;
  hipLaunchKernelGGL(k_step3, dim3(S.n_b), dim3(kAttnWaves * 64), 0, st, P, B, S);
  return hipGetLastError();
}

hipError_t launch_step4(const Pools& P, const ReqBatch& B, const StepArgs& S, hipStream_t st) {
  if (B.n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_step4, dim3(4 * B.n), dim3(256), 0, st, P, B, S);
  return hipGetLastError();
}

}  // namespace hsa
