// attend.hip - heterogeneous decode attention over the two pools (hsa_decode_attend).
//
// Keys of request i, in this order: the min(L, n_win) SWA tokens (oldest first),
// the HCA entry of each of its nb sealed blocks (layers with HCA entries), then the
// C4 entries named in the first min(k, 32 nb) slots of its top-k row (layers with
// C4 entries; -1 and out-of-range ordinals are skipped). One softmax over all of them per head, scale 1/sqrt(128). The
// streaming core and its page citations are in attn_dev.h.
#include "attn_dev.h"
#include "device.h"
#include "kernels.h"

namespace hsa {

namespace {

__device__ __forceinline__ int n_keys(const Pools& P, const Req& R, int32_t k) {
  const int swa = R.len < P.n_win ? R.len : P.n_win;
  const int nc = c4_cands(P.c4, P.eager, R);
  return swa + (P.hca ? R.nb : 0) + (k < nc ? k : nc);
}

// K and V rows of key x of request R (nullptrs for a skipped top-k slot).
__device__ __forceinline__ KeyAddr key_addr(const Pools& P, const Req& R, int x, const int32_t* sel) {
  const int swa = R.len < P.n_win ? R.len : P.n_win;
  KeyAddr a;
  a.k = a.v = nullptr;
  if (x < swa) {
    const int64_t p = (int64_t)R.len - swa + x;
    const C4Addr c = ring_addr(P, (int64_t)R.state * P.n_win + p % P.n_win);
    a.k = c.k;
    a.v = c.v;
    return a;
  }
  x -= swa;
  const int32_t* tab = P.table + (int64_t)R.state * P.table_stride;
  const int nh = P.hca ? R.nb : 0;
  if (x < nh) {
    const int32_t id = tab[x];
    if (id < 0 || id >= P.max_blocks) return a;   // never taken: tables are written before use
    const C4Addr c = hca_addr(P, id);
    a.k = c.k;
    a.v = c.v;
    return a;
  }
  x -= nh;
  const int32_t j = sel[x];
  if (j < 0 || j >= c4_cands(P.c4, P.eager, R)) return a;
  const int32_t id = tab[j / kC4];   // the open block's entry holds max_blocks + state (eager)
  if (id < 0 || id >= P.c4_ids) return a;
  const C4Addr c = c4_addr(P, (int64_t)id * kC4 + j % kC4);
  a.k = c.k;
  a.v = c.v;
  return a;
}

// One workgroup per chunk of a request's keys; it writes an unnormalised partial,
// or the output itself when the request is a single chunk. k_merge combines the
// partials in the next launch: a kernel boundary costs far less on this GPU than a
// device-scope fence in every workgroup. KV8: FP8 SWA ring and HCA entries; F8: FP8
// C4 entries.
template <bool KV8, bool F8>
__global__ __launch_bounds__(kAttnWaves * 64) void k_attend(Pools P, ReqBatch B, int32_t chunk,
                                                           const uint16_t* q, const int32_t* topk,
                                                           int32_t k, float* part_acc,
                                                           float* part_ml, float* out) {
  __shared__ AttnShared sh;
  int r, w, first;
  find_item(B.n, blockIdx.x, [&](int i) { return (n_keys(P, B.r[i], k) + chunk - 1) / chunk; }, r, w,
            first);
  const Req R = B.r[r];
  const int nk = n_keys(P, R, k);
  const int nch = (nk + chunk - 1) / chunk;
  const int32_t* sel = topk ? topk + (int64_t)r * k : nullptr;
  const C4Addr dm = dummy_rows(P, R.state);   // valid rows (L >= 1)
  float M, L, A8[8];
  // keys below the C4 entries (SWA tokens, HCA entries) follow the KV format
  attend_keys<kAttnWaves, ring_depth<kAttnWaves>(), KV8, F8>(
      [&](int x) { return key_addr(P, R, x, sel); }, w * chunk, min(nk, (w + 1) * chunk), q + (int64_t)r * kRow,
      dm.k, dm.v, sh, M, L, A8, (R.len < P.n_win ? R.len : P.n_win) + (P.hca ? R.nb : 0));
  if (nch == 1)
    store_output(out + (int64_t)r * kRow, L, A8);
  else
    store_partial(part_acc, part_ml, blockIdx.x, M, L, A8);
}

// One workgroup per (request, group of 4 heads) of the requests with two or more
// chunks.
__global__ __launch_bounds__(256) void k_merge(Pools P, ReqBatch B, int32_t chunk, int32_t k,
                                               const float* part_acc, const float* part_ml,
                                               float* out) {
  const int r = blockIdx.x >> 2;
  int c0, nch;
  prefix_of(B.n, r, [&](int i) { return (n_keys(P, B.r[i], k) + chunk - 1) / chunk; }, c0, nch);
  if (nch < 2) return;            // written directly by k_attend
  const int h = 4 * (blockIdx.x & 3) + (threadIdx.x >> 6);
  merge_partials([&](int j) { return (int64_t)(c0 + j); }, nch, h, part_acc, part_ml,
                 out + (int64_t)r * kRow);
}

}  // namespace

hipError_t launch_attend(const Pools& P, const ReqBatch& B, int64_t total_chunks, int32_t chunk,
                         const void* q, const int32_t* topk, int32_t k, float* part_acc,
                         float* part_ml, float* out, hipStream_t st,
                 const LaunchEv& ev) {
  if (total_chunks == 0) return hipSuccess;
  const dim3 g((unsigned)total_chunks), t(kAttnWaves * 64);
  const uint16_t* q16 = static_cast<const uint16_t*>(q);
  if (P.kv8)
    return P.fp8 ? launch_k(k_attend<true, true>, g, t, st, ev, P, B, chunk, q16, topk, k, part_acc, part_ml, out)
                 : launch_k(k_attend<true, false>, g, t, st, ev, P, B, chunk, q16, topk, k, part_acc, part_ml, out);
  return P.fp8 ? launch_k(k_attend<false, true>, g, t, st, ev, P, B, chunk, q16, topk, k, part_acc, part_ml, out)
               : launch_k(k_attend<false, false>, g, t, st, ev, P, B, chunk, q16, topk, k, part_acc, part_ml, out);
}

hipError_t launch_merge(const Pools& P, const ReqBatch& B, int32_t chunk, int32_t k,
                        const float* part_acc, const float* part_ml, float* out, hipStream_t st,
                 const LaunchEv& ev) {
  if (B.n == 0) return hipSuccess;
  return launch_k(k_merge, dim3(4 * B.n), dim3(256), st, ev, P, B, chunk, k, part_acc, part_ml,
                     out);
}

}  // namespace hsa
