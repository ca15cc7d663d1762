// append_seal.hip - append tokens to the State and seal full blocks into the Block Cache.
//
// Pages: [Q&A] "V4 为何要分池？块对齐与尾缓冲怎么配合？" §3.1 (a token goes to the
// tail; a full block is compressed and appended to the Classical pool), §4 (the
// decode step: write the tail, compress on fill, slide the SWA); [Ch12] "Ch 12 ·
// 推理框架 — KV 的异构调度" §2.2 (each 128-token block yields 32 CSA + 1 HCA + 128
// indexer keys).
//
// The compressor is not defined on the pages; the stand-in is gated pooling: per
// head h, g_t = <W[h], K_t[h]>, alpha = softmax over the group's tokens, entry =
// sum_t alpha_t (K_t[h], V_t[h]), stored as bf16 (round to nearest even). C4 entry
// j of a block pools tokens 4j..4j+3 with W_csa; the HCA entry pools all 128 with
// W_hca.
//
// Thread layout of a seal workgroup (256 lanes): lane t owns head t/16 and dims
// (t%16)*8 .. +8 of every token, i.e. 16 contiguous bytes of each 4 KiB K or V row,
// so one token is one coalesced 4 KiB read per workgroup and the 16 lanes of a head
// form one DPP row for the gate reduction.
#include "device.h"
#include "kernels.h"

namespace hsa {

namespace {

// Where token t of the block being sealed lives: in the state (ring slot, indexer
// tail slot) if its position precedes len_old, else in the packed input.
struct TokSrc {
  const uint16_t* ring_k;
  const uint16_t* ring_v;
  const float* tail_i;
  const uint16_t* in_k;
  const uint16_t* in_v;
  const float* in_i;
  int64_t pos0, len_old;
  int32_t n_win;

  __device__ __forceinline__ bool resident(int t) const { return pos0 + t < len_old; }
  __device__ __forceinline__ const uint16_t* k(int t) const {
    const int64_t p = pos0 + t;
    return p < len_old ? ring_k + (p % n_win) * kRow : in_k + (p - len_old) * kRow;
  }
  __device__ __forceinline__ const uint16_t* v(int t) const {
    const int64_t p = pos0 + t;
    return p < len_old ? ring_v + (p % n_win) * kRow : in_v + (p - len_old) * kRow;
  }
  __device__ __forceinline__ const float* i(int t) const {
    const int64_t p = pos0 + t;
    return p < len_old ? tail_i + (p % kBlk) * kIRow : in_i + (p - len_old) * kIRow;
  }
};

constexpr int kSubTok = kBlk / kSealSplit;   // 16 tokens per seal partial

// Seal tokens [t0, t0 + 16) of one block: writes their 4 C4 entries and 16
// indexer keys, and returns the HCA softmax partial (m, l, acc) of these tokens
// for this lane's 8 dims. Both seal paths build the HCA entry from the same eight
// partials merged in the same order, so bulk and one-token appends give
// bit-identical blocks.
__device__ __forceinline__ void seal_part(const Pools& P, const TokSrc& src, int32_t id, int t0,
                                          float& m, float& l, float* acck, float* accv) {
  const int tid = threadIdx.x;
  const int h = tid >> 4;
  const int d0 = (tid & 15) * 8;
  const int off = h * kD + d0;     // == tid * 8
  float wc[8], wh[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    wc[i] = P.gate_csa[off + i];
    wh[i] = P.gate_hca[off + i];
  }
  uint16_t* csa_k = P.csa_k + (int64_t)id * kC4 * kRow;
  uint16_t* csa_v = P.csa_v + (int64_t)id * kC4 * kRow;
  float* idx_dst = P.idx_k + (int64_t)id * kBlk * kIRow;

  m = -INFINITY;
  l = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) acck[i] = accv[i] = 0.f;

  for (int g = 0; g < kSubTok / 4; ++g) {
    const int tb = t0 + 4 * g;
    uint4 kw[4], vw[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      kw[u] = *reinterpret_cast<const uint4*>(src.k(tb + u) + off);
      vw[u] = *reinterpret_cast<const uint4*>(src.v(tb + u) + off);
    }
    // indexer keys of the 4 tokens: 4 x 64 float4, one per lane
    {
      const int u = tid >> 6, c = tid & 63;
      const float4 iv = reinterpret_cast<const float4*>(src.i(tb + u))[c];
      reinterpret_cast<float4*>(idx_dst + (int64_t)(tb + u) * kIRow)[c] = iv;
    }
    float kf[4][8], vf[4][8], gc[4], gh[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      unpack8(kw[u], kf[u]);
      unpack8(vw[u], vf[u]);
      float a = 0.f, b = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        a = fmaf(wc[i], kf[u][i], a);
        b = fmaf(wh[i], kf[u][i], b);
      }
      gc[u] = row_sum16(a);
      gh[u] = row_sum16(b);
    }
    // C4 entry (tokens tb .. tb+3): softmax of the 4 CSA gates
    {
      const float mx = fmaxf(fmaxf(gc[0], gc[1]), fmaxf(gc[2], gc[3]));
      float e[4], s = 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        e[u] = __expf(gc[u] - mx);
        s += e[u];
      }
      const float inv = 1.f / s;
      float ck[8], cv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float a = 0.f, b = 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          a = fmaf(e[u], kf[u][i], a);
          b = fmaf(e[u], vf[u][i], b);
        }
        ck[i] = a * inv;
        cv[i] = b * inv;
      }
      const int slot = tb >> 2;
      uint4 ok, ov;
      ok.x = pack_bf2(ck[0], ck[1]); ok.y = pack_bf2(ck[2], ck[3]);
      ok.z = pack_bf2(ck[4], ck[5]); ok.w = pack_bf2(ck[6], ck[7]);
      ov.x = pack_bf2(cv[0], cv[1]); ov.y = pack_bf2(cv[2], cv[3]);
      ov.z = pack_bf2(cv[4], cv[5]); ov.w = pack_bf2(cv[6], cv[7]);
      *reinterpret_cast<uint4*>(csa_k + (int64_t)slot * kRow + off) = ok;
      *reinterpret_cast<uint4*>(csa_v + (int64_t)slot * kRow + off) = ov;
    }
    // HCA running softmax over the block's tokens
    {
      const float mx = fmaxf(m, fmaxf(fmaxf(gh[0], gh[1]), fmaxf(gh[2], gh[3])));
      const float sc = __expf(m - mx);   // m = -inf on the first group -> 0
      float e[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) e[u] = __expf(gh[u] - mx);
      l = l * sc + ((e[0] + e[1]) + (e[2] + e[3]));
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float a = acck[i] * sc, b = accv[i] * sc;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          a = fmaf(e[u], kf[u][i], a);
          b = fmaf(e[u], vf[u][i], b);
        }
        acck[i] = a;
        accv[i] = b;
      }
      m = mx;
    }
  }
}

// Fold partial (m, l, acc) into the running HCA state (M, L, K, V).
__device__ __forceinline__ void merge_part(float& M, float& L, float* K, float* V, float m, float l,
                                          const float* acck, const float* accv) {
  const float Mn = fmaxf(M, m);
  const float a = __expf(M - Mn);   // 0 when M = -inf (first partial)
  const float b = __expf(m - Mn);
  L = L * a + l * b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    K[i] = fmaf(acck[i], b, K[i] * a);
    V[i] = fmaf(accv[i], b, V[i] * a);
  }
  M = Mn;
}

__device__ __forceinline__ void store_hca(const Pools& P, int32_t id, float l, const float* acck,
                                          const float* accv) {
  const int off = threadIdx.x * 8;
  const float inv = 1.f / l;
  uint4 ok, ov;
  ok.x = pack_bf2(acck[0] * inv, acck[1] * inv); ok.y = pack_bf2(acck[2] * inv, acck[3] * inv);
  ok.z = pack_bf2(acck[4] * inv, acck[5] * inv); ok.w = pack_bf2(acck[6] * inv, acck[7] * inv);
  ov.x = pack_bf2(accv[0] * inv, accv[1] * inv); ov.y = pack_bf2(accv[2] * inv, accv[3] * inv);
  ov.z = pack_bf2(accv[4] * inv, accv[5] * inv); ov.w = pack_bf2(accv[6] * inv, accv[7] * inv);
  *reinterpret_cast<uint4*>(P.hca_k + (int64_t)id * kRow + off) = ok;
  *reinterpret_cast<uint4*>(P.hca_v + (int64_t)id * kRow + off) = ov;
}

// Decode append (one token per request) with the seal fused in.
// Workgroups [0, n): write request i's token into ring slot p mod n_win and
// indexer-tail slot p mod 128 (p = len - 1), and record a new block id in the
// device block table. Workgroups [n, n + 8 * n_seal): seal one eighth of a
// sealing request's block (4 C4 entries, 16 indexer keys, one HCA partial).
// No slot written by the first group is read by the second: the new token's
// ring slot differs from the 127 older ones (n_win >= 128), and its tail slot is
// 127, which the seal reads from the input instead.
__global__ __launch_bounds__(256) void k_decode_append(Pools P, ReqBatch B, const uint16_t* kin,
                                                       const uint16_t* vin, const float* iin,
                                                       float* part) {
  const int tid = threadIdx.x;
  const int bid = blockIdx.x;
  if (bid < B.n) {
    const Req r = B.r[bid];
    const int64_t p = r.len - 1;
    const int64_t ring = ((int64_t)r.state * P.n_win + (p % P.n_win)) * kRow;
    reinterpret_cast<uint4*>(P.swa_k + ring)[tid] =
        reinterpret_cast<const uint4*>(kin + (int64_t)bid * kRow)[tid];
    reinterpret_cast<uint4*>(P.swa_v + ring)[tid] =
        reinterpret_cast<const uint4*>(vin + (int64_t)bid * kRow)[tid];
    if (tid < kIRow / 4) {
      const int64_t ti = ((int64_t)r.state * kBlk + (p % kBlk)) * kIRow;
      reinterpret_cast<float4*>(P.idx_tail + ti)[tid] =
          reinterpret_cast<const float4*>(iin + (int64_t)bid * kIRow)[tid];
    }
    if (tid == 0 && r.aux >= 0) P.table[(int64_t)r.state * P.table_stride + (r.nb - 1)] = r.aux;
    return;
  }
  const int item = (bid - B.n) / kSealSplit;
  const int sub = (bid - B.n) % kSealSplit;
  const int ri = B.seal_req[item];
  const Req r = B.r[ri];
  TokSrc src;
  src.ring_k = P.swa_k + (int64_t)r.state * P.n_win * kRow;
  src.ring_v = P.swa_v + (int64_t)r.state * P.n_win * kRow;
  src.tail_i = P.idx_tail + (int64_t)r.state * kBlk * kIRow;
  src.in_k = kin + (int64_t)ri * kRow;
  src.in_v = vin + (int64_t)ri * kRow;
  src.in_i = iin + (int64_t)ri * kIRow;
  src.len_old = r.len - 1;
  src.pos0 = (int64_t)(r.nb - 1) * kBlk;
  src.n_win = P.n_win;

  float m, l, acck[8], accv[8];
  seal_part(P, src, r.aux, sub * kSubTok, m, l, acck, accv);

  // HCA partial of this eighth -> scratch; k_seal_merge folds the eight together
  float* mine = part + (int64_t)(item * kSealSplit + sub) * kPartFloats;
  const int h = tid >> 4;
  if ((tid & 15) == 0) {
    mine[h] = m;
    mine[kH + h] = l;
  }
  float4* pk = reinterpret_cast<float4*>(mine + 2 * kH + tid * 8);
  float4* pv = reinterpret_cast<float4*>(mine + 2 * kH + kRow + tid * 8);
  pk[0] = make_float4(acck[0], acck[1], acck[2], acck[3]);
  pk[1] = make_float4(acck[4], acck[5], acck[6], acck[7]);
  pv[0] = make_float4(accv[0], accv[1], accv[2], accv[3]);
  pv[1] = make_float4(accv[4], accv[5], accv[6], accv[7]);
}

// One workgroup per block sealed by k_decode_append (next launch, so the partials
// are visible without a device-scope fence): fold its eight partials in order, the
// same arithmetic as the bulk seal, and store the HCA entry.
__global__ __launch_bounds__(256) void k_seal_merge(Pools P, ReqBatch B, const float* part) {
  const int item = blockIdx.x;
  const Req r = B.r[B.seal_req[item]];
  const int tid = threadIdx.x;
  const int h = tid >> 4;
  const float* base = part + (int64_t)item * kSealSplit * kPartFloats;
  float M = -INFINITY, L = 0.f, K8[8] = {}, V8[8] = {};
  for (int s = 0; s < kSealSplit; ++s) {
    const float* q = base + s * kPartFloats;
    float pk[8], pv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pk[i] = q[2 * kH + tid * 8 + i];
      pv[i] = q[2 * kH + kRow + tid * 8 + i];
    }
    merge_part(M, L, K8, V8, q[h], q[kH + h], pk, pv);
  }
  store_hca(P, r.aux, L, K8, V8);
}

// Bulk seal: one workgroup per block, its eight 16-token partials merged in
// registers in order.
__global__ __launch_bounds__(256) void k_bulk_seal(Pools P, const SealDesc* seals,
                                                   const uint16_t* kin, const uint16_t* vin,
                                                   const float* iin) {
  const SealDesc d = seals[blockIdx.x];
  TokSrc src;
  src.ring_k = P.swa_k + (int64_t)d.state * P.n_win * kRow;
  src.ring_v = P.swa_v + (int64_t)d.state * P.n_win * kRow;
  src.tail_i = P.idx_tail + (int64_t)d.state * kBlk * kIRow;
  // rows of positions >= len_old (row0 < 0 only when every token is resident)
  const int64_t row0 = d.row0 < 0 ? 0 : d.row0;
  src.in_k = kin ? kin + row0 * kRow : nullptr;
  src.in_v = vin ? vin + row0 * kRow : nullptr;
  src.in_i = iin ? iin + row0 * kIRow : nullptr;
  src.len_old = d.len_old;
  src.pos0 = d.pos0;
  src.n_win = P.n_win;
  float M = -INFINITY, L = 0.f, K8[8] = {}, V8[8] = {};
  for (int sub = 0; sub < kSealSplit; ++sub) {
    float m, l, acck[8], accv[8];
    seal_part(P, src, d.id, sub * kSubTok, m, l, acck, accv);
    merge_part(M, L, K8, V8, m, l, acck, accv);
  }
  store_hca(P, d.id, L, K8, V8);
  if (threadIdx.x == 0) P.table[(int64_t)d.state * P.table_stride + d.pos0 / kBlk] = d.id;
}

// Bulk ring / indexer-tail write: token positions [w0, len_new) of each request go
// to ring slot p mod n_win; those of the open block (p >= 128 * nb_new) also to
// indexer-tail slot p mod 128. One workgroup per token, grid-strided.
__global__ __launch_bounds__(256) void k_bulk_write(Pools P, const WriteDesc* w, int32_t n_req,
                                                    int64_t total, const uint16_t* kin,
                                                    const uint16_t* vin, const float* iin) {
  const int tid = threadIdx.x;
  for (int64_t x = blockIdx.x; x < total; x += gridDim.x) {
    int r = 0;
    while (r + 1 < n_req && w[r + 1].cum <= x) ++r;
    const WriteDesc d = w[r];
    const int64_t p = d.w0 + (x - d.cum);
    const int64_t row = d.row0 + (p - d.len_old);
    const int64_t ring = ((int64_t)d.state * P.n_win + (p % P.n_win)) * kRow;
    reinterpret_cast<uint4*>(P.swa_k + ring)[tid] = reinterpret_cast<const uint4*>(kin + row * kRow)[tid];
    reinterpret_cast<uint4*>(P.swa_v + ring)[tid] = reinterpret_cast<const uint4*>(vin + row * kRow)[tid];
    if (p >= (int64_t)d.nb_new * kBlk && tid < kIRow / 4) {
      const int64_t ti = ((int64_t)d.state * kBlk + (p % kBlk)) * kIRow;
      reinterpret_cast<float4*>(P.idx_tail + ti)[tid] = reinterpret_cast<const float4*>(iin + row * kIRow)[tid];
    }
  }
}

}  // namespace

hipError_t launch_decode_append(const Pools& P, const ReqBatch& B, const void* kin, const void* vin,
                                const float* iin, float* part, hipStream_t st) {
  const int grid = B.n + kSealSplit * B.n_seal;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(k_decode_append, dim3(grid), dim3(256), 0, st, P, B,
                     static_cast<const uint16_t*>(kin), static_cast<const uint16_t*>(vin), iin, part);
  return hipGetLastError();
}

hipError_t launch_seal_merge(const Pools& P, const ReqBatch& B, const float* part, hipStream_t st) {
  if (B.n_seal == 0) return hipSuccess;
  hipLaunchKernelGGL(k_seal_merge, dim3(B.n_seal), dim3(256), 0, st, P, B, part);
  return hipGetLastError();
}

hipError_t launch_bulk_seal(const Pools& P, const SealDesc* seals, int64_t n_seals, const void* kin,
                            const void* vin, const float* iin, hipStream_t st) {
  if (n_seals == 0) return hipSuccess;
  hipLaunchKernelGGL(k_bulk_seal, dim3((unsigned)n_seals), dim3(256), 0, st, P, seals,
                     static_cast<const uint16_t*>(kin), static_cast<const uint16_t*>(vin), iin);
  return hipGetLastError();
}

hipError_t launch_bulk_write(const Pools& P, const WriteDesc* w, int32_t n_req, int64_t total,
                             const void* kin, const void* vin, const float* iin, hipStream_t st) {
  if (total == 0) return hipSuccess;
  const int64_t grid = total < 65536 ? total : 65536;
  hipLaunchKernelGGL(k_bulk_write, dim3((unsigned)grid), dim3(256), 0, st, P, w, n_req, total,
                     static_cast<const uint16_t*>(kin), static_cast<const uint16_t*>(vin), iin);
  return hipGetLastError();
}

}  // namespace hsa
