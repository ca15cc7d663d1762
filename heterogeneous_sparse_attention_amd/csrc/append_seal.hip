// append_seal.hip - append tokens to the State and seal full blocks into the Block Cache.
//
// Pages: [Q&A] "V4 为何要分池？块对齐与尾缓冲怎么配合？" §3.1 (a token goes to the
// tail; a full block is compressed and appended to the Classical pool), §4 (the
// decode step: write the tail, compress on fill, slide the SWA); [Ch12] "Ch 12 ·
// 推理框架 — KV 的异构调度" §2.2 (each 128-token block yields 32 CSA + 1 HCA + 128
// indexer keys). The compressor stand-in and the seal thread layout are in
// seal_dev.h.
#include "device.h"
#include "kernels.h"
#include "seal_dev.h"

namespace hsa {

namespace {

// Decode append (one token per request) with the seal fused in.
// Workgroups [0, n): write request i's token into ring slot p mod n_win and
// indexer-tail slot p mod 128 (p = len - 1), and record a new block id in the
// device block table. Workgroups [n, n + kSealSplit * n_seal): seal one piece of
// a sealing request's block (2 C4 entries, 8 indexer keys, one HCA partial).
// No slot written by the first group is read by the second: the new token's
// ring slot differs from the 127 older ones (n_win >= 128), and its tail slot is
// 127, which the seal reads from the input instead.
// Templates: FP8 C4 entries; C4 false for layers without C4 entries; KV8 FP8 KV.
template <bool FP8, bool C4, bool KV8>
__global__ __launch_bounds__(256) void k_decode_append(Pools P, ReqBatch B, const uint16_t* kin,
                                                       const uint16_t* vin, const float* iin,
                                                       float* part) {
  const int bid = blockIdx.x;
  if (bid < B.n) {
    append_token<C4>(P, B.r[bid], bid, kin, vin, iin);
    return;
  }
  const int item = (bid - B.n) / kSealSplit;
  const int sub = (bid - B.n) % kSealSplit;
  const int ri = B.seal_req[item];
  seal_piece<FP8, C4, KV8>(P, B.r[ri], ri, item, sub, kin, vin, iin, part);
}

// One workgroup per block sealed by k_decode_append (next launch, so the partials
// are visible without a device-scope fence).
__global__ __launch_bounds__(256) void k_seal_merge(Pools P, ReqBatch B, const float* part) {
  seal_merge(P, B.r[B.seal_req[blockIdx.x]].aux, part, blockIdx.x);
}

// Bulk seal: one workgroup per block, its sixteen 8-token partials merged in
// registers in order. Templates: FP8 C4 entries; the layer keeps C4 entries (C4)
// and HCA entries (HCA); KV8 FP8 KV.
template <bool FP8, bool C4, bool HCA, bool KV8>
__global__ __launch_bounds__(256) void k_bulk_seal(Pools P, const SealDesc* seals,
                                                   const uint16_t* kin, const uint16_t* vin,
                                                   const float* iin) {
  const SealDesc d = seals[blockIdx.x];
  TokSrc src;
  ring_src(P, d.state, src);
  src.tail_i = P.idx_tail + (int64_t)d.state * kBlk * kIRow;
  // rows of positions >= len_old (row0 < 0 only when every token is resident)
  const int64_t row0 = d.row0 < 0 ? 0 : d.row0;
  src.in_k = kin ? kin + row0 * kRow : nullptr;
  src.in_v = vin ? vin + row0 * kRow : nullptr;
  src.in_i = iin ? iin + row0 * kIRow : nullptr;
  src.len_old = d.len_old;
  src.at_block(d.pos0, P.n_win);
  float M = -INFINITY, L = 0.f, K8[8] = {}, V8[8] = {};
  for (int sub = 0; sub < kSealSplit; ++sub) {
    float m, l, acck[8], accv[8];
    seal_part<FP8, C4, KV8>(P, src, d.id, sub * kSubTok, m, l, acck, accv);
    merge_part(M, L, K8, V8, m, l, acck, accv);
  }
  if constexpr (HCA) store_hca(P, d.id, L, K8, V8);
  if (threadIdx.x == 0) P.table[(int64_t)d.state * P.table_stride + d.pos0 / kBlk] = d.id;
}

// Bulk ring / indexer-tail write: token positions [w0, len_new) of each request go
// to ring slot p mod n_win; those of the open block (p >= 128 * nb_new) also to
// indexer-tail slot p mod 128. One workgroup per token, grid-strided.
__global__ __launch_bounds__(256) void k_bulk_write(Pools P, const WriteDesc* w, int32_t n_req,
                                                    int64_t total, const uint16_t* kin,
                                                    const uint16_t* vin, const float* iin) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  for (int64_t x = blockIdx.x; x < total; x += gridDim.x) {
    // the request owning token x: the number of descriptors with cum <= x, minus one
    // (cum is nondecreasing), counted 64 descriptors per ballot
    int r = -1;
    for (int base = 0; base < n_req; base += 64) {
      const int i = base + lane;
      const int c = __popcll(__ballot(i < n_req && w[i].cum <= x));
      r = base + c - 1;
      if (c < 64) break;
    }
    r = uniform(r);
    const WriteDesc d = w[r];
    const int64_t p = d.w0 + (x - d.cum);
    const int64_t row = d.row0 + (p - d.len_old);
    write_ring_token(P, (int64_t)d.state * P.n_win + (p % P.n_win), kin + row * kRow, vin + row * kRow);
    if (P.c4 && p >= (int64_t)d.nb_new * kBlk && tid < kIRow / 4) {
      const int64_t ti = ((int64_t)d.state * kBlk + (p % kBlk)) * kIRow;
      reinterpret_cast<float4*>(P.idx_tail + ti)[tid] = reinterpret_cast<const float4*>(iin + row * kIRow)[tid];
    }
  }
}

// Per-row FP8 storage: 16 rows of 128 floats per workgroup, lanes 16r .. 16r+15
// holding row r as 8 values each (the seal's per-head layout).
__global__ __launch_bounds__(256) void k_fp8_rows(const float* x, int64_t n_rows, uint8_t* codes,
                                                  float* scales) {
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  if (row >= n_rows) return;   // whole 16-lane rows, so the per-row max stays within active lanes
  const int col = (threadIdx.x & 15) * 8;
  const float4 a = reinterpret_cast<const float4*>(x + row * kD + col)[0];
  const float4 b = reinterpret_cast<const float4*>(x + row * kD + col)[1];
  const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  float sc;
  const uint2 q = quantize8_e4m3(v, sc);
  *reinterpret_cast<uint2*>(codes + row * kD + col) = q;
  if ((threadIdx.x & 15) == 0) scales[row] = sc;
}

// Eager C4: one workgroup per open-block entry, every token from the state's ring.
__global__ __launch_bounds__(256) void k_open_c4(Pools P, const OpenDesc* d) {
  const OpenDesc o = d[blockIdx.x];
  open_entry(P, o.state, o.nb, o.gi, -1, nullptr, nullptr);
}

// Table rows of attached states: one workgroup per state copies its block ids.
__global__ __launch_bounds__(256) void k_attach_rows(int32_t* table, int64_t stride, const AttachDesc* d,
                                                     const int32_t* ids) {
  const AttachDesc a = d[blockIdx.x];
  for (int64_t j = threadIdx.x; j < a.nb; j += 256)
    table[(int64_t)a.state * stride + j] = ids[a.off + j];
}

// Batched copy: chunk x belongs to the last segment whose first chunk is <= x
// (counted 64 segments per ballot); its workgroup moves up to 64 KiB, every thread
// with 16 loads in flight before its stores.
__global__ __launch_bounds__(256) void k_copy_segs(const CopySeg* s, int32_t n, int64_t total) {
  const int lane = threadIdx.x & 63;
  for (int64_t x = blockIdx.x; x < total; x += gridDim.x) {
    int r = -1;
    for (int base = 0; base < n; base += 64) {
      const int i = base + lane;
      const int c = __popcll(__ballot(i < n && s[i].first <= x));
      r = base + c - 1;
      if (c < 64) break;
    }
    r = uniform(r);
    const CopySeg d = s[r];
    const int64_t base = (x - d.first) * kCopyChunk16;
    const int64_t len = min((int64_t)kCopyChunk16, d.n16 - base);
    const HSA_GLOBAL u32x4_v* src = as_global(reinterpret_cast<const u32x4_v*>(d.src + base));
    HSA_GLOBAL u32x4_v* dst = as_global(reinterpret_cast<u32x4_v*>(d.dst + base));
    if (len == kCopyChunk16) {   // a whole chunk: unguarded, so the words stay in registers
      u32x4_v v[kCopyChunk16 / 256];
#pragma unroll
      for (int u = 0; u < kCopyChunk16 / 256; ++u) v[u] = src[threadIdx.x + u * 256];
#pragma unroll
      for (int u = 0; u < kCopyChunk16 / 256; ++u) dst[threadIdx.x + u * 256] = v[u];
    } else {
      for (int64_t w = threadIdx.x; w < len; w += 256) dst[w] = src[w];
    }
  }
}

// MXFP4 storage of indexer key rows (256 fp32 each), exactly as the seal stores
// them: a wave per row, 4 rows per workgroup.
__global__ __launch_bounds__(256) void k_mx4_rows(const float* x, int64_t n_rows, uint8_t* codes,
                                                  uint8_t* scales) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n_rows) return;   // whole waves, so the 8-lane scale reduction stays within active lanes
  const int c = threadIdx.x & 63;
  const float4 v = reinterpret_cast<const float4*>(x + row * kIRow)[c];
  mx4_store_row(v, c, codes + row * kIRowQ, scales + row * kIRowE);
}

}  // namespace

hipError_t launch_open_c4(const Pools& P, const OpenDesc* d, int32_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  return launch_k(k_open_c4, dim3((unsigned)n), dim3(256), st, LaunchEv{}, P, d);
}

hipError_t launch_copy_segs(const CopySeg* d, int32_t n, int64_t total, hipStream_t st) {
  if (n <= 0 || total <= 0) return hipSuccess;
  const int64_t grid = std::min<int64_t>(total, 8 * 256);   // grid-strided beyond 8 per CU
  return launch_k(k_copy_segs, dim3((unsigned)grid), dim3(256), st, LaunchEv{}, d, n, total);
}

hipError_t launch_attach_rows(const Pools& P, const AttachDesc* d, int32_t n, const int32_t* ids,
                              hipStream_t st) {
  if (n <= 0) return hipSuccess;
  return launch_k(k_attach_rows, dim3((unsigned)n), dim3(256), st, LaunchEv{}, P.table, P.table_stride, d,
                  ids);
}

hipError_t launch_mx4_rows(const float* x, int64_t n_rows, uint8_t* codes, uint8_t* scales,
                           hipStream_t st) {
  if (n_rows <= 0) return hipSuccess;
  return launch_k(k_mx4_rows, dim3((unsigned)((n_rows + 3) / 4)), dim3(256), st, LaunchEv{}, x,
                  n_rows, codes, scales);
}

hipError_t launch_fp8_rows(const float* x, int64_t n_rows, uint8_t* codes, float* scales,
                           hipStream_t st) {
  if (n_rows <= 0) return hipSuccess;
  return launch_k(k_fp8_rows, dim3((unsigned)((n_rows + 15) / 16)), dim3(256), st, LaunchEv{}, x,
                  n_rows, codes, scales);
}

hipError_t launch_decode_append(const Pools& P, const ReqBatch& B, const void* kin, const void* vin,
                                const float* iin, float* part, hipStream_t st,
                 const LaunchEv& ev) {
  const int grid = B.n + kSealSplit * B.n_seal;
  if (grid == 0) return hipSuccess;
  const uint16_t* k = static_cast<const uint16_t*>(kin);
  const uint16_t* v = static_cast<const uint16_t*>(vin);
  const dim3 g(grid), t(256);
  if (P.kv8) {
    if (!P.c4) return launch_k(k_decode_append<false, false, true>, g, t, st, ev, P, B, k, v, iin, part);
    if (P.fp8) return launch_k(k_decode_append<true, true, true>, g, t, st, ev, P, B, k, v, iin, part);
    return launch_k(k_decode_append<false, true, true>, g, t, st, ev, P, B, k, v, iin, part);
  }
  if (!P.c4) return launch_k(k_decode_append<false, false, false>, g, t, st, ev, P, B, k, v, iin, part);
  if (P.fp8) return launch_k(k_decode_append<true, true, false>, g, t, st, ev, P, B, k, v, iin, part);
  return launch_k(k_decode_append<false, true, false>, g, t, st, ev, P, B, k, v, iin, part);
}

hipError_t launch_seal_merge(const Pools& P, const ReqBatch& B, const float* part, hipStream_t st,
                 const LaunchEv& ev) {
  if (B.n_seal == 0) return hipSuccess;
  return launch_k(k_seal_merge, dim3(B.n_seal), dim3(256), st, ev, P, B, part);
}

hipError_t launch_bulk_seal(const Pools& P, const SealDesc* seals, int64_t n_seals, const void* kin,
                            const void* vin, const float* iin, hipStream_t st,
                 const LaunchEv& ev) {
  if (n_seals == 0) return hipSuccess;
  const dim3 g((unsigned)n_seals);
  const uint16_t* k = static_cast<const uint16_t*>(kin);
  const uint16_t* v = static_cast<const uint16_t*>(vin);
  const dim3 t(256);
  if (P.kv8) {
    if (!P.c4) return launch_k(k_bulk_seal<false, false, true, true>, g, t, st, ev, P, seals, k, v, iin);
    if (P.fp8 && P.hca) return launch_k(k_bulk_seal<true, true, true, true>, g, t, st, ev, P, seals, k, v, iin);
    if (P.fp8) return launch_k(k_bulk_seal<true, true, false, true>, g, t, st, ev, P, seals, k, v, iin);
    if (P.hca) return launch_k(k_bulk_seal<false, true, true, true>, g, t, st, ev, P, seals, k, v, iin);
    return launch_k(k_bulk_seal<false, true, false, true>, g, t, st, ev, P, seals, k, v, iin);
  }
  if (!P.c4) return launch_k(k_bulk_seal<false, false, true, false>, g, t, st, ev, P, seals, k, v, iin);
  if (P.fp8 && P.hca) return launch_k(k_bulk_seal<true, true, true, false>, g, t, st, ev, P, seals, k, v, iin);
  if (P.fp8) return launch_k(k_bulk_seal<true, true, false, false>, g, t, st, ev, P, seals, k, v, iin);
  if (P.hca) return launch_k(k_bulk_seal<false, true, true, false>, g, t, st, ev, P, seals, k, v, iin);
  return launch_k(k_bulk_seal<false, true, false, false>, g, t, st, ev, P, seals, k, v, iin);
}

hipError_t launch_bulk_write(const Pools& P, const WriteDesc* w, int32_t n_req, int64_t total,
                             const void* kin, const void* vin, const float* iin, hipStream_t st,
                 const LaunchEv& ev) {
  if (total == 0) return hipSuccess;
  const int64_t grid = total < 65536 ? total : 65536;
  return launch_k(k_bulk_write, dim3((unsigned)grid), dim3(256), st, ev, P, w, n_req, total,
                     static_cast<const uint16_t*>(kin), static_cast<const uint16_t*>(vin), iin);
}

}  // namespace hsa
