// seal_dev.h - compression of a full 128-token block (device code).
//
// Pages: [Q&A] "V4 为何要分池？块对齐与尾缓冲怎么配合？" §2.1 (m consecutive tokens'
// K/V compress into one entry, aligned to the block), §3.1 (a full block is
// compressed and appended to the Classical pool); [Ch12] "Ch 12 · 推理框架 — KV 的
// 异构调度" §2.2 (each block yields 32 CSA + 1 HCA + 128 indexer keys).
//
// The compressor is not defined on the pages; the stand-in is gated pooling: per
// head h, g_t = <W[h], K_t[h]>, alpha = softmax over the group's tokens, entry =
// sum_t alpha_t (K_t[h], V_t[h]), stored as bf16 (round to nearest even). C4 entry
// j of a block pools tokens 4j..4j+3 with W_csa; the HCA entry pools all 128 with
// W_hca, as sixteen 8-token softmax partials folded in order.
//
// Thread layout (256 lanes): lane t owns head t/16 and dims (t%16)*8 .. +8 of every
// token, i.e. 16 contiguous bytes of each 4 KiB K or V row, so a token is one
// coalesced 4 KiB read per workgroup and the 16 lanes of a head form one DPP row
// for the gate reduction.
#pragma once

#include "device.h"

namespace hsa {

// Where token t of the block being sealed lives: in the state (ring slot, indexer
// tail slot) if its position precedes len_old, else in the packed input. With FP8
// KV the ring slots hold codes and scales (ring_q, ring_s: the state's first slot).
struct TokSrc {
  const uint16_t* ring_k;
  const uint16_t* ring_v;
  const uint8_t* ring_q;
  const float* ring_s;
  const float* tail_i;
  const uint16_t* in_k;
  const uint16_t* in_v;
  const float* in_i;
  int64_t pos0, len_old;
  int32_t slot0;   // ring slot of position pos0

  // pos0 is a block start and n_win a multiple of 128, so slot0 is a multiple of 128
  // and token t's ring slot slot0 + t (tail slot t) needs no division: a 64-bit
  // modulo per token would put each token's loads in a block of its own
  __device__ __forceinline__ void at_block(int64_t p0, int32_t n_win) {
    pos0 = p0;
    slot0 = (int32_t)(p0 % n_win);
  }
  __device__ __forceinline__ bool resident(int t) const { return pos0 + t < len_old; }
  __device__ __forceinline__ const uint16_t* k(int t) const {
    const int64_t p = pos0 + t;
    return p < len_old ? ring_k + (int64_t)(slot0 + t) * kRow : in_k + (p - len_old) * kRow;
  }
  __device__ __forceinline__ const uint16_t* v(int t) const {
    const int64_t p = pos0 + t;
    return p < len_old ? ring_v + (int64_t)(slot0 + t) * kRow : in_v + (p - len_old) * kRow;
  }
  __device__ __forceinline__ const float* i(int t) const {
    const int64_t p = pos0 + t;
    return p < len_old ? tail_i + (int64_t)t * kIRow : in_i + (p - len_old) * kIRow;
  }
  __device__ __forceinline__ const uint16_t* in_krow(int t) const { return in_k + (pos0 + t - len_old) * kRow; }
  __device__ __forceinline__ const uint16_t* in_vrow(int t) const { return in_v + (pos0 + t - len_old) * kRow; }
  __device__ __forceinline__ int64_t slot(int t) const { return slot0 + t; }
};

// This lane's 8 values (at off = 8 tid: head tid / 16) of token t's K and V, as the
// State stores them. bf16 KV: the bf16 values, scales 1. FP8 KV (KV8): the E4M3
// code values as exact bf16 pairs and the head's K and V scales (value = code *
// scale); a token still in the input is quantised here exactly as the ring write
// stores it (same lanes, same per-head maximum), so both give the same bits.
__device__ __forceinline__ void load_ring_tok(const TokSrc& src, int t, int off, uint4& kw, uint4& vw,
                                              float& sk, float& sv) {
  const int h = threadIdx.x >> 4;
  const int64_t g = src.slot(t);
  const uint8_t* q = src.ring_q + g * kC4Bytes;
  kw = e4m3x8_to_bf16(*reinterpret_cast<const uint2*>(q + off));
  vw = e4m3x8_to_bf16(*reinterpret_cast<const uint2*>(q + kRow + off));
  const float* sc = src.ring_s + g * kC4Scales;
  sk = sc[4 * (h & 3) + (h >> 2)];
  sv = sc[kH + 4 * (h & 3) + (h >> 2)];
}
__device__ __forceinline__ void load_input_tok(const TokSrc& src, int t, int off, uint4& kw, uint4& vw,
                                               float& sk, float& sv) {
  float f[8];
  unpack8(*reinterpret_cast<const uint4*>(src.in_krow(t) + off), f);
  kw = e4m3x8_to_bf16(quantize8_e4m3(f, sk));
  unpack8(*reinterpret_cast<const uint4*>(src.in_vrow(t) + off), f);
  vw = e4m3x8_to_bf16(quantize8_e4m3(f, sv));
}

template <bool KV8>
__device__ __forceinline__ void load_tok(const TokSrc& src, int t, int off, uint4& kw, uint4& vw, float& sk,
                                         float& sv) {
  if constexpr (!KV8) {
    kw = *reinterpret_cast<const uint4*>(src.k(t) + off);
    vw = *reinterpret_cast<const uint4*>(src.v(t) + off);
    sk = sv = 1.f;
  } else {
    if (src.resident(t))   // workgroup-uniform
      load_ring_tok(src, t, off, kw, vw, sk, sv);
    else
      load_input_tok(src, t, off, kw, vw, sk, sv);
  }
}

// The 4 tokens tb .. tb + 3 of a group. With FP8 KV, one uniform branch per group
// (positions increase with t: the whole group in the ring, the whole group in the
// input, or, once per block at most, split between them), so that the group's loads
// are issued together: a load inside a per-token branch makes the compiler wait for
// every load in flight where the branch joins.
template <bool KV8>
__device__ __forceinline__ void load_group(const TokSrc& src, int tb, int off, uint4* kw, uint4* vw, float* sk,
                                           float* sv) {
  if constexpr (!KV8) {
#pragma unroll
    for (int u = 0; u < 4; ++u) load_tok<false>(src, tb + u, off, kw[u], vw[u], sk[u], sv[u]);
  } else {
    if (src.resident(tb + 3)) {
#pragma unroll
      for (int u = 0; u < 4; ++u) load_ring_tok(src, tb + u, off, kw[u], vw[u], sk[u], sv[u]);
    } else if (!src.resident(tb)) {
#pragma unroll
      for (int u = 0; u < 4; ++u) load_input_tok(src, tb + u, off, kw[u], vw[u], sk[u], sv[u]);
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) load_tok<true>(src, tb + u, off, kw[u], vw[u], sk[u], sv[u]);
    }
  }
}

constexpr int kSubTok = kBlk / kSealSplit;   // 8 tokens per seal partial

// C4 entry of 4 tokens: this lane's 8 dims of each (packed bf16) and their CSA gate
// logits gc (<W_csa[h], K_t[h]>); softmax over the 4 gates, the weighted sums of K
// and V, stored in C4 row `row` as bf16 or, with FP8, as per-head E4M3 codes and a
// scale (lanes 16h .. 16h+15 hold head h, so the scale's max runs over one DPP row).
// The seal and the eager entries of an open block both store through it, so an
// entry is the same bits before and after its block seals.
// With FP8 KV (KV8) the tokens' values are code values and sk / sv their per-token
// K and V scales, folded into the pooling weights.
template <bool FP8, bool KV8 = false>
__device__ __forceinline__ void c4_pool_store(const Pools& P, int64_t row, const uint4* kw, const uint4* vw,
                                              const float* gc, const float* sk = nullptr,
                                              const float* sv = nullptr) {
  const int tid = threadIdx.x;
  const int h = tid >> 4;
  const int off = tid * 8;
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
  for (int i = 0; i < 8; ++i) ck[i] = cv[i] = 0.f;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    float kf[8], vf[8];
    unpack8(kw[u], kf);
    unpack8(vw[u], vf);
    const float ek = KV8 ? e[u] * sk[u] : e[u];
    const float ev = KV8 ? e[u] * sv[u] : e[u];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ck[i] = fmaf(ek, kf[i], ck[i]);
      cv[i] = fmaf(ev, vf[i], cv[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    ck[i] *= inv;
    cv[i] *= inv;
  }
  if (FP8) {
    (void)h;
    store_row_fp8(ck, P.c4q + row * kC4Bytes, P.c4s + row * kC4Scales);
    store_row_fp8(cv, P.c4q + row * kC4Bytes + kRow, P.c4s + row * kC4Scales + kH);
  } else {
    uint4 ok, ov;
    ok.x = pack_bf2(ck[0], ck[1]); ok.y = pack_bf2(ck[2], ck[3]);
    ok.z = pack_bf2(ck[4], ck[5]); ok.w = pack_bf2(ck[6], ck[7]);
    ov.x = pack_bf2(cv[0], cv[1]); ov.y = pack_bf2(cv[2], cv[3]);
    ov.z = pack_bf2(cv[4], cv[5]); ov.w = pack_bf2(cv[6], cv[7]);
    *reinterpret_cast<uint4*>(P.csa_k + row * kRow + off) = ok;
    *reinterpret_cast<uint4*>(P.csa_v + row * kRow + off) = ov;
  }
}

// Eager C4: entry `gi` of state `state`'s open block (logical block nb), from the
// state's ring, except the token at position `in_pos`, read from `in_k` / `in_v`
// (the token appended in the same launch; -1: none). Gate logits and pooling are
// the seal's own, so the entry is bit-identical to the one the seal stores later.
// Also points the table entry of the open block at the state's open block.
__device__ __forceinline__ void open_entry(const Pools& P, int32_t state, int32_t nb, int gi,
                                           int64_t in_pos, const uint16_t* in_k, const uint16_t* in_v) {
  const int tid = threadIdx.x;
  const int off = tid * 8;
  float wc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) wc[i] = P.gate_csa[off + i];
  const int64_t p0 = (int64_t)kBlk * nb + 4 * gi;
  uint4 kw[4], vw[4];
  float gc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t p = p0 + u;
    const int64_t ring = ((int64_t)state * P.n_win + p % P.n_win) * kRow;
    kw[u] = *reinterpret_cast<const uint4*>((p == in_pos ? in_k : P.swa_k + ring) + off);
    vw[u] = *reinterpret_cast<const uint4*>((p == in_pos ? in_v : P.swa_v + ring) + off);
    float kf[8];
    unpack8(kw[u], kf);
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) a = fmaf(wc[i], kf[i], a);
    gc[u] = row_sum16(a);
  }
  c4_pool_store<false>(P, (int64_t)(P.max_blocks + state) * kC4 + gi, kw, vw, gc);
  if (tid == 0) P.table[(int64_t)state * P.table_stride + nb] = P.max_blocks + state;
}

// Seal tokens [t0, t0 + kSubTok) of one block (C4 entries bf16, or FP8 when FP8,
// which the caller sets from P.fp8; C4 false for layers without C4 entries, set
// from P.c4): writes their kSubTok / 4 C4 entries and kSubTok indexer keys, and
// returns the HCA softmax partial (m, l, acc) of these tokens for this lane's 8
// dims. Both seal paths build the HCA entry from the same kSealSplit partials
// merged in the same order, so bulk and one-token appends give bit-identical
// blocks.
template <bool FP8, bool C4, bool KV8 = false>
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
  float* idx_dst = P.idx_k + (int64_t)id * kBlk * kIRow;

  m = -INFINITY;
  l = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) acck[i] = accv[i] = 0.f;

#pragma unroll 1
  for (int g = 0; g < kSubTok / 4; ++g) {
    const int tb = t0 + 4 * g;
    uint4 kw[4], vw[4];
    float sk[4], sv[4];   // FP8 KV: the tokens' per-head scales (1 with bf16 KV)
    load_group<KV8>(src, tb, off, kw, vw, sk, sv);
    // indexer keys of the 4 tokens: 4 x 64 float4, one per lane (stored as MXFP4
    // when P.mx4, a wave per key); layers without C4 entries keep none
    if constexpr (C4) {
      const int u = tid >> 6, c = tid & 63;
      const float4 iv = reinterpret_cast<const float4*>(src.i(tb + u))[c];
      if (P.mx4) {
        const int64_t kr = (int64_t)id * kBlk + tb + u;
        mx4_store_row(iv, c, P.idx_q + kr * kIRowQ, P.idx_e + kr * kIRowE);
      } else {
        reinterpret_cast<float4*>(idx_dst + (int64_t)(tb + u) * kIRow)[c] = iv;
      }
    }
    // the tokens stay packed (bf16 pairs) and are unpacked where used, which keeps
    // the register count low enough for the scoring workgroups of the same launch
    float gc[4], gh[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float kf[8];
      unpack8(kw[u], kf);
      float a = 0.f, b = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        a = fmaf(wc[i], kf[i], a);
        b = fmaf(wh[i], kf[i], b);
      }
      gc[u] = row_sum16(a);
      gh[u] = row_sum16(b);
      if constexpr (KV8) {
        gc[u] *= sk[u];
        gh[u] *= sk[u];
      }
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
        acck[i] *= sc;
        accv[i] *= sc;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float kf[8], vf[8];
        unpack8(kw[u], kf);
        unpack8(vw[u], vf);
        const float ek = KV8 ? e[u] * sk[u] : e[u];
        const float ev = KV8 ? e[u] * sv[u] : e[u];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          acck[i] = fmaf(ek, kf[i], acck[i]);
          accv[i] = fmaf(ev, vf[i], accv[i]);
        }
      }
      m = mx;
    }
    // C4 entry (tokens tb .. tb+3) after the HCA update, so the packed tokens are
    // dead while an FP8 entry is quantised
    if constexpr (C4) c4_pool_store<FP8, KV8>(P, (int64_t)id * kC4 + (tb >> 2), kw, vw, gc, sk, sv);
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
  if (P.kv8) {   // FP8 KV: per-head E4M3 codes and scales
    float k8[8], v8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      k8[i] = acck[i] * inv;
      v8[i] = accv[i] * inv;
    }
    store_row_fp8(k8, P.hcq + (int64_t)id * kC4Bytes, P.hcs + (int64_t)id * kC4Scales);
    store_row_fp8(v8, P.hcq + (int64_t)id * kC4Bytes + kRow, P.hcs + (int64_t)id * kC4Scales + kH);
    return;
  }
  uint4 ok, ov;
  ok.x = pack_bf2(acck[0] * inv, acck[1] * inv); ok.y = pack_bf2(acck[2] * inv, acck[3] * inv);
  ok.z = pack_bf2(acck[4] * inv, acck[5] * inv); ok.w = pack_bf2(acck[6] * inv, acck[7] * inv);
  ov.x = pack_bf2(accv[0] * inv, accv[1] * inv); ov.y = pack_bf2(accv[2] * inv, accv[3] * inv);
  ov.z = pack_bf2(accv[4] * inv, accv[5] * inv); ov.w = pack_bf2(accv[6] * inv, accv[7] * inv);
  *reinterpret_cast<uint4*>(P.hca_k + (int64_t)id * kRow + off) = ok;
  *reinterpret_cast<uint4*>(P.hca_v + (int64_t)id * kRow + off) = ov;
}

// Decode-time append of request i's one new token (position p = r.len - 1): ring
// slot p mod n_win, indexer-tail slot p mod 128, and the device table entry of a
// block the token seals (r.aux = its id, else -1). 256 threads.
// Write one token's K and V rows (bf16 input rows krow, vrow) into ring slot g =
// state * n_win + p % n_win, as bf16 or (FP8 KV) as per-head codes and scales.
// 256 threads, each 8 values of each row.
__device__ __forceinline__ void write_ring_token(const Pools& P, int64_t g, const uint16_t* krow,
                                                 const uint16_t* vrow) {
  const int tid = threadIdx.x;
  const uint4 kw = reinterpret_cast<const uint4*>(krow)[tid];
  const uint4 vw = reinterpret_cast<const uint4*>(vrow)[tid];
  if (P.kv8) {
    float f[8];
    unpack8(kw, f);
    store_row_fp8(f, P.swq + g * kC4Bytes, P.sws + g * kC4Scales);
    unpack8(vw, f);
    store_row_fp8(f, P.swq + g * kC4Bytes + kRow, P.sws + g * kC4Scales + kH);
    return;
  }
  reinterpret_cast<uint4*>(P.swa_k + g * kRow)[tid] = kw;
  reinterpret_cast<uint4*>(P.swa_v + g * kRow)[tid] = vw;
}

template <bool C4>
__device__ __forceinline__ void append_token(const Pools& P, const Req& r, int i,
                                             const uint16_t* kin, const uint16_t* vin,
                                             const float* iin) {
  const int tid = threadIdx.x;
  const int64_t p = r.len - 1;
  write_ring_token(P, (int64_t)r.state * P.n_win + (p % P.n_win), kin + (int64_t)i * kRow, vin + (int64_t)i * kRow);
  if (C4 && tid < kIRow / 4) {   // the indexer tail (layers with C4 entries)
    const int64_t ti = ((int64_t)r.state * kBlk + (p % kBlk)) * kIRow;
    reinterpret_cast<float4*>(P.idx_tail + ti)[tid] =
        reinterpret_cast<const float4*>(iin + (int64_t)i * kIRow)[tid];
  }
  if (tid == 0 && r.aux >= 0) P.table[(int64_t)r.state * P.table_stride + (r.nb - 1)] = r.aux;
}

// The state's ring as a token source of the seal (bf16 rows, or FP8 codes and scales).
__device__ __forceinline__ void ring_src(const Pools& P, int32_t state, TokSrc& src) {
  const int64_t g0 = (int64_t)state * P.n_win;
  src.ring_k = P.kv8 ? nullptr : P.swa_k + g0 * kRow;
  src.ring_v = P.kv8 ? nullptr : P.swa_v + g0 * kRow;
  src.ring_q = P.kv8 ? P.swq + g0 * kC4Bytes : nullptr;
  src.ring_s = P.kv8 ? P.sws + g0 * kC4Scales : nullptr;
}

// One piece (kSubTok = 8 tokens) of the decode-time seal of request i's block r.aux:
// its 2 C4 entries, 8 indexer keys and one HCA partial to part[item * kSealSplit +
// sub]. The newest token (position r.len - 1) is read from input row i, so this
// may run in the same launch as append_token. 256 threads.
template <bool FP8, bool C4, bool KV8 = false>
__device__ __forceinline__ void seal_piece(const Pools& P, const Req& r, int i, int item, int sub,
                                           const uint16_t* kin, const uint16_t* vin,
                                           const float* iin, float* part) {
  const int tid = threadIdx.x;
  TokSrc src;
  ring_src(P, r.state, src);
  src.tail_i = P.idx_tail + (int64_t)r.state * kBlk * kIRow;
  src.in_k = kin + (int64_t)i * kRow;
  src.in_v = vin + (int64_t)i * kRow;
  src.in_i = iin + (int64_t)i * kIRow;
  src.len_old = r.len - 1;
  src.at_block((int64_t)(r.nb - 1) * kBlk, P.n_win);
  float m, l, acck[8], accv[8];
  seal_part<FP8, C4, KV8>(P, src, r.aux, sub * kSubTok, m, l, acck, accv);
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

// Fold the kSealSplit HCA partials of seal `item` in order (the arithmetic of the bulk
// seal) and store block id's HCA entry. Threads 0..255 take part (of 256 or more).
__device__ __forceinline__ void seal_merge(const Pools& P, int32_t id, const float* part, int item) {
  const int tid = threadIdx.x;
  if (tid >= 256) return;
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
  store_hca(P, id, L, K8, V8);
}

}  // namespace hsa
