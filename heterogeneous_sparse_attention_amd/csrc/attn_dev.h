// attn_dev.h - streaming core of the heterogeneous decode attention (device code).
//
// Pages: [Q&A] "V4 为何要分池？块对齐与尾缓冲怎么配合？" §4 step 4 (attention reads the
// compressed entries of the Classical pool sparsely / densely plus the exact tail
// and SWA of the State pool); [Layout] "V4 KV Layout：Classical + State 双池",
// Classical KV cache (HCA entries attended densely, CSA entries through top-k).
//
// Each key is one 4 KiB K row and one 4 KiB V row (16 heads x 128 bf16). The
// contraction is 16 independent 128-long dot products per key (no operand is
// shared across heads), about 1 flop per byte, so it is bound by HBM bandwidth and
// runs on the vector ALUs. A wave takes one key at a time as four coalesced 1 KiB
// loads per row; lane l holds heads {l/16 + 4c} x dims (l%16)*8..+8 for c = 0..3,
// and the 16 lanes of a DPP row reduce one head's dot product. Key addresses of 64
// keys are resolved at once, one per lane, and broadcast with readlane, so the
// load stream has no dependent address loads; a ring of 4 or 5 keys per wave keeps
// all but one of them in flight while one is consumed.
#pragma once

#include "device.h"

namespace hsa {

constexpr int kAttnWaves = 4;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNoMax = -1e30f;   // running-max start: finite, so exp2 never sees inf - inf
constexpr float kQScale = 1.4426950408889634f * 0.08838834764831845f;   // log2(e) / sqrt(128)

struct KeyAddr {
  const uint16_t* k;
  const uint16_t* v;
};

template <int WAVES>
struct AttnSharedT {
  float acc[WAVES][kRow];
  float m[WAVES][kH];
  float l[WAVES][kH];
};
using AttnShared = AttnSharedT<kAttnWaves>;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b),
                                         c, false);
}

__device__ __forceinline__ const uint16_t* lane_ptr(uint64_t p, int i) {
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)p, i);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(p >> 32), i);
  return reinterpret_cast<const uint16_t*>(((uint64_t)hi << 32) | lo);
}

// Keys in the load ring of a wave: RING - 1 keys stay in flight while one is
// consumed. 5 keys fit the 512 VGPRs of a wave that has a SIMD to itself (4-wave
// workgroups); 8-wave workgroups (two waves per SIMD, 256 VGPRs each) take 3, as 4
// would spill.
template <int WAVES>
constexpr int ring_depth() { return WAVES > 4 ? 3 : 5; }

// Ring of the three-launch decode step's attention (8 waves, one workgroup per CU):
// one key in flight per wave while another is consumed. On the b32 workload this
// measured faster than 3 or 4: with every CU streaming, fewer requests in flight
// gather random rows from HBM at a higher rate.
constexpr int kMixedRing = 2;

// One key in the load ring. bf16 key: chunk c of the K and V rows (8 values each).
// FP8 key: .x/.y hold the chunk's 8 E4M3 codes and .z the scale of its head.
struct KeyRegs {
  uint4 k[4];
  uint4 v[4];
};

// Issue the loads of one key. bf16 key: pk / pv are its K and V rows. FP8 key: pk
// is its code row (K codes, then V codes) and pv its scale row (K scales, then V
// scales, head h at 4 (h % 4) + h / 4, so lane l's heads l/16 + 4c are 4 consecutive
// floats). The format is a template parameter, so every path of a loop issues the
// same number of loads and the compiler's wait counts stay exact.
template <bool F8>
__device__ __forceinline__ void load_key(KeyRegs& R, const uint16_t* pk, const uint16_t* pv, int lane) {
  if constexpr (!F8) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      R.k[c] = load_stream(reinterpret_cast<const uint4*>(pk + c * 512) + lane);
      R.v[c] = load_stream(reinterpret_cast<const uint4*>(pv + c * 512) + lane);
    }
  } else {
    const uint8_t* pq = reinterpret_cast<const uint8_t*>(pk);
    const float* ps = reinterpret_cast<const float*>(pv) + 4 * (lane >> 4);
    const float4 sk = load_global(reinterpret_cast<const float4*>(ps));
    const float4 sv = load_global(reinterpret_cast<const float4*>(ps + kH));
    const float skc[4] = {sk.x, sk.y, sk.z, sk.w};
    const float svc[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint2 a = load_stream(reinterpret_cast<const uint2*>(pq + c * 512) + lane);
      const uint2 b = load_stream(reinterpret_cast<const uint2*>(pq + kRow + c * 512) + lane);
      R.k[c] = make_uint4(a.x, a.y, __float_as_uint(skc[c]), 0u);
      R.v[c] = make_uint4(b.x, b.y, __float_as_uint(svc[c]), 0u);
    }
  }
}

// Online softmax update of this lane's 4 heads with one FP8 key: the codes become
// exact bf16 pairs for the dot product, whose sum takes the K scale; the V scale
// multiplies the softmax weight.
__device__ __forceinline__ void compute_key_fp8(const KeyRegs& R, bool ok, const uint4* qw, float* m,
                                                float* l, float (*acc)[8]) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    float kf[8];
    e4m3x4_to_f32(R.k[c].x, kf);
    e4m3x4_to_f32(R.k[c].y, kf + 4);
    float a = dot2(qw[c].x, pack_exact_bf2(kf[0], kf[1]), 0.f);
    a = dot2(qw[c].y, pack_exact_bf2(kf[2], kf[3]), a);
    a = dot2(qw[c].z, pack_exact_bf2(kf[4], kf[5]), a);
    a = dot2(qw[c].w, pack_exact_bf2(kf[6], kf[7]), a);
    const float s = ok ? row_sum16(a) * (kQScale * __uint_as_float(R.k[c].z)) : -INFINITY;
    const float mx = fmaxf(m[c], s);
    const float sc = exp2f(m[c] - mx);
    const float p = exp2f(s - mx);
    l[c] = fmaf(l[c], sc, p);
    // a skipped slot holds the bytes of a dummy bf16 row, which may read as the E4M3
    // NaN code: its codes are zeroed, so its weight 0 multiplies zeros
    const float pv = ok ? p * __uint_as_float(R.v[c].z) : 0.f;
    float vf[8];
    e4m3x4_to_f32(ok ? R.v[c].x : 0u, vf);
    e4m3x4_to_f32(ok ? R.v[c].y : 0u, vf + 4);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[c][i] = fmaf(pv, vf[i], acc[c][i] * sc);
    m[c] = mx;
  }
}

// Online softmax update of this lane's 4 heads with one key (bf16, or FP8 when F8).
template <bool F8>
__device__ __forceinline__ void compute_key(const KeyRegs& R, bool ok, const uint4* qw, float* m,
                                            float* l, float (*acc)[8]) {
  if constexpr (F8) {
    compute_key_fp8(R, ok, qw, m, l, acc);
    return;
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    float a = dot2(qw[c].x, R.k[c].x, 0.f);
    a = dot2(qw[c].y, R.k[c].y, a);
    a = dot2(qw[c].z, R.k[c].z, a);
    a = dot2(qw[c].w, R.k[c].w, a);
    const float s = ok ? row_sum16(a) * kQScale : -INFINITY;
    const float mx = fmaxf(m[c], s);
    const float sc = exp2f(m[c] - mx);
    const float p = exp2f(s - mx);
    l[c] = fmaf(l[c], sc, p);
    float vf[8];
    unpack8(R.v[c], vf);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[c][i] = fmaf(p, vf[i], acc[c][i] * sc);
    m[c] = mx;
  }
}

// The loads of keys [x0, min(x0 + RING - 1, x1)) of the current 64-key group into
// ring slots 0, 1, ... (lane x of kp / vp holds key x's rows).
template <int RING, bool F8>
__device__ __forceinline__ void ring_fill(KeyRegs (&ring)[RING], int x0, int x1, uint64_t kp, uint64_t vp,
                                          int lane) {
#pragma unroll
  for (int u = 0; u < RING - 1; ++u)
    if (x0 + u < x1) load_key<F8>(ring[u], lane_ptr(kp, x0 + u), lane_ptr(vp, x0 + u), lane);
}

// Keys [x0, x1) of the current 64-key group through the ring: on entry slot u holds
// key x0 + u (RING - 1 of them in flight); each step issues the loads of the key
// RING - 1 ahead and consumes one. A load issued on some paths only would make the
// compiler's wait for a key also wait for the loads behind it, so the steps issue
// one load each on every path: a 2-key ring loads a dummy row (dummy_k / dummy_v,
// valid rows of at least 4 KiB) past x1, one key's cost per run; deeper rings run
// unconditional passes while keys remain for every step of a pass, and only their
// last one or two passes load conditionally (a dummy per slot would cost more than
// the short waits it saves on runs of a few keys).
template <int RING, bool F8>
__device__ __forceinline__ void ring_run(KeyRegs (&ring)[RING], int x0, int x1, uint64_t kp, uint64_t vp,
                                         const uint16_t* dummy_k, const uint16_t* dummy_v, uint64_t okmask,
                                         const uint4* qw, float* m, float* l, float (*acc)[8], int lane) {
  int i = x0;
  if constexpr (RING == 2) {
    for (; i < x1; i += 2) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int x = i + u;
        if (x >= x1) break;
        const bool live = x + 1 < x1;
        const int j = live ? x + 1 : 0;
        load_key<F8>(ring[(u + 1) % 2], live ? lane_ptr(kp, j) : dummy_k, live ? lane_ptr(vp, j) : dummy_v, lane);
        compute_key<F8>(ring[u], (okmask >> x) & 1ull, qw, m, l, acc);
      }
    }
  } else {
    for (; i + 2 * RING - 2 < x1; i += RING) {
#pragma unroll
      for (int u = 0; u < RING; ++u) {
        const int x = i + u;
        load_key<F8>(ring[(u + RING - 1) % RING], lane_ptr(kp, x + RING - 1), lane_ptr(vp, x + RING - 1), lane);
        compute_key<F8>(ring[u], (okmask >> x) & 1ull, qw, m, l, acc);
      }
    }
    for (; i < x1; i += RING) {
#pragma unroll
      for (int u = 0; u < RING; ++u) {
        const int x = i + u;
        if (x >= x1) break;
        if (x + RING - 1 < x1)
          load_key<F8>(ring[(u + RING - 1) % RING], lane_ptr(kp, x + RING - 1), lane_ptr(vp, x + RING - 1),
                       lane);
        compute_key<F8>(ring[u], (okmask >> x) & 1ull, qw, m, l, acc);
      }
    }
  }
}

// Keys [x0, x1) of the current group, those below `split` in format F8LO and the
// others in F8HI: one ring run per format (a format change drains the ring).
template <int RING, bool F8LO, bool F8HI>
__device__ __forceinline__ void ring_runs(KeyRegs (&ring)[RING], int x0, int x1, int split, uint64_t kp,
                                          uint64_t vp, const uint16_t* dummy_k, const uint16_t* dummy_v,
                                          uint64_t okmask, const uint4* qw, float* m, float* l, float (*acc)[8],
                                          int lane) {
  if constexpr (F8LO == F8HI) {
    ring_fill<RING, F8LO>(ring, x0, x1, kp, vp, lane);
    ring_run<RING, F8LO>(ring, x0, x1, kp, vp, dummy_k, dummy_v, okmask, qw, m, l, acc, lane);
  } else {
    const int s = min(max(split, x0), x1);
    if (x0 < s) {
      ring_fill<RING, F8LO>(ring, x0, s, kp, vp, lane);
      ring_run<RING, F8LO>(ring, x0, s, kp, vp, dummy_k, dummy_v, okmask, qw, m, l, acc, lane);
    }
    if (s < x1) {
      ring_fill<RING, F8HI>(ring, s, x1, kp, vp, lane);
      ring_run<RING, F8HI>(ring, s, x1, kp, vp, dummy_k, dummy_v, okmask, qw, m, l, acc, lane);
    }
  }
}

// Merge the waves' running softmax states in LDS. On return threads t < 256 hold
// head t/16, dims (t%16)*8 .. +8 of the workgroup's unnormalised result.
template <int WAVES>
__device__ __forceinline__ void merge_waves(const float* m, const float* l, const float (*acc)[8],
                                            AttnSharedT<WAVES>& sh, float& M, float& L, float* A8) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int h = 4 * c + (lane >> 4);
    float4* dst = reinterpret_cast<float4*>(&sh.acc[wave][h * kD + (lane & 15) * 8]);
    dst[0] = make_float4(acc[c][0], acc[c][1], acc[c][2], acc[c][3]);
    dst[1] = make_float4(acc[c][4], acc[c][5], acc[c][6], acc[c][7]);
    if ((lane & 15) == 0) {
      sh.m[wave][h] = m[c];
      sh.l[wave][h] = l[c];
    }
  }
  __syncthreads();
  const int h = (tid >> 4) & (kH - 1);
  const int d0 = (tid & 15) * 8;
  M = kNoMax;
#pragma unroll
  for (int v = 0; v < WAVES; ++v) M = fmaxf(M, sh.m[v][h]);
  L = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) A8[i] = 0.f;
#pragma unroll
  for (int v = 0; v < WAVES; ++v) {
    const float wgt = exp2f(sh.m[v][h] - M);
    L = fmaf(wgt, sh.l[v][h], L);
#pragma unroll
    for (int i = 0; i < 8; ++i) A8[i] = fmaf(wgt, sh.acc[v][h * kD + d0 + i], A8[i]);
  }
}

// Attention of one workgroup of WAVES waves over keys [x0, x1) of one request:
// wave w streams a contiguous share. key_of(x) gives the K and V rows of key x (for
// an FP8 key: its code and scale rows) or nullptrs for a skipped slot; keys x <
// split are FP8 when F8LO, the others when F8HI. dummy_k / dummy_v are valid rows
// (at least 4 KiB) read in place of skipped keys. On return threads t < 256 hold
// head t/16, dims (t%16)*8 .. +8 of the unnormalised result: running max M (log2
// units), sum L, accumulator A8.
template <int WAVES, int RING, bool F8LO, bool F8HI, class KeyFn>
__device__ __forceinline__ void attend_keys(KeyFn key_of, int x0, int x1, const uint16_t* qrow,
                                            const uint16_t* dummy_k, const uint16_t* dummy_v,
                                            AttnSharedT<WAVES>& sh, float& M, float& L, float* A8,
                                            int split = 0x7fffffff) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int per = (x1 - x0 + WAVES - 1) / WAVES;
  const int w0 = x0 + wave * per;
  const int w1 = min(w0 + per, x1);

  uint4 qw[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) qw[c] = reinterpret_cast<const uint4*>(qrow + c * 512)[lane];
  float m[4], l[4], acc[4][8];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    m[c] = kNoMax;
    l[c] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[c][i] = 0.f;
  }
  KeyRegs ring[RING];
  for (int g = w0; g < w1; g += 64) {
    KeyAddr a;
    a.k = a.v = nullptr;
    if (g + lane < w1) a = key_of(g + lane);
    const bool okl = a.k != nullptr;
    const uint64_t okmask = __ballot(okl);
    const uint64_t kp = reinterpret_cast<uint64_t>(okl ? a.k : dummy_k);
    const uint64_t vp = reinterpret_cast<uint64_t>(okl ? a.v : dummy_v);
    ring_runs<RING, F8LO, F8HI>(ring, 0, min(64, w1 - g), split - g, kp, vp, dummy_k, dummy_v, okmask, qw, m, l,
                                acc, lane);
  }
  merge_waves<WAVES>(m, l, acc, sh, M, L, A8);
}

// Attention of one workgroup over two key lists of one request, A = [a0, a1) and
// B = [b0, b1), in one online softmax; A keys are in format F8A, B keys in F8B. The
// workgroup's keys are the list A then B; wave w takes positions w, w + WAVES,
// w + 2 WAVES, ... of it, so no wave has more than one key above the average, and
// every wave's A keys come first. The addresses of the B keys are known only after
// mid(), work that every wave of the workgroup runs once (it may hold barriers and
// must issue no global load). The loads of the A keys among each wave's first
// RING - 1 keys are issued before mid(), so they arrive while mid() runs; pre() runs
// just before (work that should wait for earlier loads first). key_a / key_b return the rows of a key (an FP8 key: its code and
// scale rows) or nullptrs for a skipped slot; dummy_k / dummy_v are valid rows (at
// least 4 KiB) read in their place. Result as attend_keys.
template <int WAVES, int RING, bool F8A, bool F8B, class KeyA, class KeyB, class Pre, class Mid>
__device__ __forceinline__ void attend_two(KeyA key_a, int a0, int a1, KeyB key_b, int b0, int b1, Pre pre, Mid mid,
                                           const uint16_t* qrow, const uint16_t* dummy_k,
                                           const uint16_t* dummy_v, AttnSharedT<WAVES>& sh, float& M,
                                           float& L, float* A8) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int nA = a1 - a0, nt = nA + (b1 - b0);
  // the wave's keys: j < n at list position wave + WAVES j; the first na are A keys
  const int n = wave < nt ? (nt - wave + WAVES - 1) / WAVES : 0;
  const int na = wave < nA ? (nA - wave + WAVES - 1) / WAVES : 0;
  auto pos = [&](int j) { return wave + WAVES * j; };

  uint4 qw[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) qw[c] = load_global(reinterpret_cast<const uint4*>(qrow + c * 512) + lane);
  float m[4], l[4], acc[4][8];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    m[c] = kNoMax;
    l[c] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[c][i] = 0.f;
  }
  auto key_j = [&](int j) { return j < na ? key_a(a0 + pos(j)) : key_b(b0 + pos(j) - nA); };

  // group 0: A addresses, then the prefetch of the wave's A keys among keys
  // [0, RING - 1)
  const int n0 = min(64, n);
  const int na0 = min(na, n0);
  KeyAddr a;
  a.k = a.v = nullptr;
  if (lane < na0) a = key_a(a0 + pos(lane));
  bool okl = a.k != nullptr;
  uint64_t kp = reinterpret_cast<uint64_t>(okl ? a.k : dummy_k);
  uint64_t vp = reinterpret_cast<uint64_t>(okl ? a.v : dummy_v);
  KeyRegs ring[RING];
  pre();
  ring_fill<RING, F8A>(ring, 0, na0, kp, vp, lane);
  mid();
  if (lane < n0 && lane >= na) {
    a = key_b(b0 + pos(lane) - nA);
    okl = a.k != nullptr;
    kp = reinterpret_cast<uint64_t>(okl ? a.k : dummy_k);
    vp = reinterpret_cast<uint64_t>(okl ? a.v : dummy_v);
  }
  uint64_t okmask = __ballot(okl);
  if constexpr (F8A == F8B) {
    // the ring's first slots past the A keys take their B keys
#pragma unroll
    for (int u = 0; u < RING - 1; ++u)
      if (u >= na0 && u < n0) load_key<F8B>(ring[u], lane_ptr(kp, u), lane_ptr(vp, u), lane);
    ring_run<RING, F8A>(ring, 0, n0, kp, vp, dummy_k, dummy_v, okmask, qw, m, l, acc, lane);
  } else {
    if (na0 > 0) ring_run<RING, F8A>(ring, 0, na0, kp, vp, dummy_k, dummy_v, okmask, qw, m, l, acc, lane);
    if (na0 < n0) {
      ring_fill<RING, F8B>(ring, na0, n0, kp, vp, lane);
      ring_run<RING, F8B>(ring, na0, n0, kp, vp, dummy_k, dummy_v, okmask, qw, m, l, acc, lane);
    }
  }
  for (int g = 64; g < n; g += 64) {
    const int ng = min(64, n - g);
    a.k = a.v = nullptr;
    if (lane < ng) a = key_j(g + lane);
    okl = a.k != nullptr;
    okmask = __ballot(okl);
    kp = reinterpret_cast<uint64_t>(okl ? a.k : dummy_k);
    vp = reinterpret_cast<uint64_t>(okl ? a.v : dummy_v);
    ring_runs<RING, F8A, F8B>(ring, 0, ng, na - g, kp, vp, dummy_k, dummy_v, okmask, qw, m, l, acc, lane);
  }
  merge_waves<WAVES>(m, l, acc, sh, M, L, A8);
}

// Store one partial: part_acc row [16][128] (thread t: head t/16, dims (t%16)*8),
// part_ml row [max 16][sum 16].
__device__ __forceinline__ void store_partial(float* part_acc, float* part_ml, int64_t idx, float M,
                                              float L, const float* A8) {
  const int tid = threadIdx.x;
  float* pa = part_acc + idx * kRow + tid * 8;
  reinterpret_cast<float4*>(pa)[0] = make_float4(A8[0], A8[1], A8[2], A8[3]);
  reinterpret_cast<float4*>(pa)[1] = make_float4(A8[4], A8[5], A8[6], A8[7]);
  if ((tid & 15) == 0) {
    part_ml[idx * 2 * kH + (tid >> 4)] = M;
    part_ml[idx * 2 * kH + kH + (tid >> 4)] = L;
  }
}

__device__ __forceinline__ void store_output(float* out_row, float L, const float* A8) {
  const float inv = 1.f / L;
  float4* o4 = reinterpret_cast<float4*>(out_row + threadIdx.x * 8);
  o4[0] = make_float4(A8[0] * inv, A8[1] * inv, A8[2] * inv, A8[3] * inv);
  o4[1] = make_float4(A8[4] * inv, A8[5] * inv, A8[6] * inv, A8[7] * inv);
}

// One extra key folded into a merge: its K and V rows and the request's query (bf16
// [16][128] each), or null pointers for none.
struct ExtraKey {
  const uint16_t* k;   // bf16 K row, or (fp8) the code row: K codes, then V codes
  const uint16_t* v;   // bf16 V row, or (fp8) the scale row: K scales, then V scales
  const uint16_t* q;
  bool fp8;
};

// Log-sum-exp merge of n partials (index of the j-th given by part_of(j), plain
// arithmetic) for one request into out_row, by one wave per head h; lane l writes
// dims 2l, 2l+1. Lane j holds partial j's max and sum; the partial rows are loaded
// together with them, so up to 32 partials cost one memory round trip. With
// xk.k set, the softmax also takes that key (score q.k / sqrt(128), weight on v),
// as one more partial of max s, sum 1 and accumulator v.
// The extra key of a merge for head h, lane l (dims 2l, 2l+1): its score xs (log2
// units, the same in every lane of the wave) and its V values; xs = kNoMax and zeros
// without one.
__device__ __forceinline__ void extra_key_lane(const ExtraKey& xk, int h, int lane, float& xs, float& xvx,
                                               float& xvy) {
  xs = kNoMax;
  xvx = xvy = 0.f;
  if (xk.k) {
    const int o = h * kD + 2 * lane;
    const uint32_t qw = *reinterpret_cast<const uint32_t*>(xk.q + o);
    float k0, k1;
    if (xk.fp8) {   // two codes of K and of V, and the head's scales
      const uint8_t* codes = reinterpret_cast<const uint8_t*>(xk.k);
      const float* sc = reinterpret_cast<const float*>(xk.v);
      const int hp = 4 * (h & 3) + (h >> 2);
      const f32x2_v kc = __builtin_amdgcn_cvt_pk_f32_fp8((int)*reinterpret_cast<const uint16_t*>(codes + o), false);
      const f32x2_v vc =
          __builtin_amdgcn_cvt_pk_f32_fp8((int)*reinterpret_cast<const uint16_t*>(codes + kRow + o), false);
      k0 = kc.x * sc[hp];
      k1 = kc.y * sc[hp];
      xvx = vc.x * sc[kH + hp];
      xvy = vc.y * sc[kH + hp];
    } else {
      const uint32_t kw = *reinterpret_cast<const uint32_t*>(xk.k + o);
      const uint32_t vw = *reinterpret_cast<const uint32_t*>(xk.v + o);
      k0 = bf_lo(kw);
      k1 = bf_hi(kw);
      xvx = bf_lo(vw);
      xvy = bf_hi(vw);
    }
    xs = wave_sum(fmaf(bf_lo(qw), k0, bf_hi(qw) * k1)) * kQScale;
  }
}

template <class PartFn>
__device__ __forceinline__ void merge_partials(PartFn part_of, int n, int h, const float* part_acc,
                                               const float* part_ml, float* out_row,
                                               ExtraKey xk = ExtraKey{nullptr, nullptr, nullptr, false}) {
  const int lane = threadIdx.x & 63;
  const float* accb = part_acc + h * kD + 2 * lane;
  float xs, xvx, xvy;
  extra_key_lane(xk, h, lane, xs, xvx, xvy);
  float ox = 0.f, oy = 0.f;
  if (n <= 64) {
    float2 a[32];
#pragma unroll
    for (int c = 0; c < 32; ++c)
      if (c < n) a[c] = *reinterpret_cast<const float2*>(accb + part_of(c) * kRow);
    float mm = kNoMax, ll = 0.f;
    if (lane < n) {
      const int64_t p = part_of(lane);
      mm = part_ml[p * 2 * kH + h];
      ll = part_ml[p * 2 * kH + kH + h];
    }
    float M = fmaxf(mm, __shfl_xor(mm, 32));
    M = fmaxf(M, __shfl_xor(M, 16));
    M = fmaxf(row_max16(M), xs);
    float w = lane < n ? exp2f(mm - M) : 0.f;
    const float xw = xk.k ? exp2f(xs - M) : 0.f;
    const float invL = 1.f / (wave_sum(w * ll) + xw);
    w *= invL;
    ox = xw * invL * xvx;
    oy = xw * invL * xvy;
#pragma unroll
    for (int c = 0; c < 32; ++c) {
      if (c < n) {
        const float wc = __shfl(w, c);
        ox = fmaf(wc, a[c].x, ox);
        oy = fmaf(wc, a[c].y, oy);
      }
    }
    if (n > 32) {
#pragma unroll
      for (int c = 0; c < 32; ++c)
        if (32 + c < n) a[c] = *reinterpret_cast<const float2*>(accb + part_of(32 + c) * kRow);
#pragma unroll
      for (int c = 0; c < 32; ++c) {
        if (32 + c < n) {
          const float wc = __shfl(w, 32 + c);
          ox = fmaf(wc, a[c].x, ox);
          oy = fmaf(wc, a[c].y, oy);
        }
      }
    }
  } else {
    float M = kNoMax;
    for (int c = lane; c < n; c += 64) M = fmaxf(M, part_ml[part_of(c) * 2 * kH + h]);
    M = fmaxf(M, __shfl_xor(M, 32));
    M = fmaxf(M, __shfl_xor(M, 16));
    M = fmaxf(row_max16(M), xs);
    float L = 0.f;
    for (int c = lane; c < n; c += 64) {
      const int64_t p = part_of(c);
      L += exp2f(part_ml[p * 2 * kH + h] - M) * part_ml[p * 2 * kH + kH + h];
    }
    const float xw = xk.k ? exp2f(xs - M) : 0.f;
    const float invL = 1.f / (wave_sum(L) + xw);
    ox = xw * invL * xvx;
    oy = xw * invL * xvy;
    // groups of 32 partials: the rows are loaded together, the weights are held by
    // lanes 0..31 and broadcast
    for (int g = 0; g < n; g += 32) {
      float2 a[32];
#pragma unroll
      for (int c = 0; c < 32; ++c)
        if (g + c < n) a[c] = *reinterpret_cast<const float2*>(accb + part_of(g + c) * kRow);
      const int cl = g + (lane & 31);
      const float w = cl < n ? exp2f(part_ml[part_of(cl) * 2 * kH + h] - M) * invL : 0.f;
#pragma unroll
      for (int c = 0; c < 32; ++c) {
        if (g + c < n) {
          const float wc = __shfl(w, c);
          ox = fmaf(wc, a[c].x, ox);
          oy = fmaf(wc, a[c].y, oy);
        }
      }
    }
  }
  *reinterpret_cast<float2*>(out_row + h * kD + 2 * lane) = make_float2(ox, oy);
}

// merge_partials for one head h of a request by a workgroup of WAVES waves, for
// requests with many partials: wave w takes partials w, w + WAVES, w + 2 WAVES, ...,
// 32 at a time (their max, sum and row loaded together, one memory round trip),
// keeping a running max, sum and unnormalised row; wave 0 combines the waves' states
// from LDS and writes dims 2l, 2l+1 in lane l. Same extra key as merge_partials.
template <int WAVES>
struct MergeShared {
  float m[WAVES];
  float s[WAVES];
  float o[WAVES][kD];
};

template <int WAVES, class PartFn>
__device__ __forceinline__ void merge_partials_split(PartFn part_of, int n, int h, const float* part_acc,
                                                     const float* part_ml, float* out_row, ExtraKey xk,
                                                     MergeShared<WAVES>& sh) {
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const float* accb = part_acc + h * kD + 2 * lane;
  const int nw = wave < n ? (n - wave + WAVES - 1) / WAVES : 0;   // partials wave + WAVES c, c < nw
  float M = kNoMax, S = 0.f, ox = 0.f, oy = 0.f;
  for (int g = 0; g < nw; g += 32) {
    float2 a[32];
#pragma unroll
    for (int c = 0; c < 32; ++c)
      if (g + c < nw) a[c] = *reinterpret_cast<const float2*>(accb + part_of(wave + WAVES * (g + c)) * kRow);
    const int cl = g + (lane & 31);
    const bool mine = lane < 32 && cl < nw;
    float mm = kNoMax, ll = 0.f;
    if (mine) {
      const int64_t p = part_of(wave + WAVES * cl);
      mm = part_ml[p * 2 * kH + h];
      ll = part_ml[p * 2 * kH + kH + h];
    }
    float Mg = fmaxf(mm, __shfl_xor(mm, 32));
    Mg = fmaxf(Mg, __shfl_xor(Mg, 16));
    const float Mn = fmaxf(M, row_max16(Mg));
    const float sc = exp2f(M - Mn);
    const float w = mine ? exp2f(mm - Mn) : 0.f;
    S = fmaf(S, sc, wave_sum(w * ll));
    ox *= sc;
    oy *= sc;
#pragma unroll
    for (int c = 0; c < 32; ++c) {
      if (g + c < nw) {
        const float wc = __shfl(w, c);
        ox = fmaf(wc, a[c].x, ox);
        oy = fmaf(wc, a[c].y, oy);
      }
    }
    M = Mn;
  }
  sh.o[wave][2 * lane] = ox;
  sh.o[wave][2 * lane + 1] = oy;
  if (lane == 0) {
    sh.m[wave] = M;
    sh.s[wave] = S;
  }
  __syncthreads();
  if (wave != 0) return;
  float xs, xvx, xvy;
  extra_key_lane(xk, h, lane, xs, xvx, xvy);
  float Mx = xs;
#pragma unroll
  for (int v = 0; v < WAVES; ++v) Mx = fmaxf(Mx, sh.m[v]);
  const float xw = xk.k ? exp2f(xs - Mx) : 0.f;
  float L = xw, rx = xw * xvx, ry = xw * xvy;
#pragma unroll
  for (int v = 0; v < WAVES; ++v) {
    const float e = exp2f(sh.m[v] - Mx);
    L = fmaf(e, sh.s[v], L);
    rx = fmaf(e, sh.o[v][2 * lane], rx);
    ry = fmaf(e, sh.o[v][2 * lane + 1], ry);
  }
  const float inv = 1.f / L;
  *reinterpret_cast<float2*>(out_row + h * kD + 2 * lane) = make_float2(rx * inv, ry * inv);
}

// Sum and max over each half of a wave (lanes 0-31, 32-63); every lane gets its half's.
__device__ __forceinline__ float half_sum(float v) {
  v = row_sum16(v);
  return v + __shfl_xor(v, 16);
}
__device__ __forceinline__ float half_max(float v) {
  v = row_max16(v);
  return fmaxf(v, __shfl_xor(v, 16));
}

// merge_partials for all 16 heads of a request by one 512-thread workgroup, so that
// the whole merge costs one memory round trip (up to 32 partials): head h is taken
// by threads 32h .. 32h + 31, lane j of them writes dims 4j .. 4j + 3 and holds the
// max and sum of partial j. Same extra key as merge_partials.
template <class PartFn>
__device__ __forceinline__ void merge_partials_wg(PartFn part_of, int n, const float* part_acc,
                                                  const float* part_ml, float* out_row, ExtraKey xk) {
  const int h = threadIdx.x >> 5;
  const int j = threadIdx.x & 31;
  const int src0 = threadIdx.x & 32;   // the wave lane that holds the half's partial 0
  const int o = h * kD + 4 * j;
  float xs = kNoMax;
  float4 xv = make_float4(0.f, 0.f, 0.f, 0.f);
  // the extra key's score and V values; its loads sit in a branch, where the compiler
  // waits for every load in flight, so it runs after the partials' loads are issued
  auto extra_key = [&]() {
    if (xk.k) {
      const uint2 qw = *reinterpret_cast<const uint2*>(xk.q + o);
      float kx[4];
      if (xk.fp8) {   // four codes of K and of V, and the head's scales
        const uint8_t* codes = reinterpret_cast<const uint8_t*>(xk.k);
        const float* sc = reinterpret_cast<const float*>(xk.v);
        const int hp = 4 * (h & 3) + (h >> 2);
        const int kc = (int)*reinterpret_cast<const uint32_t*>(codes + o);
        const int vc = (int)*reinterpret_cast<const uint32_t*>(codes + kRow + o);
        const float ks = sc[hp], vs = sc[kH + hp];
        const f32x2_v k01 = __builtin_amdgcn_cvt_pk_f32_fp8(kc, false), k23 = __builtin_amdgcn_cvt_pk_f32_fp8(kc, true);
        const f32x2_v v01 = __builtin_amdgcn_cvt_pk_f32_fp8(vc, false), v23 = __builtin_amdgcn_cvt_pk_f32_fp8(vc, true);
        kx[0] = k01.x * ks;
        kx[1] = k01.y * ks;
        kx[2] = k23.x * ks;
        kx[3] = k23.y * ks;
        xv = make_float4(v01.x * vs, v01.y * vs, v23.x * vs, v23.y * vs);
      } else {
        const uint2 kw = *reinterpret_cast<const uint2*>(xk.k + o);
        const uint2 vw = *reinterpret_cast<const uint2*>(xk.v + o);
        kx[0] = bf_lo(kw.x);
        kx[1] = bf_hi(kw.x);
        kx[2] = bf_lo(kw.y);
        kx[3] = bf_hi(kw.y);
        xv = make_float4(bf_lo(vw.x), bf_hi(vw.x), bf_lo(vw.y), bf_hi(vw.y));
      }
      const float d = fmaf(bf_lo(qw.x), kx[0], bf_hi(qw.x) * kx[1]) + fmaf(bf_lo(qw.y), kx[2], bf_hi(qw.y) * kx[3]);
      xs = half_sum(d) * kQScale;
    }
  };
  if (n > 32) extra_key();   // the merge in passes below: the key first, as its loads wait anyway
  float4 acc;
  auto add = [&](float w, const float4& a) {
    acc.x = fmaf(w, a.x, acc.x);
    acc.y = fmaf(w, a.y, acc.y);
    acc.z = fmaf(w, a.z, acc.z);
    acc.w = fmaf(w, a.w, acc.w);
  };
  if (n <= 32) {   // rows, maxima and sums in one round trip
    float4 a[32];
#pragma unroll
    for (int c = 0; c < 32; ++c)
      if (c < n) a[c] = *reinterpret_cast<const float4*>(part_acc + part_of(c) * kRow + o);
    float mm = kNoMax, ll = 0.f;
    if (j < n) {
      const int64_t p = part_of(j);
      mm = part_ml[p * 2 * kH + h];
      ll = part_ml[p * 2 * kH + kH + h];
    }
    extra_key();
    const float M = fmaxf(half_max(mm), xs);
    float w = j < n ? exp2f(mm - M) : 0.f;
    const float xw = xk.k ? exp2f(xs - M) : 0.f;
    const float invL = 1.f / (half_sum(w * ll) + xw);
    w *= invL;
    const float xwn = xw * invL;
    acc = make_float4(xwn * xv.x, xwn * xv.y, xwn * xv.z, xwn * xv.w);
#pragma unroll
    for (int c = 0; c < 32; ++c)
      if (c < n) add(__shfl(w, src0 + c), a[c]);
  } else {   // maxima, then sums, then the rows 32 partials at a time
    float M = kNoMax;
    for (int c = j; c < n; c += 32) M = fmaxf(M, part_ml[part_of(c) * 2 * kH + h]);
    M = fmaxf(half_max(M), xs);
    float L = 0.f;
    for (int c = j; c < n; c += 32) {
      const int64_t p = part_of(c);
      L += exp2f(part_ml[p * 2 * kH + h] - M) * part_ml[p * 2 * kH + kH + h];
    }
    const float xw = xk.k ? exp2f(xs - M) : 0.f;
    const float invL = 1.f / (half_sum(L) + xw);
    const float xwn = xw * invL;
    acc = make_float4(xwn * xv.x, xwn * xv.y, xwn * xv.z, xwn * xv.w);
    for (int g = 0; g < n; g += 32) {
      float4 a[32];
#pragma unroll
      for (int c = 0; c < 32; ++c)
        if (g + c < n) a[c] = *reinterpret_cast<const float4*>(part_acc + part_of(g + c) * kRow + o);
      const int cl = g + j;
      const float w = cl < n ? exp2f(part_ml[part_of(cl) * 2 * kH + h] - M) * invL : 0.f;
#pragma unroll
      for (int c = 0; c < 32; ++c)
        if (g + c < n) add(__shfl(w, src0 + c), a[c]);
    }
  }
  *reinterpret_cast<float4*>(out_row + o) = acc;
}

// Log-sum-exp merge of n partials of one request into one partial (unnormalised)
// at index dst, by one wave per head h; lane l holds dims 2l, 2l+1.
template <class PartFn>
__device__ __forceinline__ void merge_to_partial(PartFn part_of, int n, int h, float* part_acc,
                                                 float* part_ml, int64_t dst) {
  const int lane = threadIdx.x & 63;
  float M = kNoMax;
  for (int c = lane; c < n; c += 64) M = fmaxf(M, part_ml[part_of(c) * 2 * kH + h]);
  M = fmaxf(M, __shfl_xor(M, 32));
  M = fmaxf(M, __shfl_xor(M, 16));
  M = row_max16(M);
  float L = 0.f, ox = 0.f, oy = 0.f;
  for (int c = 0; c < n; ++c) {
    const int64_t p = part_of(c);
    const float w = exp2f(part_ml[p * 2 * kH + h] - M);
    L = fmaf(w, part_ml[p * 2 * kH + kH + h], L);
    const float2 v = *reinterpret_cast<const float2*>(part_acc + p * kRow + h * kD + 2 * lane);
    ox = fmaf(w, v.x, ox);
    oy = fmaf(w, v.y, oy);
  }
  *reinterpret_cast<float2*>(part_acc + dst * kRow + h * kD + 2 * lane) = make_float2(ox, oy);
  if (lane == 0) {
    part_ml[dst * 2 * kH + h] = M;
    part_ml[dst * 2 * kH + kH + h] = L;
  }
}

// For a workgroup-uniform index w over requests laid end to end with cnt(i) items
// each (i < n <= 64), find its request r and offset in it. Lane i evaluates
// cnt(i); a wave scan gives the prefix.
template <class CntFn>
__device__ __forceinline__ void find_item(int n, int w, CntFn cnt, int& r, int& off, int& first) {
  const int lane = threadIdx.x & 63;
  const int c = lane < n ? cnt(lane) : 0;
  int incl = c;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  const unsigned long long bal = __ballot(lane < n && incl > w);
  r = bal ? (int)__ffsll((long long)bal) - 1 : n - 1;
  first = __shfl(incl - c, r);
  off = w - first;
}

// Prefix (sum over i < r of cnt(i)) and total, lane-parallel as find_item.
template <class CntFn>
__device__ __forceinline__ void prefix_of(int n, int r, CntFn cnt, int& first, int& count) {
  const int lane = threadIdx.x & 63;
  const int c = lane < n ? cnt(lane) : 0;
  int incl = c;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  first = __shfl(incl - c, r);
  count = __shfl(c, r);
}

}  // namespace hsa
