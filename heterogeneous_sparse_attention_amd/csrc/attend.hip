// attend.hip - heterogeneous decode attention over the two pools.
//
// Pages: [Q&A] "V4 为何要分池？块对齐与尾缓冲怎么配合？" §4 step 4 (attention reads the
// compressed entries of the Classical pool sparsely / densely plus the exact tail
// and SWA of the State pool); [Layout] "V4 KV Layout：Classical + State 双池",
// Classical KV cache (HCA entries are attended densely, CSA entries through
// top-k).
//
// Keys of request i, in this order: the min(L, n_win) SWA tokens (oldest first),
// the HCA entry of each of its nb sealed blocks, then the C4 entries named in the
// first min(k, 32 nb) slots of its top-k row (-1 and out-of-range ordinals are
// skipped). One softmax over all of them per head, scale 1/sqrt(128).
//
// Each key is one 4 KiB K row and one 4 KiB V row (16 heads x 128 bf16). The
// contraction is 16 independent 128-long dot products per key (no operand is
// shared across heads), about 1 flop per byte, so the kernel is bound by HBM
// bandwidth and runs on the vector ALUs: a wave takes one key at a time as four
// coalesced 1 KiB loads per row; lane l holds heads {l/16 + 4c} x dims
// (l%16)*8..+8 for c = 0..3, and the 16 lanes of a DPP row reduce one head's dot.
#include "device.h"
#include "kernels.h"

namespace hsa {

namespace {

constexpr int kWaves = 4;
constexpr int kStage = 2;          // keys per pipeline stage; two stages in flight per wave
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int n_keys(const Pools& P, const Req& R, int32_t k) {
  const int swa = R.len < P.n_win ? R.len : P.n_win;
  const int nc = kC4 * R.nb;
  return swa + R.nb + (k < nc ? k : nc);
}

__device__ __forceinline__ int n_chunks(const Pools& P, const Req& R, int32_t k, int32_t chunk) {
  return (n_keys(P, R, k) + chunk - 1) / chunk;
}

// Addresses of key x's K row and V row, or nullptr when the key is a skipped
// top-k slot.
struct KeyAddr {
  const uint16_t* k;
  const uint16_t* v;
};

__device__ __forceinline__ KeyAddr key_addr(const Pools& P, const Req& R, int x, const int32_t* sel) {
  const int swa = R.len < P.n_win ? R.len : P.n_win;
  KeyAddr a;
  if (x < swa) {
    const int64_t p = (int64_t)R.len - swa + x;
    const int64_t off = ((int64_t)R.state * P.n_win + p % P.n_win) * kRow;
    a.k = P.swa_k + off;
    a.v = P.swa_v + off;
    return a;
  }
  x -= swa;
  const int32_t* tab = P.table + (int64_t)R.state * P.table_stride;
  if (x < R.nb) {
    const int32_t id = tab[x];
    if (id < 0 || id >= P.max_blocks) {   // never taken: tables are written before use
      a.k = a.v = nullptr;
      return a;
    }
    const int64_t off = (int64_t)id * kRow;
    a.k = P.hca_k + off;
    a.v = P.hca_v + off;
    return a;
  }
  x -= R.nb;
  const int32_t j = sel[x];
  if (j < 0 || j >= kC4 * R.nb) {
    a.k = a.v = nullptr;
    return a;
  }
  const int32_t id = tab[j / kC4];
  if (id < 0 || id >= P.max_blocks) {
    a.k = a.v = nullptr;
    return a;
  }
  const int64_t off = ((int64_t)id * kC4 + j % kC4) * kRow;
  a.k = P.csa_k + off;
  a.v = P.csa_v + off;
  return a;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b),
                                         c, false);
}

constexpr float kNoMax = -1e30f;   // running-max start: finite, so exp2 never sees inf - inf

// Keys of one pipeline stage: four 16-byte pieces of the K row and of the V row
// per lane, and whether each key counts (skipped slots read a valid dummy row).
struct Stage {
  uint4 k[kStage][4];
  uint4 v[kStage][4];
  bool ok[kStage];
};

__device__ __forceinline__ const uint16_t* lane_ptr(uint64_t p, int i) {
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)p, i);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(p >> 32), i);
  return reinterpret_cast<const uint16_t*>(((uint64_t)hi << 32) | lo);
}

// Issue the loads of keys i .. i+kStage-1 of the current 64-key group (their
// addresses sit in lanes i.. of kp / vp); no branch around the loads.
__device__ __forceinline__ void load_stage(Stage& S, uint64_t kp, uint64_t vp, uint64_t okmask,
                                           int i, int lane) {
#pragma unroll
  for (int u = 0; u < kStage; ++u) {
    const int j = (i + u) & 63;
    const uint16_t* pk = lane_ptr(kp, j);
    const uint16_t* pv = lane_ptr(vp, j);
    S.ok[u] = (i + u < 64) && ((okmask >> j) & 1ull);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      S.k[u][c] = reinterpret_cast<const uint4*>(pk + c * 512)[lane];
      S.v[u][c] = reinterpret_cast<const uint4*>(pv + c * 512)[lane];
    }
  }
}

// Online softmax update of this lane's 4 heads with the keys of one stage.
__device__ __forceinline__ void compute_stage(const Stage& S, const uint4* qw, float qs, float* m,
                                              float* l, float (*acc)[8]) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    float s[kStage];
    float mx = m[c];
#pragma unroll
    for (int u = 0; u < kStage; ++u) {
      float a = dot2(qw[c].x, S.k[u][c].x, 0.f);
      a = dot2(qw[c].y, S.k[u][c].y, a);
      a = dot2(qw[c].z, S.k[u][c].z, a);
      a = dot2(qw[c].w, S.k[u][c].w, a);
      s[u] = S.ok[u] ? row_sum16(a) * qs : -INFINITY;
      mx = fmaxf(mx, s[u]);
    }
    const float sc = exp2f(m[c] - mx);
    float p[kStage];
    float ps = 0.f;
#pragma unroll
    for (int u = 0; u < kStage; ++u) {
      p[u] = exp2f(s[u] - mx);
      ps += p[u];
    }
    l[c] = l[c] * sc + ps;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[c][i] *= sc;
#pragma unroll
    for (int u = 0; u < kStage; ++u) {
      float vf[8];
      unpack8(S.v[u][c], vf);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[c][i] = fmaf(p[u], vf[i], acc[c][i]);
    }
    m[c] = mx;
  }
}

// One workgroup per chunk of a request's keys: four waves stream contiguous
// quarters of the chunk with two stages of loads in flight, merge in LDS and write
// one unnormalised partial (acc, max, sum per head), or the output itself when the
// request is a single chunk. k_merge combines the partials in the next launch: a
// kernel boundary costs far less on this GPU than a device-scope fence in every
// workgroup.
__global__ __launch_bounds__(kWaves * 64) void k_attend(Pools P, ReqBatch B, int32_t chunk,
                                                       const uint16_t* q, const int32_t* topk,
                                                       int32_t k, float* part_acc, float* part_ml,
                                                       float* out) {
  __shared__ float s_acc[kWaves][kRow];
  __shared__ float s_m[kWaves][kH];
  __shared__ float s_l[kWaves][kH];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);

  // which request and which chunk of its keys
  int w = blockIdx.x, r = 0, nch = 0;
  for (; r < B.n; ++r) {
    nch = n_chunks(P, B.r[r], k, chunk);
    if (w < nch || r == B.n - 1) break;
    w -= nch;
  }
  const Req R = B.r[r];
  const int nk = n_keys(P, R, k);
  const int per_wave = chunk / kWaves;
  const int x0 = w * chunk + wave * per_wave;
  const int x1 = min(x0 + per_wave, nk);
  const int32_t* sel = topk ? topk + (int64_t)r * k : nullptr;

  // q for this lane's 4 heads x 8 dims (bf16 pairs); scores are scaled by
  // log2(e) / sqrt(128) so exp2 gives the softmax
  uint4 qw[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
    qw[c] = reinterpret_cast<const uint4*>(q + (int64_t)r * kRow + c * 512)[lane];
  const float qs = kLog2e * 0.08838834764831845f;
  float m[4], l[4], acc[4][8];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    m[c] = kNoMax;
    l[c] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[c][i] = 0.f;
  }

  // a valid row for skipped slots: the state's first ring slot (L >= 1)
  const uint16_t* dummy_k = P.swa_k + (int64_t)R.state * P.n_win * kRow;
  const uint16_t* dummy_v = P.swa_v + (int64_t)R.state * P.n_win * kRow;
  for (int g = x0; g < x1; g += 64) {
    // lane i resolves the rows of key g + i (coalesced top-k / table gathers)
    KeyAddr a;
    a.k = a.v = nullptr;
    if (g + lane < x1) a = key_addr(P, R, g + lane, sel);
    const bool okl = a.k != nullptr;
    const uint64_t okmask = __ballot(okl);
    const uint64_t kp = reinterpret_cast<uint64_t>(okl ? a.k : dummy_k);
    const uint64_t vp = reinterpret_cast<uint64_t>(okl ? a.v : dummy_v);
    const int n = min(64, x1 - g);
    Stage A, Bs;
    load_stage(A, kp, vp, okmask, 0, lane);
    for (int i = 0; i < n; i += 2 * kStage) {
      load_stage(Bs, kp, vp, okmask, i + kStage, lane);
      compute_stage(A, qw, qs, m, l, acc);
      if (i + kStage >= n) break;
      load_stage(A, kp, vp, okmask, i + 2 * kStage, lane);
      compute_stage(Bs, qw, qs, m, l, acc);
    }
  }

  // merge the four waves in LDS
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int h = 4 * c + (lane >> 4);
    float4* dst = reinterpret_cast<float4*>(&s_acc[wave][h * kD + (lane & 15) * 8]);
    dst[0] = make_float4(acc[c][0], acc[c][1], acc[c][2], acc[c][3]);
    dst[1] = make_float4(acc[c][4], acc[c][5], acc[c][6], acc[c][7]);
    if ((lane & 15) == 0) {
      s_m[wave][h] = m[c];
      s_l[wave][h] = l[c];
    }
  }
  __syncthreads();
  const int h = tid >> 4;
  const int d0 = (tid & 15) * 8;
  float M = kNoMax;
#pragma unroll
  for (int v = 0; v < kWaves; ++v) M = fmaxf(M, s_m[v][h]);
  float L = 0.f, A8[8] = {};
#pragma unroll
  for (int v = 0; v < kWaves; ++v) {
    const float wgt = exp2f(s_m[v][h] - M);
    L = fmaf(wgt, s_l[v][h], L);
#pragma unroll
    for (int i = 0; i < 8; ++i) A8[i] = fmaf(wgt, s_acc[v][h * kD + d0 + i], A8[i]);
  }
  float4* o4 = reinterpret_cast<float4*>(out + (int64_t)r * kRow + tid * 8);
  if (nch == 1) {          // the request fits in one chunk: no partials
    const float inv = 1.f / L;
    o4[0] = make_float4(A8[0] * inv, A8[1] * inv, A8[2] * inv, A8[3] * inv);
    o4[1] = make_float4(A8[4] * inv, A8[5] * inv, A8[6] * inv, A8[7] * inv);
    return;
  }
  float* pa = part_acc + (int64_t)blockIdx.x * kRow + tid * 8;
  reinterpret_cast<float4*>(pa)[0] = make_float4(A8[0], A8[1], A8[2], A8[3]);
  reinterpret_cast<float4*>(pa)[1] = make_float4(A8[4], A8[5], A8[6], A8[7]);
  if ((tid & 15) == 0) {
    part_ml[(int64_t)blockIdx.x * 2 * kH + h] = M;
    part_ml[(int64_t)blockIdx.x * 2 * kH + kH + h] = L;
  }
}

// Merge of a request's chunk partials (log-sum-exp), one workgroup per (request,
// group of 4 heads); wave w takes head 4g + w, lane l dims 2l and 2l + 1. Lane c
// holds chunk c's max and sum, so the max, the total and the chunk weights are wave
// reductions and the partial rows are read with independent loads.
__global__ __launch_bounds__(256) void k_merge(Pools P, ReqBatch B, int32_t chunk, int32_t k,
                                               const float* part_acc, const float* part_ml,
                                               float* out) {
  const int r = blockIdx.x >> 2;
  const int hg = blockIdx.x & 3;
  const int nch = n_chunks(P, B.r[r], k, chunk);
  if (nch < 2) return;            // written directly by k_attend
  int c0 = 0;
  for (int i = 0; i < r; ++i) c0 += n_chunks(P, B.r[i], k, chunk);
  const int lane = threadIdx.x & 63;
  const int h = 4 * hg + (threadIdx.x >> 6);
  const float* ml = part_ml + (int64_t)c0 * 2 * kH;
  float M = kNoMax;
  for (int c = lane; c < nch; c += 64) M = fmaxf(M, ml[c * 2 * kH + h]);
  M = fmaxf(M, __shfl_xor(M, 32));
  M = fmaxf(M, __shfl_xor(M, 16));
  M = row_max16(M);
  float L = 0.f;
  for (int c = lane; c < nch; c += 64) L += exp2f(ml[c * 2 * kH + h] - M) * ml[c * 2 * kH + kH + h];
  L = wave_sum(L);
  const float invL = 1.f / L;
  const float* pa = part_acc + (int64_t)c0 * kRow + h * kD + 2 * lane;
  float ox = 0.f, oy = 0.f;
  for (int g = 0; g < nch; g += 64) {
    const int n = min(64, nch - g);
    const float w = (g + lane < nch) ? exp2f(ml[(g + lane) * 2 * kH + h] - M) * invL : 0.f;
#pragma unroll 8
    for (int c = 0; c < n; ++c) {
      const float wc = __shfl(w, c);
      const float2 a = *reinterpret_cast<const float2*>(pa + (int64_t)(g + c) * kRow);
      ox = fmaf(wc, a.x, ox);
      oy = fmaf(wc, a.y, oy);
    }
  }
  *reinterpret_cast<float2*>(out + (int64_t)r * kRow + h * kD + 2 * lane) = make_float2(ox, oy);
}

}  // namespace

hipError_t launch_attend(const Pools& P, const ReqBatch& B, int64_t total_chunks, int32_t chunk,
                         const void* q, const int32_t* topk, int32_t k, float* part_acc,
                         float* part_ml, float* out, hipStream_t st) {
  if (total_chunks == 0) return hipSuccess;
  hipLaunchKernelGGL(k_attend, dim3((unsigned)total_chunks), dim3(kWaves * 64), 0, st, P, B, chunk,
                     static_cast<const uint16_t*>(q), topk, k, part_acc, part_ml, out);
  return hipGetLastError();
}

hipError_t launch_merge(const Pools& P, const ReqBatch& B, int32_t chunk, int32_t k,
                        const float* part_acc, const float* part_ml, float* out, hipStream_t st) {
  if (B.n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_merge, dim3(4 * B.n), dim3(256), 0, st, P, B, chunk, k, part_acc, part_ml,
                     out);
  return hipGetLastError();
}

}  // namespace hsa
