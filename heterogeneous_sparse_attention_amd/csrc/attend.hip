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

struct Stage {
  uint4 k[kStage][4];
  uint4 v[kStage][4];
  bool ok[kStage];
};

__device__ __forceinline__ void load_stage(Stage& S, const Pools& P, const Req& R, int x, int x1,
                                           const int32_t* sel, int lane) {
#pragma unroll
  for (int u = 0; u < kStage; ++u) {
    KeyAddr a;
    a.k = a.v = nullptr;
    if (x + u < x1) a = key_addr(P, R, x + u, sel);
    S.ok[u] = a.k != nullptr;
    if (S.ok[u]) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        S.k[u][c] = reinterpret_cast<const uint4*>(a.k + c * 512)[lane];
        S.v[u][c] = reinterpret_cast<const uint4*>(a.v + c * 512)[lane];
      }
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
      if (S.ok[u]) {
        float a = dot2(qw[c].x, S.k[u][c].x, 0.f);
        a = dot2(qw[c].y, S.k[u][c].y, a);
        a = dot2(qw[c].z, S.k[u][c].z, a);
        a = dot2(qw[c].w, S.k[u][c].w, a);
        s[u] = row_sum16(a) * qs;
      } else {
        s[u] = -INFINITY;
      }
      mx = fmaxf(mx, s[u]);
    }
    if (mx == -INFINITY) continue;   // no valid key for this head yet
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
      if (S.ok[u]) {
        float vf[8];
        unpack8(S.v[u][c], vf);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[c][i] = fmaf(p[u], vf[i], acc[c][i]);
      }
    }
    m[c] = mx;
  }
}

// One workgroup per chunk of a request's keys: four waves stream contiguous
// quarters of the chunk with two stages of loads in flight, merge in LDS and write
// one unnormalised partial (acc, max, sum per head). The last chunk of a request
// to finish (ticket) merges all of the request's partials and writes the output.
__global__ __launch_bounds__(kWaves * 64) void k_attend(Pools P, ReqBatch B, int32_t chunk,
                                                       const uint16_t* q, const int32_t* topk,
                                                       int32_t k, float* part_acc, float* part_ml,
                                                       int32_t* tickets, float* out) {
  __shared__ float s_acc[kWaves][kRow];
  __shared__ float s_m[kWaves][kH];
  __shared__ float s_l[kWaves][kH];
  __shared__ int s_last;
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
  const int c0 = blockIdx.x - w;   // first chunk of request r
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
    m[c] = -INFINITY;
    l[c] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[c][i] = 0.f;
  }

  Stage A, Bs;
  if (x0 < x1) load_stage(A, P, R, x0, x1, sel, lane);
  for (int x = x0; x < x1; x += 2 * kStage) {
    const bool more_b = x + kStage < x1;
    if (more_b) load_stage(Bs, P, R, x + kStage, x1, sel, lane);
    compute_stage(A, qw, qs, m, l, acc);
    if (!more_b) break;
    if (x + 2 * kStage < x1) load_stage(A, P, R, x + 2 * kStage, x1, sel, lane);
    compute_stage(Bs, qw, qs, m, l, acc);
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
  float M = -INFINITY;
#pragma unroll
  for (int v = 0; v < kWaves; ++v) M = fmaxf(M, s_m[v][h]);
  float L = 0.f, A8[8] = {};
#pragma unroll
  for (int v = 0; v < kWaves; ++v) {
    const float wgt = (s_m[v][h] == -INFINITY) ? 0.f : exp2f(s_m[v][h] - M);
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
  __threadfence();
  __syncthreads();
  if (tid == 0) s_last = (atomicAdd(&tickets[r], 1) == nch - 1);
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  // last chunk of the request: log-sum-exp merge of its nch partials
  float GM = -INFINITY, GL = 0.f, G[8] = {};
#pragma unroll 4
  for (int c = c0; c < c0 + nch; ++c) {
    const float mc = part_ml[(int64_t)c * 2 * kH + h];
    const float lc = part_ml[(int64_t)c * 2 * kH + kH + h];
    const float4* pc = reinterpret_cast<const float4*>(part_acc + (int64_t)c * kRow + tid * 8);
    const float4 a0 = pc[0], a1 = pc[1];
    if (mc == -INFINITY) continue;
    const float Mn = fmaxf(GM, mc);
    const float sa = exp2f(GM - Mn), sb = exp2f(mc - Mn);
    GL = GL * sa + lc * sb;
    G[0] = fmaf(a0.x, sb, G[0] * sa); G[1] = fmaf(a0.y, sb, G[1] * sa);
    G[2] = fmaf(a0.z, sb, G[2] * sa); G[3] = fmaf(a0.w, sb, G[3] * sa);
    G[4] = fmaf(a1.x, sb, G[4] * sa); G[5] = fmaf(a1.y, sb, G[5] * sa);
    G[6] = fmaf(a1.z, sb, G[6] * sa); G[7] = fmaf(a1.w, sb, G[7] * sa);
    GM = Mn;
  }
  const float inv = 1.f / GL;
  o4[0] = make_float4(G[0] * inv, G[1] * inv, G[2] * inv, G[3] * inv);
  o4[1] = make_float4(G[4] * inv, G[5] * inv, G[6] * inv, G[7] * inv);
  if (tid == 0) atomicExch(&tickets[r], 0);   // ready for the next launch
}

}  // namespace

hipError_t launch_attend(const Pools& P, const ReqBatch& B, int64_t total_chunks, int32_t chunk,
                         const void* q, const int32_t* topk, int32_t k, float* part_acc,
                         float* part_ml, int32_t* tickets, float* out, hipStream_t st) {
  if (total_chunks == 0) return hipSuccess;
  hipLaunchKernelGGL(k_attend, dim3((unsigned)total_chunks), dim3(kWaves * 64), 0, st, P, B, chunk,
                     static_cast<const uint16_t*>(q), topk, k, part_acc, part_ml, tickets, out);
  return hipGetLastError();
}

}  // namespace hsa
