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
constexpr int kUnroll = 4;          // keys in flight per wave
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int n_keys(const Pools& P, const Req& R, int32_t k) {
  const int swa = R.len < P.n_win ? R.len : P.n_win;
  const int nc = kC4 * R.nb;
  return swa + R.nb + (k < nc ? k : nc);
}

__device__ __forceinline__ int n_chunks(const Pools& P, const Req& R, int32_t k, int32_t chunk) {
  return (n_keys(P, R, k) + chunk - 1) / chunk;
}

// Address of key x's K row (V row at the same offset in the V pool), or -1 when
// the key is a skipped top-k slot.
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

__global__ __launch_bounds__(kWaves * 64) void k_attend(Pools P, ReqBatch B, int32_t chunk,
                                                       const uint16_t* q, const int32_t* topk,
                                                       int32_t k, float* part_acc, float* part_ml) {
  __shared__ float s_acc[kWaves][kRow];
  __shared__ float s_m[kWaves][kH];
  __shared__ float s_l[kWaves][kH];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);

  // which request and which chunk of its keys
  int w = blockIdx.x, r = 0;
  for (; r < B.n - 1; ++r) {
    const int c = n_chunks(P, B.r[r], k, chunk);
    if (w < c) break;
    w -= c;
  }
  const Req R = B.r[r];
  const int nk = n_keys(P, R, k);
  const int per_wave = chunk / kWaves;
  const int x0 = w * chunk + wave * per_wave;
  const int x1 = min(x0 + per_wave, nk);
  const int32_t* sel = topk ? topk + (int64_t)r * k : nullptr;

  // q for this lane's 4 heads x 8 dims, pre-scaled so exp2 gives the softmax
  float qf[4][8];
  const float qs = kLog2e * 0.08838834764831845f;   // log2(e) / sqrt(128)
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint4 w4 = reinterpret_cast<const uint4*>(q + (int64_t)r * kRow + c * 512)[lane];
    unpack8(w4, qf[c]);
#pragma unroll
    for (int i = 0; i < 8; ++i) qf[c][i] *= qs;
  }
  float m[4], l[4], acc[4][8];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    m[c] = -INFINITY;
    l[c] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[c][i] = 0.f;
  }

  for (int xb = x0; xb < x1; xb += kUnroll) {
    uint4 kw[kUnroll][4], vw[kUnroll][4];
    bool ok[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int x = xb + u;
      KeyAddr a;
      a.k = a.v = nullptr;
      if (x < x1) a = key_addr(P, R, x, sel);
      ok[u] = a.k != nullptr;
      if (ok[u]) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          kw[u][c] = reinterpret_cast<const uint4*>(a.k + c * 512)[lane];
          vw[u][c] = reinterpret_cast<const uint4*>(a.v + c * 512)[lane];
        }
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float s[kUnroll];
      float mx = m[c];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        if (ok[u]) {
          float kf[8];
          unpack8(kw[u][c], kf);
          float a = 0.f;
#pragma unroll
          for (int i = 0; i < 8; ++i) a = fmaf(qf[c][i], kf[i], a);
          s[u] = row_sum16(a);
        } else {
          s[u] = -INFINITY;
        }
        mx = fmaxf(mx, s[u]);
      }
      if (mx == -INFINITY) continue;   // nothing valid yet for this head
      const float sc = exp2f(m[c] - mx);
      float p[kUnroll];
      float ps = 0.f;
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        p[u] = exp2f(s[u] - mx);
        ps += p[u];
      }
      l[c] = l[c] * sc + ps;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[c][i] *= sc;
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        if (ok[u]) {
          float vf[8];
          unpack8(vw[u][c], vf);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[c][i] = fmaf(p[u], vf[i], acc[c][i]);
        }
      }
      m[c] = mx;
    }
  }

  // merge the four waves in LDS, then write one unnormalised partial
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int h = 4 * c + (lane >> 4);
    float* dst = &s_acc[wave][h * kD + (lane & 15) * 8];
#pragma unroll
    for (int i = 0; i < 8; ++i) dst[i] = acc[c][i];
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
  float L = 0.f, A[8] = {};
#pragma unroll
  for (int v = 0; v < kWaves; ++v) {
    const float wgt = (s_m[v][h] == -INFINITY) ? 0.f : exp2f(s_m[v][h] - M);
    L = fmaf(wgt, s_l[v][h], L);
#pragma unroll
    for (int i = 0; i < 8; ++i) A[i] = fmaf(wgt, s_acc[v][h * kD + d0 + i], A[i]);
  }
  float* pa = part_acc + (int64_t)blockIdx.x * kRow + tid * 8;
  reinterpret_cast<float4*>(pa)[0] = make_float4(A[0], A[1], A[2], A[3]);
  reinterpret_cast<float4*>(pa)[1] = make_float4(A[4], A[5], A[6], A[7]);
  if ((tid & 15) == 0) {
    part_ml[(int64_t)blockIdx.x * 2 * kH + h] = M;
    part_ml[(int64_t)blockIdx.x * 2 * kH + kH + h] = L;
  }
}

// One workgroup per request: merge its chunk partials (log-sum-exp) and normalise.
__global__ __launch_bounds__(256) void k_combine(Pools P, ReqBatch B, int32_t chunk, int32_t k,
                                                 const float* part_acc, const float* part_ml,
                                                 float* out) {
  const int r = blockIdx.x;
  int c0 = 0;
  for (int i = 0; i < r; ++i) c0 += n_chunks(P, B.r[i], k, chunk);
  const int nc = n_chunks(P, B.r[r], k, chunk);
  const int tid = threadIdx.x;
  const int h = tid >> 4;
  float M = -INFINITY;
  for (int c = 0; c < nc; ++c) M = fmaxf(M, part_ml[(int64_t)(c0 + c) * 2 * kH + h]);
  float L = 0.f, A[8] = {};
  for (int c = 0; c < nc; ++c) {
    const float mc = part_ml[(int64_t)(c0 + c) * 2 * kH + h];
    const float wgt = (mc == -INFINITY) ? 0.f : exp2f(mc - M);
    L = fmaf(wgt, part_ml[(int64_t)(c0 + c) * 2 * kH + kH + h], L);
    const float4* pa = reinterpret_cast<const float4*>(part_acc + (int64_t)(c0 + c) * kRow + tid * 8);
    const float4 a0 = pa[0], a1 = pa[1];
    A[0] = fmaf(wgt, a0.x, A[0]); A[1] = fmaf(wgt, a0.y, A[1]);
    A[2] = fmaf(wgt, a0.z, A[2]); A[3] = fmaf(wgt, a0.w, A[3]);
    A[4] = fmaf(wgt, a1.x, A[4]); A[5] = fmaf(wgt, a1.y, A[5]);
    A[6] = fmaf(wgt, a1.z, A[6]); A[7] = fmaf(wgt, a1.w, A[7]);
  }
  const float inv = 1.f / L;
  float4* o = reinterpret_cast<float4*>(out + (int64_t)r * kRow + tid * 8);
  o[0] = make_float4(A[0] * inv, A[1] * inv, A[2] * inv, A[3] * inv);
  o[1] = make_float4(A[4] * inv, A[5] * inv, A[6] * inv, A[7] * inv);
}

}  // namespace

hipError_t launch_attend(const Pools& P, const ReqBatch& B, int64_t total_chunks, int32_t chunk,
                         const void* q, const int32_t* topk, int32_t k, float* part_acc,
                         float* part_ml, hipStream_t st) {
  if (total_chunks == 0) return hipSuccess;
  hipLaunchKernelGGL(k_attend, dim3((unsigned)total_chunks), dim3(kWaves * 64), 0, st, P, B, chunk,
                     static_cast<const uint16_t*>(q), topk, k, part_acc, part_ml);
  return hipGetLastError();
}

hipError_t launch_combine(const Pools& P, const ReqBatch& B, int32_t chunk, int32_t k,
                          const float* part_acc, const float* part_ml, float* out, hipStream_t st) {
  if (B.n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_combine, dim3(B.n), dim3(256), 0, st, P, B, chunk, k, part_acc, part_ml, out);
  return hipGetLastError();
}

}  // namespace hsa
