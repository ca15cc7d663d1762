// score_dev.h - indexer scores and top-k selection (device code).
//
// Pages: [Ch12] "Ch 12 · 推理框架 — KV 的异构调度" 名词速通 (the indexer holds tiny
// K-only keys used for top-k selection) and §2.2 (each block keeps its 128
// tokens' indexer keys); [Layout] "V4 KV Layout：Classical + State 双池", Classical KV
// cache (CSA entries are read sparsely through top-k).
//
// The score is not defined on the pages. Reading used: score of token t = sum over
// 4 heads x 64 dims of q_idx * k_idx_t; score of C4 entry j = mean of the scores
// of its tokens 4j..4j+3. Top-k keeps the kk = min(k, N_c) entries first by score
// descending, ties to the lowest C4 ordinal, written in ascending ordinal order
// (or in that selection order on request).
#pragma once

#include "device.h"

namespace hsa {

// Scores of 4 * EPW consecutive C4 entries of one block by one workgroup of 256
// threads: wave w takes entries EPW w .. EPW w + EPW - 1. Lane l owns dims
// 4l..4l+3 of every token row, so a token row is one coalesced 1 KiB read per wave;
// the 4 tokens of an entry are summed per lane before one wave reduction. row(t)
// is the keys of the t-th token of the range, out the range's first score.
template <int EPW = 8, class RowFn>
__device__ __forceinline__ void score_block(RowFn row, const float* q_row, float* out32,
                                            int n_valid = 0x7fffffff) {
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const float4 q = reinterpret_cast<const float4*>(q_row)[lane];
  float4 kv[EPW][4];
#pragma unroll
  for (int e = 0; e < EPW; ++e)
#pragma unroll
    for (int u = 0; u < 4; ++u) kv[e][u] = load_stream(reinterpret_cast<const float4*>(row((EPW * wave + e) * 4 + u)) + lane);
  float* out = out32 + EPW * wave;
#pragma unroll
  for (int e = 0; e < EPW; ++e) {
    float a = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      a = fmaf(q.x, kv[e][u].x, a);
      a = fmaf(q.y, kv[e][u].y, a);
      a = fmaf(q.z, kv[e][u].z, a);
      a = fmaf(q.w, kv[e][u].w, a);
    }
    a = wave_sum(a);
    // entries from n_valid on (an open block's incomplete groups) score -inf
    if (lane == e) out[e] = EPW * wave + e < n_valid ? a * 0.25f : -INFINITY;
  }
}

// ---- MXFP4 keys. Lane l of a wave takes token l / 8 of a group of 8 and MX block
// b = l % 8 of it (32 values: one 16-byte code load and one scale byte), so a wave
// load covers 8 tokens = 2 C4 entries.

typedef float mx_f2 __attribute__((ext_vector_type(2)));

// Sum over the lane's 32 values of q * value, times 2^E. With the codes' values
// (multiples of 1/2 up to 6) and fp32 queries, the lane sum is exact whenever the
// query's values share a fine enough grid, as the dyadic synthetic queries do.
__device__ __forceinline__ float mx_dot(const uint4& w, int E, const float* q) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  float a = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const mx_f2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(ws[j], 1.f, 0);
    const mx_f2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(ws[j], 1.f, 1);
    const mx_f2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(ws[j], 1.f, 2);
    const mx_f2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(ws[j], 1.f, 3);
    a = fmaf(q[8 * j + 0], p0.x, a);
    a = fmaf(q[8 * j + 1], p0.y, a);
    a = fmaf(q[8 * j + 2], p1.x, a);
    a = fmaf(q[8 * j + 3], p1.y, a);
    a = fmaf(q[8 * j + 4], p2.x, a);
    a = fmaf(q[8 * j + 5], p2.y, a);
    a = fmaf(q[8 * j + 6], p3.x, a);
    a = fmaf(q[8 * j + 7], p3.y, a);
  }
  return ldexpf(a, E);
}

__device__ __forceinline__ void mx_load_q(const float* q_row, int b, float* q) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 v = reinterpret_cast<const float4*>(q_row + kMxBlk * b)[i];
    q[4 * i] = v.x;
    q[4 * i + 1] = v.y;
    q[4 * i + 2] = v.z;
    q[4 * i + 3] = v.w;
  }
}

// C4 scores of a group's 2 entries from the lanes' block sums: lanes 0..31 hold
// entry 0's 4 tokens, lanes 32..63 entry 1's; written as the mean of the token scores.
__device__ __forceinline__ void mx_write_pair(float a, float* out2) {
  a = row_sum16(a);
  a += __shfl_xor(a, 16);
  const int lane = threadIdx.x & 63;
  if ((lane & 31) == 0) out2[lane >> 5] = a * 0.25f;
}

// Scores of 32 * NG tokens (8 * NG C4 entries) of stored MXFP4 keys: key rows
// [0, 32 NG) at codes + t * kIRowQ, scales + t * kIRowE; wave w takes groups
// w NG .. w NG + NG - 1 of 8 tokens.
template <int NG>
__device__ __forceinline__ void score_block_mx(const uint8_t* codes, const uint8_t* scales,
                                               const float* q_row, float* out) {
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int b = lane & 7;
  uint4 w[NG];
  int e[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int t = (wave * NG + g) * 8 + (lane >> 3);
    w[g] = load_stream(reinterpret_cast<const uint4*>(codes + (int64_t)t * kIRowQ) + b);
    e[g] = scales[(int64_t)t * kIRowE + b];
  }
  float q[32];
  mx_load_q(q_row, b, q);
#pragma unroll
  for (int g = 0; g < NG; ++g) mx_write_pair(mx_dot(w[g], e[g] - 127, q), out + 2 * (wave * NG + g));
}

// The same scores for keys not yet stored (the block being sealed in the same
// launch): each lane quantises its 32 fp32 values as the seal does (the block's
// maximum is the same however it is reduced), then takes the stored path's sum.
template <int NG, typename RowFn>
__device__ __forceinline__ void score_block_mx_raw(RowFn row, const float* q_row, float* out) {
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int b = lane & 7;
  float q[32];
  mx_load_q(q_row, b, q);
#pragma unroll 1
  for (int g = 0; g < NG; ++g) {
    const int t = (wave * NG + g) * 8 + (lane >> 3);
    const float4* src = reinterpret_cast<const float4*>(row(t) + kMxBlk * b);
    float x[32];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 v = src[i];
      x[4 * i] = v.x;
      x[4 * i + 1] = v.y;
      x[4 * i + 2] = v.z;
      x[4 * i + 3] = v.w;
    }
    float am = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) am = fmaxf(am, fabsf(x[i]));
    const int E = mx_exp(am);
    uint32_t ws[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 32; ++i) ws[i >> 3] |= e2m1_code(x[i], E) << (4 * (i & 7));
    mx_write_pair(mx_dot(make_uint4(ws[0], ws[1], ws[2], ws[3]), E, q), out + 2 * (wave * NG + g));
  }
}

// Order-preserving map of a float score to uint32 (larger score -> larger key);
// -0 is folded onto +0 so equal scores compare equal.
__device__ __forceinline__ uint32_t okey(float f) {
  uint32_t b = __float_as_uint(f);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float okey_inv(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kBins = 2048;        // radix digits of 11, 11 and 10 bits
constexpr int kTabCache = 1024;    // block-table entries kept in LDS for the row output

struct SelShared {
  uint32_t keys[kCacheN];
  uint32_t hist[3][kBins];
  unsigned long long cand[kMaxTopk];
  int32_t tab[kTabCache];
  int sh[3];
  int cnt[2][2][kSelWaves];   // [parity][above tau, equal to tau][wave]
};

constexpr int kSelBatch = 8;   // float4 loads in flight per thread when scores stream from L2

// f(i, key) for every score i < N (N a multiple of 4) read from global memory: each
// thread keeps kSelBatch float4 loads in flight, so a pass costs about N / (NT * 32)
// memory latencies rather than one per element.
template <int NT, class F>
__device__ __forceinline__ void for_each_key(int N, const float* S, F f) {
  const int n4 = N >> 2;
  const float4* S4 = reinterpret_cast<const float4*>(S);
  for (int b = 0; b < n4; b += NT * kSelBatch) {
    float4 v[kSelBatch];
    // unconditional loads (an index past the row re-reads its last float4): a load
    // inside a branch makes the compiler wait for every earlier one where the branch
    // joins, which would serialise the batch
#pragma unroll
    for (int u = 0; u < kSelBatch; ++u) v[u] = S4[min(b + u * NT + (int)threadIdx.x, n4 - 1)];
#pragma unroll
    for (int u = 0; u < kSelBatch; ++u) {
      const int j = b + u * NT + (int)threadIdx.x;
      if (j < n4) {
        f(4 * j, okey(v[u].x));
        f(4 * j + 1, okey(v[u].y));
        f(4 * j + 2, okey(v[u].z));
        f(4 * j + 3, okey(v[u].w));
      }
    }
  }
}

// Exclusive prefix sum over the wave's lanes, and the wave total in `total`.
__device__ __forceinline__ int wave_excl_scan(int v, int& total) {
  const int lane = threadIdx.x & 63;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  total = __shfl(incl, 63);
  return incl - v;
}

// Top-k of one request's N scores S by one workgroup of NT threads. Radix select
// over the order-preserving keys finds tau, the key of the kk-th entry under (score
// desc, ordinal asc), and `rem`, how many entries equal to tau make the cut (the
// passes stop early once the bucket at the cut is taken whole; tau is then that
// bucket's leading digits). One ordered pass then takes every entry above tau and
// the first `rem` entries equal to tau, writing them in ascending ordinal order
// (ballot + prefix counts). With `sorted`, the taken entries are instead ordered by
// (score desc, ordinal asc) with a bitonic sort in LDS.
// With `rows`, also writes each taken entry's physical C4 row (table[j / 32] * 32 +
// j % 32) from the state's block table `tab` (nb_tab blocks), in ascending ordinal
// order. The ordinal written for entry i is i + ord0, or ord_map[i] when a map is
// given. NT = threads of the workgroup.
template <int NT = kSelThreads>
__device__ __forceinline__ void select_run(int N, int32_t k, int32_t sorted, const float* S,
                                           int32_t* io, float* so, SelShared& sh,
                                           const int32_t* tab = nullptr, int32_t* rows = nullptr,
                                           int nb_tab = 0, int32_t ord0 = 0,
                                           const int32_t* ord_map = nullptr, int kmax = 0x7fffffff) {
  static_assert(NT % 64 == 0 && NT <= kSelThreads && NT >= 256, "select workgroup size");
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x;
  const int kk = min(min(k, N), kmax);   // kmax: candidates of the row (eager rows end in -inf)
  const bool cached = N <= kCacheN;
  const bool tab_lds = rows && nb_tab <= kTabCache;
  auto row_of = [&](int j) -> int32_t {
    if (j < 0) return -1;
    const int32_t id = tab_lds ? sh.tab[j / kC4] : tab[j / kC4];
    return id * kC4 + j % kC4;
  };
  auto ord_of = [&](int i) -> int32_t { return ord_map ? ord_map[i] : i + ord0; };

  if (kk > 0) {
    if (cached) {   // N is a multiple of 32: float4 loads
      for (int i = tid; i < N / 4; i += NT) {
        const float4 v = reinterpret_cast<const float4*>(S)[i];
        sh.keys[4 * i] = okey(v.x);
        sh.keys[4 * i + 1] = okey(v.y);
        sh.keys[4 * i + 2] = okey(v.z);
        sh.keys[4 * i + 3] = okey(v.w);
      }
    }

    for (int b = tid; b < 3 * kBins; b += NT) (&sh.hist[0][0])[b] = 0u;
    if (tab_lds)
      for (int b = tid; b < nb_tab; b += NT) sh.tab[b] = tab[b];
    __syncthreads();
    uint32_t prefix = 0u, pmask = 0u;
    int rem = kk;
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
      const uint32_t dmask = pass == 2 ? 1023u : 2047u;
      uint32_t* hist = sh.hist[pass];
      auto count = [&](int, uint32_t u) {
        if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & dmask], 1u);
      };
      if (cached) {
        for (int i = tid; i < N; i += NT) count(i, sh.keys[i]);
      } else {
        for_each_key<NT>(N, S, count);
      }
      __syncthreads();
      if (tid < 64) {
        // lane l holds digits 2047-32l down to 2016-32l
        const uint4* h4 = reinterpret_cast<const uint4*>(hist + kBins - 32 * (tid + 1));
        uint32_t tot = 0u;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const uint4 v = h4[q];
          tot += v.x + v.y + v.z + v.w;
        }
        uint32_t incl = tot;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const uint32_t y = __shfl_up(incl, o);
          if (tid >= o) incl += y;
        }
        const unsigned long long bal = __ballot(incl >= (uint32_t)rem);
        const int first = (int)__ffsll((long long)bal) - 1;
        const uint32_t base = __shfl(incl - tot, first);
        // lanes 0..31 take the 32 digits of lane `first`, highest first
        const int d = kBins - 1 - 32 * first - (tid & 31);
        const uint32_t c = tid < 32 ? hist[d] : 0u;
        uint32_t ci = c;
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) {
          const uint32_t y = __shfl_up(ci, o);
          if ((tid & 31) >= o) ci += y;
        }
        const unsigned long long b2 = __ballot(tid < 32 && base + ci >= (uint32_t)rem);
        const int dl = (int)__ffsll((long long)b2) - 1;
        if (tid == dl) {
          sh.sh[0] = d;
          sh.sh[1] = (int)(base + ci - c);
          sh.sh[2] = (int)c;
        }
      }
      __syncthreads();
      prefix |= (uint32_t)sh.sh[0] << shift;
      pmask |= dmask << shift;
      rem -= sh.sh[1];
      if (sh.sh[2] == rem) break;   // every key of the cut's bucket is taken (uniform)
    }
    // tau: the cut's digits so far (the keys under pmask); the later digits cannot
    // change what is taken once the cut's bucket is taken whole
    auto above = [&](uint32_t u) { return (u & pmask) > prefix; };
    auto at_tau = [&](uint32_t u) { return (u & pmask) == prefix; };
    // ordered pass: take entries above tau and the first `rem` equal to tau; the
    // entries taken before i are (above tau before i) + min(equal before i, rem)
    const int lane = tid & 63, wv = tid >> 6;
    // a taken entry is staged in LDS at its output position; its ordinal, score and
    // row are written after the pass, so their global lookups (ord_map, the block
    // table) are not waited for inside the pass
    auto take = [&](int i, uint32_t u, int pos) { sh.cand[pos] = ((unsigned long long)u << 32) | (uint32_t)i; };
    if (!cached) {
      // Scores stream from L2: wave w owns a contiguous range of float4s. Count its
      // entries above / equal to tau, exchange the wave totals once, then write in
      // order with in-wave prefix sums (no barrier per element).
      const int n4 = N >> 2;
      const int per = ((n4 + NW - 1) / NW + 63) & ~63;
      const int j0 = wv * per, j1 = min(n4, j0 + per);
      const float4* S4 = reinterpret_cast<const float4*>(S);
      // kSelBatch float4s of the wave's range per lane are loaded before any is used
      // (unconditionally: an index past the range re-reads its last float4)
      int gt_w = 0, eq_w = 0;
      for (int jb = j0; jb < j1; jb += 64 * kSelBatch) {
        float4 v[kSelBatch];
#pragma unroll
        for (int u = 0; u < kSelBatch; ++u) v[u] = S4[min(jb + 64 * u + lane, j1 - 1)];
#pragma unroll
        for (int u = 0; u < kSelBatch; ++u) {
          if (jb + 64 * u + lane >= j1) continue;
          const uint32_t e[4] = {okey(v[u].x), okey(v[u].y), okey(v[u].z), okey(v[u].w)};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            gt_w += above(e[q]);
            eq_w += at_tau(e[q]);
          }
        }
      }
      int tot;
      wave_excl_scan(gt_w, tot);
      gt_w = tot;
      wave_excl_scan(eq_w, tot);
      eq_w = tot;
      if (lane == 0) {
        sh.cnt[0][0][wv] = gt_w;
        sh.cnt[0][1][wv] = eq_w;
      }
      __syncthreads();
      int base_gt = 0, base_eq = 0;
      for (int w = 0; w < wv; ++w) {
        base_gt += sh.cnt[0][0][w];
        base_eq += sh.cnt[0][1][w];
      }
      for (int jb0 = j0; jb0 < j1; jb0 += 64 * kSelBatch) {
        float4 v[kSelBatch];
#pragma unroll
        for (int u = 0; u < kSelBatch; ++u) v[u] = S4[min(jb0 + 64 * u + lane, j1 - 1)];
#pragma unroll
        for (int u = 0; u < kSelBatch; ++u) {
          const int jb = jb0 + 64 * u;
          if (jb >= j1) break;   // wave-uniform
          const int j = jb + lane;
          uint32_t e[4] = {0u, 0u, 0u, 0u};
          int g = 0, q_eq = 0;
          if (j < j1) {
            e[0] = okey(v[u].x); e[1] = okey(v[u].y); e[2] = okey(v[u].z); e[3] = okey(v[u].w);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              g += above(e[q]);
              q_eq += at_tau(e[q]);
            }
          }
          int g_tot, e_tot;
          int gb = base_gt + wave_excl_scan(g, g_tot);
          int eb = base_eq + wave_excl_scan(q_eq, e_tot);
          if (j < j1) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const bool gt = above(e[q]), eq = at_tau(e[q]);
              if (gt || (eq && eb < rem)) take(4 * j + q, e[q], gb + min(eb, rem));
              gb += gt;
              eb += eq;
            }
          }
          base_gt += g_tot;
          base_eq += e_tot;
        }
      }
    }
    int base_gt = 0, base_eq = 0, parity = 0;
    for (int c0 = 0; cached && c0 < N; c0 += NT, parity ^= 1) {
      const int i = c0 + tid;
      const uint32_t u = i < N ? sh.keys[i] : 0u;
      const bool gt = i < N && above(u);
      const bool eq = i < N && at_tau(u);
      const unsigned long long bg = __ballot(gt), be = __ballot(eq);
      if (lane == 0) {
        sh.cnt[parity][0][wv] = __popcll(bg);
        sh.cnt[parity][1][wv] = __popcll(be);
      }
      __syncthreads();
      int gt_before = base_gt, eq_before = base_eq;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const int cg = sh.cnt[parity][0][w], ce = sh.cnt[parity][1][w];
        gt_before += (w < wv) ? cg : 0;
        eq_before += (w < wv) ? ce : 0;
        base_gt += cg;
        base_eq += ce;
      }
      const unsigned long long below = (1ull << lane) - 1ull;
      gt_before += __popcll(bg & below);
      eq_before += __popcll(be & below);
      if (gt || (eq && eq_before < rem)) take(i, u, gt_before + min(eq_before, rem));
      if (base_gt + min(base_eq, rem) >= kk) break;   // every entry taken (uniform)
    }
    __syncthreads();   // every taken entry staged
    for (int p = tid; p < kk; p += NT) {
      const unsigned long long c = sh.cand[p];
      const uint32_t u = (uint32_t)(c >> 32);
      const int32_t j = ord_of((int32_t)(c & 0xffffffffull));
      if (sorted) {
        sh.cand[p] = ((unsigned long long)(~u) << 32) | (c & 0xffffffffull);
      } else {
        io[p] = j;
        if (so) so[p] = okey_inv(u);
      }
      if (rows) rows[p] = row_of(j);
    }
    if (sorted) {
      int n2 = 1;
      while (n2 < kk) n2 <<= 1;
      for (int i = kk + tid; i < n2; i += NT) sh.cand[i] = ~0ull;
      __syncthreads();
      for (int size = 2; size <= n2; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
          for (int t = tid; t < n2 / 2; t += NT) {
            const int i = 2 * t - (t & (stride - 1));
            const int j = i + stride;
            const bool asc = (i & size) == 0;
            const unsigned long long a = sh.cand[i], b = sh.cand[j];
            if ((a > b) == asc) {
              sh.cand[i] = b;
              sh.cand[j] = a;
            }
          }
          __syncthreads();
        }
      }
      for (int i = tid; i < kk; i += NT) {
        const unsigned long long c = sh.cand[i];
        const int32_t j = ord_of((int32_t)(c & 0xffffffffull));
        io[i] = j;
        if (so) so[i] = okey_inv(~(uint32_t)(c >> 32));
      }
    }
  }
  for (int i = kk + tid; i < k; i += NT) {
    io[i] = -1;
    if (so) so[i] = -INFINITY;
  }
}


// Round 1 of the top-k (see SelPlan), workgroup `bid`: the whole selection of an
// unsliced row, or one slice.
template <int NT>
__device__ __forceinline__ void select_round1(int bid, int n_req, const Req* reqs, const SelPlan& SP,
                                              int32_t k, int32_t sorted, const float* scores,
                                              int64_t ld, int32_t* topk, float* score_out,
                                              SelShared& sh, const int32_t* table, int64_t stride,
                                              int32_t* rows) {
  const int r = owner_of(SP.first, n_req, bid);
  const int g = bid - SP.first[r];
  const int G = SP.first[r + 1] - SP.first[r];
  const Req R = reqs[r];
  const int N = c4_rowlen(1, SP.eager, R);
  const float* S = scores + (int64_t)r * ld;
  if (G == 1) {
    select_run<NT>(N, k, sorted, S, topk + (int64_t)r * k, score_out ? score_out + (int64_t)r * k : nullptr,
                   sh, table ? table + (int64_t)R.state * stride : nullptr,
                   rows ? rows + (int64_t)r * k : nullptr, N / kC4, 0, nullptr, c4_cands(1, SP.eager, R));
    return;
  }
  const int base = g * SP.slice;
  const int64_t c0 = ((int64_t)r * SP.gmax + g) * SP.k1;
  select_run<NT>(min(SP.slice, N - base), SP.k1, 0, S + base, SP.cand_ord + c0, SP.cand_score + c0, sh,
                 nullptr, nullptr, 0, base);
}

// Round 2 for request `r` (no-op for an unsliced row).
template <int NT>
__device__ __forceinline__ void select_round2(int r, const Req* reqs, const SelPlan& SP, int32_t k,
                                              int32_t sorted, int32_t* topk, float* score_out,
                                              SelShared& sh, const int32_t* table, int64_t stride,
                                              int32_t* rows) {
  const int G = SP.first[r + 1] - SP.first[r];
  if (G == 1) return;
  const Req R = reqs[r];
  const int64_t c0 = (int64_t)r * SP.gmax * SP.k1;
  select_run<NT>(G * SP.k1, k, sorted, SP.cand_score + c0, topk + (int64_t)r * k,
                 score_out ? score_out + (int64_t)r * k : nullptr, sh,
                 table ? table + (int64_t)R.state * stride : nullptr, rows ? rows + (int64_t)r * k : nullptr,
                 c4_rowlen(1, SP.eager, R) / kC4, 0, SP.cand_ord + c0, c4_cands(1, SP.eager, R));
}


// ---------------------------------------------------------------- selection from LDS
//
// Inclusive prefix sum over the 64 lanes of a wave with DPP moves: shifts by 1, 2, 4
// and 8 lanes within each row of 16, then the row totals carried forward with the
// row broadcasts of lane 15 (into rows 1 and 3) and lane 31 (into rows 2 and 3).
__device__ __forceinline__ uint32_t wave_incl_scan_dpp(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);   // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);   // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);   // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);   // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);   // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);   // row_bcast:31
  return v;
}
//
// For a row of at most kCacheN scores whose workgroup prefetches attention keys
// before selecting: the row is first loaded into registers, so the selection that
// follows issues no global load. Global loads complete in order, so a load issued
// after the prefetch would wait for all of it.

template <int NT>
struct SelPre {
  float4 s[kCacheN / 4 / NT];
  int32_t tab;
};

// Load row S (N scores, N a multiple of 32, at most kCacheN) and table entry t < nb
// of the state. Every load is issued: out-of-row indexes read the row's first float4
// (16 readable bytes are kept there) or table entry 0, and are ignored.
template <int NT>
__device__ __forceinline__ void sel_preload(int N, const float* S, const int32_t* tab, int nb,
                                            SelPre<NT>& pre) {
  static_assert(kCacheN % (4 * NT) == 0 && NT >= kCacheN / kC4 && NT <= kTabCache,
                "selection preload shape");
  const int tid = threadIdx.x;
  const float4* S4 = reinterpret_cast<const float4*>(S);
#pragma unroll
  for (int q = 0; q < kCacheN / 4 / NT; ++q) {
    const int i = tid + q * NT;
    pre.s[q] = load_global(S4 + (i < N / 4 ? i : 0));
  }
  pre.tab = load_global(tab + (tid < nb ? tid : 0));
}

// Which part of the selection one workgroup writes: output positions [x0, x1) of the
// ascending-ordinal list (ordinals and scores, and the physical C4 row of position x
// into rows[x - x0]); with `pad`, also the padding of positions [kk, k).
struct SelWin {
  int x0, x1;
  bool pad;
};

// Top-k of the staged row (N scores, N / 32 blocks) by one workgroup of NT threads,
// in ascending ordinal order, writing what `win` asks for.
// Same selection as select_run: radix passes of 11, 11 and 10 bits over the
// order-preserving keys find the cut; the passes stop early once the bucket at the
// cut is taken whole. One ordered pass then takes every key above the cut and the
// first `rem` keys at it: each thread owns a run of consecutive keys, and one
// workgroup-wide prefix count gives every run its output position.
// Stage the preloaded row in LDS as order-preserving keys, with the table entries,
// and clear the histograms; this waits for the row's loads. Every thread writes its
// slots unconditionally (entries past the row are never read). The first barrier of
// select_lds publishes the writes.
template <int NT>
__device__ __forceinline__ void select_stage(const SelPre<NT>& pre, SelShared& sh) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int q = 0; q < kCacheN / 4 / NT; ++q) {
    const int i = tid + q * NT;
    const float4 v = pre.s[q];
    *reinterpret_cast<uint4*>(&sh.keys[4 * i]) = make_uint4(okey(v.x), okey(v.y), okey(v.z), okey(v.w));
  }
  sh.tab[tid] = pre.tab;
  for (int b = tid; b < 3 * kBins; b += NT) (&sh.hist[0][0])[b] = 0u;
}

template <int NT>
__device__ __forceinline__ void select_lds(int N, int32_t k, int32_t* io, float* so, SelShared& sh,
                                           int32_t* rows, SelWin win, int kmax) {
  constexpr int NW = NT / 64;
  constexpr int PMAX = kCacheN / NT;   // keys per thread in the ordered pass, at most
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int kk = min(min(k, N), kmax);   // kmax: candidates of the row (eager rows end in -inf)
  HSA_GLOBAL int32_t* gio = as_global(io);
  HSA_GLOBAL float* gso = so ? as_global(so) : nullptr;
  if (kk > 0) {
    __syncthreads();   // the staged row
    uint32_t prefix = 0u, pmask = 0u;
    int rem = kk;
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
      const uint32_t dmask = pass == 2 ? 1023u : 2047u;
      uint32_t* hist = sh.hist[pass];
      for (int i = tid; i < N; i += NT) {
        const uint32_t u = sh.keys[i];
        if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & dmask], 1u);
      }
      __syncthreads();
      if (tid < 64) {
        // lane l holds digits 2047-32l down to 2016-32l
        const uint4* h4 = reinterpret_cast<const uint4*>(hist + kBins - 32 * (tid + 1));
        uint32_t tot = 0u;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const uint4 v = h4[q];
          tot += v.x + v.y + v.z + v.w;
        }
        const uint32_t incl = wave_incl_scan_dpp(tot);
        const unsigned long long bal = __ballot(incl >= (uint32_t)rem);
        const int first = uniform((int)__ffsll((long long)bal) - 1);
        const uint32_t base = (uint32_t)__builtin_amdgcn_readlane((int)(incl - tot), first);
        const int d = kBins - 1 - 32 * first - (tid & 31);
        const uint32_t c = tid < 32 ? hist[d] : 0u;
        const uint32_t ci = wave_incl_scan_dpp(c);   // lanes 32..63 add zeros
        const unsigned long long b2 = __ballot(tid < 32 && base + ci >= (uint32_t)rem);
        const int dl = (int)__ffsll((long long)b2) - 1;
        if (tid == dl) {
          sh.sh[0] = d;
          sh.sh[1] = (int)(base + ci - c);
          sh.sh[2] = (int)c;
        }
      }
      __syncthreads();
      prefix |= (uint32_t)sh.sh[0] << shift;
      pmask |= dmask << shift;
      rem -= sh.sh[1];
      if (sh.sh[2] == rem) break;   // every key of the cut's bucket is taken (uniform)
    }
    // ordered pass over runs of consecutive keys
    const int run = (N + NT - 1) / NT;
    const int i0 = tid * run;
    uint32_t e[PMAX];
    int g = 0, q_eq = 0;
#pragma unroll
    for (int j = 0; j < PMAX; ++j) {
      const bool ok = j < run && i0 + j < N;
      e[j] = ok ? sh.keys[i0 + j] : 0u;
      g += ok && (e[j] & pmask) > prefix;
      q_eq += ok && (e[j] & pmask) == prefix;
    }
    const int packed = (g << 16) | q_eq;
    const int incl = (int)wave_incl_scan_dpp((uint32_t)packed);
    int before = incl - packed;
    if (lane == 63) sh.cnt[0][0][wv] = incl;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NW; ++w) before += w < wv ? sh.cnt[0][0][w] : 0;
    int gb = before >> 16, eb = before & 0xffff;
#pragma unroll
    for (int j = 0; j < PMAX; ++j) {
      if (j < run && i0 + j < N) {
        const uint32_t m = e[j] & pmask;
        const bool gt = m > prefix, eq = m == prefix;
        if (gt || (eq && eb < rem)) {
          const int pos = gb + min(eb, rem);
          if (pos >= win.x0 && pos < win.x1) {
            const int32_t i = i0 + j;
            gio[pos] = i;
            if (gso) gso[pos] = okey_inv(e[j]);
            rows[pos - win.x0] = sh.tab[i / kC4] * kC4 + i % kC4;
          }
        }
        gb += gt;
        eb += eq;
      }
    }
  }
  if (win.pad) {
    for (int i = kk + tid; i < k; i += NT) {
      gio[i] = -1;
      if (gso) gso[i] = -INFINITY;
    }
  }
}

}  // namespace hsa
