// device.h - layout constants, launch descriptors and wavefront helpers shared by
// the gfx950 kernels of the heterogeneous KV cache.
//
// HBM layout (structure of arrays, indexed by physical id):
//   swa_k, swa_v  [max_states][n_win][16][128] bf16   token p of state s in slot p mod n_win
//   idx_tail      [max_states][128][4][64]   fp32     token p in slot p mod 128
//   csa_k, csa_v  [max_blocks][32][16][128]  bf16     C4 entry j of a block = tokens 4j..4j+3
//   (FP8 entries instead: c4q [max_blocks * 32][K, V][16][128] E4M3 codes and
//    c4s [max_blocks * 32][K, V][16] fp32 per-head scales, head h at 4 (h % 4) + h / 4)
//   hca_k, hca_v  [max_blocks][16][128]      bf16
//   idx_k         [max_blocks][128][4][64]   fp32
//   (MXFP4 indexer keys instead: idx_q [max_blocks][128][128] E2M1 code pairs and
//    idx_e [max_blocks][128][8] E8M0 scales, one per 32 values)
//   (FP8 KV instead of swa_k, swa_v and hca_k, hca_v: swq [max_states * n_win][K, V][16][128]
//    and hcq [max_blocks][K, V][16][128] E4M3 codes, sws and hcs [..][K, V][16] fp32
//    scales, the C4 FP8 row layout)
//   table         [max_states][table_stride] int32    logical block -> physical id
// One K or V row (a token or an entry) is 16 x 128 bf16 = 4 KiB contiguous, so every
// row read is a fully coalesced 4 KiB burst; one indexer row is 1 KiB.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace hsa {

constexpr int kH = 16;
constexpr int kD = 128;
constexpr int kRow = kH * kD;      // 2048 bf16 per K or V row
constexpr int kHi = 4;
constexpr int kDi = 64;
constexpr int kIRow = kHi * kDi;   // 256 fp32 per indexer row
constexpr int kBlk = 128;          // tokens per block = lcm(4, 128)
constexpr int kC4 = 32;            // C4 entries per block
constexpr int kMaxReq = 64;        // requests per launch descriptor
constexpr int kSealSplit = 16;     // workgroups per decode-time seal (8 tokens each)
#ifndef HSA_SCORE_SPLIT
#define HSA_SCORE_SPLIT 2
#endif
constexpr int kScoreSplit = HSA_SCORE_SPLIT;   // decode-step scoring workgroups per sealed block
constexpr int kPartFloats = 2 * kH + 2 * kRow;  // one HCA seal partial: m, l, acc K, acc V
constexpr int kMaxTopk = 4096;
constexpr int kC4Bytes = 2 * kRow;      // FP8 C4 row: K codes then V codes, 2048 B each
constexpr int kC4Scales = 2 * kH;       // FP8 C4 row: K scales then V scales
constexpr float kE4M3Max = 448.f;       // largest finite OCP E4M3 value
constexpr int kCacheN = 4096;      // top-k: scores kept in LDS (16 KiB); larger rows read through L2
constexpr int kMxBlk = 32;              // MXFP4 indexer keys: values per shared scale
constexpr int kIRowQ = kIRow / 2;       // MXFP4 indexer key: 128 bytes of E2M1 codes
constexpr int kIRowE = kIRow / kMxBlk;  // MXFP4 indexer key: 8 E8M0 scale bytes
constexpr int kMxUnitMax = 8;           // MXFP4 keys: at most 8 sealed blocks (136 KiB) per scoring workgroup
constexpr int kMxPass = 3;              // MXFP4 keys: sealed blocks whose loads a scoring pass issues together
                                        // (the most that keeps the 4-workgroup k_step1 instances free of spills)

// MXFP4 keys: scoring workgroups of a block sealed within the step, whose keys are
// quantised from the fp32 tail as they are scored (32 tokens each)
constexpr int kMxRawSplit = 4;

// Decode-step scoring workgroups of a request with nb sealed blocks: kScoreSplit per
// block of fp32 keys (64 KiB each, mx_unit 0), or one per mx_unit stored blocks of
// MXFP4 keys (17 KiB each) plus kMxRawSplit for a block sealed in the step.
__host__ __device__ inline int64_t score_units(int64_t nb, int mx_unit, bool sealed_now) {
  const int64_t s = sealed_now ? 1 : 0;
  return mx_unit > 0 ? (nb - s + mx_unit - 1) / mx_unit + s * kMxRawSplit : (int64_t)kScoreSplit * nb;
}

struct Pools {
  uint16_t* swa_k;
  uint16_t* swa_v;
  float* idx_tail;
  uint16_t* csa_k;
  uint16_t* csa_v;
  uint16_t* hca_k;
  uint16_t* hca_v;
  float* idx_k;
  int32_t* table;
  int64_t table_stride;
  const float* gate_csa;
  const float* gate_hca;
  uint8_t* c4q;         // FP8 entries: codes of C4 row r (block * 32 + slot) at r * kC4Bytes
  float* c4s;           // FP8 entries: scales of C4 row r at r * kC4Scales
  uint8_t* idx_q;       // MXFP4 keys: codes of key row r (block * 128 + token) at r * kIRowQ
  uint8_t* idx_e;       // MXFP4 keys: scale bytes of key row r at r * kIRowE
  uint8_t* swq;         // FP8 KV: codes of ring slot g (state * n_win + p % n_win) at g * kC4Bytes
  float* sws;           // FP8 KV: scales of ring slot g at g * kC4Scales
  uint8_t* hcq;         // FP8 KV: codes of block id's HCA entry at id * kC4Bytes
  float* hcs;           // FP8 KV: scales of block id's HCA entry at id * kC4Scales
  int32_t n_win;
  int32_t max_blocks;   // physical ids are in [0, max_blocks)
  int32_t fp8;          // 1: C4 entries are stored as FP8 (c4q, c4s); 0: bf16 (csa_k, csa_v)
  int32_t mx4;          // 1: sealed indexer keys are MXFP4 (idx_q, idx_e); 0: fp32 (idx_k)
  int32_t c4;           // layer type: 1 if the layer keeps C4 entries, indexer keys and tail
  int32_t hca;          // layer type: 1 if the layer keeps HCA entries
  int32_t eager;        // 1: the open block's complete groups have C4 entries (eager C4)
  int32_t kv8;          // 1: SWA ring tokens and HCA entries are FP8 (swq, sws, hcq, hcs); 0: bf16
  int32_t c4_ids;       // C4 block ids in [0, c4_ids): the blocks, then (eager) one open
                        // block per state at max_blocks + state
};


// One request of a launch: its state, its length and sealed-block count after the
// call, and a kernel-specific field (decode append: id of the block this token
// seals, or -1).
struct Req {
  int32_t state;
  int32_t len;
  int32_t nb;
  int32_t aux;
};

struct ReqBatch {
  int32_t n;
  int32_t n_seal;              // decode append: how many requests seal
  int32_t n_open;              // eager C4: how many requests complete a group of the open block
  int32_t pad_;
  Req r[kMaxReq];
  int8_t seal_req[kMaxReq];    // decode append: batch index of each sealing request
  int8_t open_req[kMaxReq];    // eager C4: batch index of each request completing a group
};

// Eager C4: complete groups of 4 tokens in request R's open block (32 with a deferred
// full tail), each with a C4 entry in the state's open block max_blocks + state.
__device__ __forceinline__ int open_groups(int eager, const Req& R) {
  return eager ? (R.len - kBlk * R.nb) >> 2 : 0;
}
// Top-k candidates of R: 32 per sealed block, then the open block's entries.
__device__ __forceinline__ int c4_cands(int c4, int eager, const Req& R) {
  return c4 ? kC4 * R.nb + open_groups(eager, R) : 0;
}
// Length of R's score row: 32 per block holding candidates (the open block's entries
// past its groups score -inf), so always a multiple of 32.
__device__ __forceinline__ int c4_rowlen(int c4, int eager, const Req& R) {
  return c4 ? kC4 * (R.nb + (open_groups(eager, R) > 0 ? 1 : 0)) : 0;
}

// Rows of more than `slice` scores are selected in two rounds, so that one long row
// is spread over many workgroups. Round 1: each slice of `slice` scores (the last
// one shorter) keeps its own top-k1 (k1 = k rounded up to a multiple of 4) in
// ascending ordinal order, padded with (-1, -inf). Round 2 (the next launch): the
// slices' candidates, concatenated in slice order (hence in ordinal order), are
// selected again. An entry of the row's top-k has fewer than k entries of its slice
// ahead of it under (score desc, ordinal asc), so it is among its slice's top-k1:
// the result is exact, ties included.
constexpr int kSliceN = 16384;   // shortest default slice

struct SelPlan {
  int32_t n_wgs;                   // round-1 workgroups of the batch
  int32_t gmax;                    // slices of the most-sliced row (1: no row is sliced)
  int32_t k1;                      // candidates kept per slice
  int32_t slice;                   // scores per slice, a multiple of 32
  int32_t eager;                   // rows include the open block's entries (eager C4)
  int32_t pad_;
  int32_t* cand_ord;               // [n][gmax][k1]
  float* cand_score;               // [n][gmax][k1]
  int32_t first[kMaxReq + 1];      // request i's round-1 workgroups: [first[i], first[i+1])
};

// A block to seal, read from device memory by the bulk seal kernel.
struct SealDesc {
  int32_t state;
  int32_t id;
  int64_t pos0;      // position of the block's first token (128 * logical block)
  int64_t len_old;   // tokens < len_old are resident in the state; others come from the input
  int64_t row0;      // packed input row of position len_old
};

// A request of a bulk append, for the ring / indexer-tail write kernel.
struct WriteDesc {
  int32_t state;
  int32_t nb_new;
  int64_t len_old;
  int64_t len_new;
  int64_t w0;        // first position written: max(len_old, len_new - n_win)
  int64_t row0;      // packed input row of position len_old
  int64_t cum;       // tokens written by earlier requests of the call
};

// Eager C4: entry gi of the open block (logical block nb) of a state, recomputed from
// its ring after a bulk append, a fork, a replay or a restore.
struct OpenDesc {
  int32_t state;
  int32_t nb;
  int32_t gi;
  int32_t pad_;
};

// One contiguous copy of a batched restore: n16 16-byte words from src to dst, as
// the launch's chunks [first, first + ceil(n16 / kCopyChunk16)).
struct CopySeg {
  const uint4* src;
  uint4* dst;
  int64_t n16;
  int64_t first;
};
constexpr int kCopyChunk16 = 4096;   // 16-byte words per chunk (64 KiB, 16 per thread)

// One state of a prefix attach: its table row takes ids[off .. off + nb).
struct AttachDesc {
  int32_t state;
  int32_t pad_;
  int64_t nb;
  int64_t off;
};

// Arguments of the four decode-step launches (one batch of <= kMaxReq requests).
struct StepArgs {
  const uint16_t* kin;   // new tokens' K, V [n][16][128] bf16 and indexer keys [n][256]
  const uint16_t* vin;
  const float* iin;
  const uint16_t* q;     // queries [n][16][128] bf16, indexer queries [n][256]
  const float* qi;
  float* scores;         // [n][ld] C4 scores (scratch)
  int64_t ld;
  float* part_acc;       // attention partials: part A [n_a] then part B [n_b]
  float* part_ml;
  float* seal_part;      // HCA partials of the blocks sealed in this step
  int32_t* topk;         // [n][k]
  int32_t* rows;         // [n][k] physical C4 rows of the selected entries (scratch,
                         // four-launch form)
  float* score_out;      // [n][k] or null
  float* out;            // [n][16][128] fp32
  int32_t k;
  int32_t sorted;
  int32_t n_score;       // scoring workgroups (score_units per request)
  int32_t n_a;           // part-A workgroups
  int32_t n_b;           // part-B workgroups
  int32_t fused;         // 1: three launches, part B selects for itself (rows <= kCacheN)
  int32_t mx_unit;       // MXFP4 keys: sealed blocks per scoring workgroup (0: fp32 keys)
  int32_t a_only;        // a layer without C4 entries: part A only, the new HCA key in the
                         // merge, padding top-k rows
  int32_t s2_append;     // S1 is not launched: S2 appends the tokens (and part A reads the
                         // newest from the input)
  SelPlan sel;           // top-k workgroups of the four-launch form (long rows are sliced)
  int32_t a_split[kMaxReq];       // request i's part-A keys [0, a_split[i]) are taken by part-A
                                  // workgroups, the rest by the three-launch form's mixed ones
  int32_t first_a[kMaxReq + 1];   // request i's part-A partials: [first_a[i], first_a[i+1])
  int32_t first_b[kMaxReq + 1];   // part-B partials: n_a + [first_b[i], first_b[i+1])
  int32_t first_s[kMaxReq + 1];   // request i's first scoring workgroup
};

// The request owning item w of a list laid out by prefix `first` (first[0] = 0,
// nondecreasing, first[n] = total, n <= 64): the largest r with first[r] <= w. Each
// lane reads one entry and a ballot counts the entries <= w, so the answer costs one
// load latency instead of a chain of dependent loads. Wave-uniform.
__device__ __forceinline__ int owner_of(const int32_t* first, int n, int w) {
  const int lane = threadIdx.x & 63;
  const int v = lane < n ? first[lane] : 0x7fffffff;
  return __builtin_amdgcn_readfirstlane(__popcll(__ballot(v <= w)) - 1);
}

// Range [x0, x1) of chunk w of c near-equal chunks over n keys.
__device__ __forceinline__ void chunk_range(int n, int c, int w, int& x0, int& x1) {
  x0 = (int)((int64_t)n * w / c);
  x1 = (int)((int64_t)n * (w + 1) / c);
}

// ---------------------------------------------------------------- helpers

// Global-memory view of a pointer: accesses through it are global (not flat)
// instructions, which count only on the vector-memory counter, so waits for LDS
// operations do not also wait for them.
#define HSA_GLOBAL __attribute__((address_space(1)))
template <class T>
__device__ __forceinline__ HSA_GLOBAL T* as_global(T* p) {
  return (HSA_GLOBAL T*)p;
}

// Streaming loads for data a step reads once (indexer keys, attention K/V rows):
// non-temporal, so they do not displace lines that are reused.
typedef float f32x4_v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 load_stream(const float4* p) {
  const f32x4_v v = __builtin_nontemporal_load(as_global(reinterpret_cast<const f32x4_v*>(p)));
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  const u32x4_v v = __builtin_nontemporal_load(as_global(reinterpret_cast<const u32x4_v*>(p)));
  return make_uint4(v.x, v.y, v.z, v.w);
}
// Plain loads as global instructions.
__device__ __forceinline__ uint4 load_global(const uint4* p) {
  const u32x4_v v = *as_global(reinterpret_cast<const u32x4_v*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 load_global(const float4* p) {
  const f32x4_v v = *as_global(reinterpret_cast<const f32x4_v*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ int32_t load_global(const int32_t* p) { return *as_global(p); }
typedef uint32_t u32x2_v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 load_stream(const uint2* p) {
  const u32x2_v v = __builtin_nontemporal_load(as_global(reinterpret_cast<const u32x2_v*>(p)));
  return make_uint2(v.x, v.y);
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16 bits, round to nearest even (finite values).
__device__ __forceinline__ uint32_t f2bf(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t pack_bf2(float a, float b) { return f2bf(a) | (f2bf(b) << 16); }

__device__ __forceinline__ void unpack8(const uint4& w, float* f) {
  f[0] = bf_lo(w.x); f[1] = bf_hi(w.x);
  f[2] = bf_lo(w.y); f[3] = bf_hi(w.y);
  f[4] = bf_lo(w.z); f[5] = bf_hi(w.z);
  f[6] = bf_lo(w.w); f[7] = bf_hi(w.w);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a DPP row; every lane of the row gets the sum.
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);  // row_half_mirror
  v += dpp<0x140>(v);  // row_mirror
  return v;
}

__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x141>(v));
  v = fmaxf(v, dpp<0x140>(v));
  return v;
}

// Sum over the 64 lanes of a wave; every lane gets the sum.
__device__ __forceinline__ float wave_sum(float v) {
  v = row_sum16(v);
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// ---------------------------------------------------------------- FP8 (OCP E4M3) entries

// ---------------------------------------------------------------- MXFP4 indexer keys
// OCP Microscaling MXFP4: a sealed key's 256 values form 8 blocks of 32 (block
// 2h + j = head h, dims 32j .. 32j + 31). A block has one E8M0 scale byte E + 127,
// E = floor(log2 max |x|) - 2 (2 being E2M1's largest exponent), at least -127 and
// -127 for an all-zero block; each value is the E2M1 code of x / 2^E, nearest of
// 0, .5, 1, 1.5, 2, 3, 4, 6 with ties to the even code, saturating at 6, sign bit for
// x < 0. Value 2i of a key sits in the low nibble of its byte i, 2i + 1 in the high.

// Shared exponent E of a block whose largest magnitude is amax (subnormals included).
__device__ __forceinline__ int mx_exp(float amax) {
  if (!(amax > 0.f)) return -127;
  const uint32_t b = __float_as_uint(amax);
  const int fe = (int)(b >> 23);
  const int l2 = fe ? fe - 127 : (31 - (int)__clz(b & 0x7fffffu)) - 149;   // floor(log2 amax)
  return l2 - 2 < -127 ? -127 : l2 - 2;
}

// E2M1 code of x / 2^E (the division by a power of two is exact).
__device__ __forceinline__ uint32_t e2m1_code(float x, int E) {
  const float y = ldexpf(fabsf(x), -E);
  const uint32_t c = (uint32_t)(y > 0.25f) + (uint32_t)(y >= 0.75f) + (uint32_t)(y > 1.25f) +
                     (uint32_t)(y >= 1.75f) + (uint32_t)(y > 2.5f) + (uint32_t)(y >= 3.5f) +
                     (uint32_t)(y > 5.f);
  return c | (x < 0.f ? 8u : 0u);
}

// Cooperative MXFP4 storage of one key row: lane c (0..63 of a wave, all active)
// holds values 4c .. 4c+3; the 8 lanes of a block share its scale through DPP.
// Writes the lane's 2 code bytes and, from the block's first lane, the scale byte.
__device__ __forceinline__ void mx4_store_row(const float4& v, int c, uint8_t* codes, uint8_t* scales) {
  float am = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
  am = fmaxf(am, dpp<0xB1>(am));    // quad_perm [1,0,3,2]
  am = fmaxf(am, dpp<0x4E>(am));    // quad_perm [2,3,0,1]
  am = fmaxf(am, dpp<0x141>(am));   // row_half_mirror: the other quad of the 8 lanes
  const int E = mx_exp(am);
  const uint32_t q = e2m1_code(v.x, E) | (e2m1_code(v.y, E) << 4) | (e2m1_code(v.z, E) << 8) |
                     (e2m1_code(v.w, E) << 12);
  reinterpret_cast<uint16_t*>(codes)[c] = (uint16_t)q;
  if ((c & 7) == 0) scales[c >> 3] = (uint8_t)(E + 127);
}

// The two rows of a key for attention: the bf16 K and V rows, or, for an FP8 key,
// its code row (K codes, then V codes) and its scale row (K scales, then V scales,
// head h at 4 (h % 4) + h / 4, see load_key).
struct C4Addr {
  const uint16_t* k;
  const uint16_t* v;
};
__device__ __forceinline__ C4Addr c4_addr(const Pools& P, int64_t row) {
  if (P.fp8)
    return C4Addr{reinterpret_cast<const uint16_t*>(P.c4q + row * kC4Bytes),
                  reinterpret_cast<const uint16_t*>(P.c4s + row * kC4Scales)};
  return C4Addr{P.csa_k + row * kRow, P.csa_v + row * kRow};
}
// Ring slot g = state * n_win + p % n_win (the token at position p).
__device__ __forceinline__ C4Addr ring_addr(const Pools& P, int64_t g) {
  if (P.kv8)
    return C4Addr{reinterpret_cast<const uint16_t*>(P.swq + g * kC4Bytes),
                  reinterpret_cast<const uint16_t*>(P.sws + g * kC4Scales)};
  return C4Addr{P.swa_k + g * kRow, P.swa_v + g * kRow};
}
// The HCA entry of block id.
__device__ __forceinline__ C4Addr hca_addr(const Pools& P, int64_t id) {
  if (P.kv8)
    return C4Addr{reinterpret_cast<const uint16_t*>(P.hcq + id * kC4Bytes),
                  reinterpret_cast<const uint16_t*>(P.hcs + id * kC4Scales)};
  return C4Addr{P.hca_k + id * kRow, P.hca_v + id * kRow};
}
// A pair of rows that is valid to read in place of a skipped key of either kind: a
// bf16 key reads 4 KiB from each, an FP8 key 4 KiB of codes and 128 B of scales.
// The state's first ring slot: its K row and V row, or (FP8 KV) its code row twice.
__device__ __forceinline__ C4Addr dummy_rows(const Pools& P, int32_t state) {
  const C4Addr a = ring_addr(P, (int64_t)state * P.n_win);
  return P.kv8 ? C4Addr{a.k, a.k} : a;
}

// Per-head FP8 storage of 8 values per lane, the 16 lanes of a DPP row holding one
// head's 128 values: with amax = max |x| over the head, the scale is s = amax / 448
// (1 where that is not a normal float32: an all-zero head, or amax below
// 448 * 2^-126) and each code is the E4M3 of x / s, rounded to nearest even. The
// stored value reads as code * s, so the quotient is taken against that same s;
// float32 throughout, each division correctly rounded. Returns the 8 codes (value i
// in byte i) and the scale.
__device__ __forceinline__ uint2 quantize8_e4m3(const float* x, float& scale) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
  amax = row_max16(amax);
  float s = amax / kE4M3Max;
  s = s >= __FLT_MIN__ ? s : 1.f;
  scale = s;
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = x[i] / s;
  int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w0, true);
  int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], w1, true);
  return make_uint2((uint32_t)w0, (uint32_t)w1);
}

// Store 8 values per lane of one K or V row of 16 heads x 128 in FP8 (256 lanes,
// lane t holding head t / 16, dims (t % 16) * 8 .. + 8): codes to q + 8 t, the head's
// scale to scale[4 (h % 4) + h / 4] from the head's first lane.
__device__ __forceinline__ void store_row_fp8(const float* x8, uint8_t* q, float* scale) {
  const int tid = threadIdx.x;
  float sc;
  const uint2 c = quantize8_e4m3(x8, sc);
  *reinterpret_cast<uint2*>(q + tid * 8) = c;
  if ((tid & 15) == 0) {
    const int h = tid >> 4;
    scale[4 * (h & 3) + (h >> 2)] = sc;
  }
}

typedef float f32x2_v __attribute__((ext_vector_type(2)));
// The four E4M3 codes of `w` (byte i = value i) as floats.
__device__ __forceinline__ void e4m3x4_to_f32(uint32_t w, float* f) {
  const f32x2_v lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const f32x2_v hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  f[0] = lo.x; f[1] = lo.y; f[2] = hi.x; f[3] = hi.y;
}
// Two values exactly representable in bf16 (every E4M3 value is) as a bf16 pair,
// a in the low half.
__device__ __forceinline__ uint32_t pack_exact_bf2(float a, float b) {
  return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}
// Eight E4M3 codes (value i in byte i) as eight exact bf16 values, packed in pairs.
__device__ __forceinline__ uint4 e4m3x8_to_bf16(uint2 c) {
  float f[8];
  e4m3x4_to_f32(c.x, f);
  e4m3x4_to_f32(c.y, f + 4);
  return make_uint4(pack_exact_bf2(f[0], f[1]), pack_exact_bf2(f[2], f[3]), pack_exact_bf2(f[4], f[5]),
                    pack_exact_bf2(f[6], f[7]));
}

}  // namespace hsa
