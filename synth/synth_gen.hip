// synth_gen.hip - the counter generator of the Python module `synth`, on the GPU, and
// the benchmark's streaming-read roof. Harness only: fills benchmark / test inputs and
// measures the GPU; holds no arithmetic of the cache.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../include/hsa_synth.h"

namespace {

__device__ __forceinline__ uint64_t mix64(uint64_t x) {
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return x ^ (x >> 31);
}

__device__ __forceinline__ float zval(uint32_t w) {
  const int s = (int)(w & 0xffu) + (int)((w >> 8) & 0xffu) + (int)((w >> 16) & 0xffu);
  return (float)(2 * s - 765) * (1.0f / 256.0f);
}

__device__ __forceinline__ uint32_t bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// one thread per pair of elements (2e, 2e+1): one 64-bit hash each
__global__ void k_synth(uint64_t seed, uint32_t stream_id, const uint32_t* keys, uint32_t key,
                        const int64_t* pos, int64_t pos0, int64_t n_rows, int32_t row_len,
                        int32_t as_bf16, void* out) {
  const int64_t half = row_len / 2;
  const int64_t total = n_rows * half;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = t / half;
    const int64_t e2 = t - r * half;
    const uint64_t kk = keys ? keys[r] : key;
    const int64_t p = pos ? pos[r] : pos0 + r;
    const uint64_t i = (uint64_t)p * (uint64_t)row_len + 2 * (uint64_t)e2;
    const uint64_t ctr = ((uint64_t)stream_id << 56) | (kk << 32) | (i >> 1);
    const uint64_t h = mix64(seed + (ctr + 1ull) * 0x9E3779B97F4A7C15ull);
    const float z0 = zval((uint32_t)h), z1 = zval((uint32_t)(h >> 32));
    if (as_bf16) {
      reinterpret_cast<uint32_t*>(out)[t] = bf16_bits(z0) | (bf16_bits(z1) << 16);
    } else {
      reinterpret_cast<float2*>(out)[t] = make_float2(z0, z1);
    }
  }
}

// Streaming read of n16 16-byte words (bandwidth roof of the benchmark): workgroup b
// reads the contiguous chunk [b chunk, (b + 1) chunk) with 8 non-temporal loads in
// flight per thread (a chunk per workgroup keeps DRAM pages open: it measured 7.0
// TB/s where a grid-stride walk read 5.9). The words are folded by XOR so the
// loads cannot be dropped; a workgroup writes its fold only if it is a marker value.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_read_roof(const u32x4* __restrict__ in, int64_t n16, int64_t chunk,
                                                   uint32_t* __restrict__ out) {
  constexpr int U = 8;
  const int64_t b0 = (int64_t)blockIdx.x * chunk;
  const int64_t b1 = b0 + chunk < n16 ? b0 + chunk : n16;
  uint32_t acc = 0u;
  for (int64_t base = b0 + threadIdx.x; base < b1; base += U * 256) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + u * 256;
      v[u] = i < b1 ? __builtin_nontemporal_load(in + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9E3779B9u) out[blockIdx.x] = acc;
}

}  // namespace

extern "C" int32_t hsa_roof_read(const void* buf, int64_t bytes, uint32_t* out, int32_t blocks, void* stream) {
  if (!buf || !out || bytes <= 0 || (bytes & 15) || blocks <= 0) return -1;
  const int64_t n16 = bytes / 16;
  hipLaunchKernelGGL(k_read_roof, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(buf), n16, (n16 + blocks - 1) / blocks, out);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" int32_t hsa_synth_rows(uint64_t seed, uint32_t stream_id, const uint32_t* keys,
                                  uint32_t key, const int64_t* pos, int64_t pos0, int64_t n_rows,
                                  int32_t row_len, int32_t as_bf16, void* out, void* stream) {
  if (n_rows < 0 || row_len <= 0 || (row_len & 1) || (n_rows > 0 && !out)) return -1;
  if (n_rows == 0) return 0;
  const int64_t total = n_rows * (row_len / 2);
  const int64_t blocks = (total + 255) / 256;
  const unsigned grid = (unsigned)(blocks < 65536 ? blocks : 65536);
  hipLaunchKernelGGL(k_synth, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream), seed,
                     stream_id, keys, key, pos, pos0, n_rows, row_len, as_bf16, out);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}
