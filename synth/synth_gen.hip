// synth_gen.hip - the counter generator of the Python module `synth`, on the GPU.
// Harness only: fills benchmark / test inputs; holds no arithmetic of the cache.
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

}  // namespace

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
