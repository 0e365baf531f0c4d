// Device implementation of the seeded input generator (test inputs at sizes
// that do not fit a host round trip): Philox4x32-10 (Salmon, Moraes, Dror,
// Shaw, SC'11) keyed by (seed, stream key), block j = counter (j lo, j hi, 0,
// 0); Box-Muller in float64 on the word pairs (0,1), (2,3) with
// u = (x + 0.5) 2^-32; value = fp32(z*std + mean), optionally bf16 (nearest
// even).  No multiply-add is fused, so that the host implementation of the
// same definition draws the same values.
#include "common.h"
#include "launch.h"

namespace {

DEV void philox(uint64_t j, uint32_t k0, uint32_t k1, uint32_t out[4]) {
  uint32_t c0 = (uint32_t)j, c1 = (uint32_t)(j >> 32), c2 = 0, c3 = 0;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
    uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c0 = n0; c1 = (uint32_t)p1; c2 = n2; c3 = (uint32_t)p0;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

__global__ void synth_normal_kernel(void* dst, int64_t n, int bf, uint32_t seed, uint32_t key,
                                    int64_t start, double sd, double mean) {
#pragma clang fp contract(off)
  const int64_t j0 = start >> 2, j1 = (start + n + 3) >> 2;
  for (int64_t j = j0 + blockIdx.x * (int64_t)blockDim.x + threadIdx.x; j < j1;
       j += (int64_t)gridDim.x * blockDim.x) {
    uint32_t w[4];
    philox((uint64_t)j, seed, key, w);
    const double inv = 1.0 / 4294967296.0;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      double u1 = ((double)w[2 * p] + 0.5) * inv;
      double u2 = ((double)w[2 * p + 1] + 0.5) * inv;
      double r = sqrt(-2.0 * log(u1));
      double t = 2.0 * 3.14159265358979323846 * u2;
      double z[2] = {r * cos(t), r * sin(t)};
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        int64_t e = 4 * j + 2 * p + q;
        if (e < start || e >= start + n) continue;
        float v = (float)(z[q] * sd + mean);
        if (bf) reinterpret_cast<uint16_t*>(dst)[e - start] = f2bf_bits(v);
        else reinterpret_cast<float*>(dst)[e - start] = v;
      }
    }
  }
}

__global__ void synth_ids_kernel(int32_t* dst, int64_t n, uint32_t vocab, uint32_t seed, uint32_t key) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    uint32_t w[4];
    philox((uint64_t)i >> 2, seed, key, w);
    dst[i] = (int32_t)(((uint64_t)w[i & 3] * vocab) >> 32);
  }
}

}  // namespace

hipError_t launch_synth_normal(void* dst, int64_t n, int dtype, uint32_t seed, uint32_t key,
                               int64_t start, double std, double mean, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = ((n + 3) / 4 + 1 + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(synth_normal_kernel, dim3((unsigned)blocks), dim3(256), 0, s, dst, n, dtype,
                     seed, key, start, std, mean);
  return hipGetLastError();
}

hipError_t launch_synth_token_ids(int32_t* dst, int64_t n, uint32_t vocab, uint32_t seed,
                                  uint32_t key, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(synth_ids_kernel, dim3((unsigned)blocks), dim3(256), 0, s, dst, n, vocab, seed, key);
  return hipGetLastError();
}
