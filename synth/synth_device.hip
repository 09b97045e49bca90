// Seeded synthetic-input generator, device implementation (gfx950).
//
// Produces, directly in device memory, the same values as synth_host.c's
// synth_normal (bit for bit): the SplitMix64 output function of Steele, Lea
// and Flood (OOPSLA 2014) driven by a counter, and an Irwin-Hall(12) normal
// built from integer sums, one exact int->float conversion, one exact
// power-of-two scale and one IEEE fp32 multiply.  Used to fill the multi-GB
// expert tables without a host round trip.  Holds none of the method's
// arithmetic.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ULL;
constexpr uint64_t kIdMul = 0xD1B54A32D192ED03ULL;

__host__ __device__ inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

__global__ void __launch_bounds__(256) normal_kernel(uint64_t base, uint64_t offset, int64_t n,
                                                     float sigma, float* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += stride) {
    const uint64_t i = offset + (uint64_t)j;
    uint32_t s = 0;
#pragma unroll
    for (uint64_t m = 0; m < 3; ++m) {
      const uint64_t z = mix64(base + (3 * i + m + 1) * kGamma);
      s += (uint32_t)(z & 0xFFFF) + (uint32_t)((z >> 16) & 0xFFFF) +
           (uint32_t)((z >> 32) & 0xFFFF) + (uint32_t)(z >> 48);
    }
    const float zf = (float)((int32_t)s - 393210) * (1.0f / 65536.0f);
    out[j] = zf * sigma;
  }
}

}  // namespace

extern "C" {

// Fills out[0..n) (device memory) with normal(offset + j) of stream
// (seed, stream_id).  Asynchronous on `stream` (a hipStream_t, may be null).
// Returns 0 on success, the hipError_t of the launch otherwise.
int synth_normal_device(uint64_t seed, uint64_t stream_id, uint64_t offset, int64_t n,
                        float sigma, float* out, void* stream) {
  if (n <= 0) return 0;
  if (out == nullptr) return (int)hipErrorInvalidValue;
  const uint64_t base = mix64(mix64(seed + kGamma) ^ (stream_id * kIdMul));
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(normal_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     base, offset, n, sigma, out);
  return (int)hipGetLastError();
}

}  // extern "C"
