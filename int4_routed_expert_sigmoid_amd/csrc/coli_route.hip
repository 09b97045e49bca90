// Sigmoid top-k routing and batch-union dispatch for gfx950.
//
// Routing is DeepSeek-V3 style (jeff.news "7440억 파라미터 GLM-5.2 ...",
// attention-and-kernels section): sigmoid scores, a per-expert bias that only
// steers selection, top-k, weights normalised over the selected set.  One
// wavefront routes one token: each lane holds up to 4 of the <= 256 experts,
// and each of the k rounds is a 64-lane arg-max under a strict total order
// (larger score first, lower index on ties), so the result is independent of
// the reduction order.
//
// Dispatch is the batch-union grouping of the alphamatch.ai page
// ("기술적 우수성"): per expert, the (token, slot) pairs that chose it, in
// ascending token order.  One wavefront owns one expert and sweeps the index
// array 64 entries at a time with a ballot, so list positions come from
// prefix popcounts: stable and deterministic without atomics.
#include "coli_internal.h"

namespace coli {
namespace {

constexpr int kWave = 64;

__device__ __forceinline__ bool better(float ca, int ea, float cb, int eb) {
  return ca > cb || (ca == cb && ea < eb);
}

__global__ void __launch_bounds__(256) route_topk_kernel(const float* __restrict__ logits,
                                                         const float* __restrict__ bias,
                                                         int64_t T, int E, int k,
                                                         float routed_scale,
                                                         int32_t* __restrict__ idx,
                                                         float* __restrict__ w) {
  const int lane = threadIdx.x % kWave;
  const int64_t t = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
  if (t >= T) return;
  float s[4], c[4];
  bool live[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + kWave * i;
    live[i] = e < E;
    s[i] = 0.0f;
    c[i] = -__builtin_inff();
    if (live[i]) {
      s[i] = sigmoid_f32(logits[t * E + e]);
      c[i] = s[i] + (bias ? bias[e] : 0.0f);
    }
  }
  int my_idx = -1;
  float my_s = 0.0f;
  for (int j = 0; j < k; ++j) {
    float bc = -__builtin_inff();
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (live[i] && better(c[i], lane + kWave * i, bc, be)) { bc = c[i]; be = lane + kWave * i; }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float oc = __shfl_xor(bc, off);
      const int oe = __shfl_xor(be, off);
      if (better(oc, oe, bc, be)) { bc = oc; be = oe; }
    }
    // be is now the same winner in every lane
    const int wl = be % kWave, wi = be / kWave;
    float ws = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) if (i == wi) ws = s[i];
    ws = __shfl(ws, wl);
    if (lane == wl) {
#pragma unroll
      for (int i = 0; i < 4; ++i) if (i == wi) live[i] = false;
    }
    if (lane == j) { my_idx = be; my_s = ws; }
  }
  float sum = 0.0f;
  for (int j = 0; j < k; ++j) sum = sum + __shfl(my_s, j);
  if (lane < k) {
    idx[t * k + lane] = my_idx;
    w[t * k + lane] = (my_s / sum) * routed_scale;
  }
}

// One wavefront per expert e in [0, E+S).
__global__ void __launch_bounds__(256) dispatch_lists_kernel(const int32_t* __restrict__ idx,
                                                             int64_t T, int k, int E, int S,
                                                             int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ lists) {
  const int lane = threadIdx.x % kWave;
  const int e = blockIdx.x * 4 + threadIdx.x / kWave;
  if (e >= E + S) return;
  int32_t* le = lists + (int64_t)e * T;
  if (e == E) {   // the shared expert serves every token, in slot k
    for (int64_t t = lane; t < T; t += kWave) le[t] = (int32_t)(t * (k + S) + k);
    if (lane == 0) counts[e] = (int32_t)T;
    return;
  }
  const int64_t n = T * k;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int64_t base = 0;
  for (int64_t i0 = 0; i0 < n; i0 += kWave) {
    const int64_t i = i0 + lane;
    const bool hit = i < n && idx[i] == e;
    const uint64_t m = __ballot(hit);
    const int64_t pos = base + __popcll(m & lt);
    if (hit && pos < T) le[pos] = (int32_t)((i / k) * (k + S) + i % k);
    base += __popcll(m);
  }
  if (lane == 0) counts[e] = (int32_t)(base < T ? base : T);
}

// Workgroup 0: compact the active-expert list and check the indices.
// Every workgroup: -8 * (sum of each Q8 block of x), the offset that turns the
// offset-binary nibble dot into the signed one.
__global__ void __launch_bounds__(256) dispatch_finish_kernel(
    const int32_t* __restrict__ idx, int64_t T, int k, int E, int S,
    const int32_t* __restrict__ counts, int32_t* __restrict__ n_active,
    int32_t* __restrict__ active, int32_t* __restrict__ err, const int8_t* __restrict__ xq,
    int64_t D, int32_t* __restrict__ xsum8) {
  if (blockIdx.x == 0) {
    __shared__ int bad_any;
    if (threadIdx.x == 0) bad_any = 0;
    __syncthreads();
    int bad = 0;
    for (int64_t i = threadIdx.x; i < T * k; i += blockDim.x) {
      const int e = idx[i];
      if (e < 0 || e >= E) { bad = 1; continue; }
      const int64_t t0 = (i / k) * k;
      for (int64_t j = t0; j < i; ++j) if (idx[j] == e) bad = 1;
    }
    if (bad) atomicOr(&bad_any, 1);
    if (threadIdx.x < kWave) {
      const int lane = threadIdx.x;
      const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
      int base = 0;
      for (int e0 = 0; e0 < E + S; e0 += kWave) {
        const int e = e0 + lane;
        const bool on = e < E + S && counts[e] > 0;
        const uint64_t m = __ballot(on);
        if (on) active[base + __popcll(m & lt)] = e;
        base += __popcll(m);
      }
      if (lane == 0) *n_active = base;
    }
    __syncthreads();
    if (threadIdx.x == 0) *err = bad_any ? (int)COLI_E_INDEX : 0;
  }
  if (xq) {
    const int64_t nb = T * (D / 32);
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nb; b += stride) {
      const int* xp = reinterpret_cast<const int*>(xq + 32 * b);
      int sum = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) sum = sdot4(xp[j], 0x01010101, sum);
      xsum8[b] = -8 * sum;
    }
  }
}

}  // namespace

hipError_t launch_route_topk(const float* logits, const float* bias, int64_t T, int E, int k,
                             float routed_scale, int32_t* idx, float* w, hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(route_topk_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, logits,
                     bias, T, E, k, routed_scale, idx, w);
  return hipGetLastError();
}

hipError_t launch_dispatch(const int32_t* idx, int64_t T, int k, int E, int S, int32_t* counts,
                           int32_t* lists, int32_t* n_active, int32_t* active, int32_t* err,
                           const int8_t* xq, int64_t D, int32_t* xsum8, hipStream_t s) {
  hipLaunchKernelGGL(dispatch_lists_kernel, dim3((unsigned)((E + S + 3) / 4)), dim3(256), 0, s,
                     idx, T, k, E, S, counts, lists);
  hipError_t rc = hipGetLastError();
  if (rc != hipSuccess) return rc;
  int64_t blocks = 1;
  if (xq) {
    blocks = (T * (D / 32) + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    if (blocks < 1) blocks = 1;
  }
  hipLaunchKernelGGL(dispatch_finish_kernel, dim3((unsigned)blocks), dim3(256), 0, s, idx, T, k,
                     E, S, counts, n_active, active, err, xq, D, xsum8);
  return hipGetLastError();
}

}  // namespace coli
