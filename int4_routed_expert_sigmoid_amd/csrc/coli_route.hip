// Sigmoid top-k routing and batch-union dispatch for gfx950.
//
// Routing is DeepSeek-V3 style (jeff.news "7440억 파라미터 GLM-5.2 ...",
// attention-and-kernels section): sigmoid scores, a per-expert bias that only
// steers selection, top-k, weights normalised over the selected set.  One
// wavefront routes one token: each lane holds up to 4 of the <= 256 experts,
// and each of the k rounds is a 64-lane max under a strict total order
// (larger score first, lower index on ties), so the result is independent of
// the reduction order.
//
// Dispatch is the batch-union grouping of the alphamatch.ai page
// ("기술적 우수성"): per expert, the (token, slot) pairs that chose it, in
// ascending token order.  One workgroup owns one expert and sweeps the index
// array with ballots, so list positions come from prefix popcounts: stable and
// deterministic without atomics.
#include "coli_internal.h"

// Wavefront max of a 32-bit value (ROCm device library, DPP-based).
extern "C" __device__ __attribute__((const)) unsigned int __ockl_wfred_max_u32(unsigned int);

namespace coli {
namespace {

constexpr int kWave = 64;

// Order-preserving unsigned image of a float (for finite values and +0;
// the selection score c = sigmoid + bias is never -0).
__device__ __forceinline__ uint32_t ordered_bits(float c) {
  const uint32_t b = __float_as_uint(c);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Routes one token with one wavefront: lane j < k receives the j-th selected
// expert and its weight.  Each candidate is one 64-bit key, the ordered bits
// of its selection score above the inverted expert index, so that a larger
// key is a larger score or, on a tie, the lower index: the strict order of
// the selection.  Each of the k rounds is one wavefront max (DPP) of the
// lanes' best remaining keys, taken as two 32-bit maxima; the winner is
// struck out.  The selected
// experts' sigmoid scores are fetched by their slot lanes from the lanes that
// computed them (no second read of the logits) and summed in slot order
// through readlane.
// KC > 0: k == KC known at compile time (the rounds and the sum unrolled).
template <int KC = 0>
__device__ __forceinline__ void route_token(const float* __restrict__ lg,
                                            const float* __restrict__ bias, int E, int k_rt,
                                            float routed_scale, int lane, int* out_idx,
                                            float* out_w) {
  const int k = KC > 0 ? KC : k_rt;
  // all eight loads first (indices clamped into [0, E)), then the scores
  float lv[4], bv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + kWave * i;
    const int ec = e < E ? e : E - 1;
    lv[i] = lg[ec];
    bv[i] = bias ? bias[ec] : 0.0f;
  }
  uint64_t key[4];
  float sg[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + kWave * i;
    key[i] = 0;   // below every real key
    sg[i] = 0.0f;
    if (e < E) {
      sg[i] = sigmoid_f32(lv[i]);
      const float c = sg[i] + bv[i];
      key[i] = ((uint64_t)ordered_bits(c) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
    }
  }
  // the lane's keys in descending order (a five-exchange sorting network);
  // real keys are distinct, so after each round only the winning lane has
  // its first key equal to the winner and shifts its keys up
  uint64_t q[4] = {key[0], key[1], key[2], key[3]};
  auto exch = [](uint64_t& x, uint64_t& y) {
    const uint64_t hi = x > y ? x : y, lo = x > y ? y : x;
    x = hi;
    y = lo;
  };
  exch(q[0], q[1]);
  exch(q[2], q[3]);
  exch(q[0], q[2]);
  exch(q[1], q[3]);
  exch(q[1], q[2]);
  int my_idx = -1;
  for (int j = 0; j < k; ++j) {
    // wavefront max of the 64-bit keys as two 32-bit maxima: the score bits,
    // then the index part among the lanes holding that score (a real key's
    // index part is never 0, so the other lanes' 0 cannot win)
    const uint32_t hi = __ockl_wfred_max_u32((uint32_t)(q[0] >> 32));
    const uint32_t lo = __ockl_wfred_max_u32((uint32_t)(q[0] >> 32) == hi ? (uint32_t)q[0] : 0u);
    const uint64_t win = ((uint64_t)hi << 32) | lo;
    const bool mine = q[0] == win;
    q[0] = mine ? q[1] : q[0];
    q[1] = mine ? q[2] : q[1];
    q[2] = mine ? q[3] : q[2];
    q[3] = mine ? 0 : q[3];
    if (lane == j) my_idx = (int)(0xFFFFFFFFu - (uint32_t)win);
  }
  // the selected expert's sigmoid score, from the lane that computed it
  // (expert e sits in lane e % 64, register e / 64)
  const int src = my_idx & (kWave - 1), reg = my_idx >> 6;
  float my_s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float v = __shfl(sg[i], src);
    my_s = reg == i ? v : my_s;
  }
  if (lane >= k) my_s = 0.0f;
  float sum = 0.0f;
  for (int j = 0; j < k; ++j)
    sum = sum + __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_s), j));
  *out_idx = my_idx;
  *out_w = (my_s / sum) * routed_scale;
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
  int my_idx;
  float my_w;
  route_token(logits + t * E, bias, E, k, routed_scale, lane, &my_idx, &my_w);
  if (lane < k) {
    idx[t * k + lane] = my_idx;
    w[t * k + lane] = my_w;
  }
}

// Batch-union dispatch, expert-major.  Workgroup e < E builds the list of
// expert e: it sweeps the tokens 1024 at a time, four consecutive tokens per
// thread; a token is listed when one of its slots holds e, at the first such
// slot (a later slot with the same expert is a repeat and is dropped); list
// positions are a workgroup-wide prefix of the threads' counts (three
// ballots), so each list is in ascending token order with no atomics and no
// scratch memory.  Workgroup E writes the
// shared expert's list (slot k of every token), checks every entry (out of
// range, or equal to an earlier entry of its token), marks the experts some
// kept entry selects, and writes the active list, n_active and the flag.
// Every workgroup reads the whole index array once, so the cost is linear in
// T (E + 1 reads of T * k entries, served by L2); with k = 8 the last
// workgroup loads four tokens' entries per thread before checking any, so its
// sweep is not a chain of dependent loads.
constexpr int kDispatchThreads = 256;
constexpr int kDispatchTokens = 4;   // consecutive tokens per thread and sweep

// Exclusive prefix of v (0 <= v < 8) over the workgroup's 256 threads, from
// one ballot per bit; returns it and sets *total.
__device__ __forceinline__ int block_prefix_count(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  int pre = 0, sum = 0;
#pragma unroll
  for (int bit = 0; bit < 3; ++bit) {
    const uint64_t m = __ballot((v >> bit) & 1);
    pre += __popcll(m & lt) << bit;
    sum += __popcll(m) << bit;
  }
  if (lane == 0) wsum[wave] = sum;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    base += w < wave ? wsum[w] : 0;
    tot += wsum[w];
  }
  __syncthreads();   // wsum is reused by the next sweep
  *total = tot;
  return base + pre;
}

template <int KC>
__global__ void __launch_bounds__(kDispatchThreads) dispatch_expert_kernel(
    const int32_t* __restrict__ idx, int64_t T, int k, int E, int S, int32_t* __restrict__ counts,
    int32_t* __restrict__ lists, int32_t* __restrict__ n_active, int32_t* __restrict__ active,
    int32_t* __restrict__ err) {
  __shared__ int wsum[4];
  __shared__ int present[COLI_MAX_EXPERTS + 1];
  __shared__ int bad_any;
  const int tid = threadIdx.x;
  const int e = (int)blockIdx.x;
  if (KC > 0) k = KC;
  if (e < E) {
    int count = 0;
    for (int64_t t0 = 0; t0 < T; t0 += kDispatchThreads * kDispatchTokens) {
      const int64_t tb = t0 + (int64_t)tid * kDispatchTokens;
      int slot[kDispatchTokens];
      int n = 0;
#pragma unroll
      for (int u = 0; u < kDispatchTokens; ++u) {
        const int64_t t = tb + u;
        int sl = -1;
        if (t < T) {
#pragma unroll
          for (int j = (KC > 0 ? KC : k) - 1; j >= 0; --j)   // the first slot holding e wins
            if (idx[t * k + j] == e) sl = j;
        }
        slot[u] = sl;
        n += sl >= 0;
      }
      int total;
      int pos = count + block_prefix_count(n, wsum, &total);
#pragma unroll
      for (int u = 0; u < kDispatchTokens; ++u)
        if (slot[u] >= 0) lists[(int64_t)e * T + pos++] = (int32_t)((tb + u) * (k + S) + slot[u]);
      count += total;
    }
    if (tid == 0) counts[e] = count;
    return;
  }
  // workgroup E: shared list, index check, active list
  for (int i = tid; i < E + S; i += kDispatchThreads) present[i] = 0;
  if (tid == 0) bad_any = 0;
  __syncthreads();
  int bad = 0;
  if constexpr (KC > 0) {
    // kDispatchTokens tokens per thread and sweep, their entries loaded
    // before any is checked, the repeat test done in registers
    for (int64_t t0 = 0; t0 < T; t0 += kDispatchThreads * kDispatchTokens) {
      int v[kDispatchTokens][KC];
#pragma unroll
      for (int u = 0; u < kDispatchTokens; ++u) {
        const int64_t t = t0 + tid + (int64_t)u * kDispatchThreads;
#pragma unroll
        for (int j = 0; j < KC; ++j) v[u][j] = t < T ? idx[t * KC + j] : 0;
      }
#pragma unroll
      for (int u = 0; u < kDispatchTokens; ++u) {
        const int64_t t = t0 + tid + (int64_t)u * kDispatchThreads;
        if (t < T) {
          if (S) lists[(int64_t)E * T + t] = (int32_t)(t * (KC + S) + KC);
#pragma unroll
          for (int j = 0; j < KC; ++j) {
            bool ok = v[u][j] >= 0 && v[u][j] < E;
#pragma unroll
            for (int i = 0; i < j; ++i) ok = ok && v[u][i] != v[u][j];
            if (ok) present[v[u][j]] = 1;
            else bad = 1;
          }
        }
      }
    }
  } else {
    for (int64_t t = tid; t < T; t += kDispatchThreads) {
      if (S) lists[(int64_t)E * T + t] = (int32_t)(t * (k + S) + k);
      for (int j = 0; j < k; ++j) {
        const int v = idx[t * k + j];
        bool ok = v >= 0 && v < E;
        for (int i = 0; i < j && ok; ++i) ok = idx[t * k + i] != v;
        if (ok) present[v] = 1;
        else bad = 1;
      }
    }
  }
  if (bad) atomicOr(&bad_any, 1);
  if (S && tid == 0) {
    counts[E] = (int32_t)T;
    present[E] = T > 0;
  }
  __syncthreads();
  if (tid < 64) {
    const int lane = tid;
    const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    int base = 0;
    for (int e0 = 0; e0 < E + S; e0 += 64) {
      const int x = e0 + lane;
      const bool on = x < E + S && present[x];
      const uint64_t msk = __ballot(on);
      if (on) active[base + __popcll(msk & lt)] = x;
      base += __popcll(msk);
    }
    if (lane == 0) {
      *n_active = base;
      *err = bad_any ? (int)COLI_E_INDEX : 0;
    }
  }
}

// -8 sum of the codes of every Q8 block of x (the GEMV's offset-binary
// nibble correction).
__global__ void __launch_bounds__(256) xsum8_kernel(const int8_t* __restrict__ xq, int64_t nb,
                                                    int32_t* __restrict__ xsum8) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nb; b += stride) {
    const int* xp = reinterpret_cast<const int*>(xq + 32 * b);
    int sum = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) sum = sdot4(xp[j], 0x01010101, sum);
    xsum8[b] = -8 * sum;
  }
}

// Workgroups of the fused front per token row in norm mode: the row's D / 4
// groups of 4 values at one per thread.
__host__ __device__ inline int norm_parts(int64_t D) { return (int)((D / 4 + 255) / 256); }

struct PrologueArgs {
  const float* x;
  const float* logits;
  const float* bias;
  int64_t T, D;
  int E, S, k;
  float routed_scale;
  int8_t* xq;
  float* xd;
  int32_t* xsum8;
  int32_t* idx;
  float* w;
  int32_t* counts;
  int32_t* lists;
  int32_t* n_active;
  int32_t* active;
  int32_t* err;
  int norm;        // 1: x is the residual stream h; quantise RMSNorm(h) (unit gain)
  float eps;
};

// One token: every wavefront routes it (the same result in each) and writes
// its share of the dispatch from registers, with no barrier.  The k experts
// are distinct and in [0, E) (k <= E), so every entry is listed at position 0
// of its expert's list and the index check passes.  KC > 0: k == KC known at
// compile time, so the selected experts are read into scalar registers once
// and every loop over them is unrolled.
template <int KC>
__device__ __forceinline__ void one_token_front(const PrologueArgs& a, int lane, int wave,
                                                int tid) {
  const int k = KC > 0 ? KC : a.k, E = a.E, S = a.S;
  int my_idx;
  float my_w;
  route_token<KC>(a.logits, a.bias, E, k, a.routed_scale, lane, &my_idx, &my_w);
  int rank = 0;   // position of this lane's expert among the selected, ascending
  for (int j = 0; j < k; ++j) rank += __builtin_amdgcn_readlane(my_idx, j) < my_idx;
  if (wave == 0 && lane < k) {
    a.idx[lane] = my_idx;
    a.w[lane] = my_w;
    a.lists[my_idx] = lane;      // pair 0 * (k + S) + slot
    a.active[rank] = my_idx;     // the shared expert E sorts after every routed one
  }
  for (int e = tid; e < E + S; e += 256) {
    int c = e == E ? 1 : 0;
    for (int j = 0; j < k; ++j) c |= __builtin_amdgcn_readlane(my_idx, j) == e;
    a.counts[e] = c;
  }
  if (tid == 0) {
    if (S) {
      a.lists[E] = k;            // the shared expert takes slot k
      a.active[k] = E;
    }
    *a.n_active = k + S;
    *a.err = 0;
  }
}

// The whole front of a small batch.  Workgroup 0 (4 wavefronts): routing (one
// wavefront per token), then the dispatch lists (one thread per routing
// entry, entries from LDS), the active-expert compaction and the index check;
// a single token takes a barrier-free path (below).  Workgroups 1..: Q8_0 of
// every token with its block sums, in parallel.
__global__ void __launch_bounds__(256) prologue_small_kernel(PrologueArgs a) {
  __shared__ int ent[kPrologueMaxEntries];
  __shared__ bool valid[kPrologueMaxEntries];
  __shared__ int cnt_lds[COLI_MAX_EXPERTS + 1];
  __shared__ int bad_any;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  if (tid == 0) bad_any = 0;
  if (blockIdx.x > 0 && a.norm) {
    // workgroups 1 + t * P + p: RMSNorm and Q8_0 of token t (the rmsnorm_q8
    // arithmetic), the quantisation split into P parts of at most 256 groups
    // of 4 values (one per thread); each part reduces the whole row itself
    __shared__ double red[4];
    __shared__ float rsh;
    const int parts = norm_parts(a.D);
    const int64_t t = (blockIdx.x - 1) / parts;
    const int part = (int)((blockIdx.x - 1) % parts);
    rmsnorm_q8_row<1>(a.x + t * a.D, a.D, a.eps, reinterpret_cast<int*>(a.xq + t * a.D),
                      a.xd + t * (a.D / 32), a.xsum8 + t * (a.D / 32), nullptr, red, &rsh, part,
                      parts);
    return;
  }
  if (blockIdx.x > 0) {
    // workgroups 1..: Q8_0 of x in groups of 4 values, 8 lanes per 32-value
    // block (groups never straddle a block: 256-thread strides, n4 % 8 == 0)
    const int64_t n4 = a.T * a.D / 4;
    const float4* x4 = reinterpret_cast<const float4*>(a.x);
    int* q4 = reinterpret_cast<int*>(a.xq);
    const int64_t stride = (int64_t)(gridDim.x - 1) * 256;
    for (int64_t g = (int64_t)(blockIdx.x - 1) * 256 + tid; g < n4; g += stride) {
      float dv;
      int sum;
      q4[g] = q8_quad(x4[g], &dv, &sum);
      if ((g & 7) == 0) {
        a.xd[g >> 3] = dv;
        a.xsum8[g >> 3] = -8 * sum;
      }
    }
    return;
  }
  if (a.T == 1) {
    if (a.k == 8) one_token_front<8>(a, lane, wave, tid);
    else one_token_front<0>(a, lane, wave, tid);
    return;
  }
  // workgroup 0: routing, one wavefront per token, then the dispatch
  for (int64_t t = wave; t < a.T; t += 4) {
    int my_idx;
    float my_w;
    route_token(a.logits + t * a.E, a.bias, a.E, a.k, a.routed_scale, lane, &my_idx, &my_w);
    if (lane < a.k) {
      a.idx[t * a.k + lane] = my_idx;
      a.w[t * a.k + lane] = my_w;
      ent[t * a.k + lane] = my_idx;
    }
  }
  for (int e = tid; e < a.E + a.S; e += 256) cnt_lds[e] = 0;
  __syncthreads();
  // dispatch, one thread per routing entry: its position in its expert's list
  // is the number of earlier entries (= earlier tokens) that chose the same
  // expert, so the lists come out in token order with no ordering pass
  const int64_t n = a.T * a.k;
  int bad = 0;
  for (int64_t i = tid; i < n; i += 256) {   // an entry is listed if in range and first in its token
    const int e = ent[i];
    bool ok = e >= 0 && e < a.E;
    for (int64_t j = (i / a.k) * a.k; ok && j < i; ++j) ok = ent[j] != e;
    valid[i] = ok;
    bad |= !ok;
  }
  __syncthreads();
  for (int64_t i = tid; i < n; i += 256) {
    if (!valid[i]) continue;
    const int e = ent[i];
    const int64_t t0 = (i / a.k) * a.k;
    int pos = 0;                               // valid entries of earlier tokens: pos <= t < T
    for (int64_t j = 0; j < t0; ++j) pos += valid[j] && ent[j] == e;
    atomicAdd(&cnt_lds[e], 1);
    a.lists[(int64_t)e * a.T + pos] = (int32_t)((i / a.k) * (a.k + a.S) + i % a.k);
  }
  if (a.S) {
    for (int64_t t = tid; t < a.T; t += 256)
      a.lists[(int64_t)a.E * a.T + t] = (int32_t)(t * (a.k + a.S) + a.k);
    if (tid == 0) cnt_lds[a.E] = (int)a.T;
  }
  if (bad) atomicOr(&bad_any, 1);
  __syncthreads();
  for (int e = tid; e < a.E + a.S; e += 256) a.counts[e] = cnt_lds[e];
  if (wave == 0) {
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int base = 0;
    for (int e0 = 0; e0 < a.E + a.S; e0 += kWave) {
      const int e = e0 + lane;
      const bool on = e < a.E + a.S && cnt_lds[e] > 0;
      const uint64_t m = __ballot(on);
      if (on) a.active[base + __popcll(m & lt)] = e;
      base += __popcll(m);
    }
    if (lane == 0) {
      *a.n_active = base;
      *a.err = bad_any ? (int)COLI_E_INDEX : 0;
    }
  }
}

}  // namespace

hipError_t launch_prologue_small(const float* x, const float* logits, const float* bias, int64_t T,
                                 int E, int S, int k, float routed_scale, int64_t D, int8_t* xq,
                                 float* xd, int32_t* xsum8, int32_t* idx, float* w,
                                 int32_t* counts, int32_t* lists, int32_t* n_active,
                                 int32_t* active, int32_t* err, bool norm, float eps,
                                 hipStream_t s) {
  PrologueArgs a = {x, logits, bias, T, D, E, S, k, routed_scale, xq, xd, xsum8, idx, w,
                    counts, lists, n_active, active, err, norm ? 1 : 0, eps};
  int64_t qgroups = (T * D / 4 + 255) / 256;   // one group of 4 values per thread
  if (qgroups > 256) qgroups = 256;
  if (norm) qgroups = T * norm_parts(D);       // norm_parts workgroups per token row
  hipLaunchKernelGGL(prologue_small_kernel, dim3((unsigned)(1 + qgroups)), dim3(256), 0, s, a);
  return hipGetLastError();
}

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
  if (k == 8)
    hipLaunchKernelGGL(dispatch_expert_kernel<8>, dim3((unsigned)(E + 1)), dim3(kDispatchThreads),
                       0, s, idx, T, k, E, S, counts, lists, n_active, active, err);
  else
    hipLaunchKernelGGL(dispatch_expert_kernel<0>, dim3((unsigned)(E + 1)), dim3(kDispatchThreads),
                       0, s, idx, T, k, E, S, counts, lists, n_active, active, err);
  hipError_t rc = hipGetLastError();
  if (rc != hipSuccess || !xq || T == 0) return rc;
  const int64_t nb = T * (D / 32);
  int64_t blocks = (nb + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(xsum8_kernel, dim3((unsigned)blocks), dim3(256), 0, s, xq, nb, xsum8);
  return hipGetLastError();
}

}  // namespace coli

// ---------------------------------------------------------------------------
// Router projection: logits[t][e] = sum_d wr[e][d] * x[t][d] with F32 router
// weights (jeff.news attention-and-kernels section: DeepSeek-V3-style router;
// aitrends.kr "알아두면 좋은 것": the router stays F32).  Every product of two
// floats is exact in fp64; the sum runs in fp64 and is rounded to fp32 once.
// The summation order differs from a sequential one only inside fp64, which
// moves the fp32 result only when the fp64 sum lies within about 2^-29 of a
// rounding boundary.
namespace coli {
namespace {

// Few tokens: one workgroup per expert row, its four wavefronts a quarter
// of the row each.  A wavefront loads its quarter once (float4, every load in
// flight together: up to 8 per lane, a quarter of up to 8,192 columns) and
// keeps it in registers for every token; per token it loads the token's
// quarter, runs four independent fp64 chains per lane and a fixed butterfly
// over the lanes, and the four quarters are summed in order.
constexpr int kRrChunks = 8;   // float4 per lane and quarter row

__global__ void __launch_bounds__(256) router_rows_kernel(const float* __restrict__ x,
                                                          const float* __restrict__ wr,
                                                          int64_t T, int64_t D, int E,
                                                          float* __restrict__ out) {
  __shared__ double part[4][16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e = blockIdx.x;
  const int64_t n4 = D / 4;              // a multiple of 16
  const int64_t q4 = (n4 + 3) / 4;       // float4 per quarter (at most 64 * kRrChunks)
  const int64_t lo = wave * q4, hi = lo + q4 < n4 ? lo + q4 : n4;
  const float4* w4 = reinterpret_cast<const float4*>(wr + (size_t)e * D);
  float4 a[kRrChunks];
#pragma unroll
  for (int u = 0; u < kRrChunks; ++u) {
    const int64_t i = lo + lane + 64 * u;
    a[u] = i < hi ? w4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  for (int64_t t = 0; t < T; ++t) {
    const float4* x4 = reinterpret_cast<const float4*>(x + (size_t)t * D);
    float4 b[kRrChunks];
#pragma unroll
    for (int u = 0; u < kRrChunks; ++u) {
      const int64_t i = lo + lane + 64 * u;
      b[u] = i < hi ? x4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    double s[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int u = 0; u < kRrChunks; ++u) {
      s[0] = __builtin_fma((double)a[u].x, (double)b[u].x, s[0]);
      s[1] = __builtin_fma((double)a[u].y, (double)b[u].y, s[1]);
      s[2] = __builtin_fma((double)a[u].z, (double)b[u].z, s[2]);
      s[3] = __builtin_fma((double)a[u].w, (double)b[u].w, s[3]);
    }
    double v = (s[0] + s[1]) + (s[2] + s[3]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    if (lane == 0) part[wave][t] = v;
  }
  __syncthreads();
  if (threadIdx.x < T)
    out[(size_t)threadIdx.x * E + e] =
        (float)((part[0][threadIdx.x] + part[1][threadIdx.x]) +
                (part[2][threadIdx.x] + part[3][threadIdx.x]));
}

// Many tokens: fp64 matrix cores (v_mfma_f64_16x16x4_f64), the fp32 inputs
// converted to fp64 as they are read from LDS, so every product is exact and
// every sum is an fp64 sum.  A workgroup owns 64 experts x 32 tokens,
// wavefront w the experts 16 w .. 16 w + 15 against the 32 tokens (two 16 x 16
// tiles).  64-column slices of the weight rows and of the tokens are staged
// in LDS as fp32 (rows 66 floats apart: the 32 lanes of each half of an
// operand read hit 32 different banks), double-buffered, the next slice's
// global loads held in registers while the current one is used.
// Operand layouts (16 x 16 x 4, fp64): A lane l = (row l % 16, k l / 16); B
// lane l = (k l / 16, column l % 16); the result's element i of lane l = (row
// l / 16 + 4 i, column l % 16).
typedef double f64x4 __attribute__((ext_vector_type(4)));
constexpr int kRmE = 64, kRmT = 32, kRmK = 64, kRmLd = kRmK + 2;

__global__ void __launch_bounds__(256) router_mfma_kernel(const float* __restrict__ x,
                                                          const float* __restrict__ wr,
                                                          int64_t T, int64_t D, int E,
                                                          float* __restrict__ out) {
  __shared__ float ws[2][kRmE * kRmLd];
  __shared__ float xs[2][kRmT * kRmLd];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int e0 = blockIdx.x * kRmE;
  const int64_t t0 = (int64_t)blockIdx.y * kRmT;
  // staging shares: weight float4 q = tid + 256 j (row q / 16, columns 4 (q % 16) ..),
  // token float4 q = tid + 256 j likewise
  float4 rw[4], rx[2];
  auto load_slice = [&](int64_t k0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int q = tid + 256 * j, r = q >> 4, c4 = q & 15;
      rw[j] = e0 + r < E ? *reinterpret_cast<const float4*>(wr + (size_t)(e0 + r) * D + k0 + 4 * c4)
                         : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int q = tid + 256 * j, r = q >> 4, c4 = q & 15;
      rx[j] = t0 + r < T ? *reinterpret_cast<const float4*>(x + (size_t)(t0 + r) * D + k0 + 4 * c4)
                         : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto store_slice = [&](int slot) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int q = tid + 256 * j, r = q >> 4, c = 4 * (q & 15);
      float2* p = reinterpret_cast<float2*>(&ws[slot][r * kRmLd + c]);
      p[0] = make_float2(rw[j].x, rw[j].y);
      p[1] = make_float2(rw[j].z, rw[j].w);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int q = tid + 256 * j, r = q >> 4, c = 4 * (q & 15);
      float2* p = reinterpret_cast<float2*>(&xs[slot][r * kRmLd + c]);
      p[0] = make_float2(rx[j].x, rx[j].y);
      p[1] = make_float2(rx[j].z, rx[j].w);
    }
  };
  f64x4 acc0 = {0.0, 0.0, 0.0, 0.0}, acc1 = {0.0, 0.0, 0.0, 0.0};
  const int ar = 16 * wave + (lane & 15), bk = lane >> 4, bc = lane & 15;
  load_slice(0);
  store_slice(0);
  __syncthreads();
  int slot = 0;
  for (int64_t k0 = 0; k0 < D; k0 += kRmK) {
    const bool more = k0 + kRmK < D;
    if (more) load_slice(k0 + kRmK);
    const float* wa = &ws[slot][ar * kRmLd + bk];
    const float* xa = &xs[slot][bc * kRmLd + bk];
    const float* xb = &xs[slot][(16 + bc) * kRmLd + bk];
#pragma unroll
    for (int kk = 0; kk < kRmK; kk += 4) {
      const double a = (double)wa[kk];
      acc0 = __builtin_amdgcn_mfma_f64_16x16x4f64(a, (double)xa[kk], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f64_16x16x4f64(a, (double)xb[kk], acc1, 0, 0, 0);
    }
    if (more) store_slice(slot ^ 1);
    __syncthreads();
    slot ^= 1;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = e0 + 16 * wave + (lane >> 4) + 4 * i;
    const int64_t ta = t0 + (lane & 15), tb = ta + 16;
    if (e < E && ta < T) out[(size_t)ta * E + e] = (float)acc0[i];
    if (e < E && tb < T) out[(size_t)tb * E + e] = (float)acc1[i];
  }
}

}  // namespace

hipError_t launch_router_logits(const float* x, const float* wr, int64_t T, int64_t D, int E,
                                float* out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (T < 16 && D / 4 <= 4 * 64 * kRrChunks) {
    hipLaunchKernelGGL(router_rows_kernel, dim3((unsigned)E), dim3(256), 0, s, x, wr, T, D, E,
                       out);
  } else {
    hipLaunchKernelGGL(router_mfma_kernel,
                       dim3((unsigned)((E + kRmE - 1) / kRmE), (unsigned)((T + kRmT - 1) / kRmT)),
                       dim3(256), 0, s, x, wr, T, D, E, out);
  }
  return hipGetLastError();
}

}  // namespace coli
