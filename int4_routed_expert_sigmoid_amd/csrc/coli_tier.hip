// Expert tier: an HBM cache of one layer's experts over a store in host
// memory, run entirely on the device.
//
// The pages keep the routed experts out of fast memory and cache them per
// layer with an LRU, a pinned hot store, and pins learned from a usage log
// (discuss.pytorch.kr colibri summary, "colibri의 핵심 아이디어"; jeff.news,
// idea section).  On MI355X the fast memory is HBM and the store is pinned
// host memory: the plan kernel decides hits, victims and loads from the
// routing already on the device, and the fetch kernel pulls the missing
// experts over the host link into their slots, both stream-ordered, so a
// decode step needs no host synchronisation and a next-layer fetch can run on
// a second stream under the current layer's forward.
//
//  - tier_init_kernel: shared expert in slot 0, pinned experts after it.
//  - tier_plan_kernel (one workgroup, state copied to LDS): selection counts,
//    the fit check, hits stamped in parallel, then each missing expert
//    (ascending id) takes the unpinned slot not used by the pass with the
//    smallest (stamp, slot) -- an argmin over at most 257 slots by the whole
//    workgroup -- and usage counts.
//  - tier_fetch_kernel: 16-byte copies of every expert in the load list,
//    store -> slot, for all four table arrays (one row of workgroups per
//    position of the load list).
#include "coli_internal.h"

namespace coli {
namespace {

constexpr int kPlanThreads = 256;
constexpr int kSlotsPerThread = (COLI_MAX_EXPERTS + 1 + kPlanThreads - 1) / kPlanThreads;

struct TierArgs {
  int32_t* slot_of;
  int32_t* expert_in;
  int32_t* stamp;
  int32_t* pinned;
  int32_t* usage;
  int32_t* loads;
  int32_t* counters;
  int E, S, slots;
};

TierArgs tier_args(const coli_expert_table& t, const coli_tier_state& st) {
  TierArgs a;
  a.slot_of = st.slot_of;
  a.expert_in = st.expert_in;
  a.stamp = st.stamp;
  a.pinned = st.pinned;
  a.usage = st.usage;
  a.loads = st.loads;
  a.counters = st.counters;
  a.E = t.n_routed;
  a.S = t.n_shared;
  a.slots = t.n_slots;
  return a;
}

struct PinList {
  int32_t e[COLI_MAX_EXPERTS + 1];
  int n;
};

__global__ void __launch_bounds__(256) tier_init_kernel(TierArgs a, PinList pin) {
  const int n = a.S + pin.n;
  for (int i = threadIdx.x; i < a.E + a.S; i += blockDim.x) {
    a.slot_of[i] = -1;
    a.usage[i] = 0;
  }
  __syncthreads();
  for (int s = threadIdx.x; s < a.slots; s += blockDim.x) {
    const int e = s < n ? (s < a.S ? a.E : pin.e[s - a.S]) : -1;
    a.expert_in[s] = e;
    a.stamp[s] = -1;
    a.pinned[s] = s < n ? 1 : 0;
    if (e >= 0) a.slot_of[e] = s;
    if (s < n) a.loads[1 + s] = s;
  }
  if (threadIdx.x == 0) {
    a.loads[0] = n;
    a.counters[0] = 0;
    a.counters[1] = 0;
    a.counters[2] = 0;
    a.counters[3] = 0;
  }
}

// (stamp, slot) packed so that a plain integer min orders by stamp, then
// slot: stamps are >= -1, so stamp + 1 is non-negative.
__device__ __forceinline__ int64_t victim_key(int stamp, int slot) {
  return ((int64_t)(stamp + 1) << 32) | (uint32_t)slot;
}

// The plan works on an LDS copy of the state (loaded once, written back once
// at the end), so every phase sees the previous one's writes after a barrier
// and a rejected pass changes nothing.
__global__ void __launch_bounds__(kPlanThreads) tier_plan_kernel(TierArgs a, const int32_t* idx,
                                                                  int64_t T, int k,
                                                                  int count_usage) {
  constexpr int N = COLI_MAX_EXPERTS + 1;
  __shared__ int count[N], slot_of[N], expert_in[N], stamp[N], pinned[N];
  __shared__ int64_t red[kPlanThreads / 64];
  __shared__ int bad, hits, nl, n_miss, n_hit_unpinned, n_unpinned;
  const int tid = threadIdx.x, A = a.E + a.S, NS = a.slots;
  const int step = a.counters[0];
  for (int e = tid; e < A; e += kPlanThreads) {
    count[e] = 0;
    slot_of[e] = a.slot_of[e];
  }
  for (int s = tid; s < NS; s += kPlanThreads) {
    expert_in[s] = a.expert_in[s];
    stamp[s] = a.stamp[s];
    pinned[s] = a.pinned[s];
  }
  if (tid == 0) {
    bad = 0;
    hits = 0;
    nl = 0;
    n_miss = 0;
    n_hit_unpinned = 0;
    n_unpinned = 0;
  }
  __syncthreads();
  for (int64_t i = tid; i < T * k; i += kPlanThreads) {
    const int e = idx[i];
    if (e < 0 || e >= a.E) {
      bad = 1;
    } else {
      atomicAdd(&count[e], 1);
    }
  }
  __syncthreads();
  if (a.S && tid == 0) count[a.E] = (int)T;
  __syncthreads();
  // the pass fits iff its missing experts fit in the unpinned slots that no
  // hit of this pass uses
  for (int e = tid; e < A; e += kPlanThreads) {
    if (count[e] == 0) continue;
    const int s = slot_of[e];
    if (s < 0) {
      atomicAdd(&n_miss, 1);
    } else if (!pinned[s]) {
      atomicAdd(&n_hit_unpinned, 1);
    }
  }
  for (int s = tid; s < NS; s += kPlanThreads)
    if (!pinned[s]) atomicAdd(&n_unpinned, 1);
  __syncthreads();
  if (bad || n_miss > n_unpinned - n_hit_unpinned) {
    if (tid == 0) {
      a.counters[3] = 1;
      a.loads[0] = 0;
    }
    return;
  }
  for (int e = tid; e < A; e += kPlanThreads) {   // hits
    if (count[e] == 0 || slot_of[e] < 0) continue;
    stamp[slot_of[e]] = step;
    atomicAdd(&hits, 1);
  }
  __syncthreads();
  for (int e = 0; e < A; ++e) {                    // misses, ascending id
    if (count[e] == 0 || slot_of[e] >= 0) continue;   // uniform (LDS)
    int64_t best = INT64_MAX;
#pragma unroll
    for (int i = 0; i < kSlotsPerThread; ++i) {
      const int s = tid + i * kPlanThreads;
      if (s < NS && !pinned[s] && stamp[s] < step) {
        const int64_t key = victim_key(stamp[s], s);
        best = key < best ? key : best;
      }
    }
    for (int off = 32; off >= 1; off >>= 1) {
      const int64_t o = __shfl_xor(best, off);
      best = o < best ? o : best;
    }
    if ((tid & 63) == 0) red[tid >> 6] = best;
    __syncthreads();
    if (tid == 0) {
      int64_t m = red[0];
      for (int w = 1; w < kPlanThreads / 64; ++w) m = red[w] < m ? red[w] : m;
      const int v = (int)(uint32_t)(m & 0xFFFFFFFF);
      const int old = expert_in[v];
      if (old >= 0) slot_of[old] = -1;
      expert_in[v] = e;
      slot_of[e] = v;
      stamp[v] = step;
      a.loads[1 + nl] = v;
      nl = nl + 1;
    }
    __syncthreads();
  }
  for (int e = tid; e < A; e += kPlanThreads) {
    a.slot_of[e] = slot_of[e];
    if (count_usage) a.usage[e] += count[e];
  }
  for (int s = tid; s < NS; s += kPlanThreads) {
    a.expert_in[s] = expert_in[s];
    a.stamp[s] = stamp[s];
  }
  if (tid == 0) {
    a.loads[0] = nl;
    a.counters[0] = step + 1;
    a.counters[1] += hits;
    a.counters[2] += nl;
  }
}

constexpr int kFetchBlocks = 64;   // workgroups per loaded expert
constexpr int kFetchUnroll = 4;    // 16-byte loads in flight per thread

struct FetchArgs {
  const int32_t* loads;
  const int32_t* expert_in;
  const uint4* src[4];   // store arrays (device-visible addresses)
  uint4* dst[4];         // tier arrays
  int64_t per[4];        // 16-byte vectors per expert in each array
};

// grid (kFetchBlocks, slots): blockIdx.y is a position in the load list
// (positions past its length return at once), blockIdx.x a slice of the
// expert.  Store reads go over the host link when the store is host memory.
__global__ void __launch_bounds__(256) tier_fetch_kernel(FetchArgs a) {
  const int j = blockIdx.y;
  if (j >= a.loads[0]) return;
  const int slot = a.loads[1 + j];
  const int e = a.expert_in[slot];
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int m = 0; m < 4; ++m) {
    const uint4* src = a.src[m] + (int64_t)e * a.per[m];
    uint4* dst = a.dst[m] + (int64_t)slot * a.per[m];
    const int64_t n = a.per[m];
    for (int64_t v0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v0 < n;
         v0 += stride * kFetchUnroll) {
      uint4 r[kFetchUnroll];
#pragma unroll
      for (int u = 0; u < kFetchUnroll; ++u) {
        const int64_t v = v0 + u * stride;
        if (v < n) r[u] = src[v];
      }
#pragma unroll
      for (int u = 0; u < kFetchUnroll; ++u) {
        const int64_t v = v0 + u * stride;
        if (v < n) dst[v] = r[u];
      }
    }
  }
}

}  // namespace

hipError_t launch_tier_init(const coli_expert_table& t, const coli_tier_state& st,
                            const int32_t* pin, int n_pin, hipStream_t s) {
  PinList p = {};
  for (int i = 0; i < n_pin; ++i) p.e[i] = pin[i];
  p.n = n_pin;
  hipLaunchKernelGGL(tier_init_kernel, dim3(1), dim3(256), 0, s, tier_args(t, st), p);
  return hipGetLastError();
}

hipError_t launch_tier_plan(const coli_expert_table& t, const coli_tier_state& st,
                            const int32_t* idx, int64_t T, int k, int count_usage,
                            hipStream_t s) {
  hipLaunchKernelGGL(tier_plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, tier_args(t, st), idx,
                     T, k, count_usage);
  return hipGetLastError();
}

hipError_t launch_tier_fetch(const coli_expert_table& t, const coli_tier_state& st,
                             const void* const src[4], hipStream_t s) {
  const int64_t D = t.d_model, F = t.d_ff, bits = t.weight_bits;
  FetchArgs a;
  a.loads = st.loads;
  a.expert_in = st.expert_in;
  const int64_t bytes[4] = {F * D * bits / 4, 2 * F * 4, D * F * bits / 8, D * 4};
  void* dst[4] = {t.gu_q, t.gu_s, t.dn_q, t.dn_s};
  for (int m = 0; m < 4; ++m) {
    a.src[m] = static_cast<const uint4*>(src[m]);
    a.dst[m] = static_cast<uint4*>(dst[m]);
    a.per[m] = bytes[m] / 16;
  }
  hipLaunchKernelGGL(tier_fetch_kernel, dim3(kFetchBlocks, (unsigned)t.n_slots), dim3(256), 0, s,
                     a);
  return hipGetLastError();
}

}  // namespace coli
