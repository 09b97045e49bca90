// Internal declarations of the gfx950 library: device math shared by its
// kernels and the host-side launchers called by the C ABI (coli_api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "coli.h"

namespace coli {

// ---------------------------------------------------------------------------
// Device math.  The fp32 op sequence is fixed (hipcc -ffp-contract=off; IEEE
// division and square root; fmaf -> v_fma_f32; rintf -> v_rndne_f32) so that
// every integer decision it feeds (top-k order, Q8 codes) is reproducible.

// exp(x): Cody & Waite reduction (1980) by n*ln2, ln2 split into a 16-bit
// high part and its remainder, |r| <= ln2/2, Taylor series of e^r to degree 7
// in Horner form (truncation < half an ulp), scaled by 2^n.  The input is
// clamped to [-87, 88.5] so results stay normal floats.
__device__ __forceinline__ float exp_f32(float x) {
  if (x > 88.5f) x = 88.5f;
  if (x < -87.0f) x = -87.0f;
  const float n = __builtin_rintf(x * 1.44269504088896341f);
  float r = __builtin_fmaf(-n, 0.693145751953125f, x);
  r = __builtin_fmaf(-n, 1.42860676533018708e-06f, r);
  float p = 1.98412698412698413e-04f;
  p = __builtin_fmaf(p, r, 1.38888888888888889e-03f);
  p = __builtin_fmaf(p, r, 8.33333333333333333e-03f);
  p = __builtin_fmaf(p, r, 4.16666666666666667e-02f);
  p = __builtin_fmaf(p, r, 1.66666666666666667e-01f);
  p = __builtin_fmaf(p, r, 0.5f);
  p = __builtin_fmaf(p, r, 1.0f);
  p = __builtin_fmaf(p, r, 1.0f);
  return __builtin_amdgcn_ldexpf(p, (int)n);
}

__device__ __forceinline__ float sigmoid_f32(float x) { return 1.0f / (1.0f + exp_f32(-x)); }
__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + exp_f32(-g)); }

// Q8_0 code of v in a block whose scale is d (d == 0: code 0).
__device__ __forceinline__ int q8_code(float v, float d) {
  if (d == 0.0f) return 0;
  float q = __builtin_rintf(v / d);
  q = q > 127.0f ? 127.0f : q;
  q = q < -127.0f ? -127.0f : q;
  return (int)q;
}

// Q8_0 of 4 consecutive values held by one lane; 8 consecutive lanes form one
// 32-value block.  Returns the 4 codes packed little-endian in an int32, the
// block scale and the block's code sum (all identical in the 8 lanes).
__device__ __forceinline__ int q8_quad(float4 v, float* d_out, int* sum_out) {
  float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
  amax = fmaxf(amax, __shfl_xor(amax, 1, 8));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 8));
  amax = fmaxf(amax, __shfl_xor(amax, 4, 8));
  const float d = amax / 127.0f;
  *d_out = d;
  const int q0 = q8_code(v.x, d), q1 = q8_code(v.y, d), q2 = q8_code(v.z, d),
            q3 = q8_code(v.w, d);
  int sum = q0 + q1 + q2 + q3;
  sum += __shfl_xor(sum, 1, 8);
  sum += __shfl_xor(sum, 2, 8);
  sum += __shfl_xor(sum, 4, 8);
  *sum_out = sum;
  return (q0 & 0xFF) | ((q1 & 0xFF) << 8) | ((q2 & 0xFF) << 16) | ((int)((unsigned)q3 << 24));
}

// RMSNorm with unit gain, then Q8_0, of one row of D values (D % 32 == 0),
// by one 256-thread workgroup: the sum of squares in fp64 (each square is
// exact; per-thread strided partials, a lane butterfly, then the four
// wavefronts' sums as (w0 + w1) + (w2 + w3)), r = (float)(1 / sqrt(ss / D +
// eps)) in fp64, x = h * r in fp32, then q8_quad.  Writes the packed codes,
// the block scales, and when non-null the blocks' -8 * code sums and r.
// red / rsh: workgroup LDS (4 doubles, 1 float).  Every thread must call it.
// RMSNorm of one row h (sum of squares in fp64, in one fixed order) and Q8_0
// of x = h * r.  part / nparts: this workgroup quantises Q8 blocks
// [part * ceil(NB / nparts), ...) of the row only; every part computes the
// same r (same data, same order), so a row may be split over workgroups.
// NQ: groups of 4 values per thread and phase (1 when a part is at most 256
// groups).
template <int NQ = 8>
__device__ __forceinline__ void rmsnorm_q8_row(const float* __restrict__ hrow, int64_t D, float eps,
                                               int* __restrict__ q, float* __restrict__ d,
                                               int32_t* __restrict__ xsum8,
                                               float* __restrict__ r_out, double* red,
                                               float* rsh, int part = 0, int nparts = 1) {
  const float4* hr = reinterpret_cast<const float4*>(hrow);
  double ss = 0.0;
  for (int64_t c = threadIdx.x; c < D / 4; c += 256) {
    const float4 v = hr[c];
    ss += (double)v.x * (double)v.x;
    ss += (double)v.y * (double)v.y;
    ss += (double)v.z * (double)v.z;
    ss += (double)v.w * (double)v.w;
  }
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  if (threadIdx.x == 0) {
    const double tot = (red[0] + red[1]) + (red[2] + red[3]);
    const float r = (float)(1.0 / sqrt(tot / (double)D + (double)eps));
    *rsh = r;
    if (r_out && part == 0) *r_out = r;
  }
  __syncthreads();
  const float r = *rsh;
  // Q8_0 of x = h * r with q8_quad's arithmetic, taken in phases over up to
  // NQ groups of 4 values per thread with branch-free codes (a zero
  // scale divides by 1 and its code is selected away), so that the lane
  // exchanges and the divisions of independent groups overlap.  A group past
  // the row (whole 8-lane blocks: D/4 and 256 are multiples of 8) computes on
  // an in-bounds copy and stores nothing.
  constexpr int kNormQuads = NQ;
  const int64_t nb = D / 32, per = (nb + nparts - 1) / nparts;
  const int64_t b0 = (int64_t)part * per, b1 = b0 + per < nb ? b0 + per : nb;
  const int64_t n4 = 8 * b1;   // end of this part's groups of 4
  for (int64_t c0 = 8 * b0; c0 < n4; c0 += 256 * kNormQuads) {
    int64_t c[kNormQuads];
    float4 x[kNormQuads];
    float amax[kNormQuads], dq[kNormQuads];
    int qv[kNormQuads][4], sum[kNormQuads];
#pragma unroll
    for (int u = 0; u < kNormQuads; ++u) {
      c[u] = c0 + 256 * u + threadIdx.x;
      const float4 v = hr[c[u] < n4 ? c[u] : (threadIdx.x & 7)];
      x[u] = make_float4(v.x * r, v.y * r, v.z * r, v.w * r);
      amax[u] = fmaxf(fmaxf(fabsf(x[u].x), fabsf(x[u].y)), fmaxf(fabsf(x[u].z), fabsf(x[u].w)));
    }
#pragma unroll
    for (int off = 1; off < 8; off <<= 1) {
#pragma unroll
      for (int u = 0; u < kNormQuads; ++u) amax[u] = fmaxf(amax[u], __shfl_xor(amax[u], off, 8));
    }
#pragma unroll
    for (int u = 0; u < kNormQuads; ++u) {
      dq[u] = amax[u] / 127.0f;
      const bool zero = dq[u] == 0.0f;
      const float dd = zero ? 1.0f : dq[u];
      const float xs[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float qf = __builtin_rintf(xs[i] / dd);
        qf = qf > 127.0f ? 127.0f : qf;
        qf = qf < -127.0f ? -127.0f : qf;
        qv[u][i] = zero ? 0 : (int)qf;
      }
      sum[u] = qv[u][0] + qv[u][1] + qv[u][2] + qv[u][3];
    }
#pragma unroll
    for (int off = 1; off < 8; off <<= 1) {
#pragma unroll
      for (int u = 0; u < kNormQuads; ++u) sum[u] += __shfl_xor(sum[u], off, 8);
    }
#pragma unroll
    for (int u = 0; u < kNormQuads; ++u) {
      if (c[u] < n4) {
        q[c[u]] = (qv[u][0] & 0xFF) | ((qv[u][1] & 0xFF) << 8) | ((qv[u][2] & 0xFF) << 16) |
                  ((int)((unsigned)qv[u][3] << 24));
        if ((c[u] & 7) == 0) {
          d[c[u] >> 3] = dq[u];
          if (xsum8) xsum8[c[u] >> 3] = -8 * sum[u];
        }
      }
    }
  }
}

// Read-only data that is uniform across a wavefront (the token's Q8 block,
// dispatch lists) is read through the constant address space: the compiler
// then issues scalar loads, which complete on lgkmcnt and leave the vector
// memory counter to the weight stream.
template <class T>
using cptr = const T __attribute__((address_space(4)))*;
template <class T>
__device__ __forceinline__ cptr<T> as_const(const T* p) {
  return (cptr<T>)(p);
}

// Signed int8 dot of four packed bytes, accumulated into c (v_dot4_i32_i8).
__device__ __forceinline__ int sdot4(int a, int b, int c) {
  return __builtin_amdgcn_sdot4(a, b, c, false);
}

// ---------------------------------------------------------------------------
// Workspace of coli_moe_forward, carved from the caller's buffer.
struct MoeWorkspace {
  int32_t* counts;   // [A]
  int32_t* lists;    // [A][T]
  int32_t* n_active; // [1]
  int32_t* active;   // [A]
  int32_t* err;      // [1]
  int32_t* xsum8;    // [T][D/32]   -8 * sum of each Q8 block of x
  int8_t* hq;        // [P][F]
  float* hd;         // [P][F/32]
  int32_t* hsum8;    // [P][F/32]   -8 * sum of each Q8 block of h
  float* o;          // [P][D]
  // one-token passes only (else null): Q8(h) again, in active-slot order, so
  // the down kernel can stage it without looking up the slot's pair
  int8_t* hq_slot;   // [A][F]
  float* hd_slot;    // [A][F/32]
  int32_t* hs_slot;  // [A][F/32]
  // grouped (matrix-core) path only
  uint16_t* xh;      // [T][D/32][32] f16 codes of xq in MFMA operand order
  uint16_t* h16;     // [P][F/32][32] f16 codes of Q8(h) in MFMA operand order
  // accumulator inputs of the matrix-core operands, per Q8 block (the memory
  // of xsum8 and hsum8, which the grouped path does not use)
  float* xbias;      // [T][D/32]
  float* hbias;      // [P][F/32]
  int32_t* chunks;   // [max chunks][2] (expert, chunk index) in execution order
  int32_t* n_chunks; // [1]
  size_t bytes;
};

// Layout for (E, S, D, F, T, k); base == nullptr only sizes it.
MoeWorkspace moe_workspace_layout(void* base, int E, int S, int64_t D, int64_t F, int64_t T, int k);

// ---------------------------------------------------------------------------
// Launchers (return hipError_t of the launch).
hipError_t launch_quant_act_q8(const float* x, int64_t rows, int64_t k, int8_t* q, float* d,
                               hipStream_t s);
hipError_t launch_quant_weight_q4(const float* w, int64_t rows, int64_t k, uint8_t* q, float* sc,
                                  hipStream_t s);
hipError_t launch_quant_weight_q8(const float* w, int64_t rows, int64_t k, int8_t* q, float* sc,
                                  hipStream_t s);
hipError_t launch_quant_weight_q2(const float* w, int64_t rows, int64_t k, uint8_t* q, float* sc,
                                  hipStream_t s);
hipError_t launch_table_set_expert(const coli_expert_table& t, int expert, const uint8_t* gate_q,
                                   const float* gate_s, const uint8_t* up_q, const float* up_s,
                                   const uint8_t* down_q, const float* down_s, hipStream_t s);
hipError_t launch_rmsnorm_q8(const float* h, int64_t T, int64_t D, float eps, int8_t* q, float* d,
                             float* r_out, hipStream_t s);
// Expert tier (coli_tier.hip).  pin: host array of n_pin experts.
hipError_t launch_tier_init(const coli_expert_table& t, const coli_tier_state& st,
                            const int32_t* pin, int n_pin, hipStream_t s);
hipError_t launch_tier_plan(const coli_expert_table& t, const coli_tier_state& st,
                            const int32_t* idx, int64_t T, int k, int count_usage, hipStream_t s);
// src: device-visible addresses of the store's gu_q, gu_s, dn_q, dn_s.
hipError_t launch_tier_fetch(const coli_expert_table& t, const coli_tier_state& st,
                             const void* const src[4], hipStream_t s);
// logits[t][e] = sum_d wr[e][d] x[t][d], fp64 sum rounded once (D % 64 == 0).
hipError_t launch_router_logits(const float* x, const float* wr, int64_t T, int64_t D, int E,
                                float* out, hipStream_t s);
hipError_t launch_route_topk(const float* logits, const float* bias, int64_t T, int E, int k,
                             float routed_scale, int32_t* idx, float* w, hipStream_t s);
// Dispatch lists + compaction + index check; xq != nullptr also fills xsum8.
hipError_t launch_dispatch(const int32_t* idx, int64_t T, int k, int E, int S, int32_t* counts,
                           int32_t* lists, int32_t* n_active, int32_t* active, int32_t* err,
                           const int8_t* xq, int64_t D, int32_t* xsum8, hipStream_t s);

// Fused front of a small batch (one workgroup): Q8_0 of x (+ block sums),
// routing, dispatch lists, compaction and the index check.  norm: x is the
// residual stream and RMSNorm(x) (unit gain, eps) is quantised instead.
hipError_t launch_prologue_small(const float* x, const float* logits, const float* bias, int64_t T,
                                 int E, int S, int k, float routed_scale, int64_t D, int8_t* xq,
                                 float* xd, int32_t* xsum8, int32_t* idx, float* w,
                                 int32_t* counts, int32_t* lists, int32_t* n_active,
                                 int32_t* active, int32_t* err, bool norm, float eps,
                                 hipStream_t s);
// Largest batch the fused front handles.
constexpr int64_t kPrologueMaxEntries = 1024;   // T * k
constexpr int64_t kPrologueMaxTokens = 64;

struct ForwardArgs {
  const coli_expert_table* table;
  const int8_t* xq;
  const float* xd;
  int64_t T;
  const int32_t* idx;
  const float* w;
  int k;
  float* y;
  int accumulate;
  MoeWorkspace ws;
  const coli_moe_trace* trace;   // may be null
  const coli_moe_events* events; // may be null
  bool dispatched;               // the workspace already holds dispatch + xsum8
  bool grouped;                  // run the grouped matrix-core path (see choose_grouped)
};
hipError_t launch_moe_forward(const ForwardArgs& a, hipStream_t s);

// Grouped (matrix-core) expert FFN, used from COLI_GROUPED_MIN_TOKENS tokens per pass.
bool mfma_path_fits(int64_t T, int64_t D, int64_t F, int k, int S);
// Whether the grouped path applies to (table, T, k): resident int4 tables only.
bool grouped_applies(const coli_expert_table& t, int64_t T, int k);
int64_t mfma_max_chunks(int64_t T, int k, int E, int S);
int mfma_quads_gate_up(int64_t F);
int mfma_quads_down(int64_t D);
// Work lists and f16 activation codes; needs the dispatch lists.
hipError_t launch_mfma_front(const coli_expert_table& t, const int8_t* xq, int64_t T,
                             const MoeWorkspace& ws, hipStream_t s);
// gate/up + SwiGLU + Q8(h), then down, writing ws.o; ev_down (may be null) is
// recorded between the two.
hipError_t launch_mfma_ffn(const coli_expert_table& t, const float* xd, int64_t T, int k,
                           const MoeWorkspace& ws, const coli_moe_trace* tr, void* ev_down,
                           hipStream_t s);

}  // namespace coli
