// Quantisers and table loading for gfx950.
//
//  - Q8_0 activations (discuss.pytorch.kr colibri summary, "colibri의 주요 기능":
//    int8 activations in the Q8_0 style): blocks of 32, d = max|x| / 127,
//    q = rint_half_even(x / d).
//  - per-row int4 weights (aitrends.kr "GLM-5.2-colibri-int4", "TL;DR" and
//    "기술적 특징": U8-packed nibbles, per-row F32 scale, np.rint = lrintf):
//    s = max|w| / 7, q = rint_half_even(w / s) in [-7, 7].
//  - per-row int8 weights, the container of the int8 speculative head
//    (discuss.pytorch.kr colibri summary, "colibri의 주요 기능", MTP bullet):
//    s = max|w| / 127, q = rint_half_even(w / s) in [-127, 127].
//  - RMSNorm with unit gain before Q8 (norm weights stay F32, same page,
//    "알아두면 좋은 것").
//  - re-laying a canonical expert container (int4 or int8) into the GEMV
//    table layout.
//
// All of these are small, HBM-bound passes; they are written for coalesced
// 128-bit loads and stores, not for MFMA.
#include "coli_internal.h"

namespace coli {
namespace {

constexpr int kWave = 64;

__global__ void __launch_bounds__(256) quant_act_q8_kernel(const float4* __restrict__ x,
                                                           int64_t n4, int* __restrict__ q,
                                                           float* __restrict__ d) {
  // grid-stride over groups of 4 values; the stride is a multiple of 8 so the
  // 8 lanes of a block stay together.
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    float dv;
    int sum;
    const int packed = q8_quad(x[i], &dv, &sum);
    q[i] = packed;
    if ((i & 7) == 0) d[i >> 3] = dv;
  }
}

// ---------------------------------------------------------------------------
// Per-row int4: one 256-thread workgroup per row.
__device__ __forceinline__ float block_max_256(float v, float* red) {
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  v = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return v;
}

__device__ __forceinline__ int q4_code(float v, float s) {
  if (s == 0.0f) return 0;
  float q = __builtin_rintf(v / s);
  q = q > 7.0f ? 7.0f : q;
  q = q < -7.0f ? -7.0f : q;
  return (int)q;
}

__global__ void __launch_bounds__(256) quant_weight_q4_kernel(const float* __restrict__ w,
                                                              int64_t k, uint32_t* __restrict__ q,
                                                              float* __restrict__ s) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const float4* wr = reinterpret_cast<const float4*>(w + row * k);
  float amax = 0.0f;
  for (int64_t c = threadIdx.x; c < k / 4; c += 256) {
    const float4 v = wr[c];
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  }
  amax = block_max_256(amax, red);
  const float sc = amax / 7.0f;
  if (threadIdx.x == 0) s[row] = sc;
  uint32_t* qr = q + row * (k / 8);
  for (int64_t c = threadIdx.x; c < k / 8; c += 256) {   // 8 columns -> one 32-bit word
    const float4 a = wr[2 * c], b = wr[2 * c + 1];
    const int v[8] = {q4_code(a.x, sc), q4_code(a.y, sc), q4_code(a.z, sc), q4_code(a.w, sc),
                      q4_code(b.x, sc), q4_code(b.y, sc), q4_code(b.z, sc), q4_code(b.w, sc)};
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) word |= (uint32_t)(v[i] & 0xF) << (4 * i);
    qr[c] = word;   // byte i: column 2i low nibble, 2i+1 high nibble
  }
}

// ---------------------------------------------------------------------------
// Per-row int8: one 256-thread workgroup per row, 4 columns per 32-bit word.
__device__ __forceinline__ uint32_t q8w_code(float v, float s) {
  if (s == 0.0f) return 0;
  float q = __builtin_rintf(v / s);
  q = q > 127.0f ? 127.0f : q;
  q = q < -127.0f ? -127.0f : q;
  return (uint32_t)(int)q & 0xFFu;
}

__global__ void __launch_bounds__(256) quant_weight_q8_kernel(const float* __restrict__ w,
                                                              int64_t k, uint32_t* __restrict__ q,
                                                              float* __restrict__ s) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const float4* wr = reinterpret_cast<const float4*>(w + row * k);
  float amax = 0.0f;
  for (int64_t c = threadIdx.x; c < k / 4; c += 256) {
    const float4 v = wr[c];
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  }
  amax = block_max_256(amax, red);
  const float sc = amax / 127.0f;
  if (threadIdx.x == 0) s[row] = sc;
  uint32_t* qr = q + row * (k / 4);
  for (int64_t c = threadIdx.x; c < k / 4; c += 256) {   // byte i of the word: column 4c + i
    const float4 v = wr[c];
    qr[c] = q8w_code(v.x, sc) | (q8w_code(v.y, sc) << 8) | (q8w_code(v.z, sc) << 16) |
            (q8w_code(v.w, sc) << 24);
  }
}

// ---------------------------------------------------------------------------
// Per-row int2 (the narrowest packing next to int8 and int4): s = max|w| / 1,
// q = rint_half_even(w / s) in [-1, 1], four 2-bit two's-complement fields
// per byte, the lowest bits holding the first column.  One 256-thread
// workgroup per row, 16 columns per 32-bit word.
__device__ __forceinline__ uint32_t q2_code(float v, float s) {
  if (s == 0.0f) return 0;
  float q = __builtin_rintf(v / s);
  q = q > 1.0f ? 1.0f : q;
  q = q < -1.0f ? -1.0f : q;
  return (uint32_t)(int)q & 3u;
}

__global__ void __launch_bounds__(256) quant_weight_q2_kernel(const float* __restrict__ w,
                                                              int64_t k, uint32_t* __restrict__ q,
                                                              float* __restrict__ s) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const float4* wr = reinterpret_cast<const float4*>(w + row * k);
  float amax = 0.0f;
  for (int64_t c = threadIdx.x; c < k / 4; c += 256) {
    const float4 v = wr[c];
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  }
  amax = block_max_256(amax, red);
  const float sc = amax / 1.0f;
  if (threadIdx.x == 0) s[row] = sc;
  uint32_t* qr = q + row * (k / 16);
  for (int64_t c = threadIdx.x; c < k / 16; c += 256) {   // 16 columns -> one word
    uint32_t word = 0;
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const float4 v = wr[4 * c + f];
      word |= (q2_code(v.x, sc) | (q2_code(v.y, sc) << 2) | (q2_code(v.z, sc) << 4) |
               (q2_code(v.w, sc) << 6)) << (8 * f);
    }
    qr[c] = word;   // byte i: columns 4i..4i+3, lowest bits first
  }
}

// Canonical int2 chunk (16 bytes, 64 columns; byte i holds columns
// 4i..4i+3, lowest bits first, two's complement) -> table chunk (word m,
// byte j, field i: column 16m + 4i + j; field = q + 2).  Field j of canonical
// byte 4m + i moves to field i of byte j of word m; XOR 2 turns a 2-bit two's
// complement value into q + 2.
__device__ __forceinline__ uint4 retile_chunk2(uint4 src) {
  const uint32_t sw[4] = {src.x, src.y, src.z, src.w};
  uint32_t dw[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t byte = (sw[m] >> (8 * i)) & 0xFFu;   // canonical byte 4m + i
        const uint32_t f = ((byte >> (2 * j)) & 3u) ^ 2u;
        word |= f << (8 * j + 2 * i);
      }
    dw[m] = word;
  }
  return make_uint4(dw[0], dw[1], dw[2], dw[3]);
}

// ---------------------------------------------------------------------------
// Canonical container chunk (16 bytes, 32 columns, column 2i in the low nibble
// of byte i, two's complement) -> table chunk (word kk, byte j: column
// 8kk+j low, 8kk+4+j high; nibble = q + 8).
__device__ __forceinline__ uint4 retile_chunk(uint4 src) {
  const uint32_t sw[4] = {src.x, src.y, src.z, src.w};
  uint32_t dw[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c0 = 8 * kk + j, c1 = 8 * kk + 4 + j;   // columns within the block
      const uint32_t n0 = (sw[c0 >> 3] >> (4 * (c0 & 7))) & 0xF;
      const uint32_t n1 = (sw[c1 >> 3] >> (4 * (c1 & 7))) & 0xF;
      word |= ((n0 ^ 8u) | ((n1 ^ 8u) << 4)) << (8 * j);
    }
    dw[kk] = word;
  }
  return make_uint4(dw[0], dw[1], dw[2], dw[3]);
}

struct SetExpertArgs {
  const uint4* gate_q;  // [F][D/32] (int4) or [F][D/16] (int8) chunks
  const uint4* up_q;
  const uint4* down_q;  // [D][F/32] or [D][F/16] chunks
  const float* gate_s;
  const float* up_s;
  const float* down_s;
  uint4* gu_q;          // this expert's slot
  float* gu_s;
  uint4* dn_q;
  float* dn_s;
  int64_t D, F;
};

// A canonical row is a run of 16-byte chunks (32 int4, 16 int8 or 64 int2
// columns each); the table puts chunk c of every lane's row side by side.
// int4 and int2 chunks are re-encoded (retile_chunk, retile_chunk2), int8
// chunks copied unchanged.
template <int BITS>
__device__ __forceinline__ uint4 retile(uint4 src) {
  if constexpr (BITS == 4) return retile_chunk(src);
  if constexpr (BITS == 2) return retile_chunk2(src);
  return src;
}

template <int BITS>
__global__ void __launch_bounds__(256) table_set_expert_kernel(SetExpertArgs a) {
  const int64_t ncd = a.D * BITS / 128, ncf = a.F * BITS / 128;   // chunks per row
  const int64_t n_gu = (a.F / 32) * ncd * 64;   // chunks in the gate/up slot
  const int64_t n_dn = (a.D / 64) * ncf * 64;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_gu + n_dn; i += stride) {
    if (i < n_gu) {
      const int64_t lane = i % 64, c = (i / 64) % ncd, g = i / (64 * ncd);
      const int64_t row = 32 * g + (lane & 31);
      const uint4 src = ((lane < 32 ? a.gate_q : a.up_q) + row * ncd)[c];
      a.gu_q[i] = retile<BITS>(src);
      if (c == 0) a.gu_s[g * 64 + lane] = lane < 32 ? a.gate_s[row] : a.up_s[row];
    } else {
      const int64_t j = i - n_gu;
      const int64_t lane = j % 64, c = (j / 64) % ncf, g = j / (64 * ncf);
      const int64_t row = 64 * g + lane;
      const uint4 src = a.down_q[row * ncf + c];
      a.dn_q[j] = retile<BITS>(src);
      if (c == 0) a.dn_s[row] = a.down_s[row];
    }
  }
}

// ---------------------------------------------------------------------------
// RMSNorm (fp64 sum of squares) + Q8_0: one 256-thread workgroup per row.
__global__ void __launch_bounds__(256) rmsnorm_q8_kernel(const float* __restrict__ h, int64_t D,
                                                         float eps, int* __restrict__ q,
                                                         float* __restrict__ d,
                                                         float* __restrict__ r_out) {
  __shared__ double red[4];
  __shared__ float rsh;
  const int64_t row = blockIdx.x;
  rmsnorm_q8_row(h + row * D, D, eps, q + row * (D / 4), d + row * (D / 32), nullptr,
                 r_out ? r_out + row : nullptr, red, &rsh);
}

int64_t grid_for(int64_t work, int64_t per_block, int64_t cap) {
  int64_t g = (work + per_block - 1) / per_block;
  if (g < 1) g = 1;
  return g > cap ? cap : g;
}

}  // namespace

hipError_t launch_quant_act_q8(const float* x, int64_t rows, int64_t k, int8_t* q, float* d,
                               hipStream_t s) {
  const int64_t n4 = rows * k / 4;
  if (n4 == 0) return hipSuccess;
  hipLaunchKernelGGL(quant_act_q8_kernel, dim3((unsigned)grid_for(n4, 256, 1 << 16)), dim3(256),
                     0, s, reinterpret_cast<const float4*>(x), n4, reinterpret_cast<int*>(q), d);
  return hipGetLastError();
}

hipError_t launch_quant_weight_q4(const float* w, int64_t rows, int64_t k, uint8_t* q, float* sc,
                                  hipStream_t s) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(quant_weight_q4_kernel, dim3((unsigned)rows), dim3(256), 0, s, w, k,
                     reinterpret_cast<uint32_t*>(q), sc);
  return hipGetLastError();
}

hipError_t launch_quant_weight_q2(const float* w, int64_t rows, int64_t k, uint8_t* q, float* sc,
                                  hipStream_t s) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(quant_weight_q2_kernel, dim3((unsigned)rows), dim3(256), 0, s, w, k,
                     reinterpret_cast<uint32_t*>(q), sc);
  return hipGetLastError();
}

hipError_t launch_quant_weight_q8(const float* w, int64_t rows, int64_t k, int8_t* q, float* sc,
                                  hipStream_t s) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(quant_weight_q8_kernel, dim3((unsigned)rows), dim3(256), 0, s, w, k,
                     reinterpret_cast<uint32_t*>(q), sc);
  return hipGetLastError();
}

hipError_t launch_table_set_expert(const coli_expert_table& t, int expert, const uint8_t* gate_q,
                                   const float* gate_s, const uint8_t* up_q, const float* up_s,
                                   const uint8_t* down_q, const float* down_s, hipStream_t s) {
  const int64_t D = t.d_model, F = t.d_ff;
  SetExpertArgs a;
  a.gate_q = reinterpret_cast<const uint4*>(gate_q);
  a.up_q = reinterpret_cast<const uint4*>(up_q);
  a.down_q = reinterpret_cast<const uint4*>(down_q);
  a.gate_s = gate_s;
  a.up_s = up_s;
  a.down_s = down_s;
  const int64_t bits = t.weight_bits;   // 4 or 8, checked by the caller
  a.gu_q = reinterpret_cast<uint4*>(t.gu_q + (size_t)expert * (size_t)(F * D * bits / 4));
  a.gu_s = t.gu_s + (size_t)expert * (size_t)(2 * F);
  a.dn_q = reinterpret_cast<uint4*>(t.dn_q + (size_t)expert * (size_t)(D * F * bits / 8));
  a.dn_s = t.dn_s + (size_t)expert * (size_t)D;
  a.D = D;
  a.F = F;
  const int64_t chunks = ((F / 32) * (D * bits / 128) + (D / 64) * (F * bits / 128)) * 64;
  const dim3 grid((unsigned)grid_for(chunks, 256, 1 << 16));
  if (bits == 8)
    hipLaunchKernelGGL(table_set_expert_kernel<8>, grid, dim3(256), 0, s, a);
  else if (bits == 2)
    hipLaunchKernelGGL(table_set_expert_kernel<2>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(table_set_expert_kernel<4>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_q8(const float* h, int64_t T, int64_t D, float eps, int8_t* q, float* d,
                             float* r_out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(rmsnorm_q8_kernel, dim3((unsigned)T), dim3(256), 0, s, h, D, eps,
                     reinterpret_cast<int*>(q), d, r_out);
  return hipGetLastError();
}

}  // namespace coli
