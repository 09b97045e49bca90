// Grouped-GEMM path of the expert FFN for batches with many tokens per expert
// (prefill and long verify passes): the same per-block integer dot products
// and the same fp32 rescale as the GEMV path, computed with matrix cores.
//
// What is computed (aitrends.kr "GLM-5.2-colibri-int4", "기술적 특징": int4
// weights with a per-row F32 scale against int8 activations; discuss.pytorch.kr
// colibri summary, "colibri의 주요 기능": integer-dot expert matmuls, Q8_0
// activations; batch-union grouping so that each expert's rows are read once
// per pass): for each dispatched (token, expert) pair and each weight row r,
//   P[r][b] = sum over the 32 columns of block b of q_w * q_x   (exact integer)
//   acc = fmaf(P[r][b], d_b, acc) for b = 0, 1, ... in order; out_r = acc * s_r.
//
// Why f16 matrix cores carry the integer dot.  The int4 codes (|q| <= 7) and
// the Q8 codes (|q| <= 127) are exact f16 values, each product is exact, and
// every partial sum of a 32-column block is an integer below 2^15, so the fp32
// accumulation inside v_mfma_f32_32x32x16_f16 is exact: it returns P[r][b]
// bit-for-bit, already as fp32.  The exact Q8_0 rescale then costs one VALU
// fmaf per (row, token, block).  With int8 matrix cores the int32 result needs
// a conversion first, which doubles that VALU stream, and the VALU stream, not
// the matrix cores, bounds this kernel on gfx950.
//
// Tiling.  One wavefront owns one 64-row group of the table (32 gate + 32 up
// rows, or 64 down rows) for up to 64 tokens (two 32-token subtiles).  Per
// 32-column block it loads the group's 1 KB of nibbles (16 B per lane), swaps
// lane halves so that each lane holds half of the columns of one row of each
// 32-row tile (v_permlane32_swap), expands nibbles to f16 in registers, and
// issues two K=16 MFMAs per 32x32 tile.  Four wavefronts of a workgroup take
// four consecutive row groups of the same tokens and share the token blocks
// through LDS.  The work list (expert, row quad, token chunk)
// is built on the device after dispatch; the launch is sized for the worst
// case and workgroups past the real count return at once.  Consecutive work
// items are mapped to the same XCD so that chunks of one expert share its
// weight rows in that XCD's L2.
#include "coli_internal.h"

namespace coli {
namespace {

constexpr int kWave = 64;
constexpr int kChunk = 64;        // tokens per work item (two 32-token subtiles)
constexpr int kGroupsPerWg = 4;   // row groups per workgroup (one per wavefront)
constexpr int kPfW = 4;           // weight blocks in flight per wavefront

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBufferConfig = 0x00020000;

// A 32-bit constant held in a VGPR, so that (x & m) | c selects v_and_or_b32
// (a VOP3 instruction here takes no literal and one scalar operand at most).
__device__ __forceinline__ uint32_t vconst(uint32_t c) {
  uint32_t r;
  asm("v_mov_b32 %0, %1" : "=v"(r) : "i"(c));
  return r;
}

struct UnpackConsts {
  uint32_t lo, hi, magic;
};

__device__ __forceinline__ UnpackConsts unpack_consts() {
  return {vconst(0x000F000Fu), vconst(0x00F000F0u), vconst(0x64006400u)};
}

// Eight offset-binary nibbles of one table word (byte j: column j in the low
// nibble, column 4 + j in the high nibble; nibble n = q + 8) as eight exact
// f16 values.  A nibble OR-ed into the low mantissa bits of 1024.0 (0x6400)
// gives 1024 + n, one OR-ed four bits higher gives 1024 + 16n; subtracting
// 1032 or 1152 leaves q or 16q.  Element order (columns): 0, 2, 4, 6, 1, 3, 5,
// 7, where the elements 2, 3, 6, 7 carry 16q; the activation operand carries
// x / 16 in those places, so every product is exactly q * x.
__device__ __forceinline__ half8 nibbles_to_f16(uint32_t w, const UnpackConsts& c) {
  const half2v b1 = {(_Float16)1032.0f, (_Float16)1032.0f};
  const half2v b16 = {(_Float16)1152.0f, (_Float16)1152.0f};
  const uint32_t w8 = w >> 8;
  const half2v h0 = __builtin_bit_cast(half2v, (w & c.lo) | c.magic) - b1;
  const half2v h1 = __builtin_bit_cast(half2v, (w & c.hi) | c.magic) - b16;
  const half2v h2 = __builtin_bit_cast(half2v, (w8 & c.lo) | c.magic) - b1;
  const half2v h3 = __builtin_bit_cast(half2v, (w8 & c.hi) | c.magic) - b16;
  half8 r;
  r[0] = h0[0]; r[1] = h0[1]; r[2] = h1[0]; r[3] = h1[1];
  r[4] = h2[0]; r[5] = h2[1]; r[6] = h3[0]; r[7] = h3[1];
  return r;
}

// The matrix-core operands of one table chunk.  Lane L of a row group holds
// row L's 32 columns as words w0..w3 (columns 0-7, 8-15, 16-23, 24-31).  A
// 32x32x16 MFMA wants lane l to hold row (l & 31) with columns 16 * (l >> 5)
// onward.  Swapping w0/w1 of the upper lanes with w2/w3 of the lower lanes
// gives every lane the right half of tile 0 (rows 0-31 of the group) in
// (t0a, t0b) and of tile 1 (rows 32-63) in (t1a, t1b).
struct TileOps {
  half8 t0a, t0b, t1a, t1b;
};

__device__ __forceinline__ TileOps tile_operands(u32x4 w, const UnpackConsts& c) {
  const auto s0 = __builtin_amdgcn_permlane32_swap(w.x, w.z, false, false);
  const auto s1 = __builtin_amdgcn_permlane32_swap(w.y, w.w, false, false);
  TileOps o;
  o.t0a = nibbles_to_f16(s0[0], c);
  o.t0b = nibbles_to_f16(s1[0], c);
  o.t1a = nibbles_to_f16(s0[1], c);
  o.t1b = nibbles_to_f16(s1[1], c);
  return o;
}

__device__ __forceinline__ f32x16 mfma(half8 a, half8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// The ordered rescale acc = fmaf(P, d, acc) of every element of a tile, kept
// where it is written: the empty volatile asm statements make P an input
// produced at this point and acc an output consumed here, so the compiler
// neither hoists the fmaf group above the preceding MFMAs nor sinks it into
// the next block.
__device__ __forceinline__ void rescale(f32x16& acc, f32x16 p, float d) {
  asm volatile("" : "+v"(p));
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = __builtin_fmaf(p[i], d, acc[i]);
  asm volatile("" : "+v"(acc));
}

// Row of a 32x32 tile held by register i of lane l; the lane's column (token)
// is l & 31.
__device__ __forceinline__ int tile_row(int i, int lane) {
  return (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
}

struct Item {
  int e, quad, chunk;
  bool ok;
};

// Work item of this workgroup: logical index L = XCD-major remap of
// blockIdx.x over the real item count.
__device__ __forceinline__ Item locate(const int2* items, const int32_t* total) {
  Item it = {};
  const int tot = *as_const(total);
  const int per = (tot + 7) >> 3;
  const int bid = (int)blockIdx.x;
  const int L = (bid & 7) * per + (bid >> 3);
  it.ok = (bid >> 3) < per && L < tot;
  if (!it.ok) return it;
  const cptr<int32_t> v = as_const(reinterpret_cast<const int32_t*>(items) + 2 * (size_t)L);
  const int x = v[0];
  it.e = x & 0xFFFF;
  it.quad = x >> 16;
  it.chunk = v[1];
  return it;
}

struct GuArgs {
  const u32x4* gu_q;
  const float* gu_s;
  const u32x4* xh;       // [T][NB][4] 16-byte pieces of f16 codes
  const float* xd;       // [T][NB]
  const int32_t* counts;
  const int32_t* lists;
  const int2* items;
  const int32_t* total;
  uint32_t* h16;         // [P][G][16] words: f16 codes of Q8(h)
  float* hd;             // [P][G]
  int8_t* hq;            // [P][F] (traced runs only)
  int64_t T, D, F;
  int k, S;
  int32_t* tr_pg;
  int32_t* tr_pu;
  float* tr_g;
  float* tr_u;
  float* tr_h;
};

struct DnArgs {
  const u32x4* dn_q;
  const float* dn_s;
  const u32x4* h16;      // [P][G][4] pieces
  const float* hd;
  const int32_t* counts;
  const int32_t* lists;
  const int2* items;
  const int32_t* total;
  float* o;              // [P][D]
  int64_t T, D, F;
  int k, S;
  int32_t* tr_pd;
};

// ---------------------------------------------------------------------------
// Streaming one row group against the chunk's tokens.
//
// Weights: a kPfW-deep register ring of 16-byte buffer loads per lane; the
// operands of block b + 1 are unpacked while the MFMAs of block b run.
// Tokens: the workgroup stages kStage blocks of its 64 tokens' f16 pieces and
// block scales in LDS (two stage slots); each wavefront loads a quarter of a
// stage into registers one stage ahead and stores it to the free slot, and a
// barrier per stage publishes it.  Inside a token's 64-byte block the four
// 16-byte pieces sit at position piece ^ ((token >> 2) & 3), so the 16 lanes
// of one LDS read hit 16 different 16-byte bank groups.
constexpr int kStage = 4;   // blocks per LDS stage (= one turn of the weight ring)
static_assert(kPfW == kStage, "one weight ring turn per stage");

struct StageLds {
  uint4 x[2][kStage][kChunk][4];
  float d[2][kChunk][kStage];
};

struct WeightRows {
  __amdgpu_buffer_rsrc_t rs;
  uint32_t off;   // this lane's chunk offset within a block (16 * lane)
};

// The lane's share of stage loads: token 16 * wave + lane / 4 of the chunk,
// piece (lane & 3) ^ swizzle, and the scales of blocks 2 * (lane & 3) + {0, 1}
// (lanes with (lane & 3) >= kStage / 2 load nothing for the scales).
struct TokenRows {
  __amdgpu_buffer_rsrc_t rs;
  uint32_t off;       // byte offset of the token row's piece in block 0
  const float* d;     // the token's scales
  int NB;
};

struct StageRegs {
  u32x4 x[kStage];
  float d0, d1;
};

__device__ __forceinline__ void stage_load(const TokenRows& t, int b0, int lane, StageRegs& r) {
#pragma unroll
  for (int j = 0; j < kStage; ++j) {
    const int b = b0 + j < t.NB ? b0 + j : t.NB - 1;
    r.x[j] = __builtin_amdgcn_raw_buffer_load_b128(t.rs, t.off + 64u * (uint32_t)b, 0, 0);
  }
  const int bd = b0 + 2 * (lane & 3);
  r.d0 = t.d[bd < t.NB ? bd : t.NB - 1];
  r.d1 = t.d[bd + 1 < t.NB ? bd + 1 : t.NB - 1];
}

__device__ __forceinline__ void stage_store(StageLds& L, int slot, int wave, int lane,
                                            const StageRegs& r) {
  uint4* xs = &L.x[slot][0][0][0] + 64 * wave + lane;
#pragma unroll
  for (int j = 0; j < kStage; ++j) xs[j * kChunk * 4] = __builtin_bit_cast(uint4, r.x[j]);
  if (2 * (lane & 3) < kStage) {
    float* ds = &L.d[slot][16 * wave + (lane >> 2)][2 * (lane & 3)];
    ds[0] = r.d0;
    ds[1] = r.d1;
  }
}

template <int NSUB>
struct Acc {
  f32x16 t0[NSUB], t1[NSUB];   // tile 0 (rows 0-31 of the group), tile 1 (rows 32-63)
};

// Token operands (two K-halves per subtile) of block J of a stage slot.
template <int NSUB>
struct BOps {
  half8 k0[NSUB], k1[NSUB];
};

template <int NSUB>
__device__ __forceinline__ void read_bops(const StageLds& L, int slot, int J, int p0, int p1,
                                          int lane, BOps<NSUB>& o) {
  const uint4* xs = &L.x[slot][J][0][0];
  const int n = lane & 31;
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    o.k0[s] = __builtin_bit_cast(half8, xs[(32 * s + n) * 4 + p0]);
    o.k1[s] = __builtin_bit_cast(half8, xs[(32 * s + n) * 4 + p1]);
  }
}

#define COLI_FENCE() __builtin_amdgcn_sched_barrier(0)

// Block b = b0 + J of stage slot `slot`, in an order that keeps the matrix
// pipe and the VALU busy together: the MFMAs of subtile 0, the first half of
// the next block's nibble expansion, the rescale of tile 0, the MFMAs of
// subtile 1, the rescale of tile 1, the second half of the expansion, then
// the rescales of subtile 1.  The next block's token operands are read from
// LDS while this block computes (within a stage).
template <int NSUB, bool TRACE, int J>
__device__ __forceinline__ void block_step(const StageLds& L, int slot, int b0, int NB,
                                           const WeightRows& wr, u32x4 (&wq)[kPfW], TileOps& cur,
                                           BOps<NSUB>& bo, const UnpackConsts& uc,
                                           const float (&dv)[NSUB][kStage], int p0, int p1,
                                           Acc<NSUB>& acc, int32_t* const (&tr0)[NSUB],
                                           int32_t* const (&tr1)[NSUB], int lane) {
  const int b = b0 + J;
  const f32x16 z = {};
  f32x16 p[NSUB][2];
  p[0][0] = mfma(cur.t0a, bo.k0[0], z);
  p[0][1] = mfma(cur.t1a, bo.k0[0], z);
  p[0][0] = mfma(cur.t0b, bo.k1[0], p[0][0]);
  p[0][1] = mfma(cur.t1b, bo.k1[0], p[0][1]);
  COLI_FENCE();
  BOps<NSUB> bn = bo;
  if (J + 1 < kStage) read_bops<NSUB>(L, slot, J + 1, p0, p1, lane, bn);
  constexpr int JN = (J + 1) % kPfW;   // ring slot of block b + 1
  const u32x4 w = wq[JN];
  const auto sa = __builtin_amdgcn_permlane32_swap(w.x, w.z, false, false);
  TileOps nx;
  nx.t0a = nibbles_to_f16(sa[0], uc);
  nx.t1a = nibbles_to_f16(sa[1], uc);
  COLI_FENCE();
  rescale(acc.t0[0], p[0][0], dv[0][J]);
  COLI_FENCE();
  if (NSUB > 1) {
    p[NSUB - 1][0] = mfma(cur.t0a, bo.k0[NSUB - 1], z);
    p[NSUB - 1][1] = mfma(cur.t1a, bo.k0[NSUB - 1], z);
    p[NSUB - 1][0] = mfma(cur.t0b, bo.k1[NSUB - 1], p[NSUB - 1][0]);
    p[NSUB - 1][1] = mfma(cur.t1b, bo.k1[NSUB - 1], p[NSUB - 1][1]);
    COLI_FENCE();
  }
  rescale(acc.t1[0], p[0][1], dv[0][J]);
  COLI_FENCE();
  const auto sb = __builtin_amdgcn_permlane32_swap(w.y, w.w, false, false);
  nx.t0b = nibbles_to_f16(sb[0], uc);
  nx.t1b = nibbles_to_f16(sb[1], uc);
  const int bnx = b + 1 + kPfW < NB ? b + 1 + kPfW : NB - 1;
  wq[JN] = __builtin_amdgcn_raw_buffer_load_b128(wr.rs, wr.off + 1024u * (uint32_t)bnx, 0, 0);
  COLI_FENCE();
  if (NSUB > 1) {
    rescale(acc.t0[NSUB - 1], p[NSUB - 1][0], dv[NSUB - 1][J]);
    rescale(acc.t1[NSUB - 1], p[NSUB - 1][1], dv[NSUB - 1][J]);
  }
  if (TRACE) {
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int rr = tile_row(i, lane);
        if (tr0[s]) tr0[s][(size_t)rr * NB + b] = (int32_t)p[s][0][i];
        if (tr1[s]) tr1[s][(size_t)rr * NB + b] = (int32_t)p[s][1][i];
      }
    }
  }
  cur = nx;
  bo = bn;
}

template <int NSUB, bool TRACE, bool GUARD, int J>
__device__ __forceinline__ void stage_steps(const StageLds& L, int slot, int b0, int NB,
                                            const WeightRows& wr, u32x4 (&wq)[kPfW],
                                            TileOps& cur, BOps<NSUB>& bo, const UnpackConsts& uc,
                                            const float (&dv)[NSUB][kStage], int p0, int p1,
                                            Acc<NSUB>& acc, int32_t* const (&tr0)[NSUB],
                                            int32_t* const (&tr1)[NSUB], int lane) {
  if constexpr (J < kStage) {
    if (!GUARD || b0 + J < NB)
      block_step<NSUB, TRACE, J>(L, slot, b0, NB, wr, wq, cur, bo, uc, dv, p0, p1, acc, tr0, tr1,
                                 lane);
    stage_steps<NSUB, TRACE, GUARD, J + 1>(L, slot, b0, NB, wr, wq, cur, bo, uc, dv, p0, p1, acc,
                                           tr0, tr1, lane);
  }
}

template <int NSUB, bool TRACE, bool GUARD>
__device__ __forceinline__ void stage_compute(const StageLds& L, int slot, int b0, int NB,
                                              const WeightRows& wr, u32x4 (&wq)[kPfW],
                                              TileOps& cur, const UnpackConsts& uc, int p0, int p1,
                                              Acc<NSUB>& acc, int32_t* const (&tr0)[NSUB],
                                              int32_t* const (&tr1)[NSUB], int lane) {
  const int n = lane & 31;
  float dv[NSUB][kStage];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    const float4 v = *reinterpret_cast<const float4*>(&L.d[slot][32 * s + n][0]);
    dv[s][0] = v.x;
    dv[s][1] = v.y;
    dv[s][2] = v.z;
    dv[s][3] = v.w;
  }
  BOps<NSUB> bo;
  read_bops<NSUB>(L, slot, 0, p0, p1, lane, bo);
  stage_steps<NSUB, TRACE, GUARD, 0>(L, slot, b0, NB, wr, wq, cur, bo, uc, dv, p0, p1, acc, tr0,
                                     tr1, lane);
}

// All NB blocks of one row group against NSUB subtiles of the chunk's tokens.
// Every wavefront of the workgroup takes part in the staging and barriers;
// COMPUTE is false for a wavefront whose row group is past the matrix.  The
// loop over full stages issues the same loads on every path (indices past the
// end are clamped), so the compiler's memory-counter waits stay exact and the
// weight and stage prefetches stay in flight; a partial last stage runs after it.
template <int NSUB, bool TRACE, bool COMPUTE>
__device__ __forceinline__ void stream_loop(StageLds& L, const WeightRows& wr,
                                            const TokenRows& tk, Acc<NSUB>& acc,
                                            int32_t* const (&tr0)[NSUB],
                                            int32_t* const (&tr1)[NSUB], int wave, int lane) {
  const int NB = tk.NB;
  const int NS = (NB + kStage - 1) / kStage, NSF = NB / kStage;
  const UnpackConsts uc = unpack_consts();
  u32x4 wq[kPfW];
  TileOps cur = {};
  if (COMPUTE) {
#pragma unroll
    for (int j = 0; j < kPfW; ++j) {
      const int b = j < NB ? j : NB - 1;
      wq[j] = __builtin_amdgcn_raw_buffer_load_b128(wr.rs, wr.off + 1024u * (uint32_t)b, 0, 0);
    }
  }
  StageRegs R;
  stage_load(tk, 0, lane, R);
  stage_store(L, 0, wave, lane, R);
  stage_load(tk, kStage, lane, R);
  if (COMPUTE) {
    cur = tile_operands(wq[0], uc);
    const int b = kPfW < NB ? kPfW : NB - 1;
    wq[0] = __builtin_amdgcn_raw_buffer_load_b128(wr.rs, wr.off + 1024u * (uint32_t)b, 0, 0);
  }
  __syncthreads();
  const int n = lane & 31, h = lane >> 5, sw = (n >> 2) & 3;
  const int p0 = (2 * h) ^ sw, p1 = (2 * h + 1) ^ sw;
  int st = 0;
  for (; st < NSF; ++st) {
    const int slot = st & 1;
    if (COMPUTE)
      stage_compute<NSUB, TRACE, false>(L, slot, st * kStage, NB, wr, wq, cur, uc, p0, p1, acc,
                                        tr0, tr1, lane);
    stage_store(L, slot ^ 1, wave, lane, R);
    stage_load(tk, (st + 2) * kStage, lane, R);
    __syncthreads();
  }
  if (COMPUTE && st < NS)
    stage_compute<NSUB, TRACE, true>(L, st & 1, st * kStage, NB, wr, wq, cur, uc, p0, p1, acc,
                                     tr0, tr1, lane);
}

template <int NSUB, bool TRACE>
__device__ __forceinline__ void stream_group(StageLds& L, const WeightRows& wr,
                                             const TokenRows& tk, bool compute, Acc<NSUB>& acc,
                                             int32_t* const (&tr0)[NSUB],
                                             int32_t* const (&tr1)[NSUB], int wave, int lane) {
  if (compute) stream_loop<NSUB, TRACE, true>(L, wr, tk, acc, tr0, tr1, wave, lane);
  else stream_loop<NSUB, TRACE, false>(L, wr, tk, acc, tr0, tr1, wave, lane);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint64_t bytes) {
  const uint32_t n = bytes > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, kBufferConfig);
}

// Chunk entry of this lane's stage loads and of its subtile columns.
struct ChunkTokens {
  int n_valid;          // tokens in the chunk (1..64)
  int load_entry;       // list entry of token 16 * wave + lane / 4 (clamped)
  int pair[2];          // list entries of the lane's columns in subtiles 0, 1 (clamped)
};

__device__ __forceinline__ ChunkTokens chunk_tokens(const int32_t* lists, int64_t T, int e,
                                                    int chunk, int cnt, int wave, int lane) {
  ChunkTokens c;
  const int rem = cnt - chunk * kChunk;
  c.n_valid = rem < kChunk ? rem : kChunk;
  const int32_t* list = lists + (size_t)e * T + (size_t)chunk * kChunk;
  const int lt = 16 * wave + (lane >> 2);
  c.load_entry = list[lt < c.n_valid ? lt : c.n_valid - 1];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int i = 32 * s + (lane & 31);
    c.pair[s] = list[i < c.n_valid ? i : c.n_valid - 1];
  }
  return c;
}

// Piece offset of a token row for this lane's stage loads.
__device__ __forceinline__ uint32_t load_piece_off(int64_t row, int NB, int wave, int lane) {
  const int lt = 16 * wave + (lane >> 2);
  const int piece = (lane & 3) ^ ((lt >> 2) & 3);
  return (uint32_t)((uint64_t)row * (uint64_t)NB * 64u) + 16u * (uint32_t)piece;
}

// ---------------------------------------------------------------------------
// gate/up: g and u of one 32-row tile pair, SwiGLU, Q8_0 of h per token.
template <int NSUB, bool TRACE>
__device__ __forceinline__ void gate_up_body(const GuArgs& a, StageLds& L, const Item& it,
                                             const ChunkTokens& ct, int grp, bool compute,
                                             int wave, int lane) {
  const int NB = (int)(a.D / 32);
  const int64_t G = a.F / 32;
  const int KS = a.k + a.S;
  const int n = lane & 31, hl = lane >> 5;
  const int nt = ct.n_valid;
  WeightRows wr;
  const int gsafe = compute ? grp : 0;
  wr.rs = make_rsrc(a.gu_q + ((size_t)it.e * G + gsafe) * (size_t)NB * kWave, (uint64_t)NB * 1024u);
  wr.off = 16u * (uint32_t)lane;
  TokenRows tk;
  tk.NB = NB;
  tk.rs = make_rsrc(a.xh, (uint64_t)a.T * (uint64_t)a.D * 2u);
  const int64_t lt = ct.load_entry / KS;
  tk.off = load_piece_off(lt, NB, wave, lane);
  tk.d = a.xd + lt * NB;
  int32_t* tr0[NSUB];
  int32_t* tr1[NSUB];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    tr0[s] = tr1[s] = nullptr;
    if (TRACE && compute && 32 * s + n < nt) {
      const size_t row0 = ((size_t)ct.pair[s] * a.F + 32 * (size_t)grp) * NB;
      if (a.tr_pg) tr0[s] = a.tr_pg + row0;
      if (a.tr_pu) tr1[s] = a.tr_pu + row0;
    }
  }
  Acc<NSUB> acc;
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
#pragma unroll
    for (int i = 0; i < 16; ++i) acc.t0[s][i] = acc.t1[s][i] = 0.0f;
  }
  stream_group<NSUB, TRACE>(L, wr, tk, compute, acc, tr0, tr1, wave, lane);
  if (!compute) return;

  const float* sg = a.gu_s + ((size_t)it.e * G + grp) * kWave;
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    const bool valid = 32 * s + n < nt;
    const size_t p = (size_t)ct.pair[s];
    float h[16];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = tile_row(i, lane);
      const float g = acc.t0[s][i] * sg[r];
      const float u = acc.t1[s][i] * sg[32 + r];
      h[i] = silu_f32(g) * u;
      amax = fmaxf(amax, fabsf(h[i]));
      if (TRACE && valid) {
        const size_t o = p * a.F + 32 * (size_t)grp + r;
        if (a.tr_g) a.tr_g[o] = g;
        if (a.tr_u) a.tr_u[o] = u;
        if (a.tr_h) a.tr_h[o] = h[i];
      }
    }
    amax = fmaxf(amax, __shfl_xor(amax, 32));   // the token's other 16 rows
    const float d = amax / 127.0f;
    int q[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) q[i] = q8_code(h[i], d);
    if (!valid) continue;
    if (hl == 0) a.hd[p * G + grp] = d;
    // f16 codes in the piece order the down projection reads: word 4m + hl
    // holds rows (8m + 4hl, 8m + 4hl + 2), word 4m + 2 + hl rows (+1, +3);
    // the upper lanes' words are operand elements 2, 3, 6, 7, stored as q / 16.
    const float sc = hl ? 0.0625f : 1.0f;
    uint32_t* hw = a.h16 + (p * G + grp) * 16;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const half2v lo = {(_Float16)((float)q[4 * m + 0] * sc), (_Float16)((float)q[4 * m + 2] * sc)};
      const half2v hi = {(_Float16)((float)q[4 * m + 1] * sc), (_Float16)((float)q[4 * m + 3] * sc)};
      hw[4 * m + hl] = __builtin_bit_cast(uint32_t, lo);
      hw[4 * m + 2 + hl] = __builtin_bit_cast(uint32_t, hi);
    }
    if (TRACE && a.hq) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        a.hq[p * a.F + 32 * (size_t)grp + tile_row(i, lane)] = (int8_t)q[i];
    }
  }
}

template <bool TRACE>
__global__ void __launch_bounds__(256) mfma_gate_up_kernel(GuArgs a) {
  __shared__ StageLds lds;
  const Item it = locate(a.items, a.total);
  if (!it.ok) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int grp = it.quad * kGroupsPerWg + wave;
  const bool compute = grp < (int)(a.F / 32);
  const int cnt = as_const(a.counts)[it.e];
  const ChunkTokens ct = chunk_tokens(a.lists, a.T, it.e, it.chunk, cnt, wave, lane);
  if (ct.n_valid > 32) gate_up_body<2, TRACE>(a, lds, it, ct, grp, compute, wave, lane);
  else gate_up_body<1, TRACE>(a, lds, it, ct, grp, compute, wave, lane);
}

// ---------------------------------------------------------------------------
// down: o = s_r * acc for 64 rows (two 32-row tiles) of the chunk's pairs.
template <int NSUB, bool TRACE>
__device__ __forceinline__ void down_body(const DnArgs& a, StageLds& L, const Item& it,
                                          const ChunkTokens& ct, int grp, bool compute, int wave,
                                          int lane) {
  const int NB = (int)(a.F / 32);
  const int64_t G = a.F / 32;
  const int64_t RG = a.D / 64;
  const int n = lane & 31, hl = lane >> 5;
  const int nt = ct.n_valid;
  WeightRows wr;
  const int gsafe = compute ? grp : 0;
  wr.rs = make_rsrc(a.dn_q + ((size_t)it.e * RG + gsafe) * (size_t)NB * kWave, (uint64_t)NB * 1024u);
  wr.off = 16u * (uint32_t)lane;
  TokenRows tk;
  tk.NB = NB;
  const int64_t P = a.T * (int64_t)(a.k + a.S);
  tk.rs = make_rsrc(a.h16, (uint64_t)P * (uint64_t)a.F * 2u);
  tk.off = load_piece_off(ct.load_entry, NB, wave, lane);
  tk.d = a.hd + (size_t)ct.load_entry * G;
  int32_t* tr0[NSUB];
  int32_t* tr1[NSUB];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    tr0[s] = tr1[s] = nullptr;
    if (TRACE && compute && 32 * s + n < nt && a.tr_pd) {
      tr0[s] = a.tr_pd + ((size_t)ct.pair[s] * a.D + 64 * (size_t)grp) * NB;
      tr1[s] = tr0[s] + (size_t)32 * NB;
    }
  }
  Acc<NSUB> acc;
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
#pragma unroll
    for (int i = 0; i < 16; ++i) acc.t0[s][i] = acc.t1[s][i] = 0.0f;
  }
  stream_group<NSUB, TRACE>(L, wr, tk, compute, acc, tr0, tr1, wave, lane);
  if (!compute) return;

  const float* sr = a.dn_s + (size_t)it.e * a.D + 64 * (size_t)grp;
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    if (32 * s + n >= nt) continue;
    float* orow = a.o + (size_t)ct.pair[s] * a.D + 64 * (size_t)grp;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int r = 8 * m + 4 * hl;   // rows r .. r + 3 of each tile
      float4 v0, v1;
      v0.x = acc.t0[s][4 * m + 0] * sr[r + 0];
      v0.y = acc.t0[s][4 * m + 1] * sr[r + 1];
      v0.z = acc.t0[s][4 * m + 2] * sr[r + 2];
      v0.w = acc.t0[s][4 * m + 3] * sr[r + 3];
      v1.x = acc.t1[s][4 * m + 0] * sr[32 + r + 0];
      v1.y = acc.t1[s][4 * m + 1] * sr[32 + r + 1];
      v1.z = acc.t1[s][4 * m + 2] * sr[32 + r + 2];
      v1.w = acc.t1[s][4 * m + 3] * sr[32 + r + 3];
      *reinterpret_cast<float4*>(orow + r) = v0;
      *reinterpret_cast<float4*>(orow + 32 + r) = v1;
    }
  }
}

template <bool TRACE>
__global__ void __launch_bounds__(256) mfma_down_kernel(DnArgs a) {
  __shared__ StageLds lds;
  const Item it = locate(a.items, a.total);
  if (!it.ok) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int grp = it.quad * kGroupsPerWg + wave;
  const bool compute = grp < (int)(a.D / 64);
  const int cnt = as_const(a.counts)[it.e];
  const ChunkTokens ct = chunk_tokens(a.lists, a.T, it.e, it.chunk, cnt, wave, lane);
  if (ct.n_valid > 32) down_body<2, TRACE>(a, lds, it, ct, grp, compute, wave, lane);
  else down_body<1, TRACE>(a, lds, it, ct, grp, compute, wave, lane);
}

// ---------------------------------------------------------------------------
// Front of the grouped path, after dispatch.  Workgroup 0 builds the work
// lists: per active expert c = ceil(count / 64) chunks, and per chunk qg
// gate/up and qd down row quads; items of one expert are contiguous, ordered
// (quad, chunk) with the chunk fastest.  The other workgroups write the f16
// codes of the Q8 activations in the piece order the MFMA operands read:
// piece 2h + m of block b holds columns 16h + 8m + {0, 2, 4, 6, 1, 3, 5, 7},
// the columns 4, 6, 5, 7 of each eight as q / 16 (exact in f16).
struct FrontArgs {
  const int32_t* counts;
  const int32_t* n_active;
  const int32_t* active;
  int2* gu_items;
  int2* dn_items;
  int32_t* totals;   // [2]: gate/up items, down items
  int qg, qd;
  const int8_t* xq;
  uint4* xh;
  int64_t T, D;
};

__global__ void __launch_bounds__(256) mfma_front_kernel(FrontArgs a) {
  if (blockIdx.x == 0) {
    __shared__ int pre[512 + 1];
    __shared__ int act[512];
    __shared__ int wsum[4];
    const int nact = *a.n_active;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    // active experts and their chunk counts, two per thread
    const int e0 = 2 * t < nact ? a.active[2 * t] : 0;
    const int e1 = 2 * t + 1 < nact ? a.active[2 * t + 1] : 0;
    const int n0 = 2 * t < nact ? a.counts[e0] : 0;
    const int n1 = 2 * t + 1 < nact ? a.counts[e1] : 0;
    act[2 * t] = e0;
    act[2 * t + 1] = e1;
    const int c0 = (n0 + kChunk - 1) / kChunk, c1 = (n1 + kChunk - 1) / kChunk;
    int v = c0 + c1;   // inclusive scan of the pair sums across the workgroup
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int u = __shfl_up(v, off);
      if (lane >= off) v += u;
    }
    if (lane == 63) wsum[wave] = v;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w) base += wsum[w];
    const int excl = base + v - (c0 + c1);
    pre[2 * t] = excl;
    pre[2 * t + 1] = excl + c0;
    if (t == 255) pre[512] = base + v;
    __syncthreads();
    const int chunks = pre[512];
    if (t == 0) {
      a.totals[0] = chunks * a.qg;
      a.totals[1] = chunks * a.qd;
    }
    for (int s = wave; s < nact; s += 4) {
      const int e = act[s];
      const int c = pre[s + 1] - pre[s];
      for (int i = lane; i < c * a.qg; i += kWave)
        a.gu_items[pre[s] * a.qg + i] = make_int2(e | ((i / c) << 16), i % c);
      for (int i = lane; i < c * a.qd; i += kWave)
        a.dn_items[pre[s] * a.qd + i] = make_int2(e | ((i / c) << 16), i % c);
    }
    return;
  }
  const int64_t pieces = a.T * (a.D / 32) * 4;
  const int64_t stride = (int64_t)(gridDim.x - 1) * blockDim.x;
  for (int64_t i = (int64_t)(blockIdx.x - 1) * blockDim.x + threadIdx.x; i < pieces; i += stride) {
    // piece i = (token, block, 2h + m): source columns 16h + 8m .. + 7 of the block
    const int64_t col0 = (i >> 2) * 32 + (i & 3) * 8;
    const uint2 src = *reinterpret_cast<const uint2*>(a.xq + col0);
    const int8_t* c = reinterpret_cast<const int8_t*>(&src);
    half8 h;
    h[0] = (_Float16)c[0];
    h[1] = (_Float16)c[2];
    h[2] = (_Float16)((float)c[4] * 0.0625f);
    h[3] = (_Float16)((float)c[6] * 0.0625f);
    h[4] = (_Float16)c[1];
    h[5] = (_Float16)c[3];
    h[6] = (_Float16)((float)c[5] * 0.0625f);
    h[7] = (_Float16)((float)c[7] * 0.0625f);
    a.xh[i] = __builtin_bit_cast(uint4, h);
  }
}

}  // namespace

bool mfma_path_fits(int64_t T, int64_t D, int64_t F, int k, int S) {
  const int64_t P = T * (int64_t)(k + S);
  return T * D * 2 < 0x7FFFFFFFll && P * F * 2 < 0x7FFFFFFFll && D % 64 == 0 && F % 32 == 0;
}

bool grouped_applies(const coli_expert_table& t, int64_t T, int k) {
  return t.weight_bits == 4 && !t.slot_of && T >= 1 &&
         mfma_path_fits(T, t.d_model, t.d_ff, k, t.n_shared);
}

int64_t mfma_max_chunks(int64_t T, int k, int E, int S) {
  return T * (int64_t)(k + S) / kChunk + (E + S);
}

int mfma_quads_gate_up(int64_t F) { return (int)((F / 32 + kGroupsPerWg - 1) / kGroupsPerWg); }
int mfma_quads_down(int64_t D) { return (int)((D / 64 + kGroupsPerWg - 1) / kGroupsPerWg); }

hipError_t launch_mfma_front(const coli_expert_table& t, const int8_t* xq, int64_t T,
                             const MoeWorkspace& ws, hipStream_t s) {
  FrontArgs f = {};
  f.counts = ws.counts;
  f.n_active = ws.n_active;
  f.active = ws.active;
  f.gu_items = reinterpret_cast<int2*>(ws.gu_items);
  f.dn_items = reinterpret_cast<int2*>(ws.dn_items);
  f.totals = ws.totals;
  f.qg = mfma_quads_gate_up(t.d_ff);
  f.qd = mfma_quads_down(t.d_model);
  f.xq = xq;
  f.xh = reinterpret_cast<uint4*>(ws.xh);
  f.T = T;
  f.D = t.d_model;
  const int64_t pieces = T * (t.d_model / 32) * 4;
  int64_t blocks = (pieces + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  hipLaunchKernelGGL(mfma_front_kernel, dim3((unsigned)(1 + blocks)), dim3(256), 0, s, f);
  return hipGetLastError();
}

hipError_t launch_mfma_ffn(const coli_expert_table& t, const float* xd, int64_t T, int k,
                           const MoeWorkspace& ws, const coli_moe_trace* tr, void* ev_down,
                           hipStream_t s) {
  const int E = t.n_routed, S = t.n_shared;
  const int64_t max_chunks = mfma_max_chunks(T, k, E, S);
  GuArgs g = {};
  g.gu_q = reinterpret_cast<const u32x4*>(t.gu_q);
  g.gu_s = t.gu_s;
  g.xh = reinterpret_cast<const u32x4*>(ws.xh);
  g.xd = xd;
  g.counts = ws.counts;
  g.lists = ws.lists;
  g.items = reinterpret_cast<const int2*>(ws.gu_items);
  g.total = ws.totals;
  g.h16 = reinterpret_cast<uint32_t*>(ws.h16);
  g.hd = ws.hd;
  g.hq = tr ? ws.hq : nullptr;
  g.T = T;
  g.D = t.d_model;
  g.F = t.d_ff;
  g.k = k;
  g.S = S;
  DnArgs d = {};
  d.dn_q = reinterpret_cast<const u32x4*>(t.dn_q);
  d.dn_s = t.dn_s;
  d.h16 = reinterpret_cast<const u32x4*>(ws.h16);
  d.hd = ws.hd;
  d.counts = ws.counts;
  d.lists = ws.lists;
  d.items = reinterpret_cast<const int2*>(ws.dn_items);
  d.total = ws.totals + 1;
  d.o = ws.o;
  d.T = T;
  d.D = t.d_model;
  d.F = t.d_ff;
  d.k = k;
  d.S = S;
  const unsigned grid_gu = (unsigned)((max_chunks * mfma_quads_gate_up(t.d_ff) + 7) / 8 * 8);
  const unsigned grid_dn = (unsigned)((max_chunks * mfma_quads_down(t.d_model) + 7) / 8 * 8);
  if (tr) {
    g.tr_pg = tr->p_gate;
    g.tr_pu = tr->p_up;
    g.tr_g = tr->g;
    g.tr_u = tr->u;
    g.tr_h = tr->h;
    d.tr_pd = tr->p_down;
    hipLaunchKernelGGL(mfma_gate_up_kernel<true>, dim3(grid_gu), dim3(256), 0, s, g);
  } else {
    hipLaunchKernelGGL(mfma_gate_up_kernel<false>, dim3(grid_gu), dim3(256), 0, s, g);
  }
  hipError_t rc = hipGetLastError();
  if (rc != hipSuccess) return rc;
  if (ev_down && (rc = hipEventRecord(static_cast<hipEvent_t>(ev_down), s)) != hipSuccess) return rc;
  if (tr) hipLaunchKernelGGL(mfma_down_kernel<true>, dim3(grid_dn), dim3(256), 0, s, d);
  else hipLaunchKernelGGL(mfma_down_kernel<false>, dim3(grid_dn), dim3(256), 0, s, d);
  return hipGetLastError();
}

}  // namespace coli
