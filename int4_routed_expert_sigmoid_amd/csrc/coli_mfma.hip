// Grouped-GEMM path of the expert FFN for batches with many tokens per expert
// (prefill and long verify passes): the same per-block integer dot products
// and the same fp32 rescale as the GEMV path, computed with matrix cores.
//
// What is computed (aitrends.kr "GLM-5.2-colibri-int4", "기술적 특징": int4
// weights with a per-row F32 scale against int8 activations; discuss.pytorch.kr
// colibri summary, "colibri의 주요 기능": integer-dot expert matmuls, Q8_0
// activations; alphamatch.ai "기술적 우수성": batch-union grouping, so that
// each expert's rows are read once per group of tokens): for each dispatched
// (token, expert) pair and each weight row r,
//   P[r][b] = sum over the 32 columns of block b of q_w * q_x   (exact integer)
//   acc = fmaf(P[r][b], d_b, acc) for b = 0, 1, ... in order; out_r = acc * s_r.
//
// Why f16 matrix cores carry the integer dot.  The int4 codes (|q| <= 7) and
// the Q8 codes (|q| <= 127) are exact f16 values, each product is exact, and
// every partial sum of a 32-column block is an integer below 2^23 (the weight
// operand carries an offset, cancelled through the accumulator input; see
// nibbles_to_f16), so the fp32 accumulation inside v_mfma_f32_16x16x32_f16
// (K = 32 = one Q8 block) is exact: it returns P[r][b] bit-for-bit, as fp32.  The exact Q8_0
// rescale then costs one VALU fmaf per (row, token, block) and nothing else;
// an int8 matrix core's int32 result would need a conversion first, doubling
// that VALU stream, which is what bounds this kernel.
//
// Tiling.  A work item is (expert, four consecutive 64-row groups, up to 128
// tokens of the expert's list); each of the workgroup's four wavefronts owns
// one row group (gate/up: 32 gate + 32 up rows; down: 64 rows) against all
// of the item's tokens, in M = ceil(tokens / 16) subtiles of 16.  Per 32-column
// block a wavefront loads its group's 1 KB of nibbles (16 B per lane, a ring
// of buffer loads 4 to 8 blocks deep), moves the four 8-column words of 16-row
// tiles into MFMA operand position with two v_permlane32_swap and two
// v_permlane16_swap, expands nibbles to f16 in registers, and issues 4 * M
// MFMAs whose results are rescaled three MFMAs later, so the fmaf chain of one
// tile overlaps the matrix pipe's work on the next.  The tokens' f16 operands
// and block scales are staged into LDS one stage ahead (two slots; a stage is
// 16 / M blocks, one barrier per stage); the 16 lanes of a 16-byte LDS read hit 16 different
// bank groups through an XOR swizzle.  The work list is built on the device
// after dispatch; the launch is sized for the worst case and workgroups past
// the real count return at once.  Each XCD takes every eighth chunk of the
// list, heaviest first, with its row quads in a row (see locate).
#include "coli_internal.h"

namespace coli {
namespace {

constexpr int kWave = 64;
constexpr int kSub = 16;                 // tokens per matrix-core subtile
constexpr int kMaxSub = 8;               // subtiles per work item
constexpr int kChunk = kSub * kMaxSub;   // tokens per work item
constexpr int kGroupsPerWg = 4;          // row groups per workgroup (one per wavefront)
constexpr int kLag = 3;                  // MFMAs between a result and its rescale

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
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
// f16 values, offset: a nibble OR-ed into the low mantissa bits of 1024.0
// (0x6400) gives 1024 + n = q + 1032, one OR-ed four bits higher gives
// 1024 + 16n = 16q + 1152.  Element order (columns): 0, 2, 4, 6, 1, 3, 5, 7,
// where the elements 2, 3, 6, 7 (columns 4-7 of each eight) carry 16q + 1152;
// the token operand carries x there as x / 16.  A block's dot product is then
// P + 1032 SL + 72 SH, SL and SH the token's code sums over the columns 0-3
// and 4-7 of each eight.  Either the offsets are subtracted here (OFFSET
// false: q and 16q, two more instructions per word), or (OFFSET true)
// -(1032 SL + 72 SH), staged with the token, is the matrix-core instruction's
// accumulator input, so its result is P all the same.  No partial sum
// reaches 2^23 (32 products of at most 1039 * 127, and the offset below
// 1104 * 16 * 127), so every step of that sum is exact in fp32.
template <bool OFFSET>
__device__ __forceinline__ half8 nibbles_to_f16(uint32_t w, const UnpackConsts& c) {
  const uint32_t w8 = w >> 8;
  half2v h0 = __builtin_bit_cast(half2v, (w & c.lo) | c.magic);
  half2v h1 = __builtin_bit_cast(half2v, (w & c.hi) | c.magic);
  half2v h2 = __builtin_bit_cast(half2v, (w8 & c.lo) | c.magic);
  half2v h3 = __builtin_bit_cast(half2v, (w8 & c.hi) | c.magic);
  if constexpr (!OFFSET) {
    const half2v b1 = {(_Float16)1032.0f, (_Float16)1032.0f};
    const half2v b16 = {(_Float16)1152.0f, (_Float16)1152.0f};
    h0 -= b1;
    h1 -= b16;
    h2 -= b1;
    h3 -= b16;
  }
  half8 r;
  r[0] = h0[0]; r[1] = h0[1]; r[2] = h1[0]; r[3] = h1[1];
  r[4] = h2[0]; r[5] = h2[1]; r[6] = h3[0]; r[7] = h3[1];
  return r;
}

// The four 16-row tile operands of one table chunk.  Lane 16 * q + j holds
// row 16 * q + j of the group as words 0..3 (columns 0-7, 8-15, 16-23,
// 24-31).  A 16x16x32 MFMA wants, in lane 16 * g + j of tile t, word g of row
// 16 * t + j: a transpose of (16-lane row, word) over 4 x 4, done as a swap of
// the off-diagonal 2 x 2 quadrants across the wavefront halves followed by a
// swap inside each 32-lane half.
__device__ __forceinline__ void tile_words(u32x4 w, uint32_t (&t)[4]) {
  const auto a = __builtin_amdgcn_permlane32_swap(w.x, w.z, false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(w.y, w.w, false, false);
  const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  const auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  t[0] = c[0];
  t[1] = c[1];
  t[2] = d[0];
  t[3] = d[1];
}

__device__ __forceinline__ f32x4 mfma(half8 a, half8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// acc = fmaf(P, d, acc) for the four elements of a tile that a lane holds.
__device__ __forceinline__ void rescale(f32x4& acc, f32x4 p, float d) {
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(p[i], d, acc[i]);
}

struct Item {
  int e, quad, chunk;
  bool ok;
};

// Work item of this workgroup: one row quad of one chunk.  The chunk list is
// sorted by descending work.  Workgroups are dispatched to the eight XCDs
// round robin by blockIdx.x, and XCD x takes chunks x, x + 8, x + 16, ...
// with all q row quads of a chunk in a row: every XCD gets the same mix of
// heavy and light chunks, and the row quads of a chunk, which stage the same
// tokens, share them in that XCD's L2.
__device__ __forceinline__ Item locate(const int2* chunks, const int32_t* n_chunks, int q) {
  Item it = {};
  const int tot = *as_const(n_chunks);
  const int bid = (int)blockIdx.x;
  const int k = bid >> 3;
  const int p = (k / q) * 8 + (bid & 7);
  it.ok = p < tot;
  if (!it.ok) return it;
  const cptr<int32_t> v = as_const(reinterpret_cast<const int32_t*>(chunks) + 2 * (size_t)p);
  it.e = v[0];
  it.quad = k % q;
  it.chunk = v[1];
  return it;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint64_t bytes) {
  const uint32_t n = bytes > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, kBufferConfig);
}

// Arguments of both matrix kernels.  Token operands: tok [rows][NB][4] 16-byte
// pieces of f16 codes (piece g of a block = its columns 8g .. 8g + 7 in the
// expansion's element order), tokd [rows][NB] block scales, tokb [rows][NB]
// the accumulator inputs -(1032 SL + 72 SH); a list entry p names row p / KS
// (gate/up: the token of pair p) or p (down: the pair).
struct GArgs {
  const u32x4* wq;        // [E+S][RG][NB][64] 16-byte lane chunks
  const float* ws;        // gate/up: [E+S][RG][64] lane-ordered; down: [E+S][D]
  const uint4* tok;
  const float* tokd;
  const float* tokb;
  const int32_t* counts;
  const int32_t* lists;
  const int2* chunks;     // (expert, chunk index) in execution order
  const int32_t* n_chunks;
  int64_t T, D, F;
  int NB, RG, KS, row_div;
  int Q;                  // row quads per chunk (items per chunk)
  // gate/up results
  uint32_t* h16;          // [P][F/32][4 pieces][4 words]
  float* hd;              // [P][F/32]
  float* hb;              // [P][F/32] accumulator inputs of Q8(h)
  int8_t* hq;             // [P][F] (traced runs only)
  // down result
  float* o;               // [P][D]
  // traces (null = skip)
  int32_t* tr_p0;         // gate partials / down partials
  int32_t* tr_p1;         // up partials
  float* tr_g;
  float* tr_u;
  float* tr_h;
};

// Pipeline shape per subtile count M.  S blocks are staged per barrier and
// the weight ring is R blocks deep: few tokens per item make a block cheap, so
// small M needs more blocks in flight per wavefront and fewer barriers, and
// has the registers for them (the accumulators are 16 M).  The staged pieces
// per thread (M * S / 4, 16 B each) stay at 16 VGPRs or less.  The ring has
// R + 1 slots and a block refills the slot the previous block consumed: the
// lane swaps that move a chunk into operand position overwrite their inputs,
// so the slot being consumed cannot take its own refill without a copy and a
// wait for the load at the loop's back edge.  U is the loop unroll: a
// multiple of R + 1 and of 2 S, so ring positions and LDS slots are
// compile-time constants; the block loop runs to NB rounded up to U (see
// stream).  Each M is one copy of the unrolled loop, so U is kept small: the
// instruction cache is shared by the workgroups of neighbouring CUs.  OFFSET
// (see nibbles_to_f16) trades two VALU instructions per weight word for one
// 16-byte LDS read per subtile and block: it pays while the expansion is
// shared by few subtiles, and costs once the LDS reads of the operands
// dominate.
template <int M>
struct Cfg {
  static constexpr bool OFFSET = M <= 2;
  static constexpr int S = M <= 2 ? 8 : M <= 4 ? 4 : 2;
  static constexpr int RS = M <= 4 ? 8 : 4;             // ring slots
  static constexpr int R = RS - 1;                      // blocks in flight
  static constexpr int U = (2 * S > RS ? 2 * S : RS);
  static constexpr int PT = (64 * M * S + 255) / 256;   // staged pieces per thread
  static constexpr int XS = 64 * M * S;                 // 16-byte pieces per stage
  static constexpr int DS = 16 * M * S;                 // scales per stage
  static_assert(U % RS == 0 && U % (2 * S) == 0, "static ring and slot positions");
  static_assert(DS <= 256, "one scale per thread");
};

// LDS of the staging: two slots of one stage each.  In block j of a stage,
// piece g of token t sits at 16-byte slot 64 M j + 4 t + (g ^ ((t >> 1) & 3)),
// so the 16 lanes of one operand read hit 16 different bank groups; the
// scales are [j][16 M], the accumulator inputs [j][16 M] four copies each
// (one 16-byte read fills the four accumulator registers of a lane).  Sized
// for the largest stage (M S = 16).
struct Stage {
  uint4 x[2][1024];
  f32x4 k[2][256];
  float d[2][256];
};

// The thread's share of a stage: pieces q = tid + 256 i (block q / 64M of the
// stage, token (q % 64M) / 4, piece q & 3) and, for tid < 16 M S, the scale of
// token tid % 16M in block tid / 16M.  Loads are issued for blocks past the
// end too (clamped to the last block), stores only for the stage's pieces.
template <int M>
struct StageSrc {
  const uint4 *x0, *x1, *x2, *x3;   // block 0 piece of the token of each share
  const float* d;                   // block 0 scale of the scale share's token
  const float* k;                   // its block 0 accumulator input
};

// Share i of a thread (named members: they must stay in registers).
template <int I, class A, class V>
__device__ __forceinline__ V& share(A& a) {
  if constexpr (I == 0) return a.x0;
  else if constexpr (I == 1) return a.x1;
  else if constexpr (I == 2) return a.x2;
  else return a.x3;
}

template <int I>
__device__ __forceinline__ uint4& pick(uint4& x0, uint4& x1, uint4& x2, uint4& x3) {
  if constexpr (I == 0) return x0;
  else if constexpr (I == 1) return x1;
  else if constexpr (I == 2) return x2;
  else return x3;
}

template <int M, int I = 0>
__device__ __forceinline__ void stage_load(const StageSrc<M>& s, int st, int NB, int tid,
                                           uint4& x0, uint4& x1, uint4& x2, uint4& x3,
                                           float& d, float& k, bool& dok) {
  using C = Cfg<M>;
  if constexpr (I < C::PT) {
    const int q = tid + 256 * I;
    int b = st * C::S + q / (64 * M);
    b = b < NB ? b : NB - 1;
    pick<I>(x0, x1, x2, x3) = share<I, const StageSrc<M>, const uint4* const>(s)[(size_t)b * 4];
    stage_load<M, I + 1>(s, st, NB, tid, x0, x1, x2, x3, d, k, dok);
  } else {
    // a block past the end gets scale 0 (applied at the store: a use of the
    // loaded value here would wait for every load issued before it)
    const int b = st * C::S + (tid < C::DS ? tid : 0) / (16 * M);
    d = s.d[b < NB ? b : NB - 1];   // issued on every path
    if constexpr (C::OFFSET) k = s.k[b < NB ? b : NB - 1];
    dok = b < NB;
  }
}

template <int M, int I = 0>
__device__ __forceinline__ void stage_store(Stage& L, int slot, int tid, uint4& x0, uint4& x1,
                                            uint4& x2, uint4& x3, float d, float k, bool dok) {
  using C = Cfg<M>;
  if constexpr (I < C::PT) {
    const int q = tid + 256 * I;
    if (C::XS % 256 == 0 || q < C::XS) {
      const int j = q / (64 * M), rr = q % (64 * M), t = rr >> 2, g = rr & 3;
      L.x[slot][64 * M * j + 4 * t + (g ^ ((t >> 1) & 3))] = pick<I>(x0, x1, x2, x3);
    }
    stage_store<M, I + 1>(L, slot, tid, x0, x1, x2, x3, d, k, dok);
  } else {
    // fmaf(P, 0, acc) leaves acc exactly as it is (acc is never -0: it starts
    // at +0 and an fmaf that cancels exactly rounds to +0)
    if (tid < C::DS) {
      L.d[slot][tid] = dok ? d : 0.0f;
      if constexpr (C::OFFSET) L.k[slot][tid] = f32x4{k, k, k, k};
    }
  }
}

// Per-wavefront state of the block loop.
template <int M>
struct Acc {
  f32x4 a[M][4];   // [subtile][tile]: rows 4 * (lane >> 4) + i of tile t, token lane & 15
};

struct Trace {
  int32_t* p[kMaxSub][4];   // row base (times NB) of each (subtile, tile) element 0, or null
};

// One block of the stream: expand the weights, read the tokens' operands,
// issue the MFMAs subtile by subtile and rescale each result kLag MFMAs later.
// The kLag results still pending at the end of the block (subtile M - 1, the
// last kLag tiles) are carried in p[] with their scale in dprev and rescaled
// at the start of the next block.
template <int M, bool TRACE>
__device__ __forceinline__ void block_step(const Stage& L, int slot, int jst, int xoff, int n,
                                           u32x4 w, const UnpackConsts& uc, Acc<M>& acc,
                                           f32x4 (&p)[4], float& dprev, const Trace& tr, int b,
                                           int NB) {
  float d[M];
#pragma unroll
  for (int s = 0; s < M; ++s) d[s] = L.d[slot][kSub * M * jst + kSub * s + n];
  const uint4* xs = &L.x[slot][64 * M * jst + xoff];
  constexpr bool OFS = Cfg<M>::OFFSET;
  const f32x4* ks = &L.k[slot][kSub * M * jst + n];
  half8 B[M];
  f32x4 K[M] = {};
  B[0] = __builtin_bit_cast(half8, xs[0]);
  if (OFS) K[0] = ks[0];
  if (M > 1) {
    B[1] = __builtin_bit_cast(half8, xs[64]);
    if (OFS) K[1] = ks[kSub];
  }
  // the operand reads go out before the expansion, which covers their latency
  __builtin_amdgcn_sched_barrier(0);
  uint32_t tw[4];
  tile_words(w, tw);
  half8 A[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) A[t] = nibbles_to_f16<OFS>(tw[t], uc);
#pragma unroll
  for (int s = 0; s < M; ++s) {
    if (s + 2 < M) {
      B[s + 2] = __builtin_bit_cast(half8, xs[64 * (s + 2)]);
      if (OFS) K[s + 2] = ks[kSub * (s + 2)];
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int i = 4 * s + t;
      p[i & 3] = mfma(A[t], B[s], K[s]);
      if (TRACE && tr.p[s][t] && b < NB) {
#pragma unroll
        for (int r = 0; r < 4; ++r) tr.p[s][t][(size_t)r * NB + b] = (int32_t)p[i & 3][r];
      }
      // the result kLag MFMAs back: this block's item i - kLag, or one of the
      // last kLag of the previous block (subtile M - 1)
      const int j = i - kLag;
      if (j >= 0) rescale(acc.a[j >> 2][j & 3], p[j & 3], d[j >> 2]);
      else rescale(acc.a[M - 1][4 + j], p[4 + j], dprev);
    }
  }
  dprev = d[M - 1];
}

// All NB blocks of one row group against the item's M subtiles.  Every
// wavefront of the workgroup takes part in the staging and the barriers;
// `compute` is false for a wavefront whose row group is past the matrix.
// Stage st is loaded into registers one stage ahead and stored to slot
// st & 1 after the barrier that ends stage st - 1 (all reads of that slot,
// two stages back, are done by then).
template <int M, bool TRACE>
__device__ __forceinline__ void stream_loop(Stage& L, const GArgs& a, __amdgpu_buffer_rsrc_t wrs,
                                            const StageSrc<M>& src, bool compute, Acc<M>& acc,
                                            const Trace& tr, int tid, int lane) {
  using C = Cfg<M>;
  const int NB = a.NB;
  const UnpackConsts uc = unpack_consts();
  // the lane's operand: piece (lane >> 4) of token (lane & 15) of each
  // subtile, at 16-byte slot xoff (+ 64 per subtile)
  const int n = lane & 15, g = lane >> 4;
  const int xoff = 4 * n + (g ^ ((n >> 1) & 3));
  const uint32_t voff = 16u * (uint32_t)lane;
  u32x4 wq[C::RS];
#pragma unroll
  for (int j = 0; j < C::R; ++j)
    wq[j] = __builtin_amdgcn_raw_buffer_load_b128(wrs, voff + 1024u * (uint32_t)(j < NB ? j : NB - 1),
                                                  0, 0);
  uint4 r0 = {}, r1 = {}, r2 = {}, r3 = {};
  float rd = 0.0f, rk = 0.0f;
  bool rok = false;
  stage_load<M>(src, 0, NB, tid, r0, r1, r2, r3, rd, rk, rok);
  stage_store<M>(L, 0, tid, r0, r1, r2, r3, rd, rk, rok);
  stage_load<M>(src, 1, NB, tid, r0, r1, r2, r3, rd, rk, rok);
  __syncthreads();
  f32x4 p[4] = {};
  float dprev = 0.0f;
  // NB rounded up to U: the blocks past the end repeat the last block's
  // weights and tokens with scale 0 (stage_load), so they change nothing
  const int NBU = (NB + C::U - 1) / C::U * C::U;
  for (int b = 0; b < NBU; b += C::U) {
#pragma unroll
    for (int j = 0; j < C::U; ++j) {
      const int bb = b + j, jst = j % C::S, slot = (j / C::S) & 1;
      {
        // block bb + R into the slot block bb - 1 used (free since then),
        // issued by every wavefront (one past the matrix reads row group 0),
        // so that the memory-counter waits of the staging are exact
        const int bn = bb + C::R < NB ? bb + C::R : NB - 1;
        wq[(j + C::R) % C::RS] =
            __builtin_amdgcn_raw_buffer_load_b128(wrs, voff + 1024u * (uint32_t)bn, 0, 0);
      }
      if (compute)
        block_step<M, TRACE>(L, slot, jst, xoff, n, wq[j % C::RS], uc, acc, p, dprev, tr, bb, NB);
      // blocks stay in program order: the scheduler would otherwise hoist the
      // next blocks' loads into this one and run out of registers
      __builtin_amdgcn_sched_barrier(0);
      if (jst == C::S - 1) {   // end of stage st = bb / S
        // unconditional, so that the memory-counter waits are exact: the
        // stores past the last stage go to a slot nobody reads, the loads past
        // the end read the last block
        stage_store<M>(L, slot ^ 1, tid, r0, r1, r2, r3, rd, rk, rok);
        stage_load<M>(src, bb / C::S + 2, NB, tid, r0, r1, r2, r3, rd, rk, rok);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  if (compute) {
#pragma unroll
    for (int t = 4 - kLag; t < 4; ++t) rescale(acc.a[M - 1][t], p[t], dprev);
  }
}

template <int M, bool TRACE>
__device__ __forceinline__ void stream(Stage& L, const GArgs& a, __amdgpu_buffer_rsrc_t wrs,
                                       const StageSrc<M>& src, bool compute, Acc<M>& acc,
                                       const Trace& tr, int tid, int lane) {
  stream_loop<M, TRACE>(L, a, wrs, src, compute, acc, tr, tid, lane);
}

// Entries of this item: list entry of token t (clamped into the valid range).
struct ChunkInfo {
  const int32_t* list;
  int nv;   // tokens in the item (1..128)
};

__device__ __forceinline__ int entry_of(const ChunkInfo& c, int t) {
  return c.list[t < c.nv ? t : c.nv - 1];
}

template <int M, int I = 0>
__device__ __forceinline__ void stage_src_share(const GArgs& a, const ChunkInfo& c, int tid,
                                                StageSrc<M>& s) {
  if constexpr (I < Cfg<M>::PT) {
    const int q = tid + 256 * I;
    const int64_t r = entry_of(c, (q % (64 * M)) >> 2) / a.row_div;
    share<I, StageSrc<M>, const uint4*>(s) = a.tok + (size_t)r * a.NB * 4 + (q & 3);
    stage_src_share<M, I + 1>(a, c, tid, s);
  }
}

template <int M>
__device__ __forceinline__ StageSrc<M> stage_src(const GArgs& a, const ChunkInfo& c, int tid) {
  using C = Cfg<M>;
  StageSrc<M> s = {};
  stage_src_share<M>(a, c, tid, s);
  const int64_t rd = entry_of(c, (tid < C::DS ? tid : 0) % (16 * M)) / a.row_div;
  s.d = a.tokd + (size_t)rd * a.NB;
  s.k = a.tokb + (size_t)rd * a.NB;
  return s;
}

// ---------------------------------------------------------------------------
// gate/up: g and u of the group's 32 rows for M subtiles of tokens, SwiGLU,
// Q8_0 of h per token (the group's 32 rows are one Q8 block of h), and the
// f16 codes of Q8(h) in the down projection's operand order.
template <int M, bool TRACE>
__device__ __forceinline__ void gate_up_item(const GArgs& a, Stage& L, const Item& it,
                                             const ChunkInfo& c, int grp, bool compute,
                                             int tid, int lane) {
  const int G16 = (int)(a.F / 32);
  const int n = lane & 15, gq = lane >> 4;
  const int gsafe = compute ? grp : 0;
  const __amdgpu_buffer_rsrc_t wrs =
      make_rsrc(a.wq + ((size_t)it.e * a.RG + gsafe) * (size_t)a.NB * kWave,
                (uint64_t)a.NB * 1024u);
  Trace tr = {};
  if (TRACE && compute) {
#pragma unroll
    for (int s = 0; s < M; ++s) {
      if (kSub * s + n >= c.nv) continue;
      const size_t pr = (size_t)c.list[kSub * s + n];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        int32_t* base = t < 2 ? a.tr_p0 : a.tr_p1;
        const int row = 32 * grp + 16 * (t & 1) + 4 * gq;
        if (base) tr.p[s][t] = base + (pr * a.F + row) * a.NB;
      }
    }
  }
  Acc<M> acc;
#pragma unroll
  for (int s = 0; s < M; ++s)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc.a[s][t] = f32x4{};
  const StageSrc<M> src = stage_src<M>(a, c, tid);
  stream<M, TRACE>(L, a, wrs, src, compute, acc, tr, tid, lane);
  if (!compute) return;

  // lane-ordered scales of the group: lane row 16 t + 4 gq + i
  const float* sg = a.ws + ((size_t)it.e * a.RG + grp) * kWave;
  float sc[4][4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[t][i] = sg[16 * t + 4 * gq + i];
  // one subtile per pass, always from acc.a[0]: the next subtile's
  // accumulators move down after each pass, so the epilogue (two divisions
  // per value) is emitted once per M rather than M times
#pragma unroll 1
  for (int s = 0; s < M; ++s) {
    const bool valid = kSub * s + n < c.nv;
    const size_t p = (size_t)entry_of(c, kSub * s + n);
    float h[2][4];
    float amax = 0.0f;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float gv = acc.a[0][hh][i] * sc[hh][i];
        const float uv = acc.a[0][2 + hh][i] * sc[2 + hh][i];
        h[hh][i] = silu_f32(gv) * uv;
        amax = fmaxf(amax, fabsf(h[hh][i]));
        if (TRACE && valid) {
          const size_t o = p * a.F + 32 * (size_t)grp + 16 * hh + 4 * gq + i;
          if (a.tr_g) a.tr_g[o] = gv;
          if (a.tr_u) a.tr_u[o] = uv;
          if (a.tr_h) a.tr_h[o] = h[hh][i];
        }
      }
    }
    // the token's 32 rows sit in lanes n, n + 16, n + 32, n + 48
    {
      const auto x16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(amax),
                                                        __float_as_uint(amax), false, false);
      amax = fmaxf(__uint_as_float(x16[0]), __uint_as_float(x16[1]));
      const auto x32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(amax),
                                                        __float_as_uint(amax), false, false);
      amax = fmaxf(__uint_as_float(x32[0]), __uint_as_float(x32[1]));
    }
    const float d = amax / 127.0f;
    int q[2][4];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int i = 0; i < 4; ++i) q[hh][i] = q8_code(h[hh][i], d);
    // accumulator input of the down operand: this lane's rows are columns
    // 4 (gq & 1) + i of their eights (rows 4..7 of an eight carry q / 16)
    int kb = (gq & 1) ? 72 : 1032;
    kb *= q[0][0] + q[0][1] + q[0][2] + q[0][3] + q[1][0] + q[1][1] + q[1][2] + q[1][3];
    {
      const auto k16 = __builtin_amdgcn_permlane16_swap((uint32_t)kb, (uint32_t)kb, false, false);
      kb = (int)k16[0] + (int)k16[1];
      const auto k32 = __builtin_amdgcn_permlane32_swap((uint32_t)kb, (uint32_t)kb, false, false);
      kb = (int)k32[0] + (int)k32[1];
    }
    // f16 pieces of Q8(h): rows 16 hh + 8 m + {0, 2, 4, 6, 1, 3, 5, 7} form
    // piece 2 hh + m, the rows 4..7 of each eight as q / 16.  This lane holds
    // rows 4 gq .. 4 gq + 3 of each half: words 0 and 2 of piece gq >> 1 for
    // even gq, words 1 and 3 for odd gq; a swap between 16-lane rows gives
    // each lane two adjacent words.
    const float scl = (gq & 1) ? 0.0625f : 1.0f;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const half2v x = {(_Float16)((float)q[hh][0] * scl), (_Float16)((float)q[hh][2] * scl)};
      const half2v y = {(_Float16)((float)q[hh][1] * scl), (_Float16)((float)q[hh][3] * scl)};
      const auto sw = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x),
                                                       __builtin_bit_cast(uint32_t, y), false,
                                                       false);
      if (valid) {
        uint32_t* dst = a.h16 + ((p * G16 + grp) * 4 + 2 * hh + (gq >> 1)) * 4 + 2 * (gq & 1);
        *reinterpret_cast<uint2*>(dst) = make_uint2(sw[0], sw[1]);
      }
    }
    if (valid && gq == 0) {
      a.hd[p * G16 + grp] = d;
      a.hb[p * G16 + grp] = -(float)kb;
    }
    if (TRACE && valid && a.hq) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          a.hq[p * a.F + 32 * (size_t)grp + 16 * hh + 4 * gq + i] = (int8_t)q[hh][i];
    }
#pragma unroll
    for (int r = 0; r + 1 < M; ++r)
#pragma unroll
      for (int t = 0; t < 4; ++t) acc.a[r][t] = acc.a[r + 1][t];
  }
}

// down: o = s_r * acc for the group's 64 rows and the item's pairs.
template <int M, bool TRACE>
__device__ __forceinline__ void down_item(const GArgs& a, Stage& L, const Item& it,
                                          const ChunkInfo& c, int grp, bool compute, int tid,
                                          int lane) {
  const int n = lane & 15, gq = lane >> 4;
  const int gsafe = compute ? grp : 0;
  const __amdgpu_buffer_rsrc_t wrs =
      make_rsrc(a.wq + ((size_t)it.e * a.RG + gsafe) * (size_t)a.NB * kWave,
                (uint64_t)a.NB * 1024u);
  Trace tr = {};
  if (TRACE && compute && a.tr_p0) {
#pragma unroll
    for (int s = 0; s < M; ++s) {
      if (kSub * s + n >= c.nv) continue;
      const size_t pr = (size_t)c.list[kSub * s + n];
#pragma unroll
      for (int t = 0; t < 4; ++t)
        tr.p[s][t] = a.tr_p0 + (pr * a.D + 64 * (size_t)grp + 16 * t + 4 * gq) * a.NB;
    }
  }
  Acc<M> acc;
#pragma unroll
  for (int s = 0; s < M; ++s)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc.a[s][t] = f32x4{};
  const StageSrc<M> src = stage_src<M>(a, c, tid);
  stream<M, TRACE>(L, a, wrs, src, compute, acc, tr, tid, lane);
  if (!compute) return;
  const float* sr = a.ws + (size_t)it.e * a.D + 64 * (size_t)grp;
  float4 sc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) sc[t] = *reinterpret_cast<const float4*>(sr + 16 * t + 4 * gq);
#pragma unroll 1
  for (int s = 0; s < M; ++s) {
    if (kSub * s + n < c.nv) {
      float* orow = a.o + (size_t)c.list[kSub * s + n] * a.D + 64 * (size_t)grp;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float4 v = make_float4(acc.a[0][t][0] * sc[t].x, acc.a[0][t][1] * sc[t].y,
                                     acc.a[0][t][2] * sc[t].z, acc.a[0][t][3] * sc[t].w);
        *reinterpret_cast<float4*>(orow + 16 * t + 4 * gq) = v;
      }
    }
#pragma unroll
    for (int r = 0; r + 1 < M; ++r)
#pragma unroll
      for (int t = 0; t < 4; ++t) acc.a[r][t] = acc.a[r + 1][t];
  }
}

template <bool DOWN, bool TRACE>
__global__ void __launch_bounds__(256, 2) mfma_ffn_kernel(GArgs a) {
  __shared__ Stage lds;
  const Item it = locate(a.chunks, a.n_chunks, a.Q);
  if (!it.ok) return;
  const int tid = (int)threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = it.quad * kGroupsPerWg + wave;
  const bool compute = grp < a.RG;
  const int cnt = as_const(a.counts)[it.e];
  ChunkInfo c;
  c.list = a.lists + (size_t)it.e * a.T + (size_t)it.chunk * kChunk;
  const int rem = cnt - it.chunk * kChunk;
  c.nv = rem < kChunk ? rem : kChunk;
  const int M = (c.nv + kSub - 1) / kSub;
#define COLI_ITEM(MM)                                                                   \
  case MM:                                                                              \
    if (DOWN) down_item<MM, TRACE>(a, lds, it, c, grp, compute, tid, lane);             \
    else gate_up_item<MM, TRACE>(a, lds, it, c, grp, compute, tid, lane);               \
    break;
  switch (M) {
    COLI_ITEM(1)
    COLI_ITEM(2)
    COLI_ITEM(3)
    COLI_ITEM(4)
    COLI_ITEM(5)
    COLI_ITEM(6)
    COLI_ITEM(7)
    COLI_ITEM(8)
    default: break;
  }
#undef COLI_ITEM
}

// ---------------------------------------------------------------------------
// Front of the grouped path, after dispatch.  Workgroup 0 builds the chunk
// list that both matrix kernels share: an expert of n tokens has n / 128 full
// chunks (M = 8) and, when n % 128 > 0, one last chunk of M = ceil((n % 128) /
// 16) subtiles; each chunk is one work item per row quad of the kernel, found
// by locate.  The list holds the M = 8 chunks first, then the last chunks by
// descending M, so workgroups running side by side mostly execute the same
// code (each M is its own unrolled loop; a last chunk of M = 8 follows the
// full ones); inside a group the experts are in ascending order.  The other
// workgroups write the f16
// codes of the Q8 activations in the piece order the MFMA operands read:
// piece g of block b holds columns 8g + {0, 2, 4, 6, 1, 3, 5, 7}, the columns
// 4, 6, 5, 7 of each eight as q / 16 (exact in f16), and each block's
// accumulator input -(1032 SL + 72 SH) (see nibbles_to_f16).
struct FrontArgs {
  const int32_t* counts;
  const int32_t* n_active;
  const int32_t* active;
  int2* chunks;
  int32_t* n_chunks;
  const int8_t* xq;
  uint4* xh;
  float* xb;
  int64_t T, D;
};

// Exclusive prefix over the workgroup of v (256 threads); *total = the sum.
__device__ __forceinline__ int wg_exclusive(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int u = __shfl_up(x, off);
    if (lane >= off) x += u;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    base += w < wave ? wsum[w] : 0;
    tot += wsum[w];
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

// nc chunks c0 .. c0 + nc - 1 of expert e from list position pos; one
// wavefront.
__device__ __forceinline__ void emit_chunks(int2* chunks, int pos, int e, int c0, int nc,
                                            int lane) {
  for (int i = lane; i < nc; i += kWave) chunks[pos + i] = make_int2(e, c0 + i);
}

__global__ void __launch_bounds__(256) mfma_front_kernel(FrontArgs a) {
  if (blockIdx.x == 0) {
    __shared__ int wsum[4];
    __shared__ int4 plan[512];   // per active expert: e, full chunks, their position, last's
    const int nact = *a.n_active;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    // two active experts per thread: full chunks f, last-chunk subtiles m
    int e[2], f[2], m[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int s = 2 * t + i;
      e[i] = s < nact ? a.active[s] : 0;
      const int n = s < nact ? a.counts[e[i]] : 0;
      f[i] = n / kChunk;
      m[i] = (n % kChunk + kSub - 1) / kSub;
    }
    int g8;
    const int p8 = wg_exclusive(f[0] + f[1], wsum, &g8);
    int start = g8;          // first chunk position of the current M group
    int last[2] = {-1, -1};  // chunk position of each expert's last chunk
#pragma unroll 1
    for (int mm = kMaxSub; mm >= 1; --mm) {   // a last chunk of 113..127 tokens has M = 8
      int gm;
      const int r = wg_exclusive((m[0] == mm) + (m[1] == mm), wsum, &gm);
      if (m[0] == mm) last[0] = start + r;
      if (m[1] == mm) last[1] = start + r + (m[0] == mm);
      start += gm;
    }
    plan[2 * t] = make_int4(e[0], f[0], p8, last[0]);
    plan[2 * t + 1] = make_int4(e[1], f[1], p8 + f[0], last[1]);
    if (t == 0) *a.n_chunks = start;
    __syncthreads();
    for (int s = wave; s < nact; s += 4) {
      const int4 pl = plan[s];
      emit_chunks(a.chunks, pl.z, pl.x, 0, pl.y, lane);
      if (pl.w >= 0) emit_chunks(a.chunks, pl.w, pl.x, pl.y, 1, lane);
    }
    return;
  }
  const int64_t pieces = a.T * (a.D / 32) * 4;
  const int64_t stride = (int64_t)(gridDim.x - 1) * blockDim.x;
  for (int64_t i = (int64_t)(blockIdx.x - 1) * blockDim.x + threadIdx.x; i < pieces; i += stride) {
    // piece i = (token, block, g): source columns 8g .. 8g + 7 of the block
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
    // the block's four pieces are lanes 4 m .. 4 m + 3 of this wavefront
    // (the piece count and the stride are multiples of 4)
    int kb = 1032 * ((int)c[0] + c[1] + c[2] + c[3]) + 72 * ((int)c[4] + c[5] + c[6] + c[7]);
    kb += __shfl_xor(kb, 1);
    kb += __shfl_xor(kb, 2);
    if ((i & 3) == 0) a.xb[i >> 2] = -(float)kb;
  }
}

}  // namespace

bool mfma_path_fits(int64_t T, int64_t D, int64_t F, int k, int S) {
  (void)T;
  (void)k;
  (void)S;
  return D % 64 == 0 && F % 32 == 0;
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
  f.chunks = reinterpret_cast<int2*>(ws.chunks);
  f.n_chunks = ws.n_chunks;
  f.xq = xq;
  f.xh = reinterpret_cast<uint4*>(ws.xh);
  f.xb = ws.xbias;
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
  GArgs g = {};
  g.wq = reinterpret_cast<const u32x4*>(t.gu_q);
  g.ws = t.gu_s;
  g.tok = reinterpret_cast<const uint4*>(ws.xh);
  g.tokd = xd;
  g.tokb = ws.xbias;
  g.counts = ws.counts;
  g.lists = ws.lists;
  g.chunks = reinterpret_cast<const int2*>(ws.chunks);
  g.n_chunks = ws.n_chunks;
  g.T = T;
  g.D = t.d_model;
  g.F = t.d_ff;
  g.NB = (int)(t.d_model / 32);
  g.RG = (int)(t.d_ff / 32);
  g.KS = k + S;
  g.row_div = k + S;
  g.Q = mfma_quads_gate_up(t.d_ff);
  g.h16 = reinterpret_cast<uint32_t*>(ws.h16);
  g.hd = ws.hd;
  g.hb = ws.hbias;
  g.hq = tr ? ws.hq : nullptr;
  GArgs d = g;
  d.wq = reinterpret_cast<const u32x4*>(t.dn_q);
  d.ws = t.dn_s;
  d.tok = reinterpret_cast<const uint4*>(ws.h16);
  d.tokd = ws.hd;
  d.tokb = ws.hbias;
  d.NB = (int)(t.d_ff / 32);
  d.RG = (int)(t.d_model / 64);
  d.row_div = 1;
  d.Q = mfma_quads_down(t.d_model);
  d.h16 = nullptr;
  d.hd = nullptr;
  d.hb = nullptr;
  d.hq = nullptr;
  d.o = ws.o;
  // enough workgroups for ceil(chunks / 8) chunks on each XCD (see locate)
  const int64_t per_xcd = (max_chunks + 7) / 8;
  const unsigned grid_gu = (unsigned)(per_xcd * 8 * mfma_quads_gate_up(t.d_ff));
  const unsigned grid_dn = (unsigned)(per_xcd * 8 * mfma_quads_down(t.d_model));
  if (tr) {
    g.tr_p0 = tr->p_gate;
    g.tr_p1 = tr->p_up;
    g.tr_g = tr->g;
    g.tr_u = tr->u;
    g.tr_h = tr->h;
    d.tr_p0 = tr->p_down;
    hipLaunchKernelGGL((mfma_ffn_kernel<false, true>), dim3(grid_gu), dim3(256), 0, s, g);
  } else {
    hipLaunchKernelGGL((mfma_ffn_kernel<false, false>), dim3(grid_gu), dim3(256), 0, s, g);
  }
  hipError_t rc = hipGetLastError();
  if (rc != hipSuccess) return rc;
  if (ev_down && (rc = hipEventRecord(static_cast<hipEvent_t>(ev_down), s)) != hipSuccess) return rc;
  if (tr) hipLaunchKernelGGL((mfma_ffn_kernel<true, true>), dim3(grid_dn), dim3(256), 0, s, d);
  else hipLaunchKernelGGL((mfma_ffn_kernel<true, false>), dim3(grid_dn), dim3(256), 0, s, d);
  return hipGetLastError();
}

}  // namespace coli
