// Decode / verify path: int4 x int8 GEMV over the batch-union expert set.
//
// The integer dot of int8 (Q8_0) activations with packed int4 weights is the
// method's hot loop (discuss.pytorch.kr colibri summary, "colibri의 주요 기능";
// jeff.news, kernel section: int4 wins in batch and loses for a single row on
// the CPU, so the path is chosen per shape).  On gfx950 a decode token reads
// every selected expert once from HBM, so these kernels are written to stream
// the table at HBM speed:
//
//  - one 64-lane wavefront owns a row group (32 gate + 32 up rows, or 64 down
//    rows); every load is one 1 KB coalesced dwordx4 per wavefront bringing
//    block b of all 64 rows, lane l holding its own row's 32 nibbles;
//  - the token's block (8 int8 words, its scale and its -8*sum) is uniform
//    across the wavefront and comes through scalar loads, so the nibble
//    unpack (3 ALU ops per word) feeds eight v_dot4_i32_i8 per block directly;
//  - each lane runs its row's accumulation acc = fmaf(P_b, d_b, acc) over b
//    in ascending order in registers: the exact op order of the numerics, with
//    no cross-lane reduction;
//  - a ring of PF outstanding 1 KB loads per wavefront keeps HBM busy;
//  - every token that selected the expert (up to MAXT per pass) is served from
//    the same weight load: the batch union of the alphamatch.ai page
//    ("기술적 우수성").
//
// Nibbles are stored offset-binary (q + 8), so a dot with them is
// sum (q+8) x = P + 8 sum x; the -8 sum x term is precomputed per block.
//
// One-token passes (decode) take their own prologue in both kernels: the
// token records (token 0 for gate/up; for down, the slot's Q8(h), which
// gate/up also stores in active-slot order) are loaded at kernel entry with
// no dependent load before them, and the whole weight ring is issued as soon
// as the active expert is known; the gate/up epilogue exchanges lanes with
// permlane swaps and DPP instead of LDS shuffles.
//
// int8 tables (the int8 speculative head: discuss.pytorch.kr colibri summary,
// "colibri의 주요 기능", MTP bullet; jeff.news, MTP section) run the same
// kernels with two 1 KB wavefront loads per 32-column block: the codes are
// already signed bytes, so they go to v_dot4_i32_i8 as loaded and the block
// dot starts from 0.  int2 tables (same page, integer-dot bullet: int8/int4/
// int2 packings) hold two blocks per 1 KB wavefront load; their 2-bit fields
// are stored q + 2 and the block dot starts from -2 sum x.
//
// The SwiGLU, the row scale and the Q8_0 re-quantisation of h are fused into
// the gate/up epilogue; the routing-weighted combine runs as its own kernel in
// slot order (shared expert first), which keeps it deterministic.  (Folding it
// into the down kernel as a last-arriver reduction measured no faster on
// MI355X: with agent-scope release/acquire fences, which write back and
// invalidate the L2 of every XCD, it was slower; with write-through output
// stores, a device-scope counter and coherent loads instead, the last
// workgroup's store-completion, atomic and load round trips cost what the
// extra launch does.)
#include "coli_internal.h"

#include <hip/hip_ext.h>

namespace coli {
namespace {

constexpr int kWave = 64;
// Word 3 of a gfx9-family buffer descriptor for raw 32-bit-element access.
constexpr int kBufferConfig = 0x00020000;
// Cache-policy operand of a buffer load: non-temporal (streamed once).
constexpr int kNonTemporal = 2;

struct GuArgs {
  const uint4* gu_q;
  const float* gu_s;
  const int8_t* xq;
  const float* xd;
  const int32_t* xsum8;
  const int32_t* counts;
  const int32_t* lists;
  const int32_t* n_active;
  const int32_t* active;
  int8_t* hq;
  float* hd;
  int32_t* hsum8;
  int8_t* hq_slot;         // one-token passes: Q8(h) also in active-slot order
  float* hd_slot;
  int32_t* hs_slot;
  const int32_t* slot_of;  // expert tier: storage position of each expert, or null
  int n_store;             // positions the table holds
  int32_t* err;
  int64_t T, D, F;
  int k, S;
  int32_t* tr_pg;
  int32_t* tr_pu;
  float* tr_g;
  float* tr_u;
  float* tr_h;
};

struct DnArgs {
  const uint4* dn_q;
  const float* dn_s;
  const int8_t* hq;
  const float* hd;
  const int32_t* hsum8;
  const int8_t* hq_slot;   // one-token passes: Q8(h) in active-slot order
  const float* hd_slot;
  const int32_t* hs_slot;
  const int32_t* counts;
  const int32_t* lists;
  const int32_t* n_active;
  const int32_t* active;
  float* o;
  const int32_t* slot_of;
  int n_store;
  int32_t* err;
  int64_t T, D, F;
  int k, S, E;
  int32_t* tr_pd;
};

// Storage position of expert e: e itself, or its tier slot.  A tier slot
// outside [0, n_store) (the expert is not resident) flags COLI_E_TIER and
// returns -1: the workgroup then skips the expert without reading it.
__device__ __forceinline__ int storage_of(const int32_t* slot_of, int n_store, int e,
                                          int32_t* err) {
  if (!slot_of) return e;
  const int p = *as_const(slot_of + e);
  if (p < 0 || p >= n_store) {
    if (threadIdx.x == 0) *err = COLI_E_TIER;
    return -1;
  }
  return p;
}

// 16-byte chunks per 32-column block (int4: 1, int8: 2); int2 packs two
// blocks in a chunk and has its own loop.
constexpr int chunks_per_block(int bits) { return bits == 8 ? 2 : 1; }
// Blocks in flight in a ring of pf chunks.
constexpr int blocks_per_ring(int pf, int bits) { return bits == 8 ? pf / 2 : bits == 4 ? pf : 2 * pf; }
// Chunks of a row group of nb blocks.
constexpr int row_chunks(int nb, int bits) { return bits == 8 ? 2 * nb : bits == 4 ? nb : nb / 2; }

// The 32 weight codes of one block as the 8 byte-vectors that line up with
// the 8 int8 words of the activation block (offset-binary nibbles for int4,
// signed bytes for int8).
struct Unpacked {
  uint32_t v[8];
};

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// A copy into a register distinct from the source ("=&v": early clobber).
// Taking a ring slot's words through it ends the slot's live range before the
// slot is refilled, so the refill load can target the same registers.
// Without it the register allocator keeps the consumed words in the slot
// registers, sends the refill elsewhere and copies the whole ring back at the
// loop's back-edge, which first waits for every load in flight (vmcnt(0)):
// the ring drains once per PF chunks.  Needed for int8 slots (used as
// loaded) and, under the register pressure of several tokens per pass, for
// int4 slots too; the one-token int4 loop is free of it without the copy.
__device__ __forceinline__ uint32_t fresh(uint32_t x) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=&v"(r) : "v"(x));
  return r;
}

// lo = w & 0x0F0F0F0F and t = w >> 4, both into registers distinct from w:
// the split ends w's live range the way fresh() does, without extra moves.
__device__ __forceinline__ void split_nibbles(uint32_t w, uint32_t& lo, uint32_t& t) {
  asm volatile("v_and_b32 %0, 0xf0f0f0f, %2\n\tv_lshrrev_b32 %1, 4, %2"
               : "=&v"(lo), "=&v"(t)
               : "v"(w));
}

// int4: one chunk holds the whole block.
template <bool COPY>
__device__ __forceinline__ Unpacked unpack_chunk(u32x4 w) {
  Unpacked u;
  if (COPY) {
    uint32_t t[4];
    split_nibbles(w.x, u.v[0], t[0]);
    split_nibbles(w.y, u.v[2], t[1]);
    split_nibbles(w.z, u.v[4], t[2]);
    split_nibbles(w.w, u.v[6], t[3]);
    u.v[1] = t[0] & 0x0F0F0F0Fu;
    u.v[3] = t[1] & 0x0F0F0F0Fu;
    u.v[5] = t[2] & 0x0F0F0F0Fu;
    u.v[7] = t[3] & 0x0F0F0F0Fu;
    return u;
  }
  u.v[0] = w.x & 0x0F0F0F0Fu;
  u.v[1] = (w.x >> 4) & 0x0F0F0F0Fu;
  u.v[2] = w.y & 0x0F0F0F0Fu;
  u.v[3] = (w.y >> 4) & 0x0F0F0F0Fu;
  u.v[4] = w.z & 0x0F0F0F0Fu;
  u.v[5] = (w.z >> 4) & 0x0F0F0F0Fu;
  u.v[6] = w.w & 0x0F0F0F0Fu;
  u.v[7] = (w.w >> 4) & 0x0F0F0F0Fu;
  return u;
}

// int8: two chunks, columns 0-15 and 16-31, bytes in column order.
__device__ __forceinline__ Unpacked int8_block(u32x4 lo, u32x4 hi) {
  Unpacked u;
  u.v[0] = lo.x;
  u.v[1] = lo.y;
  u.v[2] = lo.z;
  u.v[3] = lo.w;
  u.v[4] = hi.x;
  u.v[5] = hi.y;
  u.v[6] = hi.z;
  u.v[7] = hi.w;
  return u;
}

// The block in ring slots [slot, slot + U), for a loop serving NT tokens.
template <int U, int NT>
__device__ __forceinline__ Unpacked take_block(const u32x4* slot) {
  if constexpr (U == 1) {
    return unpack_chunk<(NT > 1)>(slot[0]);
  } else {
    return int8_block(slot[0], slot[1]);
  }
}

// The token blocks of one pass live in LDS, block-major: record b (R bytes)
// holds block b's 32 int8 activations of every token slot j of the pass (at
// 32 j), then each slot's pair (d, bitcast(-8 * sum)) (at 32 MAXT + 8 j).  So
// one address serves every token of a block, and the blocks of an unrolled
// ring pass sit at immediate offsets from one base: no per-token address
// arithmetic in the loop.  One wavefront stages the records once per pass
// (slots past the pass's token count repeat its last token), then reads them
// with broadcast LDS loads one block ahead of use; LDS returns in order, so
// those waits never drain the weight ring.  The records run on past the last
// block, zero-filled, up to a whole number of ring passes plus one (the
// read-ahead of the last block): a block past the end of the row then has
// activations 0 and scale 0 and adds exactly +0, so the loop needs no guard.
template <int MAXT>
struct PassLds {
  static constexpr int R = (40 * MAXT + 15) / 16 * 16;
  static constexpr int DM = 32 * MAXT;
};

// Records of a pass over nb blocks, pb blocks per ring pass.
constexpr int64_t pass_records(int64_t nb, int pb) { return (nb + pb - 1) / pb * pb + 1; }

constexpr size_t pass_lds_bytes(int maxt, int64_t nb, int pb) {
  return (size_t)pass_records(nb, pb) * (size_t)((40 * maxt + 15) / 16 * 16);
}

__device__ __forceinline__ unsigned char* gemv_lds() {
  extern __shared__ __align__(16) unsigned char coli_lds[];
  return coli_lds;
}

// Zero-fills the records past the last block (once per kernel: the passes
// only write records 0..NB-1).  Threads tid of nth of the workgroup.
template <int MAXT>
__device__ __forceinline__ void clear_tail_records(int NB, int pb, int tid, int nth) {
  constexpr int R = PassLds<MAXT>::R;
  uint4* tail = reinterpret_cast<uint4*>(gemv_lds() + (size_t)NB * R);
  const int n = (int)(pass_records(NB, pb) - NB) * (R / 16);
  for (int i = tid; i < n; i += nth) tail[i] = make_uint4(0, 0, 0, 0);
}

// The block's sum term is staged as -8 sum x (int4: nibbles are q + 8) or
// -2 sum x (int2: fields are q + 2; sum_shift 2, exact since -8 sum x is a
// multiple of 8); int8 blocks do not use it.
//
// Every load of a round (up to kStageX 16-byte code loads and kStageD scale/sum
// pairs per thread; one round covers d_model 8192 at 64 threads) is issued
// before the first LDS store, so staging costs one memory round trip, not
// one per load.  Memory waits retire in issue order, so the kernels issue
// only the head of their weight ring before the staging loads and the rest
// of it from after_loads(), which runs once the first round's loads are out:
// the staging then waits for the ring head, not for the whole ring.
constexpr int kStageX = 8;
constexpr int kStageD = 4;

template <int MAXT, typename F>
__device__ __forceinline__ void stage_round(unsigned char* lds, int j, const u32x4* xg,
                                            const float* __restrict__ drow,
                                            const int32_t* __restrict__ srow, int NB, int tid,
                                            int nth, int sum_shift, int r, F&& after_loads) {
  constexpr int R = PassLds<MAXT>::R;
  const int n = 2 * NB;
  // Indices past the end are clamped to the last element, for the loads and
  // the stores alike (a clamped lane rewrites that element with its own
  // value): the round is branch-free, so its loads stay together.
  int xi[kStageX], bi[kStageD];
  u32x4 v[kStageX];
  float d[kStageD];
  int32_t s[kStageD];
#pragma unroll
  for (int u = 0; u < kStageX; ++u) {
    const int i = (r * kStageX + u) * nth + tid;
    xi[u] = i < n ? i : n - 1;
    v[u] = xg[xi[u]];
  }
#pragma unroll
  for (int u = 0; u < kStageD; ++u) {
    const int b = (r * kStageD + u) * nth + tid;
    bi[u] = b < NB ? b : NB - 1;
    d[u] = drow[bi[u]];
    s[u] = srow[bi[u]];
  }
  after_loads();
  // the loaded values are taken here, after every load of the round has been
  // issued (otherwise the compiler sinks each load down to its store)
#pragma unroll
  for (int u = 0; u < kStageX; ++u) asm volatile("" : "+v"(v[u]));
#pragma unroll
  for (int u = 0; u < kStageX; ++u)
    *reinterpret_cast<u32x4*>(lds + (size_t)(xi[u] >> 1) * R + 32 * j + 16 * (xi[u] & 1)) = v[u];
#pragma unroll
  for (int u = 0; u < kStageD; ++u)
    *reinterpret_cast<float2*>(lds + (size_t)bi[u] * R + PassLds<MAXT>::DM + 8 * j) =
        make_float2(d[u], __int_as_float(s[u] >> sum_shift));
}

template <int MAXT, typename F>
__device__ __forceinline__ void stage_token(unsigned char* lds, int j,
                                            const int8_t* __restrict__ xrow,
                                            const float* __restrict__ drow,
                                            const int32_t* __restrict__ srow, int NB, int tid,
                                            int nth, int sum_shift, F&& after_loads) {
  const u32x4* xg = reinterpret_cast<const u32x4*>(xrow);
  stage_round<MAXT>(lds, j, xg, drow, srow, NB, tid, nth, sum_shift, 0, after_loads);
  for (int r = 1; r * nth * kStageX < 2 * NB || r * nth * kStageD < NB; ++r)
    stage_round<MAXT>(lds, j, xg, drow, srow, NB, tid, nth, sum_shift, r, [] {});
}

struct XBlock {
  uint4 lo, hi;
  float2 dm;
};

// Token slot j of the block whose record starts at rec.
template <int MAXT>
__device__ __forceinline__ XBlock read_xblock(const unsigned char* rec, int j) {
  XBlock v;
  v.lo = *reinterpret_cast<const uint4*>(rec + 32 * j);
  v.hi = *reinterpret_cast<const uint4*>(rec + 32 * j + 16);
  v.dm = *reinterpret_cast<const float2*>(rec + PassLds<MAXT>::DM + 8 * j);
  return v;
}

// P_b of one row with one activation block: sum over 32 of q_w * q_x
// (int4: the offset-binary sum plus the block's -8 sum x).
template <int U>
__device__ __forceinline__ int block_dot(const Unpacked& u, const XBlock& xb) {
  int s = U == 1 ? __float_as_int(xb.dm.y) : 0;
  s = sdot4((int)u.v[0], (int)xb.lo.x, s);
  s = sdot4((int)u.v[1], (int)xb.lo.y, s);
  s = sdot4((int)u.v[2], (int)xb.lo.z, s);
  s = sdot4((int)u.v[3], (int)xb.lo.w, s);
  s = sdot4((int)u.v[4], (int)xb.hi.x, s);
  s = sdot4((int)u.v[5], (int)xb.hi.y, s);
  s = sdot4((int)u.v[6], (int)xb.hi.z, s);
  s = sdot4((int)u.v[7], (int)xb.hi.w, s);
  return s;
}

// The weight ring of one row group: PF outstanding 16-byte loads per lane,
// over the NU chunks (1 KB per wavefront each) of the row group.
template <int PF>
struct Ring {
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t loff;
  int NU;
  u32x4 buf[PF];

  // Issues slots [0, N0) (the ring head), in slot order so that slot 0 lands
  // first; issue<N0>() issues the rest.
  template <int N0>
  __device__ __forceinline__ void start(const char* wbase, uint32_t lane_off, int nu) {
    rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(wbase), 0, nu * 1024, kBufferConfig);
    loff = lane_off;
    NU = nu;
    issue_range<0, N0>();
  }
  template <int N0>
  __device__ __forceinline__ void issue() {
    issue_range<N0, PF>();
  }
  template <int A, int B>
  __device__ __forceinline__ void issue_range() {
#pragma unroll
    for (int i = A; i < B; ++i) {
      buf[i] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, loff, (i < NU ? i : NU - 1) * 1024,
                                                     kNonTemporal);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
};

// Ring slots issued before the token staging (the rest follow its loads).
constexpr int ring_head(int pf, int maxt) { return maxt >= 8 || pf < 4 ? pf : 4; }

// Refills the U slots of ring position i (block b) with the chunks of block
// b + PB, clamped into the row group.
template <int PF, int U, int PB>
__device__ __forceinline__ void refill(Ring<PF>& ring, int b, int i) {
  const int NU = ring.NU;
#pragma unroll
  for (int c = 0; c < U; ++c) {
    const int un = U * (b + PB) + c < NU ? U * (b + PB) + c : NU - 1;
    ring.buf[U * i + c] =
        __builtin_amdgcn_raw_buffer_load_b128(ring.rsrc, ring.loff, un * 1024, kNonTemporal);
  }
}

// Streams the NB blocks of one row group (lane-owned rows) and accumulates
// exactly NT tokens.  The body is branch-free so the waitcnt pass can keep
// the ring of PF weight loads in flight: every refill is unconditional (its
// index is clamped into the row group), and a block past the end of the row
// (only when PF / U does not divide NB) is computed on clamped weights and a
// zero record, which leaves the accumulator bit-identical (it starts at +0
// and so is never -0).  Buffer loads: the row group is one descriptor (scalar
// registers), the lane's 16-byte column a constant vector offset and the
// chunk a scalar offset; each ring slot is consumed before it is refilled, so
// the ring stays PF deep across the loop back-edge.  Weight loads are
// non-temporal: each byte is used once.
// A block is U consecutive chunks, so PF / U blocks are in flight.
template <int NT, int MAXT, int PF, int U, bool TRACE>
__device__ __forceinline__ void stream_rows(Ring<PF>& ring, float* acc,
                                            int32_t* const* trace_row) {
  static_assert(PF % U == 0, "the ring holds whole blocks");
  constexpr int PB = PF / U;
  constexpr int R = PassLds<MAXT>::R;
  const unsigned char* lds = gemv_lds();
  const int NU = ring.NU;
  const int NB = NU / U;
  XBlock cur[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) cur[j] = read_xblock<MAXT>(lds, j);
  for (int b0 = 0; b0 < NB; b0 += PB) {
    const unsigned char* rec = lds + (size_t)b0 * R;
#pragma unroll
    for (int i = 0; i < PB; ++i) {
      const int b = b0 + i;
      const Unpacked u = take_block<U, NT>(&ring.buf[U * i]);
      __builtin_amdgcn_sched_barrier(0);
      // int4 slots are refilled as soon as they are unpacked; int8 slots feed
      // the dots as loaded, so they are refilled after the block's dots (the
      // load can then reuse the slot's registers).
      if constexpr (U == 1) refill<PF, U, PB>(ring, b, i);
      XBlock nxt[NT];
#pragma unroll
      for (int j = 0; j < NT; ++j) nxt[j] = read_xblock<MAXT>(rec + (i + 1) * R, j);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int p = block_dot<U>(u, cur[j]);
        if (TRACE) {
          if (trace_row[j] && b < NB) trace_row[j][b] = p;
        }
        acc[j] = __builtin_fmaf((float)p, cur[j].dm.x, acc[j]);
        cur[j] = nxt[j];
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (U == 2) {
        refill<PF, U, PB>(ring, b, i);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
}

// int2: one 16-byte chunk holds two blocks (64 columns).  Word m of the
// chunk covers columns 16m..16m+15; its byte j holds, from the lowest bits
// up, 2-bit fields for columns 16m + 4i + j (i = 0..3), offset binary
// (q + 2), so (w >> 2i) & 0x03030303 is the byte vector of activation word
// 4m + i.  The first split of each word writes fresh registers (early
// clobber), which ends the ring slot's live range before its refill.
__device__ __forceinline__ void split_pairs(uint32_t w, uint32_t& f0, uint32_t& t) {
  asm volatile("v_and_b32 %0, 0x3030303, %2\n\tv_lshrrev_b32 %1, 2, %2"
               : "=&v"(f0), "=&v"(t)
               : "v"(w));
}

__device__ __forceinline__ void unpack_int2(u32x4 w, Unpacked* u) {
  const uint32_t word[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    uint32_t t;
    Unpacked& ub = u[m >> 1];
    const int base = 4 * (m & 1);
    split_pairs(word[m], ub.v[base], t);
    ub.v[base + 1] = t & 0x03030303u;
    ub.v[base + 2] = (t >> 2) & 0x03030303u;
    ub.v[base + 3] = (t >> 4) & 0x03030303u;
  }
}

// stream_rows for int2 tables: ring slot i holds blocks 2i and 2i + 1 of the
// ring pass, so PF chunks are 2 PF blocks in flight.  The block dot starts
// from the staged -2 sum x (codes are stored as q + 2).
template <int NT, int MAXT, int PF, bool TRACE>
__device__ __forceinline__ void stream_rows2(Ring<PF>& ring, float* acc,
                                             int32_t* const* trace_row) {
  constexpr int PB = 2 * PF;
  constexpr int R = PassLds<MAXT>::R;
  const unsigned char* lds = gemv_lds();
  const int NU = ring.NU;
  const int NB = 2 * NU;
  XBlock cur[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) cur[j] = read_xblock<MAXT>(lds, j);
  for (int b0 = 0; b0 < NB; b0 += PB) {
    const unsigned char* rec = lds + (size_t)b0 * R;
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      Unpacked u[2];
      unpack_int2(ring.buf[i], u);
      __builtin_amdgcn_sched_barrier(0);
      const int c = b0 / 2 + i + PF;
      ring.buf[i] = __builtin_amdgcn_raw_buffer_load_b128(ring.rsrc, ring.loff,
                                                          (c < NU ? c : NU - 1) * 1024,
                                                          kNonTemporal);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int b = b0 + 2 * i + h;
        XBlock nxt[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) nxt[j] = read_xblock<MAXT>(rec + (2 * i + h + 1) * R, j);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const int p = block_dot<1>(u[h], cur[j]);
          if (TRACE) {
            if (trace_row[j] && b < NB) trace_row[j][b] = p;
          }
          acc[j] = __builtin_fmaf((float)p, cur[j].dm.x, acc[j]);
          cur[j] = nxt[j];
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
}

// Token slots a pass of nt tokens computes: the next power of two (at most
// MAXT); slots from nt on repeat the last token and their results are unused.
template <int MAXT>
__device__ __forceinline__ int pass_slots(int nt) {
  return (MAXT >= 8 && nt > 4) ? 8 : (MAXT >= 4 && nt > 2) ? 4 : (MAXT >= 2 && nt == 2) ? 2 : 1;
}

// Runs the loop of the table's container for NT token slots.
template <int NT, int MAXT, int PF, int BITS, bool TRACE>
__device__ __forceinline__ void stream_slots(Ring<PF>& ring, float* acc,
                                             int32_t* const* trace_row) {
  if constexpr (BITS == 2) {
    stream_rows2<NT, MAXT, PF, TRACE>(ring, acc, trace_row);
  } else {
    stream_rows<NT, MAXT, PF, chunks_per_block(BITS), TRACE>(ring, acc, trace_row);
  }
}

// Runs the loop for the nt (1..MAXT) tokens of one pass.
template <int MAXT, int PF, int BITS, bool TRACE>
__device__ __forceinline__ void stream_pass(int nt, Ring<PF>& ring, float* acc,
                                            int32_t* const* trace_row) {
  switch (pass_slots<MAXT>(nt)) {
    case 8: stream_slots<(MAXT >= 8 ? 8 : 1), MAXT, PF, BITS, TRACE>(ring, acc, trace_row); break;
    case 4: stream_slots<(MAXT >= 4 ? 4 : 1), MAXT, PF, BITS, TRACE>(ring, acc, trace_row); break;
    case 2: stream_slots<(MAXT >= 2 ? 2 : 1), MAXT, PF, BITS, TRACE>(ring, acc, trace_row); break;
    default: stream_slots<1, MAXT, PF, BITS, TRACE>(ring, acc, trace_row); break;
  }
}

// A workgroup is W wavefronts on W consecutive row groups of one expert:
// they share one copy of the pass's token records, so a pass needs 1 / W of
// the LDS per wavefront (the 4- and 8-token records would otherwise cap the
// resident workgroups per CU below the wavefronts the chip can hold).  A
// trailing wavefront without a row group of its own recomputes the last one
// and stores nothing.
constexpr int gemv_waves(int maxt) { return maxt >= 4 ? 4 : 1; }

// Maximum / sum over each 32-lane half of the wavefront, returned in every
// lane of the half: rotations within the 16-lane rows (DPP row_ror 1, 2, 4,
// 8), then the half's two rows combined through v_permlane16_swap (its two
// results hold, in every lane, the lane's own row and the other row of its
// pair).  Both are exact in any order.
constexpr int kDppRowRor = 0x120;
template <int N>
__device__ __forceinline__ float ror_max(float x) {
  return fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kDppRowRor + N,
                                                             0xF, 0xF, false)));
}
template <int N>
__device__ __forceinline__ int ror_add(int x) {
  return x + __builtin_amdgcn_update_dpp(0, x, kDppRowRor + N, 0xF, 0xF, false);
}
__device__ __forceinline__ float half_max(float x) {
  x = ror_max<8>(ror_max<4>(ror_max<2>(ror_max<1>(x))));
  const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ int half_sum(int x) {
  x = ror_add<8>(ror_add<4>(ror_add<2>(ror_add<1>(x))));
  const auto s = __builtin_amdgcn_permlane16_swap((unsigned)x, (unsigned)x, false, false);
  return (int)s[0] + (int)s[1];
}

// gate/up of a one-token pass (one wavefront per row group).  The token is
// token 0 whatever the routing, so its blocks are staged first, with no
// dependent load before them; the expert's weight ring starts as soon as the
// active-expert load returns, between the staging loads and the LDS stores.
template <int PF, int BITS, bool TRACE>
__device__ __forceinline__ void gate_up_one_token(const GuArgs& a) {
  const int slot = blockIdx.y, lane = (int)threadIdx.x;
  const int NB = (int)(a.D / 32);
  const int64_t G = a.F / 32;
  const int grp = (int)blockIdx.x;       // grid.x == G at one wavefront per workgroup
  const int NU = row_chunks(NB, BITS);
  unsigned char* lds = gemv_lds();
  Ring<PF> ring;
  int e = 0, es = -1;
  stage_token<1>(lds, 0, a.xq, a.xd, a.xsum8, NB, lane, kWave, BITS == 2 ? 2 : 0, [&] {
    const int n_active = *as_const(a.n_active);
    e = as_const(a.active)[slot];
    es = slot < n_active ? storage_of(a.slot_of, a.n_store, e, a.err) : -1;
    // issued on every path (expert 0 stands in when there is none), so the
    // memory-counter waits after it count the whole ring
    const int esafe = es < 0 ? 0 : es;
    ring.template start<PF>(
        reinterpret_cast<const char*>(a.gu_q + ((size_t)esafe * G + grp) * (size_t)NU * kWave),
        16u * (uint32_t)lane, NU);
  });
  if (es < 0) return;                    // uniform: one wavefront
  clear_tail_records<1>(NB, blocks_per_ring(PF, BITS), lane, kWave);
  const float rs = a.gu_s[((size_t)es * G + grp) * kWave + lane];
  const int pair = as_const(a.lists)[(size_t)e * a.T];
  int32_t* trow[1] = {nullptr};
  if (TRACE) {
    int32_t* base = lane < 32 ? a.tr_pg : a.tr_pu;
    if (base) trow[0] = base + ((size_t)pair * a.F + 32 * (size_t)grp + (lane & 31)) * NB;
  }
  __syncthreads();
  float acc[1] = {0.0f};
  stream_pass<1, PF, BITS, TRACE>(1, ring, acc, trow);
  const float v = acc[0] * rs;              // g (lanes 0-31) or u (lanes 32-63)
  // lanes 0-31 receive their up row (lane + 32)
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                   false);
  const float up = __uint_as_float(sw[1]);
  const float h = silu_f32(v) * up;
  const float amax = half_max(fabsf(h));
  const float d = amax / 127.0f;
  const int q = q8_code(h, d);
  const int qs = half_sum(q);
  if (lane < 32) {
    const size_t p = (size_t)pair;
    const size_t r = 32 * (size_t)grp + lane;
    a.hq[p * a.F + r] = (int8_t)q;
    if (a.hq_slot) a.hq_slot[(size_t)slot * a.F + r] = (int8_t)q;
    if (lane == 0) {
      a.hd[p * G + grp] = d;
      a.hsum8[p * G + grp] = -8 * qs;
      if (a.hq_slot) {
        a.hd_slot[(size_t)slot * G + grp] = d;
        a.hs_slot[(size_t)slot * G + grp] = -8 * qs;
      }
    }
    if (TRACE) {
      if (a.tr_g) a.tr_g[p * a.F + r] = v;
      if (a.tr_u) a.tr_u[p * a.F + r] = up;
      if (a.tr_h) a.tr_h[p * a.F + r] = h;
    }
  }
}

template <int MAXT, int PF, int BITS, bool TRACE>
__global__ void __launch_bounds__(64 * gemv_waves(MAXT)) gate_up_kernel(GuArgs a) {
  if constexpr (MAXT == 1) {
    if (a.T == 1) {
      gate_up_one_token<PF, BITS, TRACE>(a);
      return;
    }
  }
  constexpr int W = gemv_waves(MAXT);
  const int slot = blockIdx.y;
  const int n_active = *as_const(a.n_active);   // both loads in flight together;
  const int e = as_const(a.active)[slot];        // e is used only once slot is valid
  if (slot >= n_active) return;
  const int wave = W > 1 ? __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave) : 0;
  const int lane = (int)threadIdx.x % kWave;
  const int NB = (int)(a.D / 32);
  const int64_t G = a.F / 32;
  const bool live = (int64_t)blockIdx.x * W + wave < G;
  const int grp = live ? (int)blockIdx.x * W + wave : (int)G - 1;
  const int KS = a.k + a.S;
  const int es = storage_of(a.slot_of, a.n_store, e, a.err);
  if (es < 0) return;                    // uniform across the workgroup
  const int NU = row_chunks(NB, BITS);   // 1 KB chunks in the row group
  const char* wbase = reinterpret_cast<const char*>(a.gu_q + ((size_t)es * G + grp) * (size_t)NU * kWave);
  const uint32_t loff = 16u * (uint32_t)lane;
  constexpr int H = ring_head(PF, MAXT);
  Ring<PF> ring;
  ring.template start<H>(wbase, loff, NU);       // the weight stream starts before anything else
  clear_tail_records<MAXT>(NB, blocks_per_ring(PF, BITS), threadIdx.x, kWave * W);
  const int cnt = as_const(a.counts)[e];
  const float rs = a.gu_s[((size_t)es * G + grp) * kWave + lane];
  const cptr<int32_t> list = as_const(a.lists + (size_t)e * a.T);
  for (int c0 = 0; c0 < cnt; c0 += MAXT) {
    const int nt = cnt - c0 < MAXT ? cnt - c0 : MAXT;
    const int ns = pass_slots<MAXT>(nt);
    int pair[MAXT];
    int32_t* trow[MAXT];
    if (c0 > 0) {
      __syncthreads();                // the previous pass has finished reading the LDS records
      ring.template start<H>(wbase, loff, NU); // each pass streams the row group again
    }
#pragma unroll
    for (int j = 0; j < MAXT; ++j) {
      pair[j] = list[c0 + (j < nt ? j : nt - 1)];
      trow[j] = nullptr;
      if (TRACE) {
        int32_t* base = lane < 32 ? a.tr_pg : a.tr_pu;
        if (base && live)
          trow[j] = base + ((size_t)pair[j] * a.F + 32 * (size_t)grp + (lane & 31)) * NB;
      }
    }
#pragma unroll
    for (int j = 0; j < MAXT; ++j) {
      if (j < ns) {   // (ns >= 1: token 0 always runs and issues the ring's rest)
        const int64_t t = __builtin_amdgcn_readfirstlane(pair[j] / KS);
        if (j == 0)
          stage_token<MAXT>(gemv_lds(), j, a.xq + t * a.D, a.xd + t * NB, a.xsum8 + t * NB, NB,
                            threadIdx.x, kWave * W, BITS == 2 ? 2 : 0,
                            [&] { ring.template issue<H>(); });
        else
          stage_token<MAXT>(gemv_lds(), j, a.xq + t * a.D, a.xd + t * NB, a.xsum8 + t * NB, NB,
                            threadIdx.x, kWave * W, BITS == 2 ? 2 : 0, [] {});
      }
    }
    __syncthreads();
    float acc[MAXT];
#pragma unroll
    for (int j = 0; j < MAXT; ++j) acc[j] = 0.0f;
    stream_pass<MAXT, PF, BITS, TRACE>(nt, ring, acc, trow);
#pragma unroll
    for (int j = 0; j < MAXT; ++j) {
      if (j < nt) {
        const float v = acc[j] * rs;              // g (lanes 0-31) or u (lanes 32-63)
        // lanes 0-31 receive their up row (lane + 32)
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                         false, false);
        const float up = __uint_as_float(sw[1]);
        const float h = silu_f32(v) * up;
        const float amax = half_max(fabsf(h));
        const float d = amax / 127.0f;
        const int q = q8_code(h, d);
        const int qs = half_sum(q);
        const size_t p = (size_t)pair[j];
        if (live && lane < 32) {
          const size_t r = 32 * (size_t)grp + lane;
          a.hq[p * a.F + r] = (int8_t)q;
          if (lane == 0) {
            a.hd[p * G + grp] = d;
            a.hsum8[p * G + grp] = -8 * qs;
          }
          if (TRACE) {
            if (a.tr_g) a.tr_g[p * a.F + r] = v;
            if (a.tr_u) a.tr_u[p * a.F + r] = up;
            if (a.tr_h) a.tr_h[p * a.F + r] = h;
          }
        }
      }
    }
  }
}

// down of a one-token pass (one wavefront per 64-row group).  Its token
// records are the slot's Q8(h), which gate/up also stored in active-slot
// order, so they are staged first with no dependent load; the weight ring
// starts as soon as the active-expert load returns, and the pair (the output
// row) is looked up while the staging completes.
template <int PF, int BITS, bool TRACE>
__device__ __forceinline__ void down_one_token(const DnArgs& a) {
  const int slot = blockIdx.y, lane = (int)threadIdx.x;
  const int NB = (int)(a.F / 32);
  const int grp = (int)blockIdx.x;       // grid.x == D / 64 at one wavefront per workgroup
  const int NU = row_chunks(NB, BITS);
  unsigned char* lds = gemv_lds();
  Ring<PF> ring;
  int e = 0, es = -1;
  stage_token<1>(lds, 0, a.hq_slot + (size_t)slot * a.F, a.hd_slot + (size_t)slot * NB,
                 a.hs_slot + (size_t)slot * NB, NB, lane, kWave, BITS == 2 ? 2 : 0, [&] {
    const int n_active = *as_const(a.n_active);
    e = as_const(a.active)[slot];
    es = slot < n_active ? storage_of(a.slot_of, a.n_store, e, a.err) : -1;
    // issued on every path (expert 0 stands in when there is none), so the
    // memory-counter waits after it count the whole ring
    const int esafe = es < 0 ? 0 : es;
    ring.template start<PF>(
        reinterpret_cast<const char*>(a.dn_q + ((size_t)esafe * (a.D / 64) + grp) * (size_t)NU * kWave),
        16u * (uint32_t)lane, NU);
  });
  if (es < 0) return;                    // uniform: one wavefront
  clear_tail_records<1>(NB, blocks_per_ring(PF, BITS), lane, kWave);
  const size_t row = 64 * (size_t)grp + lane;
  const float rs = a.dn_s[(size_t)es * a.D + row];
  const int pair = as_const(a.lists)[(size_t)e * a.T];
  int32_t* trow[1] = {(TRACE && a.tr_pd) ? a.tr_pd + ((size_t)pair * a.D + row) * NB : nullptr};
  __syncthreads();
  float acc[1] = {0.0f};
  stream_pass<1, PF, BITS, TRACE>(1, ring, acc, trow);
  a.o[(size_t)pair * a.D + row] = acc[0] * rs;
}

template <int MAXT, int PF, int BITS, bool TRACE>
__global__ void __launch_bounds__(64 * gemv_waves(MAXT)) down_kernel(DnArgs a) {
  if constexpr (MAXT == 1) {
    if (a.T == 1 && a.hq_slot) {
      down_one_token<PF, BITS, TRACE>(a);
      return;
    }
  }
  constexpr int W = gemv_waves(MAXT);
  const int slot = blockIdx.y;
  const int n_active = *as_const(a.n_active);   // both loads in flight together;
  const int e = as_const(a.active)[slot];        // e is used only once slot is valid
  if (slot >= n_active) return;
  const int wave = W > 1 ? __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave) : 0;
  const int lane = (int)threadIdx.x % kWave;
  const int64_t G = a.D / 64;
  const bool live = (int64_t)blockIdx.x * W + wave < G;
  const int grp = live ? (int)blockIdx.x * W + wave : (int)G - 1;
  const int NB = (int)(a.F / 32);
  const int NU = row_chunks(NB, BITS);
  const int es = storage_of(a.slot_of, a.n_store, e, a.err);
  if (es < 0) return;                    // uniform across the workgroup
  const char* wbase =
      reinterpret_cast<const char*>(a.dn_q + ((size_t)es * (a.D / 64) + grp) * (size_t)NU * kWave);
  const uint32_t loff = 16u * (uint32_t)lane;
  constexpr int H = ring_head(PF, MAXT);
  Ring<PF> ring;
  ring.template start<H>(wbase, loff, NU);       // the weight stream starts before anything else
  clear_tail_records<MAXT>(NB, blocks_per_ring(PF, BITS), threadIdx.x, kWave * W);
  const int cnt = as_const(a.counts)[e];
  const size_t row = 64 * (size_t)grp + lane;
  const float rs = a.dn_s[(size_t)es * a.D + row];
  const cptr<int32_t> list = as_const(a.lists + (size_t)e * a.T);
  for (int c0 = 0; c0 < cnt; c0 += MAXT) {
    const int nt = cnt - c0 < MAXT ? cnt - c0 : MAXT;
    const int ns = pass_slots<MAXT>(nt);
    int pair[MAXT];
    int32_t* trow[MAXT];
    if (c0 > 0) {
      __syncthreads();
      ring.template start<H>(wbase, loff, NU);
    }
#pragma unroll
    for (int j = 0; j < MAXT; ++j) {
      pair[j] = list[c0 + (j < nt ? j : nt - 1)];
      trow[j] = (TRACE && a.tr_pd && live) ? a.tr_pd + ((size_t)pair[j] * a.D + row) * NB : nullptr;
    }
#pragma unroll
    for (int j = 0; j < MAXT; ++j) {
      if (j < ns) {   // (ns >= 1: token 0 always runs and issues the ring's rest)
        const size_t p = (size_t)__builtin_amdgcn_readfirstlane(pair[j]);
        if (j == 0)
          stage_token<MAXT>(gemv_lds(), j, a.hq + p * a.F, a.hd + p * NB, a.hsum8 + p * NB, NB,
                            threadIdx.x, kWave * W, BITS == 2 ? 2 : 0,
                            [&] { ring.template issue<H>(); });
        else
          stage_token<MAXT>(gemv_lds(), j, a.hq + p * a.F, a.hd + p * NB, a.hsum8 + p * NB, NB,
                            threadIdx.x, kWave * W, BITS == 2 ? 2 : 0, [] {});
      }
    }
    __syncthreads();
    float acc[MAXT];
#pragma unroll
    for (int j = 0; j < MAXT; ++j) acc[j] = 0.0f;
    stream_pass<MAXT, PF, BITS, TRACE>(nt, ring, acc, trow);
#pragma unroll
    for (int j = 0; j < MAXT; ++j)
      if (live && j < nt) a.o[(size_t)pair[j] * a.D + row] = acc[j] * rs;
  }
}

__device__ __forceinline__ float4 fma4(float w, float4 a, float4 acc) {
  return make_float4(__builtin_fmaf(w, a.x, acc.x), __builtin_fmaf(w, a.y, acc.y),
                     __builtin_fmaf(w, a.z, acc.z), __builtin_fmaf(w, a.w, acc.w));
}

// y[t][r] = o_shared + sum_j w_j o_j, as y = fmaf(w_j, o_j, y) in slot order,
// four rows per thread.  KU > 0: k == KU, unrolled, every slot's load issued
// before the ordered fmaf chain; KU == 0: any k.  Slots the dispatch drops
// are skipped (their o rows were never written): an index outside [0, E), or
// one equal to an earlier slot's of the same token.
template <int KU>
__global__ void __launch_bounds__(256) combine_kernel(const float* __restrict__ o,
                                                      const int32_t* __restrict__ idx,
                                                      const float* __restrict__ w, int64_t D,
                                                      int k, int E, int S, float* __restrict__ y,
                                                      int accumulate) {
  const int64_t t = blockIdx.y;
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // 4-row group
  if (4 * q >= D) return;
  const int KS = k + S;
  const float4* ot = reinterpret_cast<const float4*>(o + (size_t)t * KS * D) + q;
  const int64_t D4 = D / 4;
  float4 acc = S ? ot[k * D4] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  if constexpr (KU > 0) {
    float4 v[KU];
    float wj[KU];
#pragma unroll
    for (int j = 0; j < KU; ++j) {   // o rows of skipped slots are read but never used,
      wj[j] = w[t * KU + j];         // so no load waits for the index check
      v[j] = ot[j * D4];
    }
    int ev[KU];
#pragma unroll
    for (int j = 0; j < KU; ++j) ev[j] = idx[t * KU + j];
#pragma unroll
    for (int j = 0; j < KU; ++j) {
      bool keep = ev[j] >= 0 && ev[j] < E;
#pragma unroll
      for (int i = 0; i < j; ++i) keep = keep && ev[i] != ev[j];
      if (keep) acc = fma4(wj[j], v[j], acc);
    }
  } else {
    for (int j = 0; j < k; ++j) {
      const int e = idx[t * k + j];
      bool keep = e >= 0 && e < E;
      for (int i = 0; i < j && keep; ++i) keep = idx[t * k + i] != e;
      if (!keep) continue;
      acc = fma4(w[t * k + j], ot[j * D4], acc);
    }
  }
  float4* yt = reinterpret_cast<float4*>(y + t * D) + q;
  if (accumulate) {
    const float4 r = *yt;
    acc = make_float4(r.x + acc.x, r.y + acc.y, r.z + acc.z, r.w + acc.w);
  }
  *yt = acc;
}

// Stage events (profiled forward only; not for stream capture, where a record
// only expresses a dependency).
hipError_t record(void* ev, hipStream_t s) {
  return ev ? hipEventRecord(reinterpret_cast<hipEvent_t>(ev), s) : hipSuccess;
}

// Weight loads (1 KB per wavefront) in flight per wavefront, by tokens per
// pass and 16-byte chunks per block, as measured at d_model 6144, d_ff 2048
// with 257 experts.  One-token gate/up passes keep 12 (576 wavefronts on the
// chip): a decode step took 36.0 us against 37.5 with 16, 38.4 with 24, 36.7
// with 8 and 40.0 with 6 (depths that divide the 192-block row; 10 ties with
// 12, 14 ran 36.8); one-token down passes are fastest at 8 (4 and 16
// slower).  int8 tables (two loads per block) keep 8 in one-token gate/up
// passes: 60.9 us per step against 62.0 with 12, 63.6 with 16, 68.0 with 6
// and 82.0 with 4; int2 tables are fastest at 12 too (28.9 us per step
// against 29.1 with 8 or 16).  Four-token passes run
// four wavefronts per workgroup on ~1,800 row groups, and the fewer loads
// each keeps in flight the better down to gate/up 4, down 2: 99.6 us per
// pass against 108.6 with 16 and 8 (gate/up 2 with down 2: 110.4); int2
// tables gain too (86.6 -> 76.2 us), int8 tables (two loads per block) lose
// (180.1 -> 184.6 us) and keep 16 and 8.  With int4 tables, two-token
// passes are fastest at 16 and 4 (65.1 us against 66.8 with 16 and 8; 8 and
// 4: 68.1, 12 and 8: 70.5) and eight-token passes at 8 and 4 (199.6 against
// 201.5 us; 4 and 2: 208).
constexpr int pf_gate_up(int maxt, int bits) {
  if (maxt <= 0 || bits <= 0) return 0;
  if (maxt == 1) return bits == 8 ? 8 : 12;
  if (maxt == 4 && bits != 8) return 4;
  if (maxt == 8 && bits == 4) return 8;
  return 16;
}
constexpr int pf_down(int maxt, int bits) {
  if (maxt <= 0 || bits <= 0) return 0;
  if (maxt == 4 && bits != 8) return 2;
  if ((maxt == 2 || maxt == 8) && bits == 4) return 4;
  return 8;
}
constexpr size_t kLdsLimit = 65536;

// Stage events of the GEMV kernels, attached to the kernels' own dispatches
// (hipExtLaunchKernelGGL): gu_start / gu_stop take the start and end of the
// gate/up kernel's execution, dn_stop the end of the down kernel's.  So the
// gate/up interval is the kernel itself, with no marker packet or dispatch
// gap inside it.  Any may be null.
struct GemvEvents {
  void* gu_start;
  void* gu_stop;
  void* dn_stop;
};

template <int MAXT, int BITS, bool TRACE>
hipError_t launch_pair(const GuArgs& g, const DnArgs& d, int maxA, const GemvEvents& ev,
                       hipStream_t s) {
  constexpr int PG = pf_gate_up(MAXT, BITS), PD = pf_down(MAXT, BITS);
  const size_t lds_gu = pass_lds_bytes(MAXT, g.D / 32, blocks_per_ring(PG, BITS));
  const size_t lds_dn = pass_lds_bytes(MAXT, d.F / 32, blocks_per_ring(PD, BITS));
  constexpr int W = gemv_waves(MAXT);
  hipExtLaunchKernelGGL((gate_up_kernel<MAXT, PG, BITS, TRACE>),
                        dim3((unsigned)((g.F / 32 + W - 1) / W), maxA), dim3(kWave * W),
                        (uint32_t)lds_gu, s, reinterpret_cast<hipEvent_t>(ev.gu_start),
                        reinterpret_cast<hipEvent_t>(ev.gu_stop), 0, g);
  hipError_t rc = hipGetLastError();
  if (rc != hipSuccess) return rc;
  hipExtLaunchKernelGGL((down_kernel<MAXT, PD, BITS, TRACE>),
                        dim3((unsigned)((d.D / 64 + W - 1) / W), maxA), dim3(kWave * W),
                        (uint32_t)lds_dn, s, nullptr, reinterpret_cast<hipEvent_t>(ev.dn_stop),
                        0, d);
  return hipGetLastError();
}

// Tokens per pass: the batch (a power of two up to 8), capped so that the
// pass's LDS token records fit in 64 KB in both kernels.
int pass_tokens(int64_t T, int64_t D, int64_t F, int bits) {
  int m = T <= 1 ? 1 : T <= 2 ? 2 : T <= 4 ? 4 : 8;
  auto fits = [&](int mt) {
    return pass_lds_bytes(mt, D / 32, blocks_per_ring(pf_gate_up(mt, bits), bits)) <= kLdsLimit &&
           pass_lds_bytes(mt, F / 32, blocks_per_ring(pf_down(mt, bits), bits)) <= kLdsLimit;
  };
  while (m > 1 && !fits(m)) m /= 2;
  return m;
}

template <int BITS, bool TRACE>
hipError_t launch_gemv_bits(const GuArgs& g, const DnArgs& d, int maxA, int64_t T,
                            const GemvEvents& ev, hipStream_t s) {
  switch (pass_tokens(T, g.D, g.F, BITS)) {
    case 1: return launch_pair<1, BITS, TRACE>(g, d, maxA, ev, s);
    case 2: return launch_pair<2, BITS, TRACE>(g, d, maxA, ev, s);
    case 4: return launch_pair<4, BITS, TRACE>(g, d, maxA, ev, s);
    default: return launch_pair<8, BITS, TRACE>(g, d, maxA, ev, s);
  }
}

template <bool TRACE>
hipError_t launch_gemv(const GuArgs& g, const DnArgs& d, int bits, int maxA, int64_t T,
                       const GemvEvents& ev, hipStream_t s) {
  switch (bits) {
    case 8: return launch_gemv_bits<8, TRACE>(g, d, maxA, T, ev, s);
    case 2: return launch_gemv_bits<2, TRACE>(g, d, maxA, T, ev, s);
    default: return launch_gemv_bits<4, TRACE>(g, d, maxA, T, ev, s);
  }
}

}  // namespace

hipError_t launch_moe_forward(const ForwardArgs& f, hipStream_t s) {
  const coli_expert_table& t = *f.table;
  const int E = t.n_routed, S = t.n_shared;
  const int64_t D = t.d_model, F = t.d_ff, T = f.T;
  if (T == 0) return hipSuccess;
  const MoeWorkspace& ws = f.ws;
  const coli_moe_events no_events = {};
  const coli_moe_events& ev = f.events ? *f.events : no_events;
  hipError_t rc = record(ev.begin, s);
  if (rc != hipSuccess) return rc;
  const bool grouped = f.grouped;
  if (!f.dispatched) {
    // the GEMV path also needs the code sums of x; the grouped path does not
    rc = launch_dispatch(f.idx, T, f.k, E, S, ws.counts, ws.lists, ws.n_active, ws.active, ws.err,
                         grouped ? nullptr : f.xq, D, ws.xsum8, s);
    if (rc != hipSuccess) return rc;
  }
  const coli_moe_trace* tr = f.trace;
  if (grouped) {
    if ((rc = launch_mfma_front(t, f.xq, T, ws, s)) != hipSuccess) return rc;
    if ((rc = record(ev.gate_up, s)) != hipSuccess) return rc;
    rc = launch_mfma_ffn(t, f.xd, T, f.k, ws, tr, ev.down, s);
  }
  if (!grouped) {
  const int64_t maxA = (T * f.k < E ? T * f.k : E) + S;

  GuArgs g = {};
  g.gu_q = reinterpret_cast<const uint4*>(t.gu_q);
  g.gu_s = t.gu_s;
  g.xq = f.xq;
  g.xd = f.xd;
  g.xsum8 = ws.xsum8;
  g.counts = ws.counts;
  g.lists = ws.lists;
  g.n_active = ws.n_active;
  g.active = ws.active;
  g.hq = ws.hq;
  g.hd = ws.hd;
  g.hsum8 = ws.hsum8;
  g.hq_slot = ws.hq_slot;
  g.hd_slot = ws.hd_slot;
  g.hs_slot = ws.hs_slot;
  g.slot_of = t.slot_of;
  g.n_store = t.slot_of ? t.n_slots : E + S;
  g.err = ws.err;
  g.T = T;
  g.D = D;
  g.F = F;
  g.k = f.k;
  g.S = S;
  DnArgs d = {};
  d.dn_q = reinterpret_cast<const uint4*>(t.dn_q);
  d.dn_s = t.dn_s;
  d.hq = ws.hq;
  d.hd = ws.hd;
  d.hsum8 = ws.hsum8;
  d.hq_slot = ws.hq_slot;
  d.hd_slot = ws.hd_slot;
  d.hs_slot = ws.hs_slot;
  d.counts = ws.counts;
  d.lists = ws.lists;
  d.n_active = ws.n_active;
  d.active = ws.active;
  d.o = ws.o;
  d.slot_of = t.slot_of;
  d.n_store = t.slot_of ? t.n_slots : E + S;
  d.err = ws.err;
  d.T = T;
  d.D = D;
  d.F = F;
  d.k = f.k;
  d.S = S;
  d.E = E;
  const GemvEvents gev = {ev.gate_up, ev.down, ev.combine};
  if (tr) {
    g.tr_pg = tr->p_gate;
    g.tr_pu = tr->p_up;
    g.tr_g = tr->g;
    g.tr_u = tr->u;
    g.tr_h = tr->h;
    d.tr_pd = tr->p_down;
    rc = launch_gemv<true>(g, d, t.weight_bits, (int)maxA, T, gev, s);
  } else {
    rc = launch_gemv<false>(g, d, t.weight_bits, (int)maxA, T, gev, s);
  }
  }
  if (rc != hipSuccess) return rc;
  // the GEMV path attaches `combine` to the end of its down kernel
  if (grouped && (rc = record(ev.combine, s)) != hipSuccess) return rc;
  const dim3 cgrid((unsigned)((D / 4 + 255) / 256), (unsigned)T);
  if (f.k == 8)
    hipLaunchKernelGGL(combine_kernel<8>, cgrid, dim3(256), 0, s, ws.o, f.idx, f.w, D, f.k, E, S,
                       f.y, f.accumulate);
  else
    hipLaunchKernelGGL(combine_kernel<0>, cgrid, dim3(256), 0, s, ws.o, f.idx, f.w, D, f.k, E, S,
                       f.y, f.accumulate);
  rc = hipGetLastError();
  if (rc == hipSuccess) rc = record(ev.end, s);
  if (rc != hipSuccess || !tr) return rc;
  // test dumps of the dispatch and of the workspace intermediates
  const int64_t A = E + S, P = T * (f.k + S);
  struct Copy { void* dst; const void* src; size_t n; };
  const Copy copies[] = {
      {tr->counts, ws.counts, sizeof(int32_t) * A},
      {tr->lists, ws.lists, sizeof(int32_t) * A * T},
      {tr->n_active, ws.n_active, sizeof(int32_t)},
      {tr->active, ws.active, sizeof(int32_t) * A},
      {tr->hq, ws.hq, (size_t)(P * F)},
      {tr->hd, ws.hd, sizeof(float) * P * (F / 32)},
      {tr->o, ws.o, sizeof(float) * P * D},
      {f.dispatched ? tr->xq : nullptr, f.xq, (size_t)(T * D)},
      {f.dispatched ? tr->xd : nullptr, f.xd, sizeof(float) * T * (D / 32)},
      {f.dispatched ? tr->idx : nullptr, f.idx, sizeof(int32_t) * T * f.k},
      {f.dispatched ? tr->w : nullptr, f.w, sizeof(float) * T * f.k},
  };
  for (const Copy& c : copies) {
    if (!c.dst) continue;
    rc = hipMemcpyAsync(c.dst, c.src, c.n, hipMemcpyDeviceToDevice, s);
    if (rc != hipSuccess) return rc;
  }
  return hipSuccess;
}

}  // namespace coli
