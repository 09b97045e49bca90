/*
 * coli.h - C ABI of the MI355X (gfx950) routed int4 MoE FFN library.
 *
 * The method (colibri, as described on the discuss.pytorch.kr, jeff.news,
 * alphamatch.ai and aitrends.kr pages about it): a DeepSeek-V3-style sigmoid
 * top-k router with a selection bias picks k of E routed experts per token;
 * activations are quantised Q8_0 style to int8; every expert is a SwiGLU FFN
 * whose int4 weights (signed nibbles packed in U8, one F32 scale per row,
 * rounded with lrintf half-to-even) are multiplied against the int8
 * activations with an integer dot product; the expert outputs are combined
 * with the normalised routing weights plus one always-on shared expert;
 * tokens that share a pass are grouped by expert (batch union) so that each
 * selected expert's weights are read once.
 *
 * Conventions for every entry point:
 *  - Bulk arrays (f32 inputs of the quantisers, packed weights, table arrays,
 *    layer outputs y, workspace) must be 16-byte aligned, every other pointer
 *    4-byte aligned (torch allocations and their row slices are);
 *    misaligned pointers return COLI_E_INVAL.
 *  - Tensor pointers are DEVICE pointers (hipMalloc / torch CUDA tensors),
 *    owned by the caller; the library never allocates, frees or keeps them.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Work is enqueued asynchronously; nothing synchronises the host except
 *    coli_moe_status(), which is documented as synchronising.
 *  - Arguments are validated on the host before anything is enqueued; a
 *    failed check returns a negative coli_status and enqueues nothing.
 *    A failed launch returns COLI_E_HIP (see coli_last_hip_error()).
 *  - Row-major layouts; int64 sizes; all shapes in elements.
 *  - Results are a deterministic function of the inputs (bit-reproducible).
 *
 * Numerics (identical op order to the oracle, so integers, quantised values
 * and the fp32 decode outputs match it bit for bit):
 *  - Q8_0: per block of 32 values, d = max|x| / 127.0f (IEEE division),
 *    q = clamp(rint_half_even(x / d), -127, 127); d == 0 gives q = 0.
 *  - int4 rows: s = max|w| / 7.0f, q = clamp(rint_half_even(w / s), -7, 7).
 *  - Dot of a packed row with a Q8 vector: int32 block partials
 *    P_b = sum_32 q_w q_x; acc = 0; acc = fmaf((float)P_b, d_b, acc) for b
 *    ascending; y = acc * s_row.
 *  - exp is a fixed fp32 algorithm (Cody-Waite reduction by ln2 split into
 *    0.693145751953125 + 1.42860676533018708e-6, degree-7 Taylor in Horner
 *    form with fmaf, input clamped to [-87, 88.5]); sigmoid(x) =
 *    1 / (1 + exp(-x)); silu(g) = g / (1 + exp(-g)).
 */
#ifndef COLI_H
#define COLI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  COLI_OK = 0,
  COLI_E_INVAL = -1,     /* null pointer or out-of-range scalar argument      */
  COLI_E_SHAPE = -2,     /* a size is not a multiple the layout needs, or too big */
  COLI_E_WORKSPACE = -3, /* workspace smaller than coli_moe_workspace_bytes()  */
  COLI_E_DEVICE = -4,    /* the current device is not gfx950                   */
  COLI_E_HIP = -5,       /* a HIP runtime call failed                          */
  COLI_E_INDEX = -6,     /* an expert index was outside [0, E) or repeated     */
  COLI_E_TIER = -7       /* expert tier: a selected expert is not resident, or
                            a pass needs more experts than the tier's slots  */
} coli_status;

/* Limits of the library. */
#define COLI_MAX_EXPERTS 256 /* routed experts per layer                    */
#define COLI_MAX_TOPK 64     /* experts selected per token                  */
#define COLI_MAX_DIM 32768   /* d_model and d_ff of an expert table         */

/* ------------------------------------------------------------------------
 * Device-resident expert table of one MoE layer.
 *
 * The pages' container is row-major U8 nibbles plus a per-row F32 scale file
 * (aitrends.kr "GLM-5.2-colibri-int4", section "기술적 특징"); coli_quant_weight_q4
 * produces exactly that.  The table holds the same codes re-laid for the
 * gfx950 GEMV: every 64-lane wavefront load of 1 KB brings one 16-byte,
 * 32-column chunk of 64 different rows, so each lane owns one row and runs
 * its block accumulation in order without cross-lane traffic.
 *
 *   gu_q  [E+S][F/32][D/32][64][16] bytes.  Group g, block b, lane l holds
 *         columns 32b..32b+31 of gate row 32g+l (l < 32) or up row
 *         32g+l-32 (l >= 32).
 *   gu_s  [E+S][F/32][64] f32, the row scales in the same lane order.
 *   dn_q  [E+S][D/64][F/32][64][16] bytes.  Group g, block b, lane l holds
 *         columns 32b..32b+31 of down row 64g+l.
 *   dn_s  [E+S][D] f32.
 *
 * Within a 16-byte chunk, 32-bit word k (0..3) holds columns 8k..8k+7 of
 * the block: byte j (0..3) has column 8k+j in its low nibble and column
 * 8k+4+j in its high nibble; each nibble stores q + 8 (0..15).
 *
 * int8 tables (weight_bits = 8): the container of the int8 speculative head
 * (discuss.pytorch.kr colibri summary, "colibri의 주요 기능", MTP bullet:
 * that head must be int8; jeff.news, MTP section).  Codes are int8 in
 * [-127, 127] with the same per-row F32 scales and the same Q8_0 block dot.
 * A block of 32 columns is two 16-byte chunks, so the chunk index runs over
 * half-blocks:
 *   gu_q  [E+S][F/32][D/16][64][16], chunk c of lane l = columns
 *         16c..16c+15 of the lane's row (gate rows l < 32, up rows l >= 32);
 *   dn_q  [E+S][D/64][F/16][64][16];
 * byte j of a chunk is column 16c+j as a two's-complement int8.  gu_s and
 * dn_s are as above.  int8 tables run the GEMV kernels at every batch size.
 *
 * int2 tables (weight_bits = 2; same page, integer-dot bullet: int8, int4 and
 * int2 packings): codes in [-2, 1] (the quantiser produces [-1, 1]), a
 * 16-byte chunk holds 64 columns (two blocks), so d_ff % 64 == 0:
 *   gu_q  [E+S][F/32][D/64][64][16], dn_q  [E+S][D/64][F/64][64][16];
 * 32-bit word m of a chunk holds columns 16m..16m+15: byte j has, from the
 * lowest bits up, 2-bit fields for columns 16m+j, 16m+4+j, 16m+8+j and
 * 16m+12+j, each stored as q + 2.  The canonical int2 container is
 * [rows][k/4] bytes, byte i holding columns 4i..4i+3 from the lowest bits
 * up in two's complement.  int2 tables run the GEMV kernels.
 *
 * The shared expert (when S = 1) is index E.  E <= 256, S in {0, 1},
 * D % 64 == 0, F % 32 == 0 (int2: F % 64 == 0), D and F <= COLI_MAX_DIM,
 * weight_bits 2, 4 or 8.
 *
 * Expert tiers (see coli_tier_* below): with slot_of != NULL the four arrays
 * hold n_slots experts, and expert e lives at position slot_of[e] (a device
 * array [E+S]; -1 = not resident).  A forward that selects a non-resident
 * expert skips it and reports COLI_E_TIER through coli_moe_status().  With
 * slot_of == NULL (n_slots ignored) expert e lives at position e.
 */
typedef struct {
  int32_t n_routed;    /* E */
  int32_t n_shared;    /* S */
  int32_t d_model;     /* D */
  int32_t d_ff;        /* F */
  int32_t weight_bits; /* 4: nibble-packed int4; 8: int8; 2: 2-bit fields */
  uint8_t* gu_q;
  float* gu_s;
  uint8_t* dn_q;
  float* dn_s;
  int32_t n_slots;        /* experts the arrays hold when slot_of != NULL */
  const int32_t* slot_of; /* device [E+S] position of each expert, or NULL */
} coli_expert_table;

/* Sizes in bytes of the four table arrays for (E, S, D, F, weight_bits).
 * Returns the total, or 0 for an unsupported shape.  Output pointers may be
 * NULL. */
size_t coli_table_bytes(int32_t n_routed, int32_t n_shared, int64_t d_model, int64_t d_ff,
                        int32_t weight_bits, size_t* gu_q, size_t* gu_s, size_t* dn_q,
                        size_t* dn_s);

/* Copies one expert, given as the pages' canonical containers (device
 * pointers), into slot `expert` (0..E+S-1) of the table.  weight_bits 4:
 * gate_q, up_q [F][D/2] bytes with scales [F], down_q [D][F/2] with scales
 * [D]; low nibble = even column, two's complement.  weight_bits 8: gate_q,
 * up_q [F][D] int8 codes, down_q [D][F] int8 codes (pass them as bytes).
 * The codes are unchanged; only their placement (and the nibble encoding)
 * change (see above). */
int coli_table_set_expert(const coli_expert_table* table, int32_t expert, const uint8_t* gate_q,
                          const float* gate_s, const uint8_t* up_q, const float* up_s,
                          const uint8_t* down_q, const float* down_s, void* stream);

/* ------------------------------------------------------------------------
 * Q8_0 activation quantisation (discuss.pytorch.kr colibri summary, section
 * "colibri의 주요 기능": int8 activations, Q8_0 style; jeff.news, kernel
 * section).  x [rows][k] f32 -> q [rows][k] int8, d [rows][k/32] f32.
 * k % 32 == 0.  rows may be 0 (no work). */
int coli_quant_act_q8(const float* x, int64_t rows, int64_t k, int8_t* q, float* d, void* stream);

/* Per-row symmetric int4 quantisation into the pages' container
 * (aitrends.kr "GLM-5.2-colibri-int4": per-row F32 scale, np.rint/lrintf).
 * w [rows][k] f32 -> q [rows][k/2] bytes (low nibble = even column, two's
 * complement) and s [rows] f32.  k % 32 == 0. */
int coli_quant_weight_q4(const float* w, int64_t rows, int64_t k, uint8_t* q, float* s,
                         void* stream);

/* Per-row symmetric int8 quantisation into the int8 container of the
 * speculative head (discuss.pytorch.kr colibri summary, "colibri의 주요
 * 기능", MTP bullet): s = max|w| / 127.0f, q = clamp(rint_half_even(w / s),
 * -127, 127), an all-zero row gives s = 0 and q = 0.  w [rows][k] f32 ->
 * q [rows][k] int8 and s [rows] f32.  k % 32 == 0. */
int coli_quant_weight_q8(const float* w, int64_t rows, int64_t k, int8_t* q, float* s,
                         void* stream);

/* Per-row symmetric int2 into the 2-bit container (discuss.pytorch.kr colibri
 * summary, "colibri의 주요 기능", integer-dot bullet): s = max|w| / 1.0f,
 * q = clamp(rint_half_even(w / s), -1, 1), an all-zero row gives s = 0 and
 * q = 0.  w [rows][k] f32 -> q [rows][k/4] bytes (byte i: columns 4i..4i+3,
 * lowest bits first, two's complement) and s [rows] f32.  k % 32 == 0. */
int coli_quant_weight_q2(const float* w, int64_t rows, int64_t k, uint8_t* q, float* s,
                         void* stream);

/* Fused RMSNorm (unit gain) + Q8_0 of the normalised vector, for a pre-norm
 * residual stack (router and norm stay F32: aitrends.kr, "알아두면 좋은 것").
 * Per row: ss = sum h^2 accumulated in fp64, r = (float)(1/sqrt(ss/D + eps))
 * in fp64, xhat = h * r in fp32, then Q8_0 of xhat.  h [T][D] f32 -> q [T][D],
 * d [T][D/32]; r_out [T] (may be NULL) receives r.  D % 32 == 0, eps >= 0. */
int coli_rmsnorm_q8(const float* h, int64_t T, int64_t D, float eps, int8_t* q, float* d,
                    float* r_out, void* stream);

/* ------------------------------------------------------------------------
 * Sigmoid top-k routing, DeepSeek-V3 style (jeff.news, attention-and-kernels
 * section; 8 of 256 experts per token).  Per token: s_e = sigmoid(logit_e);
 * selection score c_e = s_e + bias_e; the k largest c are chosen, a tie
 * going to the lower expert index, and listed in descending c; weights
 * w_j = (s_j / sum) * routed_scale with sum the fp32 sum of the selected s
 * in that order.  logits [T][E] f32, bias [E] f32 (NULL = no bias) ->
 * idx [T][k] int32, w [T][k] f32.  1 <= E <= 256, 1 <= k <= min(E, 64). */
int coli_route_topk(const float* logits, const float* bias, int64_t T, int32_t E, int32_t k,
                    float routed_scale, int32_t* idx, float* w, void* stream);

/* Router projection: the logits of coli_route_topk from the hidden state and
 * the F32 router weights (the router is the DeepSeek-V3-style gate of
 * jeff.news, attention-and-kernels section; its weights stay F32, aitrends.kr
 * "알아두면 좋은 것").  logits[t][e] = sum_d wr[e][d] * x[t][d]: each product
 * exact in fp64, summed in fp64, rounded to fp32 once (the summation order
 * inside fp64 is the kernel's; it changes the fp32 result only when the fp64
 * sum lies within ~2^-29 relative of a rounding boundary).
 * x [T][D] f32, wr [E][D] f32 (caller-owned device buffers, 16-byte aligned)
 * -> logits [T][E] f32.  D % 64 == 0, 1 <= E <= 256.  Errors: COLI_E_SHAPE,
 * COLI_E_INVAL (null or misaligned pointer), COLI_E_DEVICE, COLI_E_HIP. */
int coli_router_logits(const float* x, const float* wr, int64_t T, int64_t D, int32_t E,
                       float* logits, void* stream);

/* ------------------------------------------------------------------------
 * Batch-union dispatch (alphamatch.ai page, "기술적 우수성": prefill groups
 * tokens by expert; discuss.pytorch.kr: the batched verify pass).  From
 * idx [T][k] builds, for every expert e in [0, E+S): counts[e] and
 * lists[e][0..counts[e]) (row stride T) of pair ids p = t*(k+S) + slot in
 * ascending token order, the shared expert E taking slot k of every token;
 * active[0..*n_active) = experts with counts > 0, ascending.  Indices outside
 * [0, E) or repeated within a token are dropped and set *err to COLI_E_INDEX
 * (else *err = 0).  counts [E+S], lists [E+S][T], n_active [1],
 * active [E+S], err [1]: int32 device arrays. */
int coli_dispatch(const int32_t* idx, int64_t T, int32_t k, int32_t E, int32_t S,
                  int32_t* counts, int32_t* lists, int32_t* n_active, int32_t* active,
                  int32_t* err, void* stream);

/* ------------------------------------------------------------------------
 * The MoE FFN forward over a device-resident table: the expert matmuls as
 * integer dots of int8 (Q8_0) activations with the packed weights
 * (discuss.pytorch.kr colibri summary, "colibri의 주요 기능", integer-dot
 * bullet; jeff.news, attention-and-kernels section: DeepSeek-V3-style MoE
 * with a shared expert; aitrends.kr "GLM-5.2-colibri-int4", "기술적 특징":
 * U8-packed int4 with per-row F32 scales), with the tokens grouped per
 * expert so that each selected expert's rows are read once per pass
 * (alphamatch.ai, "기술적 우수성").
 *   xq [T][D] int8, xd [T][D/32] f32: the Q8_0 tokens.
 *   idx [T][k] int32, w [T][k] f32: the routing (coli_route_topk).
 *   y [T][D] f32: y = moe (accumulate = 0) or y + moe (accumulate = 1), with
 *   moe = o_shared + sum_j w_j o_idx_j accumulated as y = fmaf(w_j, o_j, y)
 *   in slot order after the shared expert.
 * Each expert: g = W_gate x, u = W_up x, h = silu(g) u, (hq, hd) = Q8_0(h),
 * o = W_down hq.  The workspace (caller-owned, device memory) must hold
 * coli_moe_workspace_bytes(table, T, k) bytes; its contents need no
 * initialisation and are clobbered.  Calls that share a workspace must not
 * overlap.  Routings from the caller may hold invalid entries: an entry
 * outside [0, E), or one equal to an earlier slot of the same token, is
 * dropped (listed for no expert; its slot contributes nothing to y, and the
 * remaining slots keep their order), coli_moe_status() reports COLI_E_INDEX,
 * and nothing faults.  coli_route_topk never produces such entries. */
size_t coli_moe_workspace_bytes(const coli_expert_table* table, int64_t T, int32_t k);

int coli_moe_forward(const coli_expert_table* table, const int8_t* xq, const float* xd,
                     int64_t T, const int32_t* idx, const float* w, int32_t k, float* y,
                     int accumulate, void* workspace, size_t ws_bytes, void* stream);

/* Per-shape path choice (jeff.news, kernel section: the pages' int4 kernel
 * wins in batch and loses to f32 for a single row, so the engine picks the
 * kernel by shape).  Two exact paths compute every forward bit-identically:
 *   COLI_PATH_GEMV     wavefront-per-row-group GEMV, 1-8 tokens per weight
 *                      pass; any table.
 *   COLI_PATH_GROUPED  grouped matrix-core GEMM over chunks of <= 128
 *                      tokens per expert; resident int4 tables only.
 *   COLI_PATH_AUTO     GROUPED from the measured crossover in tokens per
 *                      pass (COLI_GROUPED_MIN_TOKENS: at d_model 6144,
 *                      d_ff 2048, 256 + 1 experts, top-8 the GEMV wins at 4
 *                      tokens, the grouped path from 5, where the GEMV
 *                      moves to its 8-token kernel), GEMV below it and
 *                      wherever GROUPED does not apply.
 * (An f32-weight path would move 8x the bytes of an HBM-bound GEMV, so it
 * is never the faster one here.) */
#define COLI_PATH_AUTO 0
#define COLI_PATH_GEMV 1
#define COLI_PATH_GROUPED 2
#define COLI_GROUPED_MIN_TOKENS 5

/* coli_moe_forward on the given path.  COLI_PATH_GROUPED on a table it does
 * not apply to returns COLI_E_SHAPE. */
int coli_moe_forward_path(const coli_expert_table* table, const int8_t* xq, const float* xd,
                          int64_t T, const int32_t* idx, const float* w, int32_t k, float* y,
                          int accumulate, void* workspace, size_t ws_bytes, int32_t path,
                          void* stream);

/* Host-only: the path COLI_PATH_AUTO takes for (table, T, k): COLI_PATH_GEMV
 * or COLI_PATH_GROUPED (or a negative status for invalid arguments). */
int coli_moe_path(const coli_expert_table* table, int64_t T, int32_t k);

/* Intermediate dumps for testing; every pointer may be NULL (not written).
 * Pair p = t*(k+S) + slot indexes per-(token, slot) arrays; pairs with an
 * invalid index are left unwritten. */
typedef struct {
  int32_t* counts;   /* [E+S]                    dispatch counts      */
  int32_t* lists;    /* [E+S][T]                 dispatch lists       */
  int32_t* n_active; /* [1]                                            */
  int32_t* active;   /* [E+S]                                          */
  int32_t* p_gate;   /* [T*(k+S)][F][D/32]       int32 block partials */
  int32_t* p_up;     /* [T*(k+S)][F][D/32]                             */
  int32_t* p_down;   /* [T*(k+S)][D][F/32]                             */
  float* g;          /* [T*(k+S)][F]                                   */
  float* u;          /* [T*(k+S)][F]                                   */
  float* h;          /* [T*(k+S)][F]                                   */
  int8_t* hq;        /* [T*(k+S)][F]                                   */
  float* hd;         /* [T*(k+S)][F/32]                                */
  float* o;          /* [T*(k+S)][D]             expert outputs       */
  /* coli_moe_layer only: its own front-end results                        */
  int8_t* xq;        /* [T][D]                   Q8_0 codes of x      */
  float* xd;         /* [T][D/32]                Q8_0 scales of x     */
  int32_t* idx;      /* [T][k]                   routing              */
  float* w;          /* [T][k]                                         */
} coli_moe_trace;

int coli_moe_forward_traced(const coli_expert_table* table, const int8_t* xq, const float* xd,
                            int64_t T, const int32_t* idx, const float* w, int32_t k, float* y,
                            int accumulate, void* workspace, size_t ws_bytes,
                            const coli_moe_trace* trace, void* stream);

/* Stage timing: hipEvent_t handles (created by the caller with timing
 * enabled, passed as void*) that the forward records on `stream`.  Any may
 * be NULL.  Used by the benchmark to time the dominant kernel.  On the
 * GEMV path (decode / verify) gate_up, down and combine are attached to the
 * GEMV kernels' own dispatches (hipExtLaunchKernel start / stop events), so
 * gate_up..down is the gate/up kernel's execution time; on the grouped path
 * they are markers between the kernels.  Not for use under stream capture
 * (a captured record expresses a dependency only). */
typedef struct {
  void* begin;   /* before the dispatch kernels (coli_moe_layer*: before
                    the front end: quantisation, routing, dispatch)     */
  void* gate_up; /* GEMV: start of the gate/up kernel; grouped: before
                    the gate/up kernel                                   */
  void* down;    /* GEMV: end of the gate/up kernel; grouped: between
                    the gate/up and down kernels                         */
  void* combine; /* GEMV: end of the down kernel; grouped: before the
                    weighted combine                                     */
  void* end;     /* after the weighted combine                         */
} coli_moe_events;

int coli_moe_forward_profiled(const coli_expert_table* table, const int8_t* xq, const float* xd,
                              int64_t T, const int32_t* idx, const float* w, int32_t k, float* y,
                              int accumulate, void* workspace, size_t ws_bytes,
                              const coli_moe_events* events, void* stream);

/* ------------------------------------------------------------------------
 * The whole layer in one call, from f32 activations and router logits (the
 * routed MoE FFN of jeff.news, attention-and-kernels section: sigmoid router
 * with a selection bias, shared + routed experts; the integer-dot expert
 * matmuls of discuss.pytorch.kr, "colibri의 주요 기능"):
 * Q8_0 of x (coli_quant_act_q8), routing (coli_route_topk, bias may be NULL),
 * then coli_moe_forward, with the same numerics as those calls.  For small
 * batches (T <= 64 and T*k <= 1024: decode and speculative verify) the
 * quantisation, routing and dispatch run fused in one single-workgroup
 * kernel, so a decode step is 4 kernels.  The workspace must hold
 * coli_moe_layer_workspace_bytes(table, T, k) bytes (no initialisation;
 * clobbered; calls sharing it must not overlap).  _ex additionally takes the
 * optional trace and stage events of the forward (both may be NULL; events
 * are not for use under stream capture). */
size_t coli_moe_layer_workspace_bytes(const coli_expert_table* table, int64_t T, int32_t k);

int coli_moe_layer(const coli_expert_table* table, const float* x, const float* logits,
                   const float* bias, int64_t T, int32_t k, float routed_scale, float* y,
                   int accumulate, void* workspace, size_t ws_bytes, void* stream);

int coli_moe_layer_ex(const coli_expert_table* table, const float* x, const float* logits,
                      const float* bias, int64_t T, int32_t k, float routed_scale, float* y,
                      int accumulate, void* workspace, size_t ws_bytes,
                      const coli_moe_trace* trace, const coli_moe_events* events, void* stream);

/* One pre-norm residual MoE block in place: h <- h + MoE(RMSNorm(h)), the
 * layer form of a deep decode stack (router and norm stay F32: aitrends.kr,
 * "알아두면 좋은 것"; shared expert and routed experts combined as in
 * coli_moe_forward).  RMSNorm has unit gain and the arithmetic of
 * coli_rmsnorm_q8; routing, forward and combine are those of coli_moe_layer
 * with accumulate = 1, so the result is bit-identical to coli_rmsnorm_q8 +
 * coli_route_topk + coli_moe_forward(accumulate = 1).  For small batches
 * (T <= 64 and T*k <= 1024) the RMSNorm + Q8_0, routing and dispatch run in
 * one kernel, so a decode block is 4 kernels.  h [T][D] f32 (device, 16-byte
 * aligned), read and overwritten; logits [T][E] f32; bias [E] f32 or NULL;
 * eps finite and >= 0.  The workspace is coli_moe_layer's
 * (coli_moe_layer_workspace_bytes(table, T, k) bytes, clobbered, calls
 * sharing it must not overlap).  Argument errors return before any launch;
 * index errors are reported by coli_moe_status. */
int coli_moe_block(const coli_expert_table* table, float* h, const float* logits,
                   const float* bias, int64_t T, int32_t k, float routed_scale, float eps,
                   void* workspace, size_t ws_bytes, void* stream);

/* coli_moe_layer for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments without the workspace, the same result bit for bit.
 * The workspace is a file-scope device array of COLI_NOALLOC_BYTES
 * (64 MiB) that each GPU the library runs on holds until the process ends;
 * the call allocates and frees nothing.  A call needing more than that
 * (coli_moe_layer_workspace_bytes(table, T, k) > COLI_NOALLOC_BYTES; at
 * d_model 6144, d_ff 2048, top-8 with a shared expert: above 222 tokens)
 * returns COLI_E_WORKSPACE before any launch.  Resident tables only
 * (slot_of == NULL, else COLI_E_INVAL): with the routing inside the call no
 * index error can arise, so no status needs reading back.  Every call on one
 * GPU uses the same array: calls on one stream are ordered, but calls that
 * overlap on one GPU (other streams, other threads) race. */
#define COLI_NOALLOC_BYTES 67108864 /* 64 MiB */
int coli_moe_layer_noalloc(const coli_expert_table* table, const float* x, const float* logits,
                           const float* bias, int64_t T, int32_t k, float routed_scale, float* y,
                           int accumulate, void* stream);

/* Synchronises `stream`, then reports the device-side checks of the last
 * forward or layer call that used `workspace`: COLI_OK, COLI_E_INDEX or
 * COLI_E_TIER. */
int coli_moe_status(const void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Expert tier: an HBM cache of one layer's experts over a store in host
 * memory.  The pages keep the routed experts out of fast memory and cache
 * them per layer with an LRU, a pinned hot store, and pins learned from a
 * usage log (discuss.pytorch.kr colibri summary, "colibri의 핵심 아이디어";
 * jeff.news, idea section; pulmap.app, "쓸수록 빨라지는 캐시": usage-learned
 * pinning and next-layer readahead).  Here the fast memory is n_slots
 * expert slots in HBM, the store is the layer's E+S experts in pinned host
 * memory, and everything runs on the device: no host round trip per pass.
 *
 * Policy (deterministic):
 *  - coli_tier_init: the shared expert takes slot 0, then the pinned experts
 *    slots 1, 2, ... in the order given; those slots are never evicted; each
 *    is a load.  The plan step counter starts at 0.
 *  - coli_tier_plan (once per pass, before the forward): the needed set is
 *    every selected expert plus the shared one.  Resident needed experts are
 *    hits (their slot's stamp becomes the current step); then the missing
 *    ones, in ascending id, each take the unpinned slot not used by this
 *    pass with the smallest stamp (the lower slot on equal stamps; empty
 *    slots have stamp -1); the evicted expert leaves the tier.  With
 *    count_usage, usage[e] grows by the tokens that selected e (the shared
 *    expert: all T).  A prefetch is a plan with count_usage = 0 on the
 *    predicted selection.  If the needed set does not fit, the plan changes
 *    nothing and sets the error flag (coli_tier_status: COLI_E_TIER).
 *  - coli_tier_fetch copies every slot of the load list from the store.
 *
 * State (device arrays, caller-owned, int32):
 */
typedef struct {
  int32_t* slot_of;   /* [E+S] slot of expert e, or -1                     */
  int32_t* expert_in; /* [slots] expert in slot s, or -1                   */
  int32_t* stamp;     /* [slots] plan step of the slot's last use, -1 never */
  int32_t* pinned;    /* [slots] 1 = pinned                                */
  int32_t* usage;     /* [E+S] selections counted                          */
  int32_t* loads;     /* [1 + slots]: count, then the slots to fill         */
  int32_t* counters;  /* [4]: plan steps, hits, loads, error flag          */
} coli_tier_state;

/* Sizes in bytes of the four arrays of a table holding `slots` experts.
 * Returns the total, or 0 for an unsupported shape. */
size_t coli_tier_table_bytes(int32_t slots, int64_t d_model, int64_t d_ff, int32_t weight_bits,
                             size_t* gu_q, size_t* gu_s, size_t* dn_q, size_t* dn_s);

/* Resets the state of `tier` (a table with slot_of == state->slot_of and
 * n_slots slots) and fills the shared and pinned slots from `store` (as
 * coli_tier_fetch).  pin: host array of n_pin distinct routed experts.
 * Requires S + n_pin <= n_slots. */
int coli_tier_init(const coli_expert_table* tier, const coli_tier_state* state,
                   const int32_t* pin, int32_t n_pin, const coli_expert_table* store,
                   void* stream);

/* One pass's plan from the routing idx [T][k] (device, int32). */
int coli_tier_plan(const coli_expert_table* tier, const coli_tier_state* state,
                   const int32_t* idx, int64_t T, int32_t k, int32_t count_usage,
                   void* stream);

/* Fills the slots of the load list from `store`: a table (slot_of NULL) of
 * the same E, S, D, F and weight_bits whose arrays are pinned host memory
 * (hipHostMalloc) or device memory.  The copy is a kernel that reads the
 * store through its device mapping, so it is stream-ordered and needs no
 * host synchronisation; run it on a second stream to overlap the next
 * layer's fetch with this layer's forward. */
int coli_tier_fetch(const coli_expert_table* tier, const coli_tier_state* state,
                    const coli_expert_table* store, void* stream);

/* Synchronises `stream`, then reports the tier's error flag: COLI_OK or
 * COLI_E_TIER (a pass needed more experts than the slots, or an index was
 * invalid). */
int coli_tier_status(const coli_tier_state* state, void* stream);

/* Host-only: the n routed experts with the largest usage (ties to the lower
 * id), in that order, for pinning on the next run.  usage: host [E]. */
int coli_tier_rank(const int32_t* usage, int32_t E, int32_t n, int32_t* out);

/* ------------------------------------------------------------------------ */
const char* coli_status_string(int status);
/* hipError_t of the most recent COLI_E_HIP on the calling thread. */
int coli_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif
