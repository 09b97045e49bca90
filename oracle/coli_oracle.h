/*
 * Oracle for the routed int4 MoE FFN with sigmoid top-k routing.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  The GPU library
 * shares no code, header, table or constant with it.
 *
 * Plain, slow, obviously-correct host C.  Every function computes the plain
 * per-token definition in the order written below; OpenMP only splits
 * independent output rows, so results do not depend on the thread count.
 * All pointers are host pointers owned by the caller.
 */
#ifndef COLI_ORACLE_H
#define COLI_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* OpenMP threads used by the parallel loops. */
int orc_num_threads(void);
void orc_set_threads(int n);

/* exp / sigmoid / silu in fp32 (Cody-Waite reduction + degree-7 Taylor). */
float orc_expf(float x);
float orc_sigmoidf(float x);
float orc_siluf(float g);
void orc_expf_vec(const float* x, int64_t n, float* out);
void orc_sigmoidf_vec(const float* x, int64_t n, float* out);
void orc_siluf_vec(const float* x, int64_t n, float* out);

/* Q8_0 activations: blocks of 32, d = max|x| / 127, q = lrintf(x / d). */
void orc_q8_quant(const float* x, int64_t n, int8_t* q, float* d);

/* per-row symmetric int4: s = max|w| / 7, q = lrintf(w / s) in [-7, 7]. */
void orc_q4_quant_row(const float* w, int64_t k, int8_t* q, float* s);
/* rows x k fp32 -> canonical container: rows x k/2 bytes + rows f32 scales. */
void orc_q4_quant(const float* w, int64_t rows, int64_t k, uint8_t* packed, float* s);

/* per-row symmetric int8 (the int8 container): s = max|w| / 127,
 * q = lrintf(w / s) in [-127, 127]; rows x k int8 + rows f32 scales. */
void orc_q8w_quant_row(const float* w, int64_t k, int8_t* q, float* s);
void orc_q8w_quant(const float* w, int64_t rows, int64_t k, int8_t* q, float* s);

/* per-row symmetric int2: s = max|w| / 1, q = lrintf(w / s) in [-1, 1];
 * 2-bit container: byte i = sum_j (q[4i+j] & 3) << 2j; decode maps field
 * f >= 2 to f - 4. */
void orc_q2_quant_row(const float* w, int64_t k, int8_t* q, float* s);
void orc_q2_quant(const float* w, int64_t rows, int64_t k, uint8_t* packed, float* s);
void orc_pack_q2(const int8_t* q, int64_t n, uint8_t* out);
void orc_unpack_q2(const uint8_t* in, int64_t n, int8_t* q);

/* nibble container: byte i = (q[2i] & 15) | (q[2i+1] & 15) << 4. */
void orc_pack_q4(const int8_t* q, int64_t n, uint8_t* out);
void orc_unpack_q4(const uint8_t* in, int64_t n, int8_t* q);

/* sigmoid top-k routing for T tokens.  idx[T][k] in descending selection
 * score, w[T][k] normalised over the selected set times routed_scale. */
void orc_route(const float* logits, const float* bias, int64_t T, int32_t E, int32_t k,
               float routed_scale, int32_t* idx, float* w);

/* Weight matrices come in one of three containers, named by `bits`: 4 = the
 * nibble container (k/2 bytes per row), 8 = the int8 container (k bytes per
 * row, one int8 code per column), 2 = the 2-bit container (k/4 bytes per
 * row).  Scales are one f32 per row in all three. */

/* int32 block partials of one weight row with a Q8 vector: P[k/32]. */
void orc_row_partials(const uint8_t* wrow, int bits, const int8_t* xq, int64_t k, int32_t* P);
/* acc = 0; for b ascending: acc = fmaf((float)P[b], d[b], acc); return acc * s. */
float orc_rescale(const int32_t* P, const float* d, int64_t nb, float s);
/* y[r] for every row of a weight matrix; P (rows x k/32) and absterm (fp64
 * sum over blocks of |s * d_b * P_b|) are optional (NULL to skip). */
void orc_matvec(const uint8_t* Wq, int bits, const float* Ws, int64_t rows, int64_t k,
                const int8_t* xq, const float* xd, float* y, int32_t* P, double* absterm);

/* One SwiGLU expert on one Q8 token.  Every output is required except the
 * optional partial/absterm dumps (NULL to skip). */
void orc_expert(const uint8_t* gate_q, const float* gate_s, const uint8_t* up_q,
                const float* up_s, const uint8_t* down_q, const float* down_s, int bits,
                int64_t D, int64_t F, const int8_t* xq, const float* xd, float* g, float* u,
                float* h, int8_t* hq, float* hd, float* o, int32_t* P_gate, int32_t* P_up,
                int32_t* P_down, double* abs_down);

/* The MoE layer for T tokens, every expert in the container `bits`.
 * experts[e*6 + m] holds, for expert e in
 * [0, E+S), the six container pointers gate_q, gate_s, up_q, up_s, down_q,
 * down_s (NULL rows are allowed for experts no token selects).  The shared
 * expert is index E.  out[T][D] = moe (accumulate = 0) or out + moe (1).
 * absterm[T][D] (optional) receives the fp64 sum of |terms| of each output.
 * keep[T][k] (optional): entries with keep == 0 are skipped (see
 * orc_keep_entries); without it every entry must be valid.
 * Returns 0, or -1 if a selected expert is missing / an index is invalid. */
int orc_moe_layer(const void* const* experts, int bits, int32_t E, int32_t S, int64_t D,
                  int64_t F, int64_t T, const int8_t* xq, const float* xd, const int32_t* idx,
                  const float* w, int32_t k, const uint8_t* keep, float* out, int accumulate,
                  double* absterm);

/* Entries a forward serves: (t, j) is kept when idx[t][j] is in [0, E) and no
 * earlier slot of token t holds the same expert.  keep[T][k] = 1 / 0; returns
 * the number of dropped entries. */
int64_t orc_keep_entries(const int32_t* idx, int64_t T, int32_t k, int32_t E, uint8_t* keep);

/* RMSNorm with unit gain: ss in fp64, r = (float)(1/sqrt(ss/D + eps)), out = h * r. */
void orc_rmsnorm(const float* h, int64_t T, int64_t D, float eps, float* out, float* r_out);

/* Router projection (jeff.news, attention-and-kernels section: the router is
 * part of the DeepSeek-V3-style MoE; aitrends.kr "알아두면 좋은 것": router
 * weights stay F32): logits[t][e] = sum_d wr[e][d] * x[t][d], each product
 * exact in fp64, summed in fp64 in ascending d, rounded once to fp32. */
void orc_router_logits(const float* x, const float* wr, int64_t T, int64_t D, int32_t E,
                       float* logits);

/* Batch-union dispatch.  For every expert e in [0, E+S): counts[e] and the
 * list lists[e*T .. e*T+counts[e]) of pair ids p = t*(k+S) + slot in
 * ascending token order (the shared expert E takes slot k of every token).
 * active[0..*n_active) lists the experts with counts > 0 in ascending id.
 * keep[T][k] (optional): only entries with keep == 1 are listed.
 * Returns 0, or -1 if a listed index is outside [0, E) or repeats within a
 * token. */
int orc_dispatch(const int32_t* idx, int64_t T, int32_t k, int32_t E, int32_t S,
                 const uint8_t* keep, int32_t* counts, int32_t* lists, int32_t* n_active,
                 int32_t* active);

/* Expert tier of one layer (per-layer LRU + pinned hot store + usage
 * counts; the full policy is stated in coli_oracle.c).  State arrays:
 * slot_of[E+S] (slot or -1), expert_in[slots] (expert or -1), stamp[slots]
 * (plan step of last use, -1 never), pinned[slots] (0/1), usage[E+S].
 * loads[] receives the slots to fill, in order.  Return 0 or -1. */
int orc_tier_init(int32_t E, int32_t S, int32_t slots, const int32_t* pin, int32_t n_pin,
                  int32_t* slot_of, int32_t* expert_in, int32_t* stamp, int32_t* pinned,
                  int32_t* usage, int32_t* loads, int32_t* n_loads);
int orc_tier_plan(int32_t E, int32_t S, int32_t slots, const int32_t* idx, int64_t T, int32_t k,
                  int32_t step, int count_usage, int32_t* slot_of, int32_t* expert_in,
                  int32_t* stamp, const int32_t* pinned, int32_t* usage, int32_t* loads,
                  int32_t* n_loads, int32_t* hits);
/* The n most used routed experts (ties to the lower id), in that order. */
void orc_tier_pin_top(int32_t E, const int32_t* usage, int32_t n, int32_t* out);

#ifdef __cplusplus
}
#endif
#endif
