/*
 * Oracle for the routed int4 MoE FFN with sigmoid top-k routing.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * CPU-baseline leg of the benchmark, never by the product path.  It shares
 * no code with the GPU library.
 *
 * What the method computes, and where the pages say so:
 *
 *  - Activations are quantised "Q8_0 style" to int8 and multiplied against
 *    quantised weights with an integer dot product (discuss.pytorch.kr,
 *    "colibri: 744B MoE ... 순수 C 추론 엔진", section "colibri의 주요 기능",
 *    integer-dot-kernel bullet; jeff.news "7440억 파라미터 GLM-5.2 ...",
 *    section on attention and kernels, integer matmul bullet).
 *  - Expert weights are int4, stored as U8-packed nibbles with a separate
 *    per-row F32 scale file, produced with np.rint so that they match the
 *    engine's lrintf rounding (aitrends.kr "GLM-5.2-colibri-int4", sections
 *    "TL;DR", "훈련 방식" and "기술적 특징").
 *  - Routing is DeepSeek-V3 style: sigmoid scores, top-k with a selection
 *    bias, plus an always-on shared expert (jeff.news, attention-and-kernels
 *    section, DeepSeek-style tricks bullet); 8 of 256 experts per token
 *    (discuss.pytorch.kr, "colibri의 핵심 아이디어"; jeff.news, disk
 *    bottleneck section: 75 layers x 8 experts).
 *  - Router and norm layers stay F32 (aitrends.kr, "알아두면 좋은 것").
 *  - Prefill and the batched verify pass group tokens by expert so that
 *    each selected expert is loaded once ("batch-union MoE", alphamatch.ai
 *    "Colibri: 25GB RAM만으로 ...", section "기술적 우수성").
 *
 * Readings where the pages are silent (each is the plainest one the rest
 * supports): Q8 blocks hold 32 values with an F32 scale max|x|/127; int4
 * rows use s = max|w|/7 and codes in [-7, 7]; int8 rows (the container of
 * the speculative head) use s = max|w|/127 and codes in [-127, 127], one
 * byte per column, through the same dot; the low nibble holds the even
 * column; the expert FFN is SwiGLU; the combine is shared + sum_j w_j o_j;
 * the hidden vector is re-quantised with Q8_0 before the down projection;
 * fp32 accumulation runs over blocks in ascending order with one fused
 * multiply-add per block; exp is a fixed fp32 algorithm (below) so that the
 * integer decisions it feeds are reproducible.
 */
#include "coli_oracle.h"

#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

/* Threads the OpenMP loops of this library use (reported with timings). */
int orc_num_threads(void) { return omp_get_max_threads(); }

/* Threads of the calling thread's later parallel regions (timing runs only). */
void orc_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }

/* ------------------------------------------------------------------------
 * exp(x) in fp32 (Cody & Waite, "Software Manual for the Elementary
 * Functions", 1980: argument reduction by n*ln2 with ln2 split in a high
 * part that has trailing zero bits and a low part).  x is clamped to
 * [-87, 88.5] so every result is a normal float; n = rint(x*log2(e));
 * r = x - n*ln2 with |r| <= ln2/2; e^r by its Taylor series to degree 7
 * (truncation < 6e-9, below half an ulp) in Horner form with fmaf; the
 * result is scaled by 2^n.
 */
float orc_expf(float x) {
  if (x > 88.5f) x = 88.5f;
  if (x < -87.0f) x = -87.0f;
  const float n = rintf(x * 1.44269504088896341f);
  float r = fmaf(-n, 0.693145751953125f, x);       /* ln2 high part, 16 bits */
  r = fmaf(-n, 1.42860676533018708e-06f, r);       /* ln2 - high part        */
  float p = 1.98412698412698413e-04f;              /* 1/7! */
  p = fmaf(p, r, 1.38888888888888889e-03f);        /* 1/6! */
  p = fmaf(p, r, 8.33333333333333333e-03f);        /* 1/5! */
  p = fmaf(p, r, 4.16666666666666667e-02f);        /* 1/4! */
  p = fmaf(p, r, 1.66666666666666667e-01f);        /* 1/3! */
  p = fmaf(p, r, 0.5f);                            /* 1/2! */
  p = fmaf(p, r, 1.0f);
  p = fmaf(p, r, 1.0f);
  return ldexpf(p, (int)n);
}

/* sigma(x) = 1 / (1 + e^-x): the sigmoid score of the router. */
float orc_sigmoidf(float x) { return 1.0f / (1.0f + orc_expf(-x)); }

/* silu(g) = g / (1 + e^-g): the SwiGLU gate activation. */
float orc_siluf(float g) { return g / (1.0f + orc_expf(-g)); }

void orc_expf_vec(const float* x, int64_t n, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_expf(x[i]);
}
void orc_sigmoidf_vec(const float* x, int64_t n, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_sigmoidf(x[i]);
}
void orc_siluf_vec(const float* x, int64_t n, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_siluf(x[i]);
}

/* ------------------------------------------------------------------------
 * Q8_0 activation quantisation, per block of 32: d = max|x| / 127 (fp32,
 * correctly rounded), q = lrintf(x / d) (round half to even, the rounding
 * the pages name for the int4 conversion), clamped to [-127, 127]; an
 * all-zero block gets d = 0 and q = 0.
 */
void orc_q8_quant(const float* x, int64_t n, int8_t* q, float* d) {
  for (int64_t b = 0; b < n / 32; ++b) {
    const float* xb = x + 32 * b;
    float amax = 0.0f;
    for (int j = 0; j < 32; ++j) {
      const float a = fabsf(xb[j]);
      if (a > amax) amax = a;
    }
    const float db = amax / 127.0f;
    d[b] = db;
    for (int j = 0; j < 32; ++j) {
      long v = 0;
      if (db != 0.0f) v = lrintf(xb[j] / db);
      if (v > 127) v = 127;
      if (v < -127) v = -127;
      q[32 * b + j] = (int8_t)v;
    }
  }
}

/* ------------------------------------------------------------------------
 * Per-row symmetric int4 (aitrends.kr "GLM-5.2-colibri-int4": per-row F32
 * scale, np.rint matching the engine's lrintf): s = max|w| / 7,
 * q = lrintf(w / s) clamped to [-7, 7]; an all-zero row gets s = 0, q = 0.
 */
void orc_q4_quant_row(const float* w, int64_t k, int8_t* q, float* s) {
  float amax = 0.0f;
  for (int64_t j = 0; j < k; ++j) {
    const float a = fabsf(w[j]);
    if (a > amax) amax = a;
  }
  const float sc = amax / 7.0f;
  *s = sc;
  for (int64_t j = 0; j < k; ++j) {
    long v = 0;
    if (sc != 0.0f) v = lrintf(w[j] / sc);
    if (v > 7) v = 7;
    if (v < -7) v = -7;
    q[j] = (int8_t)v;
  }
}

/* ------------------------------------------------------------------------
 * Per-row symmetric int2, the narrowest packing the pages name next to int8
 * and int4 (discuss.pytorch.kr, "colibri의 주요 기능", integer-dot bullet:
 * the int8/int4/int2 packings match the int8 container bit for bit).
 * Reading: the int4 rule with one level a side, s = max|w| / 1,
 * q = lrintf(w / s) clamped to [-1, 1]; packed four 2-bit two's-complement
 * fields per byte, the lowest bits holding the first column.  The container
 * decodes all four field values (-2 included), like the nibble one.
 */
void orc_q2_quant_row(const float* w, int64_t k, int8_t* q, float* s) {
  float amax = 0.0f;
  for (int64_t j = 0; j < k; ++j) {
    const float a = fabsf(w[j]);
    if (a > amax) amax = a;
  }
  const float s2 = amax / 1.0f;
  *s = s2;
  for (int64_t j = 0; j < k; ++j) {
    long v = 0;
    if (s2 != 0.0f) v = lrintf(w[j] / s2);
    if (v > 1) v = 1;
    if (v < -1) v = -1;
    q[j] = (int8_t)v;
  }
}

void orc_pack_q2(const int8_t* q, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n / 4; ++i) {
    uint8_t byte = 0;
    for (int j = 0; j < 4; ++j) byte |= (uint8_t)(((uint8_t)q[4 * i + j] & 3u) << (2 * j));
    out[i] = byte;
  }
}

/* Two's-complement 2-bit field f -> f - 4 if f >= 2. */
void orc_unpack_q2(const uint8_t* in, int64_t n, int8_t* q) {
  for (int64_t i = 0; i < n / 4; ++i)
    for (int j = 0; j < 4; ++j) {
      const int f = (in[i] >> (2 * j)) & 3;
      q[4 * i + j] = (int8_t)(f >= 2 ? f - 4 : f);
    }
}

void orc_q2_quant(const float* w, int64_t rows, int64_t k, uint8_t* packed, float* s) {
#pragma omp parallel
  {
    int8_t* q = (int8_t*)malloc((size_t)k);
#pragma omp for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
      orc_q2_quant_row(w + r * k, k, q, s + r);
      orc_pack_q2(q, k, packed + r * (k / 4));
    }
    free(q);
  }
}

/* Signed nibbles packed two per U8 byte, low nibble = even column. */
void orc_pack_q4(const int8_t* q, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n / 2; ++i)
    out[i] = (uint8_t)(((uint8_t)q[2 * i] & 0x0F) | (((uint8_t)q[2 * i + 1] & 0x0F) << 4));
}

/* Two's-complement nibble n -> n - 16 if n >= 8. */
void orc_unpack_q4(const uint8_t* in, int64_t n, int8_t* q) {
  for (int64_t i = 0; i < n / 2; ++i) {
    const int lo = in[i] & 0x0F, hi = in[i] >> 4;
    q[2 * i] = (int8_t)(lo >= 8 ? lo - 16 : lo);
    q[2 * i + 1] = (int8_t)(hi >= 8 ? hi - 16 : hi);
  }
}

void orc_q4_quant(const float* w, int64_t rows, int64_t k, uint8_t* packed, float* s) {
#pragma omp parallel
  {
    int8_t* q = (int8_t*)malloc((size_t)k);
#pragma omp for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
      orc_q4_quant_row(w + r * k, k, q, s + r);
      orc_pack_q4(q, k, packed + r * (k / 2));
    }
    free(q);
  }
}

/* ------------------------------------------------------------------------
 * Per-row symmetric int8, the container of the speculative-decoding head
 * (discuss.pytorch.kr, "colibri의 주요 기능": that head has to stay int8,
 * and the int8 container is what the packed forms are checked against;
 * jeff.news, MTP section).  Same rule as int4 with 127 levels a side:
 * s = max|w| / 127, q = lrintf(w / s) clamped to [-127, 127]; an all-zero
 * row gets s = 0, q = 0.  The container is rows x k int8 + rows f32 scales.
 */
void orc_q8w_quant_row(const float* w, int64_t k, int8_t* q, float* s) {
  float amax = 0.0f;
  for (int64_t j = 0; j < k; ++j) {
    const float a = fabsf(w[j]);
    if (a > amax) amax = a;
  }
  const float sw = amax / 127.0f;
  *s = sw;
  for (int64_t j = 0; j < k; ++j) {
    long v = 0;
    if (sw != 0.0f) v = lrintf(w[j] / sw);
    if (v > 127) v = 127;
    if (v < -127) v = -127;
    q[j] = (int8_t)v;
  }
}

void orc_q8w_quant(const float* w, int64_t rows, int64_t k, int8_t* q, float* s) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) orc_q8w_quant_row(w + r * k, k, q + r * k, s + r);
}

/* ------------------------------------------------------------------------
 * Sigmoid top-k routing (DeepSeek-V3 style, jeff.news attention-and-kernels
 * section).  Per token: s_e = sigma(logit_e); the selection score is
 * c_e = s_e + bias_e (the bias steers selection only); the k largest c are
 * taken, a tie going to the lower expert index, listed in descending c;
 * the routing weights are w_j = (s_idx_j / sum) * routed_scale where sum
 * adds the selected s in that order in fp32.
 */
void orc_route(const float* logits, const float* bias, int64_t T, int32_t E, int32_t k,
               float routed_scale, int32_t* idx, float* w) {
  float* s = (float*)malloc(sizeof(float) * (size_t)E);
  float* c = (float*)malloc(sizeof(float) * (size_t)E);
  char* taken = (char*)malloc((size_t)E);
  for (int64_t t = 0; t < T; ++t) {
    for (int32_t e = 0; e < E; ++e) {
      s[e] = orc_sigmoidf(logits[t * E + e]);
      c[e] = s[e] + bias[e];
      taken[e] = 0;
    }
    for (int32_t j = 0; j < k; ++j) {
      int32_t best = -1;
      for (int32_t e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || c[e] > c[best]) best = e;
      }
      taken[best] = 1;
      idx[t * k + j] = best;
    }
    float sum = 0.0f;
    for (int32_t j = 0; j < k; ++j) sum = sum + s[idx[t * k + j]];
    for (int32_t j = 0; j < k; ++j) w[t * k + j] = (s[idx[t * k + j]] / sum) * routed_scale;
  }
  free(s);
  free(c);
  free(taken);
}

/* ------------------------------------------------------------------------
 * Integer dot of one weight row with a Q8 vector, per block of 32:
 * P_b = sum_j q_w * q_x, exact in int32 (|P_b| <= 32*127*127).  bits = 4:
 * the row is the nibble container (k/2 bytes); bits = 8: the int8 container
 * (k bytes, one code per column); bits = 2: four 2-bit fields per byte
 * (k/4 bytes).
 */
void orc_row_partials(const uint8_t* wrow, int bits, const int8_t* xq, int64_t k, int32_t* P) {
  for (int64_t b = 0; b < k / 32; ++b) {
    int32_t acc = 0;
    if (bits == 8) {
      const int8_t* w8 = (const int8_t*)wrow + 32 * b;
      for (int j = 0; j < 32; ++j) acc += (int32_t)w8[j] * (int32_t)xq[32 * b + j];
      P[b] = acc;
      continue;
    }
    if (bits == 2) {
      for (int j = 0; j < 32; ++j) {
        const int f = (wrow[(32 * b + j) / 4] >> (2 * (j % 4))) & 3;
        acc += (f >= 2 ? f - 4 : f) * (int32_t)xq[32 * b + j];
      }
      P[b] = acc;
      continue;
    }
    for (int j = 0; j < 16; ++j) {
      const uint8_t byte = wrow[16 * b + j];
      const int lo = byte & 0x0F, hi = byte >> 4;
      const int w0 = lo >= 8 ? lo - 16 : lo, w1 = hi >= 8 ? hi - 16 : hi;
      acc += w0 * (int32_t)xq[32 * b + 2 * j] + w1 * (int32_t)xq[32 * b + 2 * j + 1];
    }
    P[b] = acc;
  }
}

/* Block rescale: acc = 0; acc = fmaf((float)P_b, d_b, acc) for b ascending;
 * the row result is acc * s (the row's F32 scale). */
float orc_rescale(const int32_t* P, const float* d, int64_t nb, float s) {
  float acc = 0.0f;
  for (int64_t b = 0; b < nb; ++b) acc = fmaf((float)P[b], d[b], acc);
  return acc * s;
}

/* y = W x for a weight matrix in either container (bits 4 or 8). */
void orc_matvec(const uint8_t* Wq, int bits, const float* Ws, int64_t rows, int64_t k,
                const int8_t* xq, const float* xd, float* y, int32_t* P, double* absterm) {
  const int64_t nb = k / 32;
#pragma omp parallel
  {
    int32_t* Pl = (int32_t*)malloc(sizeof(int32_t) * (size_t)nb);
#pragma omp for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
      orc_row_partials(Wq + r * (k * bits / 8), bits, xq, k, Pl);
      y[r] = orc_rescale(Pl, xd, nb, Ws[r]);
      if (P) memcpy(P + r * nb, Pl, sizeof(int32_t) * (size_t)nb);
      if (absterm) {
        double m = 0.0;
        for (int64_t b = 0; b < nb; ++b) m += fabs((double)Ws[r] * (double)xd[b] * (double)Pl[b]);
        absterm[r] = m;
      }
    }
    free(Pl);
  }
}

/* ------------------------------------------------------------------------
 * One SwiGLU expert: g = W_gate x, u = W_up x (both from the Q8 token),
 * h = silu(g) * u, (hq, hd) = Q8_0(h), o = W_down hq.
 */
void orc_expert(const uint8_t* gate_q, const float* gate_s, const uint8_t* up_q,
                const float* up_s, const uint8_t* down_q, const float* down_s, int bits,
                int64_t D, int64_t F, const int8_t* xq, const float* xd, float* g, float* u,
                float* h, int8_t* hq, float* hd, float* o, int32_t* P_gate, int32_t* P_up,
                int32_t* P_down, double* abs_down) {
  orc_matvec(gate_q, bits, gate_s, F, D, xq, xd, g, P_gate, NULL);
  orc_matvec(up_q, bits, up_s, F, D, xq, xd, u, P_up, NULL);
  for (int64_t r = 0; r < F; ++r) h[r] = orc_siluf(g[r]) * u[r];
  orc_q8_quant(h, F, hq, hd);
  orc_matvec(down_q, bits, down_s, D, F, hq, hd, o, P_down, abs_down);
}

/* ------------------------------------------------------------------------
 * Which routing entries a forward serves.  The router never selects an
 * expert twice for one token nor one outside [0, E), but the forward also
 * takes routings from its caller; the reading used on both sides: an entry
 * (t, j) is kept when 0 <= idx[t][j] < E and no earlier slot i < j of the
 * same token holds the same expert; a dropped entry is not listed for any
 * expert and contributes nothing to the token's output.  keep[t*k + j] = 1
 * for a kept entry, else 0; returns the number of dropped entries.
 */
int64_t orc_keep_entries(const int32_t* idx, int64_t T, int32_t k, int32_t E, uint8_t* keep) {
  int64_t dropped = 0;
  for (int64_t t = 0; t < T; ++t)
    for (int32_t j = 0; j < k; ++j) {
      const int32_t e = idx[t * k + j];
      int ok = e >= 0 && e < E;
      for (int32_t i = 0; i < j; ++i)
        if (idx[t * k + i] == e) ok = 0;
      keep[t * k + j] = (uint8_t)ok;
      dropped += !ok;
    }
  return dropped;
}

/* ------------------------------------------------------------------------
 * The MoE layer, token by token: y = o_shared (0 without a shared expert),
 * then y = fmaf(w_j, o_idx_j, y) for j = 0..k-1; out = y or out + y.
 * keep == NULL: every entry must be valid (else -1); otherwise the entries
 * with keep[t*k + j] == 0 are skipped (orc_keep_entries).
 */
int orc_moe_layer(const void* const* experts, int bits, int32_t E, int32_t S, int64_t D,
                  int64_t F, int64_t T, const int8_t* xq, const float* xd, const int32_t* idx,
                  const float* w, int32_t k, const uint8_t* keep, float* out, int accumulate,
                  double* absterm) {
  float* g = (float*)malloc(sizeof(float) * (size_t)F);
  float* u = (float*)malloc(sizeof(float) * (size_t)F);
  float* h = (float*)malloc(sizeof(float) * (size_t)F);
  int8_t* hq = (int8_t*)malloc((size_t)F);
  float* hd = (float*)malloc(sizeof(float) * (size_t)(F / 32));
  float* o = (float*)malloc(sizeof(float) * (size_t)D);
  float* y = (float*)malloc(sizeof(float) * (size_t)D);
  double* m = (double*)malloc(sizeof(double) * (size_t)D);
  double* my = (double*)malloc(sizeof(double) * (size_t)D);
  int rc = 0;
  for (int64_t t = 0; t < T && rc == 0; ++t) {
    const int8_t* xt = xq + t * D;
    const float* dt = xd + t * (D / 32);
    for (int64_t r = 0; r < D; ++r) { y[r] = 0.0f; my[r] = 0.0; }
    for (int32_t j = -S; j < k; ++j) {   /* j = -1: the shared expert first */
      if (j >= 0 && keep && !keep[t * k + j]) continue;
      const int32_t e = j < 0 ? E : idx[t * k + j];
      if (e < 0 || e >= E + S) { rc = -1; break; }
      const void* const* ex = experts + 6 * (int64_t)e;
      if (!ex[0] || !ex[1] || !ex[2] || !ex[3] || !ex[4] || !ex[5]) { rc = -1; break; }
      orc_expert((const uint8_t*)ex[0], (const float*)ex[1], (const uint8_t*)ex[2],
                 (const float*)ex[3], (const uint8_t*)ex[4], (const float*)ex[5], bits, D, F,
                 xt, dt, g, u, h, hq, hd, o, NULL, NULL, NULL, m);
      if (j < 0) {
        for (int64_t r = 0; r < D; ++r) { y[r] = o[r]; my[r] = m[r]; }
      } else {
        const float wj = w[t * k + j];
        for (int64_t r = 0; r < D; ++r) {
          y[r] = fmaf(wj, o[r], y[r]);
          my[r] += fabs((double)wj) * m[r];
        }
      }
    }
    for (int64_t r = 0; r < D; ++r) {
      out[t * D + r] = accumulate ? out[t * D + r] + y[r] : y[r];
      if (absterm) absterm[t * D + r] = my[r];
    }
  }
  free(g); free(u); free(h); free(hq); free(hd); free(o); free(y); free(m); free(my);
  return rc;
}

/* ------------------------------------------------------------------------
 * RMSNorm with unit gain (norm weights are F32 on the pages; the deep stack
 * uses gain 1): ss = sum h_i^2 in fp64 (each square exact), r =
 * (float)(1 / sqrt(ss / D + eps)) computed in fp64, out_i = h_i * r in fp32.
 */
void orc_rmsnorm(const float* h, int64_t T, int64_t D, float eps, float* out, float* r_out) {
  for (int64_t t = 0; t < T; ++t) {
    double ss = 0.0;
    for (int64_t i = 0; i < D; ++i) ss += (double)h[t * D + i] * (double)h[t * D + i];
    const float r = (float)(1.0 / sqrt(ss / (double)D + (double)eps));
    if (r_out) r_out[t] = r;
    for (int64_t i = 0; i < D; ++i) out[t * D + i] = h[t * D + i] * r;
  }
}

/* ------------------------------------------------------------------------
 * Router projection: the F32 router weight matrix applied to the hidden
 * state.  A product of two floats has at most 48 significant bits, so it is
 * exact in fp64; the sum runs in fp64 in ascending d and is rounded to fp32
 * once.
 */
void orc_router_logits(const float* x, const float* wr, int64_t T, int64_t D, int32_t E,
                       float* logits) {
#pragma omp parallel for schedule(static) if (T * (int64_t)E * D > (1 << 22))
  for (int64_t te = 0; te < T * (int64_t)E; ++te) {
    const int64_t t = te / E, e = te % E;
    double s = 0.0;
    for (int64_t d = 0; d < D; ++d) s += (double)wr[e * D + d] * (double)x[t * D + d];
    logits[te] = (float)s;
  }
}

/* ------------------------------------------------------------------------
 * Batch-union dispatch: the expert-major view of the routing so that each
 * selected expert's weights are read once per pass.
 */
int orc_dispatch(const int32_t* idx, int64_t T, int32_t k, int32_t E, int32_t S,
                 const uint8_t* keep, int32_t* counts, int32_t* lists, int32_t* n_active,
                 int32_t* active) {
  for (int32_t e = 0; e < E + S; ++e) counts[e] = 0;
  for (int64_t t = 0; t < T; ++t)
    for (int32_t j = 0; j < k; ++j) {
      if (keep && !keep[t * k + j]) continue;   /* a dropped entry is not listed */
      if (idx[t * k + j] < 0 || idx[t * k + j] >= E) return -1;
      for (int32_t i = 0; i < j; ++i)
        if (idx[t * k + i] == idx[t * k + j]) return -1;   /* top-k never repeats */
    }
  for (int32_t e = 0; e < E + S; ++e) {
    for (int64_t t = 0; t < T; ++t) {
      if (e == E) {
        lists[(int64_t)e * T + counts[e]++] = (int32_t)(t * (k + S) + k);
        continue;
      }
      for (int32_t j = 0; j < k; ++j)
        if (idx[t * k + j] == e && (!keep || keep[t * k + j]))
          lists[(int64_t)e * T + counts[e]++] = (int32_t)(t * (k + S) + j);
    }
  }
  int32_t na = 0;
  for (int32_t e = 0; e < E + S; ++e)
    if (counts[e] > 0) active[na++] = e;
  *n_active = na;
  return 0;
}

/* ------------------------------------------------------------------------
 * Expert tier of one layer.  The pages keep the routed experts out of the
 * fast memory and cache them per layer: an LRU cache per layer, a pinned
 * hot store for the most used experts, and a usage log from which the next
 * run pins the most frequently selected experts (discuss.pytorch.kr colibri
 * summary, "colibri의 핵심 아이디어"; jeff.news, the idea section).  Here
 * the fast memory is `slots` expert slots and the policy is, in full:
 *
 *  - init: the shared expert (S = 1) takes slot 0, then the pinned experts
 *    take slots 1, 2, ... in the order given; those slots are pinned and are
 *    never evicted; each of them is a load.  Other slots start empty.
 *  - plan (one per pass, `step` counting the plans of this layer): the
 *    needed set is every expert some token selected plus the shared expert.
 *    A needed expert already in a slot is a hit and that slot's stamp
 *    becomes `step`.  Then the missing experts, in ascending id, each take
 *    the unpinned slot not used by this pass (stamp < step) with the
 *    smallest stamp, the lower slot on equal stamps (empty slots have stamp
 *    -1, so they go first); the evicted expert leaves the tier; the slot is
 *    a load.  With count_usage, usage[e] grows by the number of tokens that
 *    selected e (the shared expert: every token).
 *  - pin_top: the n routed experts with the largest usage, the lower id on
 *    equal counts, in that order.
 *
 * Returns 0, or -1 (and changes nothing) if an index is invalid or the
 * missing experts do not fit in the unpinned slots the pass's hits leave.
 */
int orc_tier_init(int32_t E, int32_t S, int32_t slots, const int32_t* pin, int32_t n_pin,
                  int32_t* slot_of, int32_t* expert_in, int32_t* stamp, int32_t* pinned,
                  int32_t* usage, int32_t* loads, int32_t* n_loads) {
  if (S + n_pin > slots) return -1;
  for (int32_t e = 0; e < E + S; ++e) { slot_of[e] = -1; usage[e] = 0; }
  for (int32_t s = 0; s < slots; ++s) { expert_in[s] = -1; stamp[s] = -1; pinned[s] = 0; }
  int32_t n = 0;
  for (int32_t i = -S; i < n_pin; ++i) {
    const int32_t e = i < 0 ? E : pin[i];
    if (e < 0 || e >= E + S || slot_of[e] >= 0) return -1;
    slot_of[e] = n;
    expert_in[n] = e;
    pinned[n] = 1;
    loads[n] = n;
    ++n;
  }
  *n_loads = n;
  return 0;
}

int orc_tier_plan(int32_t E, int32_t S, int32_t slots, const int32_t* idx, int64_t T, int32_t k,
                  int32_t step, int count_usage, int32_t* slot_of, int32_t* expert_in,
                  int32_t* stamp, const int32_t* pinned, int32_t* usage, int32_t* loads,
                  int32_t* n_loads, int32_t* hits) {
  int32_t* count = (int32_t*)calloc((size_t)(E + S), sizeof(int32_t));
  int rc = 0;
  for (int64_t i = 0; i < T * k; ++i) {
    if (idx[i] < 0 || idx[i] >= E) { rc = -1; break; }
    count[idx[i]] += 1;
  }
  if (S) count[E] = (int32_t)T;
  if (rc == 0) {   /* the pass must fit: its misses in the unpinned slots its hits leave */
    int32_t miss = 0, hit_unpinned = 0, unpinned = 0;
    for (int32_t e = 0; e < E + S; ++e) {
      if (count[e] == 0) continue;
      if (slot_of[e] < 0) ++miss;
      else if (!pinned[slot_of[e]]) ++hit_unpinned;
    }
    for (int32_t s = 0; s < slots; ++s) unpinned += pinned[s] ? 0 : 1;
    if (miss > unpinned - hit_unpinned) rc = -1;
  }
  int32_t nh = 0, nl = 0;
  for (int32_t e = 0; e < E + S && rc == 0; ++e) {     /* hits */
    if (count[e] == 0 || slot_of[e] < 0) continue;
    stamp[slot_of[e]] = step;
    ++nh;
  }
  for (int32_t e = 0; e < E + S && rc == 0; ++e) {     /* misses, ascending id */
    if (count[e] == 0 || slot_of[e] >= 0) continue;
    int32_t v = -1;
    for (int32_t s = 0; s < slots; ++s) {
      if (pinned[s] || stamp[s] >= step) continue;
      if (v < 0 || stamp[s] < stamp[v]) v = s;
    }
    if (v < 0) { rc = -1; break; }
    if (expert_in[v] >= 0) slot_of[expert_in[v]] = -1;
    expert_in[v] = e;
    slot_of[e] = v;
    stamp[v] = step;
    loads[nl++] = v;
  }
  if (rc == 0 && count_usage)
    for (int32_t e = 0; e < E + S; ++e) usage[e] += count[e];
  *n_loads = nl;
  *hits = nh;
  free(count);
  return rc;
}

void orc_tier_pin_top(int32_t E, const int32_t* usage, int32_t n, int32_t* out) {
  char* taken = (char*)calloc((size_t)E, 1);
  for (int32_t i = 0; i < n && i < E; ++i) {
    int32_t best = -1;
    for (int32_t e = 0; e < E; ++e) {
      if (taken[e]) continue;
      if (best < 0 || usage[e] > usage[best]) best = e;
    }
    taken[best] = 1;
    out[i] = best;
  }
  free(taken);
}
