// C ABI of the gfx950 routed int4 MoE library: argument validation on the
// host (before anything is enqueued), device check, workspace layout and the
// calls into the kernel launchers.  No entry point allocates memory.
#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>

#include "coli_internal.h"

namespace {

thread_local int g_last_hip_error = 0;

int hip_fail(hipError_t e) {
  g_last_hip_error = (int)e;
  return COLI_E_HIP;
}

// Per-device memo of the architecture check: 0 unknown, 1 gfx950, 2 other.
std::atomic<int> g_device_ok[64];

int check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return COLI_E_DEVICE;
  }
  if (dev < 0 || dev >= 64) return COLI_E_DEVICE;
  int st = g_device_ok[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) {
      g_last_hip_error = (int)e;
      return COLI_E_DEVICE;
    }
    st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_device_ok[dev].store(st, std::memory_order_relaxed);
  }
  return st == 1 ? COLI_OK : COLI_E_DEVICE;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// The kernels use 16-byte vector accesses on bulk arrays and 4-byte scalar
// loads elsewhere; misaligned pointers are rejected instead of faulting.
bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
bool al4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3) == 0; }

int table_check(const coli_expert_table* t) {
  if (!t) return COLI_E_INVAL;
  if (t->n_routed < 1 || t->n_routed > COLI_MAX_EXPERTS) return COLI_E_SHAPE;
  if (t->n_shared < 0 || t->n_shared > 1) return COLI_E_SHAPE;
  if (t->d_model <= 0 || t->d_model % 64 != 0 || t->d_ff <= 0 || t->d_ff % 32 != 0)
    return COLI_E_SHAPE;
  if (t->d_model > COLI_MAX_DIM || t->d_ff > COLI_MAX_DIM) return COLI_E_SHAPE;
  if (t->weight_bits != 2 && t->weight_bits != 4 && t->weight_bits != 8) return COLI_E_SHAPE;
  if (t->weight_bits == 2 && t->d_ff % 64) return COLI_E_SHAPE;   // int2 chunks: 64 columns
  if (t->slot_of && (t->n_slots < 1 || t->n_slots > t->n_routed + t->n_shared))
    return COLI_E_SHAPE;
  if (t->slot_of && !al4(t->slot_of)) return COLI_E_INVAL;
  if (!t->gu_q || !t->gu_s || !t->dn_q || !t->dn_s) return COLI_E_INVAL;
  if (!al16(t->gu_q) || !al16(t->dn_q) || !al4(t->gu_s) || !al4(t->dn_s)) return COLI_E_INVAL;
  return COLI_OK;
}

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }


}  // namespace

namespace coli {

MoeWorkspace moe_workspace_layout(void* base, int E, int S, int64_t D, int64_t F, int64_t T,
                                  int k) {
  MoeWorkspace w = {};
  char* p = static_cast<char*>(base);
  size_t off = 0;
  auto take = [&](size_t bytes) -> void* {
    void* r = p ? p + off : nullptr;
    off += align256(bytes);
    return r;
  };
  const size_t A = (size_t)(E + S), P = (size_t)T * (size_t)(k + S);
  w.err = static_cast<int32_t*>(take(sizeof(int32_t)));   // first: coli_moe_status reads it
  w.n_active = static_cast<int32_t*>(take(sizeof(int32_t)));
  w.counts = static_cast<int32_t*>(take(sizeof(int32_t) * A));
  w.active = static_cast<int32_t*>(take(sizeof(int32_t) * A));
  w.lists = static_cast<int32_t*>(take(sizeof(int32_t) * A * (size_t)T));
  w.xsum8 = static_cast<int32_t*>(take(sizeof(int32_t) * (size_t)T * (size_t)(D / 32)));
  w.hq = static_cast<int8_t*>(take(P * (size_t)F));
  w.hd = static_cast<float*>(take(sizeof(float) * P * (size_t)(F / 32)));
  w.hsum8 = static_cast<int32_t*>(take(sizeof(int32_t) * P * (size_t)(F / 32)));
  w.o = static_cast<float*>(take(sizeof(float) * P * (size_t)D));
  if (T == 1) {
    w.hq_slot = static_cast<int8_t*>(take(A * (size_t)F));
    w.hd_slot = static_cast<float*>(take(sizeof(float) * A * (size_t)(F / 32)));
    w.hs_slot = static_cast<int32_t*>(take(sizeof(int32_t) * A * (size_t)(F / 32)));
  }
  const size_t chunks = (size_t)mfma_max_chunks(T, k, E, S);
  w.xh = static_cast<uint16_t*>(take(2 * (size_t)T * (size_t)D));
  w.h16 = static_cast<uint16_t*>(take(2 * P * (size_t)F));
  w.xbias = reinterpret_cast<float*>(w.xsum8);
  w.hbias = reinterpret_cast<float*>(w.hsum8);
  w.chunks = static_cast<int32_t*>(take(8 * chunks));
  w.n_chunks = static_cast<int32_t*>(take(sizeof(int32_t)));
  w.bytes = off;
  return w;
}

}  // namespace coli

extern "C" {

const char* coli_status_string(int status) {
  switch (status) {
    case COLI_OK: return "ok";
    case COLI_E_INVAL: return "invalid argument (null pointer or scalar out of range)";
    case COLI_E_SHAPE: return "unsupported shape";
    case COLI_E_WORKSPACE: return "workspace too small";
    case COLI_E_DEVICE: return "current device is not gfx950 (or no device)";
    case COLI_E_HIP: return "HIP runtime error";
    case COLI_E_INDEX: return "expert index out of range or repeated within a token";
    case COLI_E_TIER: return "expert tier: expert not resident, or a pass needs more slots";
    default: return "unknown status";
  }
}

int coli_last_hip_error(void) { return g_last_hip_error; }

size_t coli_table_bytes(int32_t E, int32_t S, int64_t D, int64_t F, int32_t bits, size_t* gu_q,
                        size_t* gu_s, size_t* dn_q, size_t* dn_s) {
  if (E < 1 || E > COLI_MAX_EXPERTS || S < 0 || S > 1 || D <= 0 || D % 64 || F <= 0 || F % 32 ||
      D > COLI_MAX_DIM || F > COLI_MAX_DIM || (bits != 2 && bits != 4 && bits != 8) ||
      (bits == 2 && F % 64))
    return 0;
  const size_t n = (size_t)(E + S);
  const size_t a = n * (size_t)(D * F * bits / 4), b = n * (size_t)(2 * F) * sizeof(float),
               c = n * (size_t)(D * F * bits / 8), d = n * (size_t)D * sizeof(float);
  if (gu_q) *gu_q = a;
  if (gu_s) *gu_s = b;
  if (dn_q) *dn_q = c;
  if (dn_s) *dn_s = d;
  return a + b + c + d;
}

int coli_table_set_expert(const coli_expert_table* table, int32_t expert, const uint8_t* gate_q,
                          const float* gate_s, const uint8_t* up_q, const float* up_s,
                          const uint8_t* down_q, const float* down_s, void* stream) {
  int rc = table_check(table);
  if (rc) return rc;
  if (expert < 0 || expert >= table->n_routed + table->n_shared) return COLI_E_INVAL;
  if (!gate_q || !gate_s || !up_q || !up_s || !down_q || !down_s) return COLI_E_INVAL;
  if (!al16(gate_q) || !al16(up_q) || !al16(down_q) || !al4(gate_s) || !al4(up_s) ||
      !al4(down_s))
    return COLI_E_INVAL;
  if ((rc = check_device())) return rc;
  hipError_t e = coli::launch_table_set_expert(*table, expert, gate_q, gate_s, up_q, up_s, down_q,
                                               down_s, as_stream(stream));
  return e == hipSuccess ? COLI_OK : hip_fail(e);
}

int coli_quant_act_q8(const float* x, int64_t rows, int64_t k, int8_t* q, float* d, void* stream) {
  if (rows < 0 || k <= 0) return COLI_E_SHAPE;
  if (k % 32) return COLI_E_SHAPE;
  if (rows == 0) return COLI_OK;
  if (!x || !q || !d) return COLI_E_INVAL;
  if (!al16(x) || !al4(q) || !al4(d)) return COLI_E_INVAL;
  int rc = check_device();
  if (rc) return rc;
  hipError_t e = coli::launch_quant_act_q8(x, rows, k, q, d, as_stream(stream));
  return e == hipSuccess ? COLI_OK : hip_fail(e);
}

int coli_quant_weight_q4(const float* w, int64_t rows, int64_t k, uint8_t* q, float* s,
                         void* stream) {
  if (rows < 0 || k <= 0 || k % 32) return COLI_E_SHAPE;
  if (rows > 0x7FFFFFFF) return COLI_E_SHAPE;
  if (rows == 0) return COLI_OK;
  if (!w || !q || !s) return COLI_E_INVAL;
  if (!al16(w) || !al4(q) || !al4(s)) return COLI_E_INVAL;
  int rc = check_device();
  if (rc) return rc;
  hipError_t e = coli::launch_quant_weight_q4(w, rows, k, q, s, as_stream(stream));
  return e == hipSuccess ? COLI_OK : hip_fail(e);
}

int coli_quant_weight_q2(const float* w, int64_t rows, int64_t k, uint8_t* q, float* s,
                         void* stream) {
  if (rows < 0 || k <= 0 || k % 32) return COLI_E_SHAPE;
  if (rows > 0x7FFFFFFF) return COLI_E_SHAPE;
  if (rows == 0) return COLI_OK;
  if (!w || !q || !s) return COLI_E_INVAL;
  if (!al16(w) || !al4(q) || !al4(s)) return COLI_E_INVAL;
  int rc = check_device();
  if (rc) return rc;
  hipError_t e = coli::launch_quant_weight_q2(w, rows, k, q, s, as_stream(stream));
  return e == hipSuccess ? COLI_OK : hip_fail(e);
}

int coli_quant_weight_q8(const float* w, int64_t rows, int64_t k, int8_t* q, float* s,
                         void* stream) {
  if (rows < 0 || k <= 0 || k % 32) return COLI_E_SHAPE;
  if (rows > 0x7FFFFFFF) return COLI_E_SHAPE;
  if (rows == 0) return COLI_OK;
  if (!w || !q || !s) return COLI_E_INVAL;
  if (!al16(w) || !al4(q) || !al4(s)) return COLI_E_INVAL;
  int rc = check_device();
  if (rc) return rc;
  hipError_t e = coli::launch_quant_weight_q8(w, rows, k, q, s, as_stream(stream));
  return e == hipSuccess ? COLI_OK : hip_fail(e);
}

int coli_rmsnorm_q8(const float* h, int64_t T, int64_t D, float eps, int8_t* q, float* d,
                    float* r_out, void* stream) {
  if (T < 0 || D <= 0 || D % 32 || T > 0x7FFFFFFF) return COLI_E_SHAPE;
  if (!(eps >= 0.0f) || std::isinf(eps)) return COLI_E_INVAL;
  if (T == 0) return COLI_OK;
  if (!h || !q || !d) return COLI_E_INVAL;
  if (!al16(h) || !al4(q) || !al4(d) || !al4(r_out)) return COLI_E_INVAL;
  int rc = check_device();
  if (rc) return rc;
  hipError_t e = coli::launch_rmsnorm_q8(h, T, D, eps, q, d, r_out, as_stream(stream));
  return e == hipSuccess ? COLI_OK : hip_fail(e);
}

int coli_route_topk(const float* logits, const float* bias, int64_t T, int32_t E, int32_t k,
                    float routed_scale, int32_t* idx, float* w, void* stream) {
  if (E < 1 || E > COLI_MAX_EXPERTS) return COLI_E_SHAPE;
  if (k < 1 || k > E || k > COLI_MAX_TOPK) return COLI_E_SHAPE;
  if (T < 0 || T > 0x7FFFFFFF / 4) return COLI_E_SHAPE;
  if (!std::isfinite(routed_scale)) return COLI_E_INVAL;
  if (T == 0) return COLI_OK;
  if (!logits || !idx || !w) return COLI_E_INVAL;
  if (!al4(logits) || !al4(bias) || !al4(idx) || !al4(w)) return COLI_E_INVAL;
  int rc = check_device();
  if (rc) return rc;
  hipError_t e = coli::launch_route_topk(logits, bias, T, E, k, routed_scale, idx, w,
                                         as_stream(stream));
  return e == hipSuccess ? COLI_OK : hip_fail(e);
}

int coli_router_logits(const float* x, const float* wr, int64_t T, int64_t D, int32_t E,
                       float* logits, void* stream) {
  if (E < 1 || E > COLI_MAX_EXPERTS) return COLI_E_SHAPE;
  if (D < 64 || D % 64 != 0 || D > COLI_MAX_DIM) return COLI_E_SHAPE;
  if (T < 0 || T > 0x7FFFFFFF / 4) return COLI_E_SHAPE;
  if (T == 0) return COLI_OK;
  if (!x || !wr || !logits) return COLI_E_INVAL;
  if (!al16(x) || !al16(wr) || !al4(logits)) return COLI_E_INVAL;
  int rc = check_device();
  if (rc) return rc;
  hipError_t e = coli::launch_router_logits(x, wr, T, D, E, logits, as_stream(stream));
  return e == hipSuccess ? COLI_OK : hip_fail(e);
}

int coli_dispatch(const int32_t* idx, int64_t T, int32_t k, int32_t E, int32_t S, int32_t* counts,
                  int32_t* lists, int32_t* n_active, int32_t* active, int32_t* err,
                  void* stream) {
  if (E < 1 || E > COLI_MAX_EXPERTS || S < 0 || S > 1) return COLI_E_SHAPE;
  if (k < 1 || k > E || k > COLI_MAX_TOPK) return COLI_E_SHAPE;
  if (T < 0 || T * (int64_t)(k + S) > 0x7FFFFFFF) return COLI_E_SHAPE;
  if (!counts || !lists || !n_active || !active || !err || (T > 0 && !idx)) return COLI_E_INVAL;
  if (!al4(idx) || !al4(counts) || !al4(lists) || !al4(n_active) || !al4(active) || !al4(err))
    return COLI_E_INVAL;
  int rc = check_device();
  if (rc) return rc;
  hipError_t e = coli::launch_dispatch(idx, T, k, E, S, counts, lists, n_active, active, err,
                                       nullptr, 0, nullptr, as_stream(stream));
  return e == hipSuccess ? COLI_OK : hip_fail(e);
}

size_t coli_moe_workspace_bytes(const coli_expert_table* table, int64_t T, int32_t k) {
  if (!table || T < 0 || k < 1) return 0;
  return coli::moe_workspace_layout(nullptr, table->n_routed, table->n_shared, table->d_model,
                                    table->d_ff, T, k)
      .bytes;
}

// The path a forward takes: AUTO is grouped from COLI_GROUPED_MIN_TOKENS
// tokens per pass where the grouped path applies (the crossover measured at
// the page shape), else the GEMV.  Returns 0 (GEMV), 1 (grouped) or < 0.
static int choose_grouped(const coli_expert_table* t, int64_t T, int k, int path) {
  const bool applies = coli::grouped_applies(*t, T, k);
  switch (path) {
    case COLI_PATH_AUTO: return applies && T >= COLI_GROUPED_MIN_TOKENS ? 1 : 0;
    case COLI_PATH_GEMV: return 0;
    case COLI_PATH_GROUPED: return applies ? 1 : COLI_E_SHAPE;
    default: return COLI_E_INVAL;
  }
}

static int forward_impl(const coli_expert_table* table, const int8_t* xq, const float* xd,
                        int64_t T, const int32_t* idx, const float* w, int32_t k, float* y,
                        int accumulate, void* workspace, size_t ws_bytes,
                        const coli_moe_trace* trace, const coli_moe_events* events,
                        void* stream, int path = COLI_PATH_AUTO) {
  int rc = table_check(table);
  if (rc) return rc;
  if (k < 1 || k > table->n_routed || k > COLI_MAX_TOPK) return COLI_E_SHAPE;
  if (T < 0 || T * (int64_t)(k + table->n_shared) > 0x7FFFFFFF) return COLI_E_SHAPE;
  if (accumulate != 0 && accumulate != 1) return COLI_E_INVAL;
  if (T == 0) return COLI_OK;
  if (!xq || !xd || !idx || !w || !y || !workspace) return COLI_E_INVAL;
  if (!al4(xq) || !al4(xd) || !al4(idx) || !al4(w) || !al16(y) || !al16(workspace))
    return COLI_E_INVAL;
  const coli::MoeWorkspace ws = coli::moe_workspace_layout(
      workspace, table->n_routed, table->n_shared, table->d_model, table->d_ff, T, k);
  if (ws_bytes < ws.bytes) return COLI_E_WORKSPACE;
  const int grouped = choose_grouped(table, T, k, path);
  if (grouped < 0) return grouped;
  if ((rc = check_device())) return rc;
  coli::ForwardArgs a;
  a.grouped = grouped == 1;
  a.table = table;
  a.xq = xq;
  a.xd = xd;
  a.T = T;
  a.idx = idx;
  a.w = w;
  a.k = k;
  a.y = y;
  a.accumulate = accumulate;
  a.ws = ws;
  a.trace = trace;
  a.events = events;
  a.dispatched = false;
  hipError_t e = coli::launch_moe_forward(a, as_stream(stream));
  return e == hipSuccess ? COLI_OK : hip_fail(e);
}

int coli_moe_forward(const coli_expert_table* table, const int8_t* xq, const float* xd, int64_t T,
                     const int32_t* idx, const float* w, int32_t k, float* y, int accumulate,
                     void* workspace, size_t ws_bytes, void* stream) {
  return forward_impl(table, xq, xd, T, idx, w, k, y, accumulate, workspace, ws_bytes, nullptr,
                      nullptr, stream);
}

int coli_moe_forward_path(const coli_expert_table* table, const int8_t* xq, const float* xd,
                          int64_t T, const int32_t* idx, const float* w, int32_t k, float* y,
                          int accumulate, void* workspace, size_t ws_bytes, int32_t path,
                          void* stream) {
  if (path < COLI_PATH_AUTO || path > COLI_PATH_GROUPED) return COLI_E_INVAL;
  return forward_impl(table, xq, xd, T, idx, w, k, y, accumulate, workspace, ws_bytes, nullptr,
                      nullptr, stream, path);
}

int coli_moe_path(const coli_expert_table* table, int64_t T, int32_t k) {
  int rc = table_check(table);
  if (rc) return rc;
  if (k < 1 || k > table->n_routed || k > COLI_MAX_TOPK || T < 0) return COLI_E_SHAPE;
  return choose_grouped(table, T, k, COLI_PATH_AUTO) == 1 ? COLI_PATH_GROUPED : COLI_PATH_GEMV;
}

int coli_moe_forward_profiled(const coli_expert_table* table, const int8_t* xq, const float* xd,
                              int64_t T, const int32_t* idx, const float* w, int32_t k, float* y,
                              int accumulate, void* workspace, size_t ws_bytes,
                              const coli_moe_events* events, void* stream) {
  if (!events) return COLI_E_INVAL;
  return forward_impl(table, xq, xd, T, idx, w, k, y, accumulate, workspace, ws_bytes, nullptr,
                      events, stream);
}

int coli_moe_forward_traced(const coli_expert_table* table, const int8_t* xq, const float* xd,
                            int64_t T, const int32_t* idx, const float* w, int32_t k, float* y,
                            int accumulate, void* workspace, size_t ws_bytes,
                            const coli_moe_trace* trace, void* stream) {
  if (!trace) return COLI_E_INVAL;
  return forward_impl(table, xq, xd, T, idx, w, k, y, accumulate, workspace, ws_bytes, trace,
                      nullptr, stream);
}

// Layer workspace: the forward's, then the front-end results.
struct LayerWorkspace {
  coli::MoeWorkspace fwd;
  int8_t* xq;
  float* xd;
  int32_t* idx;
  float* w;
  size_t bytes;
};

static LayerWorkspace layer_workspace_layout(void* base, const coli_expert_table* t, int64_t T,
                                             int k) {
  LayerWorkspace l;
  l.fwd = coli::moe_workspace_layout(base, t->n_routed, t->n_shared, t->d_model, t->d_ff, T, k);
  size_t off = l.fwd.bytes;
  char* p = static_cast<char*>(base);
  auto take = [&](size_t bytes) -> void* {
    void* r = p ? p + off : nullptr;
    off += align256(bytes);
    return r;
  };
  l.xq = static_cast<int8_t*>(take((size_t)(T * t->d_model)));
  l.xd = static_cast<float*>(take(sizeof(float) * (size_t)(T * (t->d_model / 32))));
  l.idx = static_cast<int32_t*>(take(sizeof(int32_t) * (size_t)(T * k)));
  l.w = static_cast<float*>(take(sizeof(float) * (size_t)(T * k)));
  l.bytes = off;
  return l;
}

size_t coli_moe_layer_workspace_bytes(const coli_expert_table* table, int64_t T, int32_t k) {
  if (!table || T < 0 || k < 1) return 0;
  return layer_workspace_layout(nullptr, table, T, k).bytes;
}

// The layer from f32 activations (norm: from the residual stream h, whose
// RMSNorm is quantised) and router logits: the fused front end for small
// batches, else Q8_0 (or RMSNorm + Q8_0) and routing kernels, then the forward.
static int layer_impl(const coli_expert_table* table, const float* x, const float* logits,
                      const float* bias, int64_t T, int32_t k, float routed_scale, float* y,
                      int accumulate, void* workspace, size_t ws_bytes,
                      const coli_moe_trace* trace, const coli_moe_events* events, bool norm,
                      float eps, void* stream) {
  int rc = table_check(table);
  if (rc) return rc;
  const int E = table->n_routed, S = table->n_shared;
  if (k < 1 || k > E || k > COLI_MAX_TOPK) return COLI_E_SHAPE;
  if (T < 0 || T * (int64_t)(k + S) > 0x7FFFFFFF) return COLI_E_SHAPE;
  if (accumulate != 0 && accumulate != 1) return COLI_E_INVAL;
  if (!std::isfinite(routed_scale)) return COLI_E_INVAL;
  if (norm && !(std::isfinite(eps) && eps >= 0.0f)) return COLI_E_INVAL;
  if (T == 0) return COLI_OK;
  if (!x || !logits || !y || !workspace) return COLI_E_INVAL;
  if (!al16(x) || !al4(logits) || !al4(bias) || !al16(y) || !al16(workspace)) return COLI_E_INVAL;
  const LayerWorkspace l = layer_workspace_layout(workspace, table, T, k);
  if (ws_bytes < l.bytes) return COLI_E_WORKSPACE;
  if ((rc = check_device())) return rc;
  const int64_t D = table->d_model;
  hipStream_t s = as_stream(stream);
  hipError_t e = hipSuccess;
  // `begin` marks the start of the front end; the forward records the rest
  coli_moe_events fwd_events = {};
  if (events) {
    fwd_events = *events;
    fwd_events.begin = nullptr;
    if (events->begin) e = hipEventRecord(reinterpret_cast<hipEvent_t>(events->begin), s);
    if (e != hipSuccess) return hip_fail(e);
  }
  const bool small = T <= coli::kPrologueMaxTokens && T * k <= coli::kPrologueMaxEntries;
  if (small) {
    e = coli::launch_prologue_small(x, logits, bias, T, E, S, k, routed_scale, D, l.xq, l.xd,
                                    l.fwd.xsum8, l.idx, l.w, l.fwd.counts, l.fwd.lists,
                                    l.fwd.n_active, l.fwd.active, l.fwd.err, norm, eps, s);
  } else {
    e = norm ? coli::launch_rmsnorm_q8(x, T, D, eps, l.xq, l.xd, nullptr, s)
             : coli::launch_quant_act_q8(x, T, D, l.xq, l.xd, s);
    if (e == hipSuccess) e = coli::launch_route_topk(logits, bias, T, E, k, routed_scale, l.idx, l.w, s);
  }
  if (e != hipSuccess) return hip_fail(e);
  coli::ForwardArgs a;
  a.grouped = choose_grouped(table, T, k, COLI_PATH_AUTO) == 1;
  a.table = table;
  a.xq = l.xq;
  a.xd = l.xd;
  a.T = T;
  a.idx = l.idx;
  a.w = l.w;
  a.k = k;
  a.y = y;
  a.accumulate = accumulate;
  a.ws = l.fwd;
  a.trace = trace;
  a.events = events ? &fwd_events : nullptr;
  a.dispatched = small;
  e = coli::launch_moe_forward(a, s);
  return e == hipSuccess ? COLI_OK : hip_fail(e);
}

int coli_moe_layer_ex(const coli_expert_table* table, const float* x, const float* logits,
                      const float* bias, int64_t T, int32_t k, float routed_scale, float* y,
                      int accumulate, void* workspace, size_t ws_bytes,
                      const coli_moe_trace* trace, const coli_moe_events* events, void* stream) {
  return layer_impl(table, x, logits, bias, T, k, routed_scale, y, accumulate, workspace,
                    ws_bytes, trace, events, false, 0.0f, stream);
}

int coli_moe_block(const coli_expert_table* table, float* h, const float* logits,
                   const float* bias, int64_t T, int32_t k, float routed_scale, float eps,
                   void* workspace, size_t ws_bytes, void* stream) {
  return layer_impl(table, h, logits, bias, T, k, routed_scale, h, 1, workspace, ws_bytes,
                    nullptr, nullptr, true, eps, stream);
}

int coli_moe_layer(const coli_expert_table* table, const float* x, const float* logits,
                   const float* bias, int64_t T, int32_t k, float routed_scale, float* y,
                   int accumulate, void* workspace, size_t ws_bytes, void* stream) {
  return coli_moe_layer_ex(table, x, logits, bias, T, k, routed_scale, y, accumulate, workspace,
                           ws_bytes, nullptr, nullptr, stream);
}

// ---------------------------------------------------------------------------
// Allocation-free layer: coli_moe_layer with its workspace in a file-scope
// device array instead of a caller's buffer.  Each device holds its own copy
// of the array (loaded with the code object, kept until the process ends);
// host code reaches it only through the device address hipGetSymbolAddress
// gives on that device, looked up once per device.
namespace {

constexpr size_t kNoAllocBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

std::mutex g_scratch_mu;
void* g_scratch[64];   // device address of `scratch` per device (null: not looked up)

int scratch_on_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= 64) return COLI_E_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e);
    if (!p) return COLI_E_DEVICE;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return COLI_OK;
}

}  // namespace

int coli_moe_layer_noalloc(const coli_expert_table* table, const float* x, const float* logits,
                           const float* bias, int64_t T, int32_t k, float routed_scale, float* y,
                           int accumulate, void* stream) {
  int rc = table_check(table);
  if (rc) return rc;
  if (table->slot_of) return COLI_E_INVAL;   // resident tables only (see coli.h)
  if (k < 1 || k > table->n_routed || k > COLI_MAX_TOPK || T < 0) return COLI_E_SHAPE;
  if (T * (int64_t)(k + table->n_shared) > 0x7FFFFFFF) return COLI_E_SHAPE;
  if (coli_moe_layer_workspace_bytes(table, T, k) > kNoAllocBytes) return COLI_E_WORKSPACE;
  if (T == 0) return COLI_OK;
  if ((rc = check_device())) return rc;
  void* ws = nullptr;
  if ((rc = scratch_on_current_device(&ws))) return rc;
  return layer_impl(table, x, logits, bias, T, k, routed_scale, y, accumulate, ws, kNoAllocBytes,
                    nullptr, nullptr, false, 0.0f, stream);
}

int coli_moe_status(const void* workspace, size_t ws_bytes, void* stream) {
  if (!workspace || ws_bytes < sizeof(int32_t)) return COLI_E_INVAL;
  int rc = check_device();
  if (rc) return rc;
  int32_t err = 0;
  hipError_t e = hipMemcpyAsync(&err, workspace, sizeof(err), hipMemcpyDeviceToHost,
                                as_stream(stream));
  if (e != hipSuccess) return hip_fail(e);
  e = hipStreamSynchronize(as_stream(stream));
  if (e != hipSuccess) return hip_fail(e);
  return err == 0 ? COLI_OK : err == COLI_E_TIER ? COLI_E_TIER : COLI_E_INDEX;
}

// ---------------------------------------------------------------------------
// Expert tier.

size_t coli_tier_table_bytes(int32_t slots, int64_t D, int64_t F, int32_t bits, size_t* gu_q,
                             size_t* gu_s, size_t* dn_q, size_t* dn_s) {
  if (slots < 1 || slots > COLI_MAX_EXPERTS + 1) return 0;
  if (D <= 0 || D % 64 || F <= 0 || F % 32 || D > COLI_MAX_DIM || F > COLI_MAX_DIM) return 0;
  if ((bits != 2 && bits != 4 && bits != 8) || (bits == 2 && F % 64)) return 0;
  const size_t n = (size_t)slots;
  const size_t a = n * (size_t)(D * F * bits / 4), b = n * (size_t)(2 * F) * sizeof(float),
               c = n * (size_t)(D * F * bits / 8), d = n * (size_t)D * sizeof(float);
  if (gu_q) *gu_q = a;
  if (gu_s) *gu_s = b;
  if (dn_q) *dn_q = c;
  if (dn_s) *dn_s = d;
  return a + b + c + d;
}

static int tier_check(const coli_expert_table* t, const coli_tier_state* st) {
  int rc = table_check(t);
  if (rc) return rc;
  if (!st || !t->slot_of || t->slot_of != st->slot_of) return COLI_E_INVAL;
  const int32_t* p[] = {st->slot_of, st->expert_in, st->stamp, st->pinned, st->usage, st->loads,
                        st->counters};
  for (const int32_t* q : p)
    if (!q || !al4(q)) return COLI_E_INVAL;
  return COLI_OK;
}

static int store_view(const coli_expert_table* tier, const coli_expert_table* store,
                      const void* src[4]);

int coli_tier_init(const coli_expert_table* tier, const coli_tier_state* st, const int32_t* pin,
                   int32_t n_pin, const coli_expert_table* store, void* stream) {
  int rc = tier_check(tier, st);
  if (rc) return rc;
  const int E = tier->n_routed, S = tier->n_shared;
  if (n_pin < 0 || (n_pin > 0 && !pin) || S + n_pin > tier->n_slots) return COLI_E_INVAL;
  for (int i = 0; i < n_pin; ++i) {
    if (pin[i] < 0 || pin[i] >= E) return COLI_E_INVAL;
    for (int j = 0; j < i; ++j)
      if (pin[j] == pin[i]) return COLI_E_INVAL;
  }
  if ((rc = check_device())) return rc;
  const void* src[4];
  if ((rc = store_view(tier, store, src))) return rc;
  hipError_t e = coli::launch_tier_init(*tier, *st, pin, n_pin, as_stream(stream));
  if (e == hipSuccess) e = coli::launch_tier_fetch(*tier, *st, src, as_stream(stream));
  return e == hipSuccess ? COLI_OK : hip_fail(e);
}

int coli_tier_plan(const coli_expert_table* tier, const coli_tier_state* st, const int32_t* idx,
                   int64_t T, int32_t k, int32_t count_usage, void* stream) {
  int rc = tier_check(tier, st);
  if (rc) return rc;
  if (T < 0 || T > 0x7FFFFFFF || k < 1 || k > COLI_MAX_TOPK || k > tier->n_routed)
    return COLI_E_SHAPE;
  if (T * (int64_t)k > 0x7FFFFFFF) return COLI_E_SHAPE;
  if ((T > 0 && !idx) || !al4(idx) || (count_usage != 0 && count_usage != 1)) return COLI_E_INVAL;
  if ((rc = check_device())) return rc;
  hipError_t e = coli::launch_tier_plan(*tier, *st, idx, T, k, count_usage, as_stream(stream));
  return e == hipSuccess ? COLI_OK : hip_fail(e);
}

// The device-visible address of a store array: device memory as it is,
// pinned host memory through its device mapping; anything else is refused.
static int device_view(const void* p, const void** out) {
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();   // clear the sticky error of the failed query
    return COLI_E_INVAL;
  }
  if (attr.type == hipMemoryTypeDevice) {
    *out = p;
    return COLI_OK;
  }
  if (attr.type == hipMemoryTypeHost && attr.devicePointer) {
    *out = attr.devicePointer;
    return COLI_OK;
  }
  return COLI_E_INVAL;
}

// Checks a store against its tier and resolves its device-visible addresses
// (call after check_device: the address query needs the device).
static int store_view(const coli_expert_table* tier, const coli_expert_table* store,
                      const void* src[4]) {
  if (!store || store->slot_of) return COLI_E_INVAL;
  if (store->n_routed != tier->n_routed || store->n_shared != tier->n_shared ||
      store->d_model != tier->d_model || store->d_ff != tier->d_ff ||
      store->weight_bits != tier->weight_bits)
    return COLI_E_SHAPE;
  if (!store->gu_q || !store->gu_s || !store->dn_q || !store->dn_s) return COLI_E_INVAL;
  if (!al16(store->gu_q) || !al16(store->gu_s) || !al16(store->dn_q) || !al16(store->dn_s) ||
      !al16(tier->gu_s) || !al16(tier->dn_s))
    return COLI_E_INVAL;
  const void* host[4] = {store->gu_q, store->gu_s, store->dn_q, store->dn_s};
  for (int m = 0; m < 4; ++m) {
    int rc = device_view(host[m], &src[m]);
    if (rc) return rc;
  }
  return COLI_OK;
}

int coli_tier_fetch(const coli_expert_table* tier, const coli_tier_state* st,
                    const coli_expert_table* store, void* stream) {
  int rc = tier_check(tier, st);
  if (rc) return rc;
  if (!store) return COLI_E_INVAL;
  if (store->n_routed != tier->n_routed || store->d_model != tier->d_model) return COLI_E_SHAPE;
  if ((rc = check_device())) return rc;
  const void* src[4];
  if ((rc = store_view(tier, store, src))) return rc;
  hipError_t e = coli::launch_tier_fetch(*tier, *st, src, as_stream(stream));
  return e == hipSuccess ? COLI_OK : hip_fail(e);
}

int coli_tier_status(const coli_tier_state* st, void* stream) {
  if (!st || !st->counters) return COLI_E_INVAL;
  int rc = check_device();
  if (rc) return rc;
  int32_t c[4] = {};
  hipError_t e = hipMemcpyAsync(c, st->counters, sizeof(c), hipMemcpyDeviceToHost,
                                as_stream(stream));
  if (e != hipSuccess) return hip_fail(e);
  e = hipStreamSynchronize(as_stream(stream));
  if (e != hipSuccess) return hip_fail(e);
  return c[3] == 0 ? COLI_OK : COLI_E_TIER;
}

int coli_tier_rank(const int32_t* usage, int32_t E, int32_t n, int32_t* out) {
  if (E < 1 || E > COLI_MAX_EXPERTS || n < 0 || n > E) return COLI_E_SHAPE;
  if (!usage || (n > 0 && !out)) return COLI_E_INVAL;
  // selection by repeated maximum: n, E <= 256
  bool taken[COLI_MAX_EXPERTS] = {};
  for (int i = 0; i < n; ++i) {
    int best = -1;
    for (int e = 0; e < E; ++e)
      if (!taken[e] && (best < 0 || usage[e] > usage[best])) best = e;
    taken[best] = true;
    out[i] = best;
  }
  return COLI_OK;
}

}  // extern "C"
