// C-ABI entry points: validate on the host, plan the caller's workspace, enqueue the
// gfx950 kernels on the caller's stream.  No allocation, no synchronisation.
#include <hip/hip_runtime.h>

#include "csa.h"
#include "launch.hpp"
#include "mqa_bwd.hpp"
#include "mqa_bwd_dkv.hpp"
#include "validate.hpp"

using namespace csa;

namespace {

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

csa_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return CSA_OK;
  set_error("%s: %s", what, hipGetErrorString(e));
  return CSA_ERR_HIP;
}

#define CSA_TRY(expr)                  \
  do {                                 \
    const csa_status_t s_ = (expr);    \
    if (s_ != CSA_OK) return s_;       \
  } while (0)

#define CSA_HIP(expr, what) CSA_TRY(hip_status((expr), what))

bool empty(const csa_params_t* p) { return (int64_t)p->B * p->S == 0; }

// Optional per-launch event recording for the traced fused calls.
struct Tracer {
  void* const* events = nullptr;
  int32_t* kinds = nullptr;
  int32_t n = 0, used = 0;
  hipError_t start(hipStream_t st) {
    if (!events) return hipSuccess;
    used = 1;
    return hipEventRecord(static_cast<hipEvent_t>(events[0]), st);
  }
  hipError_t mark(csa_kernel_t k, hipStream_t st) {
    if (!events) return hipSuccess;
    kinds[used - 1] = k;
    return hipEventRecord(static_cast<hipEvent_t>(events[used++]), st);
  }
};

int32_t n_chunks(const WsPlan& plan, int32_t S) {
  return plan.chunk_rows > 0 ? (S + plan.chunk_rows - 1) / plan.chunk_rows : 0;
}

// the indexer options that need a key pass before the scoring kernel
bool index_prologue(const csa_params_t& p) {
  return (p.flags & (CSA_FLAG_INDEX_PROLOGUE | CSA_FLAG_INDEX_FP8)) != 0;
}

// Kernel launches of the indexer/top-k stage: the key prologue (with the flag), then
// one fused launch, or two per chunk.
int32_t index_launches(const csa_params_t& p, const WsPlan& plan) {
  return (index_prologue(p) ? 1 : 0) + (p.topk <= kFusedTopkMax ? 1 : 2 * n_chunks(plan, p.S));
}

csa_status_t check_ws(const csa_params_t* p, int32_t op, void* ws, size_t ws_bytes, WsPlan* plan) {
  *plan = plan_workspace(*p, op);
  if (plan->total == 0) return CSA_OK;
  if (ws_bytes < plan->total) {
    set_error("workspace of %zu bytes is below the %zu bytes this op needs", ws_bytes, plan->total);
    return CSA_ERR_WORKSPACE;
  }
  return check_ptr(ws, "ws");
}

// Indexer scores and top-k over query chunks that fit the scores workspace.
csa_status_t run_index_topk(const csa_params_t* p, const void* q_idx, const float* w_idx,
                            const void* k_idx, int32_t* idx, int32_t* nvis, unsigned char* ws,
                            const WsPlan& plan, hipStream_t st, Tracer* tr = nullptr) {
  Tracer none;
  if (!tr) tr = &none;
  if (index_prologue(*p)) {  // transformed keys into the workspace; queries transform in-kernel
    void* k_rot = ws + plan.k_rot;
    CSA_HIP(launch_index_keys(*p, k_idx, k_rot, st), "indexer key prologue launch");
    CSA_HIP(tr->mark(CSA_KERNEL_INDEX_KEYS, st), "event record");
    k_idx = k_rot;
  }
  if (p->topk <= kFusedTopkMax) {
    CSA_HIP(launch_index_topk(*p, q_idx, w_idx, k_idx, idx, nvis, st), "indexer/top-k launch");
    CSA_HIP(tr->mark(CSA_KERNEL_INDEX_TOPK, st), "event record");
    return CSA_OK;
  }
  float* scores = reinterpret_cast<float*>(ws + plan.scores);
  for (int32_t t0 = 0; t0 < p->S; t0 += plan.chunk_rows) {
    const int32_t rows = p->S - t0 < plan.chunk_rows ? p->S - t0 : plan.chunk_rows;
    CSA_HIP(launch_index_scores(*p, q_idx, w_idx, k_idx, scores, plan.ld, t0, rows, st), "indexer launch");
    CSA_HIP(tr->mark(CSA_KERNEL_INDEXER, st), "event record");
    CSA_HIP(launch_topk(*p, scores, plan.ld, t0, rows, idx, nvis, st), "top-k launch");
    CSA_HIP(tr->mark(CSA_KERNEL_TOPK, st), "event record");
  }
  return CSA_OK;
}

csa_status_t check_inputs_compress(const csa_params_t* p, const void* va, const void* ga,
                                   const void* vb, const void* gb, const float* bias) {
  CSA_TRY(check_ptr(va, "va"));
  CSA_TRY(check_ptr(ga, "ga"));
  CSA_TRY(check_ptr(bias, "bias"));
  if (p->overlap) {
    CSA_TRY(check_ptr(vb, "vb"));
    CSA_TRY(check_ptr(gb, "gb"));
  } else if (vb || gb) {
    set_error("vb/gb must be NULL when overlap == 0");
    return CSA_ERR_INVALID_ARG;
  }
  return CSA_OK;
}

csa_status_t check_inputs_index(const void* q_idx, const float* w_idx, const void* k_idx) {
  CSA_TRY(check_ptr(q_idx, "q_idx"));
  CSA_TRY(check_ptr(w_idx, "w_idx"));
  CSA_TRY(check_ptr(k_idx, "k_idx"));
  return CSA_OK;
}

csa_status_t check_optional(const void* ptr, const char* name) {
  return ptr ? check_ptr(ptr, name) : CSA_OK;
}

}  // namespace

extern "C" {

int32_t csa_abi_version(void) { return CSA_ABI_VERSION; }

const char* csa_last_error(void) { return last_error(); }

const char* csa_status_str(csa_status_t s) {
  switch (s) {
    case CSA_OK: return "CSA_OK";
    case CSA_ERR_INVALID_ARG: return "CSA_ERR_INVALID_ARG";
    case CSA_ERR_WORKSPACE: return "CSA_ERR_WORKSPACE";
    case CSA_ERR_UNSUPPORTED: return "CSA_ERR_UNSUPPORTED";
    case CSA_ERR_HIP: return "CSA_ERR_HIP";
  }
  return "CSA_ERR_UNKNOWN";
}

size_t csa_workspace_bytes(const csa_params_t* p, int32_t op) {
  uint32_t need = 0;
  switch (op) {
    case CSA_OP_COMPRESS: need = uint32_t(Need::COMPRESS); break;
    case CSA_OP_INDEX_TOPK: need = uint32_t(Need::INDEX); break;
    case CSA_OP_SPARSE_MQA: need = uint32_t(Need::MQA); break;
    case CSA_OP_CSA_FWD: need = Need::COMPRESS | Need::INDEX | Need::MQA; break;
    case CSA_OP_HCA_FWD: need = Need::COMPRESS | Need::MQA; break;
    case CSA_OP_SPARSE_MQA_BWD: need = uint32_t(Need::MQA); break;
    default: set_error("unknown op %d", op); return 0;
  }
  // the attention workspace (rotated window latents) does not depend on the entries,
  // so it is sized for the window-only case too
  if (validate_params(p, need, op == CSA_OP_SPARSE_MQA || op == CSA_OP_SPARSE_MQA_BWD) != CSA_OK) return 0;
  return plan_workspace(*p, op).total;
}

csa_status_t csa_compress(const csa_params_t* p, const void* va, const void* ga, const void* vb,
                          const void* gb, const float* bias, void* kv_c, void* stream) {
  CSA_TRY(validate_params(p, uint32_t(Need::COMPRESS), false));
  if (empty(p)) return CSA_OK;
  CSA_TRY(check_inputs_compress(p, va, ga, vb, gb, bias));
  CSA_TRY(check_ptr(kv_c, "kv_c"));
  CSA_HIP(launch_compress(*p, va, ga, vb, gb, bias, kv_c, as_stream(stream)), "compress launch");
  return CSA_OK;
}

csa_status_t csa_index_scores(const csa_params_t* p, const void* q_idx, const float* w_idx,
                              const void* k_idx, float* scores, int64_t ld, int32_t t0,
                              int32_t nrows, void* stream) {
  CSA_TRY(validate_params(p, uint32_t(Need::INDEX), false));
  if (t0 < 0 || nrows < 0 || (int64_t)t0 + nrows > p->S) {
    set_error("rows %d..%d outside 0..S=%d", t0, t0 + nrows, p->S);
    return CSA_ERR_INVALID_ARG;
  }
  if (ld < (int64_t)(p->ratio > 0 ? p->S / p->ratio : 0)) {
    set_error("ld=%lld is below S/ratio", (long long)ld);
    return CSA_ERR_INVALID_ARG;
  }
  if (p->B == 0 || nrows == 0) return CSA_OK;
  CSA_TRY(check_inputs_index(q_idx, w_idx, k_idx));
  CSA_TRY(check_ptr(scores, "scores"));
  CSA_HIP(launch_index_scores(*p, q_idx, w_idx, k_idx, scores, ld, t0, nrows, as_stream(stream)),
          "indexer launch");
  return CSA_OK;
}

csa_status_t csa_index_keys(const csa_params_t* p, const void* k_idx, void* k_out, void* stream) {
  CSA_TRY(validate_params(p, uint32_t(Need::INDEX_KEYS), false));
  if (empty(p)) return CSA_OK;
  CSA_TRY(check_ptr(k_idx, "k_idx"));
  CSA_TRY(check_ptr(k_out, "k_out"));
  const size_t rows = (size_t)p->B * (size_t)(p->S / p->ratio);
  const size_t in_bytes = rows * (size_t)p->idx_dim * (p->dtype == CSA_BF16 ? 2 : 4);
  const size_t out_bytes = (p->flags & CSA_FLAG_INDEX_FP8) ? rows * (size_t)(p->idx_dim + 16) : in_bytes;
  const uintptr_t a = reinterpret_cast<uintptr_t>(k_idx), b = reinterpret_cast<uintptr_t>(k_out);
  if (a < b + out_bytes && b < a + in_bytes) {
    set_error("k_out overlaps k_idx");
    return CSA_ERR_INVALID_ARG;
  }
  CSA_HIP(launch_index_keys(*p, k_idx, k_out, as_stream(stream)), "indexer key prologue launch");
  return CSA_OK;
}

csa_status_t csa_index_topk(const csa_params_t* p, const void* q_idx, const float* w_idx,
                            const void* k_idx, int32_t* idx, int32_t* n_visible, void* ws,
                            size_t ws_bytes, void* stream) {
  CSA_TRY(validate_params(p, uint32_t(Need::INDEX), false));
  if (empty(p)) return CSA_OK;
  CSA_TRY(check_inputs_index(q_idx, w_idx, k_idx));
  CSA_TRY(check_ptr(idx, "idx"));
  CSA_TRY(check_optional(n_visible, "n_visible"));
  WsPlan plan;
  CSA_TRY(check_ws(p, CSA_OP_INDEX_TOPK, ws, ws_bytes, &plan));
  return run_index_topk(p, q_idx, w_idx, k_idx, idx, n_visible, static_cast<unsigned char*>(ws),
                        plan, as_stream(stream));
}

static csa_status_t sparse_mqa_fwd(const csa_params_t* p, const void* q, const void* kv_c,
                                   const void* kv_raw, const int32_t* idx, const float* sinks,
                                   void* o, float* lse, bool want_lse, void* ws, size_t ws_bytes,
                                   void* stream);

csa_status_t csa_sparse_mqa_fwd(const csa_params_t* p, const void* q, const void* kv_c,
                                const void* kv_raw, const int32_t* idx, void* o, void* ws,
                                size_t ws_bytes, void* stream) {
  return csa_sparse_mqa_fwd_sink(p, q, kv_c, kv_raw, idx, nullptr, o, ws, ws_bytes, stream);
}

csa_status_t csa_sparse_mqa_fwd_sink(const csa_params_t* p, const void* q, const void* kv_c,
                                     const void* kv_raw, const int32_t* idx, const float* sinks,
                                     void* o, void* ws, size_t ws_bytes, void* stream) {
  return sparse_mqa_fwd(p, q, kv_c, kv_raw, idx, sinks, o, nullptr, false, ws, ws_bytes, stream);
}

csa_status_t csa_sparse_mqa_fwd_lse(const csa_params_t* p, const void* q, const void* kv_c,
                                    const void* kv_raw, const int32_t* idx, const float* sinks,
                                    void* o, float* lse, void* ws, size_t ws_bytes, void* stream) {
  return sparse_mqa_fwd(p, q, kv_c, kv_raw, idx, sinks, o, lse, true, ws, ws_bytes, stream);
}

static csa_status_t sparse_mqa_fwd(const csa_params_t* p, const void* q, const void* kv_c,
                                   const void* kv_raw, const int32_t* idx, const float* sinks,
                                   void* o, float* lse, bool want_lse, void* ws, size_t ws_bytes,
                                   void* stream) {
  const bool window_only = kv_c == nullptr;
  CSA_TRY(validate_params(p, uint32_t(Need::MQA) | (idx ? uint32_t(Need::SELECT) : 0u), window_only));
  if (window_only && idx) {
    set_error("idx given without kv_c");
    return CSA_ERR_INVALID_ARG;
  }
  if (empty(p)) return CSA_OK;
  CSA_TRY(check_ptr(q, "q"));
  CSA_TRY(check_ptr(kv_raw, "kv_raw"));
  CSA_TRY(check_ptr(o, "o"));
  if (want_lse) CSA_TRY(check_ptr(lse, "lse"));
  CSA_TRY(check_optional(kv_c, "kv_c"));
  CSA_TRY(check_optional(idx, "idx"));
  CSA_TRY(check_optional(sinks, "sinks"));
  WsPlan plan;
  CSA_TRY(check_ws(p, CSA_OP_SPARSE_MQA, ws, ws_bytes, &plan));
  unsigned char* w = static_cast<unsigned char*>(ws);
  const hipStream_t st = as_stream(stream);
  void* kv_w = w + plan.kv_w;
  CSA_HIP(launch_window_rope(*p, kv_raw, kv_w, st), "window rope launch");
  const MqaMode mode = window_only ? MQA_WINDOW_ONLY : (idx ? MQA_SELECTED : MQA_DENSE);
  CSA_HIP(launch_sparse_mqa(*p, mode, q, kv_c, kv_w, idx, sinks, o, lse, st), "attention launch");
  return CSA_OK;
}

csa_status_t csa_sparse_mqa_bwd_dq(const csa_params_t* p, const void* q, const void* kv_c,
                                   const void* kv_raw, const int32_t* idx, const float* sinks,
                                   const void* o, const void* d_o, void* dq, void* ws,
                                   size_t ws_bytes, void* stream) {
  const bool window_only = kv_c == nullptr;
  CSA_TRY(validate_params(p, uint32_t(Need::MQA) | (idx ? uint32_t(Need::SELECT) : 0u), window_only));
  if (window_only && idx) {
    set_error("idx given without kv_c");
    return CSA_ERR_INVALID_ARG;
  }
  if (empty(p)) return CSA_OK;
  CSA_TRY(check_ptr(q, "q"));
  CSA_TRY(check_ptr(kv_raw, "kv_raw"));
  CSA_TRY(check_ptr(o, "o"));
  CSA_TRY(check_ptr(d_o, "d_o"));
  CSA_TRY(check_ptr(dq, "dq"));
  CSA_TRY(check_optional(kv_c, "kv_c"));
  CSA_TRY(check_optional(idx, "idx"));
  CSA_TRY(check_optional(sinks, "sinks"));
  WsPlan plan;
  CSA_TRY(check_ws(p, CSA_OP_SPARSE_MQA, ws, ws_bytes, &plan));
  unsigned char* w = static_cast<unsigned char*>(ws);
  const hipStream_t st = as_stream(stream);
  void* kv_w = w + plan.kv_w;
  CSA_HIP(launch_window_rope(*p, kv_raw, kv_w, st), "window rope launch");
  const MqaMode mode = window_only ? MQA_WINDOW_ONLY : (idx ? MQA_SELECTED : MQA_DENSE);
  CSA_HIP(launch_mqa_bwd_dq(*p, mode, q, kv_c, kv_w, idx, sinks, o, d_o, dq, st), "dq launch");
  return CSA_OK;
}

csa_status_t csa_sparse_mqa_bwd_dkv(const csa_params_t* p, const void* q, const void* kv_c,
                                    const void* kv_raw, const int32_t* idx, const float* sinks,
                                    const void* o, const float* lse, const void* d_o, float* dkv_c,
                                    float* dkv_raw, float* dsinks, void* ws, size_t ws_bytes,
                                    void* stream) {
  const bool window_only = kv_c == nullptr;
  CSA_TRY(validate_params(p, uint32_t(Need::MQA) | (idx ? uint32_t(Need::SELECT) : 0u), window_only));
  if (window_only && idx) {
    set_error("idx given without kv_c");
    return CSA_ERR_INVALID_ARG;
  }
  if (p->dtype == CSA_F32 && p->D > 256) {
    set_error("the key-side backward holds fp32 operands for D <= 256, not D=%d", p->D);
    return CSA_ERR_UNSUPPORTED;
  }
  if (!dkv_c != window_only) {
    set_error(window_only ? "dkv_c given without kv_c" : "dkv_c is NULL");
    return CSA_ERR_INVALID_ARG;
  }
  if (!dsinks != !sinks) {
    set_error(sinks ? "dsinks is NULL" : "dsinks given without sinks");
    return CSA_ERR_INVALID_ARG;
  }
  if (dsinks) CSA_TRY(check_ptr(dsinks, "dsinks"));
  const hipStream_t st = as_stream(stream);
  if (empty(p)) {  // nothing contributes: the sink gradient is zero
    if (dsinks) CSA_HIP(launch_zero_f32(dsinks, (size_t)p->H, st), "zero launch");
    return CSA_OK;
  }
  CSA_TRY(check_ptr(q, "q"));
  CSA_TRY(check_ptr(kv_raw, "kv_raw"));
  CSA_TRY(check_ptr(o, "o"));
  CSA_TRY(check_ptr(lse, "lse"));
  CSA_TRY(check_ptr(d_o, "d_o"));
  CSA_TRY(check_ptr(dkv_raw, "dkv_raw"));
  CSA_TRY(check_optional(kv_c, "kv_c"));
  CSA_TRY(check_optional(dkv_c, "dkv_c"));
  CSA_TRY(check_optional(idx, "idx"));
  CSA_TRY(check_optional(sinks, "sinks"));
  WsPlan plan;
  CSA_TRY(check_ws(p, CSA_OP_SPARSE_MQA_BWD, ws, ws_bytes, &plan));
  unsigned char* w = static_cast<unsigned char*>(ws);
  void* kv_w = w + plan.kv_w;
  CSA_HIP(launch_window_rope(*p, kv_raw, kv_w, st), "window rope launch");
  DkvWs dw;
  dw.interm = w + plan.interm;
  dw.ds_row = reinterpret_cast<float*>(w + plan.ds_row);
  dw.sink_part = reinterpret_cast<float*>(w + plan.sink_part);
  dw.cnt = reinterpret_cast<int32_t*>(w + plan.cnt);
  dw.tot = reinterpret_cast<int32_t*>(w + plan.tot);
  dw.base = reinterpret_cast<int32_t*>(w + plan.base);
  dw.segbase = reinterpret_cast<int32_t*>(w + plan.segbase);
  dw.list = reinterpret_cast<int32_t*>(w + plan.list);
  dw.partial = reinterpret_cast<float*>(w + plan.partial);
  const MqaMode mode = window_only ? MQA_WINDOW_ONLY : (idx ? MQA_SELECTED : MQA_DENSE);
  CSA_HIP(launch_mqa_bwd_dkv(*p, mode, q, kv_c, kv_w, kv_raw, idx, sinks, o, lse, d_o, dkv_c, dkv_raw,
                             dsinks, dw, st),
          "key-side backward launch");
  return CSA_OK;
}

csa_status_t csa_kl_target(const csa_params_t* p, const void* q, const void* kv_c,
                           const int32_t* idx, float* target, void* stream) {
  CSA_TRY(validate_params(p, Need::MQA | Need::SELECT, false));
  if (empty(p)) return CSA_OK;
  CSA_TRY(check_ptr(q, "q"));
  CSA_TRY(check_ptr(kv_c, "kv_c"));
  CSA_TRY(check_ptr(idx, "idx"));
  CSA_TRY(check_ptr(target, "target"));
  CSA_HIP(launch_kl_target(*p, q, kv_c, idx, target, as_stream(stream)), "KL target launch");
  return CSA_OK;
}

static csa_status_t fused(const csa_params_t* p, const csa_inputs_t* in, void* o, void* ws,
                          size_t ws_bytes, void* stream, bool csa_layer, Tracer* tr) {
  const uint32_t need = csa_layer ? (Need::COMPRESS | Need::INDEX | Need::MQA) : (Need::COMPRESS | Need::MQA);
  CSA_TRY(validate_params(p, need, false));
  if (p->overlap != (csa_layer ? 1 : 0)) {
    set_error(csa_layer ? "csa_fwd needs overlap == 1" : "hca_fwd needs overlap == 0");
    return CSA_ERR_INVALID_ARG;
  }
  if (!in) {
    set_error("inputs is NULL");
    return CSA_ERR_INVALID_ARG;
  }
  if (empty(p)) return CSA_OK;
  CSA_TRY(check_ptr(in->q, "q"));
  CSA_TRY(check_ptr(in->kv_raw, "kv_raw"));
  CSA_TRY(check_ptr(o, "o"));
  CSA_TRY(check_inputs_compress(p, in->va, in->ga, in->vb, in->gb, in->bias));
  if (csa_layer) CSA_TRY(check_inputs_index(in->q_idx, in->w_idx, in->k_idx));
  CSA_TRY(check_optional(in->kv_c_out, "kv_c_out"));
  CSA_TRY(check_optional(in->idx_out, "idx_out"));
  CSA_TRY(check_optional(in->n_visible_out, "n_visible_out"));
  CSA_TRY(check_optional(in->sinks, "sinks"));
  CSA_TRY(check_optional(in->lse_out, "lse_out"));
  WsPlan plan;
  CSA_TRY(check_ws(p, csa_layer ? CSA_OP_CSA_FWD : CSA_OP_HCA_FWD, ws, ws_bytes, &plan));
  unsigned char* w = static_cast<unsigned char*>(ws);
  const hipStream_t st = as_stream(stream);
  void* kv_c = in->kv_c_out ? in->kv_c_out : static_cast<void*>(w + plan.kv_c);
  void* kv_w = w + plan.kv_w;
  if (tr->events) {
    const int32_t need = 4 + (csa_layer ? index_launches(*p, plan) : 0);
    if (tr->n < need || !tr->kinds) {
      set_error("traced call needs %d events and a kinds array, got %d", need, tr->n);
      return CSA_ERR_INVALID_ARG;
    }
  }
  CSA_HIP(tr->start(st), "event record");
  CSA_HIP(launch_compress(*p, in->va, in->ga, in->vb, in->gb, in->bias, kv_c, st), "compress launch");
  CSA_HIP(tr->mark(CSA_KERNEL_COMPRESS, st), "event record");
  CSA_HIP(launch_window_rope(*p, in->kv_raw, kv_w, st), "window rope launch");
  CSA_HIP(tr->mark(CSA_KERNEL_WINDOW_ROPE, st), "event record");
  int32_t* idx = nullptr;
  if (csa_layer) {
    idx = in->idx_out ? in->idx_out : reinterpret_cast<int32_t*>(w + plan.idx);
    int32_t* nvis = in->n_visible_out ? in->n_visible_out : reinterpret_cast<int32_t*>(w + plan.nvis);
    CSA_TRY(run_index_topk(p, in->q_idx, in->w_idx, in->k_idx, idx, nvis, w, plan, st, tr));
  }
  CSA_HIP(launch_sparse_mqa(*p, csa_layer ? MQA_SELECTED : MQA_DENSE, in->q, kv_c, kv_w, idx, in->sinks, o, in->lse_out, st),
          "attention launch");
  CSA_HIP(tr->mark(CSA_KERNEL_ATTENTION, st), "event record");
  return CSA_OK;
}

csa_status_t csa_fwd(const csa_params_t* p, const csa_inputs_t* in, void* o, void* ws,
                     size_t ws_bytes, void* stream) {
  Tracer none;
  return fused(p, in, o, ws, ws_bytes, stream, true, &none);
}

csa_status_t hca_fwd(const csa_params_t* p, const csa_inputs_t* in, void* o, void* ws,
                     size_t ws_bytes, void* stream) {
  Tracer none;
  return fused(p, in, o, ws, ws_bytes, stream, false, &none);
}

int32_t csa_trace_events(const csa_params_t* p, int32_t op) {
  if (op != CSA_OP_CSA_FWD && op != CSA_OP_HCA_FWD) {
    set_error("op %d has no traced variant", op);
    return 0;
  }
  const bool csa_layer = op == CSA_OP_CSA_FWD;
  const uint32_t need = csa_layer ? (Need::COMPRESS | Need::INDEX | Need::MQA) : (Need::COMPRESS | Need::MQA);
  if (validate_params(p, need, false) != CSA_OK) return 0;
  return 4 + (csa_layer ? index_launches(*p, plan_workspace(*p, op)) : 0);
}

static csa_status_t traced(const csa_params_t* p, const csa_inputs_t* in, void* o, void* ws,
                           size_t ws_bytes, void* stream, void* const* events, int32_t* kinds,
                           int32_t n_events, bool csa_layer) {
  if (!events || !kinds) {
    set_error("events and kinds must be non-NULL");
    return CSA_ERR_INVALID_ARG;
  }
  Tracer tr;
  tr.events = events;
  tr.kinds = kinds;
  tr.n = n_events;
  return fused(p, in, o, ws, ws_bytes, stream, csa_layer, &tr);
}

csa_status_t csa_fwd_traced(const csa_params_t* p, const csa_inputs_t* in, void* o, void* ws,
                            size_t ws_bytes, void* stream, void* const* events, int32_t* kinds,
                            int32_t n_events) {
  return traced(p, in, o, ws, ws_bytes, stream, events, kinds, n_events, true);
}

csa_status_t hca_fwd_traced(const csa_params_t* p, const csa_inputs_t* in, void* o, void* ws,
                            size_t ws_bytes, void* stream, void* const* events, int32_t* kinds,
                            int32_t n_events) {
  return traced(p, in, o, ws, ws_bytes, stream, events, kinds, n_events, false);
}

csa_status_t csa_debug_layout(const csa_params_t* p, int32_t* comp_pos, int32_t* n_visible,
                              int32_t* win_lo, void* stream) {
  if (!p) {
    set_error("params is NULL");
    return CSA_ERR_INVALID_ARG;
  }
  if (p->S < 0 || p->ratio < 1 || p->window < 0) {
    set_error("S=%d ratio=%d window=%d", p->S, p->ratio, p->window);
    return CSA_ERR_INVALID_ARG;
  }
  CSA_HIP(launch_debug_layout(*p, comp_pos, n_visible, win_lo, as_stream(stream)), "layout launch");
  return CSA_OK;
}

}  // extern "C"
