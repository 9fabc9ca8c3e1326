// Host stand-ins for the kernel launchers of libcsa: each records the call and writes
// every byte the real kernel writes (computed from the params), so a workspace plan
// that is too small, or an output placed past the caller's buffer, becomes an
// AddressSanitizer error in the host test.  Inputs are read at their first and last
// byte for the same reason.
#include <string.h>

#include <string>
#include <vector>

#include "launch.hpp"
#include "mqa_bwd.hpp"
#include "mqa_bwd_dkv.hpp"
#include "validate.hpp"

std::vector<std::string> g_calls;
hipError_t g_fail = hipSuccess;  // returned by every launcher when set
int g_events = 0;

const char* hipGetErrorString(hipError_t e) { return e == hipSuccess ? "hipSuccess" : "stub launch failure"; }
hipError_t hipEventRecord(hipEvent_t, hipStream_t) {
  ++g_events;
  return hipSuccess;
}

namespace {
size_t es(const csa_params_t& p) { return p.dtype == CSA_BF16 ? 2 : 4; }
void touch_out(void* p, size_t n) {
  if (n) memset(p, 0x5a, n);
}
volatile unsigned char g_sink;
void touch_in(const void* p, size_t n) {
  if (!n) return;
  const unsigned char* c = static_cast<const unsigned char*>(p);
  g_sink = c[0];
  g_sink = c[n - 1];
}
size_t n_ent(const csa_params_t& p) { return p.ratio > 0 ? (size_t)(p.S / p.ratio) : 0; }
size_t bs(const csa_params_t& p) { return (size_t)p.B * (size_t)p.S; }
hipError_t done(const char* name) {
  g_calls.push_back(name);
  return g_fail;
}
}  // namespace

namespace csa {

hipError_t launch_compress(const csa_params_t& p, const void* va, const void* ga, const void* vb,
                           const void* gb, const float* bias, void* kv_c, hipStream_t) {
  const size_t in = bs(p) * p.D * es(p);
  touch_in(va, in);
  touch_in(ga, in);
  if (p.overlap) {
    touch_in(vb, in);
    touch_in(gb, in);
  }
  touch_in(bias, (size_t)(p.overlap ? 2 : 1) * p.ratio * p.D * 4);
  touch_out(kv_c, (size_t)p.B * n_ent(p) * p.D * es(p));
  return done("compress");
}

hipError_t launch_window_rope(const csa_params_t& p, const void* kv_raw, void* kv_w, hipStream_t) {
  touch_in(kv_raw, bs(p) * p.D * es(p));
  touch_out(kv_w, bs(p) * p.D * es(p));
  return done("window_rope");
}

static size_t key_row_bytes(const csa_params_t& p) {
  return (p.flags & CSA_FLAG_INDEX_FP8) ? (size_t)p.idx_dim + 16 : (size_t)p.idx_dim * es(p);
}

hipError_t launch_index_scores(const csa_params_t& p, const void* q_idx, const float* w_idx,
                               const void* k_idx, float* scores, int64_t ld, int32_t t0,
                               int32_t nrows, hipStream_t) {
  touch_in(q_idx, bs(p) * p.idx_heads * p.idx_dim * es(p));
  touch_in(w_idx, bs(p) * p.idx_heads * 4);
  touch_in(k_idx, (size_t)p.B * n_ent(p) * key_row_bytes(p));
  (void)t0;
  touch_out(scores, (size_t)p.B * (size_t)nrows * (size_t)ld * 4);
  return done("index_scores");
}

hipError_t launch_index_keys(const csa_params_t& p, const void* k_idx, void* k_out, hipStream_t) {
  touch_in(k_idx, (size_t)p.B * n_ent(p) * p.idx_dim * es(p));
  touch_out(k_out, (size_t)p.B * n_ent(p) * key_row_bytes(p));
  return done("index_keys");
}

hipError_t launch_index_topk(const csa_params_t& p, const void* q_idx, const float* w_idx,
                             const void* k_idx, int32_t* idx, int32_t* n_visible, hipStream_t) {
  touch_in(q_idx, bs(p) * p.idx_heads * p.idx_dim * es(p));
  touch_in(w_idx, bs(p) * p.idx_heads * 4);
  touch_in(k_idx, (size_t)p.B * n_ent(p) * key_row_bytes(p));
  touch_out(idx, bs(p) * p.topk * 4);
  if (n_visible) touch_out(n_visible, bs(p) * 4);
  return done("index_topk");
}

hipError_t launch_topk(const csa_params_t& p, const float* scores, int64_t ld, int32_t t0,
                       int32_t nrows, int32_t* idx, int32_t* n_visible, hipStream_t) {
  touch_in(scores, (size_t)p.B * (size_t)nrows * (size_t)ld * 4);
  for (int32_t b = 0; b < p.B; ++b) {
    touch_out(idx + ((size_t)b * p.S + t0) * p.topk, (size_t)nrows * p.topk * 4);
    if (n_visible) touch_out(n_visible + (size_t)b * p.S + t0, (size_t)nrows * 4);
  }
  return done("topk");
}

hipError_t launch_sparse_mqa(const csa_params_t& p, MqaMode mode, const void* q, const void* kv_c,
                             const void* kv_w, const int32_t* idx, const float* sinks, void* o,
                             float* lse, hipStream_t) {
  touch_in(q, bs(p) * p.H * p.D * es(p));
  if (mode != MQA_WINDOW_ONLY) touch_in(kv_c, (size_t)p.B * n_ent(p) * p.D * es(p));
  touch_in(kv_w, bs(p) * p.D * es(p));
  if (mode == MQA_SELECTED) touch_in(idx, bs(p) * p.topk * 4);
  if (sinks) touch_in(sinks, (size_t)p.H * 4);
  touch_out(o, bs(p) * p.H * p.D * es(p));
  if (lse) touch_out(lse, bs(p) * p.H * 4);
  return done(mode == MQA_SELECTED ? "mqa_selected" : mode == MQA_DENSE ? "mqa_dense" : "mqa_window");
}

hipError_t launch_kl_target(const csa_params_t& p, const void* q, const void* kv_c, const int32_t* idx,
                            float* target, hipStream_t) {
  touch_in(q, bs(p) * p.H * p.D * es(p));
  touch_in(kv_c, (size_t)p.B * n_ent(p) * p.D * es(p));
  touch_in(idx, bs(p) * p.topk * 4);
  touch_out(target, bs(p) * p.topk * 4);
  return done("kl_target");
}

hipError_t launch_debug_layout(const csa_params_t& p, int32_t* comp_pos, int32_t* n_visible,
                               int32_t* win_lo, hipStream_t) {
  if (comp_pos) touch_out(comp_pos, n_ent(p) * 4);
  if (n_visible) touch_out(n_visible, (size_t)p.S * 4);
  if (win_lo) touch_out(win_lo, (size_t)p.S * 4);
  return done("debug_layout");
}

hipError_t launch_mqa_bwd_dq(const csa_params_t& p, MqaMode mode, const void* q, const void* kv_c,
                             const void* kv_w, const int32_t* idx, const float* sinks, const void* o,
                             const void* d_o, void* dq, hipStream_t) {
  touch_in(q, bs(p) * p.H * p.D * es(p));
  if (mode != MQA_WINDOW_ONLY) touch_in(kv_c, (size_t)p.B * n_ent(p) * p.D * es(p));
  touch_in(kv_w, bs(p) * p.D * es(p));
  if (mode == MQA_SELECTED) touch_in(idx, bs(p) * p.topk * 4);
  if (sinks) touch_in(sinks, (size_t)p.H * 4);
  touch_in(o, bs(p) * p.H * p.D * es(p));
  touch_in(d_o, bs(p) * p.H * p.D * es(p));
  touch_out(dq, bs(p) * p.H * p.D * es(p));
  return done("bwd_dq");
}

hipError_t launch_zero_f32(float* p, size_t n, hipStream_t) {
  touch_out(p, n * 4);
  return done("zero");
}

// Writes what the real launcher writes, chunk by chunk: the outputs, and in each chunk
// the intermediate rows and the counting-sort and segment regions at their per-chunk
// extents, so a plan smaller than any chunk needs shows up under the sanitizer.
hipError_t launch_mqa_bwd_dkv(const csa_params_t& p, MqaMode mode, const void* q, const void* kv_c,
                              const void* kv_w, const void* kv_raw, const int32_t* idx, const float* sinks,
                              const void* o, const float* lse, const void* d_o, float* dkv_c, float* dkv_raw,
                              float* dsinks, const DkvWs& w, hipStream_t) {
  const size_t act = bs(p) * p.H * p.D * es(p);
  const size_t n = mode == MQA_WINDOW_ONLY ? 0 : n_ent(p);
  touch_in(q, act);
  touch_in(o, act);
  touch_in(d_o, act);
  touch_in(lse, bs(p) * p.H * 4);
  touch_in(kv_w, bs(p) * p.D * es(p));
  touch_in(kv_raw, bs(p) * p.D * es(p));
  if (mode != MQA_WINDOW_ONLY) touch_in(kv_c, (size_t)p.B * n * p.D * es(p));
  if (mode == MQA_SELECTED) touch_in(idx, bs(p) * p.topk * 4);
  if (sinks) touch_in(sinks, (size_t)p.H * 4);
  if (dkv_c) touch_out(dkv_c, (size_t)p.B * n * p.D * 4);
  touch_out(dkv_raw, bs(p) * p.D * 4);
  const DkvShape sh = dkv_shape(p, mode == MQA_SELECTED ? 0 : (mode == MQA_DENSE ? 1 : 2));
  const int64_t rows = (int64_t)bs(p);
  for (int64_t r0 = 0; r0 < rows; r0 += sh.rows) {
    const int64_t nr = rows - r0 < sh.rows ? rows - r0 : sh.rows;
    touch_out(w.interm, (size_t)nr * sh.kw * p.D * es(p));
    if (sh.kmax > 0) {
      const int64_t nkeys = ((r0 + nr - 1) / p.S - r0 / p.S + 1) * (int64_t)n;
      const int64_t nblk = (nr + kDkvRowBlock - 1) / kDkvRowBlock;
      touch_out(w.cnt, (size_t)(nblk * nkeys) * 4);
      touch_out(w.tot, (size_t)nkeys * 4);
      touch_out(w.base, (size_t)(nkeys + 1) * 4);
      touch_out(w.segbase, (size_t)(nkeys + 1) * 4);
      touch_out(w.list, (size_t)(nr * sh.kmax) * 4);
      touch_out(w.partial, (size_t)(nr * sh.kmax / kDkvSeg + nkeys + 1) * p.D * 4);
    }
  }
  if (sinks) {
    touch_out(w.ds_row, bs(p) * p.H * 4);
    touch_out(w.sink_part, (size_t)kDkvSinkGroups * p.H * 4);
    touch_out(dsinks, (size_t)p.H * 4);
  }
  return done("bwd_dkv");
}

}  // namespace csa
