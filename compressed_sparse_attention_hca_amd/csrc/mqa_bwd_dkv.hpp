// Launcher of the key-side backward of the sparse attention (mqa_bwd_dkv.hip).
#pragma once

#include "launch.hpp"

namespace csa {

// Workspace regions (device pointers), laid out by plan_workspace(p, CSA_OP_SPARSE_MQA_BWD).
struct DkvWs {
  void* interm;       // per-pair key gradients of one chunk of rows
  float* ds_row;      // per-query sink terms [B,S,H]
  float* sink_part;   // partial sums of the sink gradient
  int32_t* cnt;       // counting-sort table [blocks][keys]
  int32_t* tot;
  int32_t* base;
  int32_t* segbase;
  int32_t* list;      // pair rows by entry
  float* partial;     // segment sums
};

// dkv_c [B,S/ratio,D] (nullptr for the window-only layer), dkv_raw [B,S,D] and dsinks
// [H] (nullptr without sinks), all fp32 and overwritten: the gradients of the forward
// of launch_sparse_mqa with the same mode, inputs and sinks, given its output o, its
// log-denominators lse [B,S,H] and d_o = dL/do.  kv_w holds the rotated window latents
// (launch_window_rope); kv_raw the raw ones (read for the window norm's gradient).
hipError_t launch_mqa_bwd_dkv(const csa_params_t& p, MqaMode mode, const void* q, const void* kv_c,
                              const void* kv_w, const void* kv_raw, const int32_t* idx, const float* sinks,
                              const void* o, const float* lse, const void* d_o, float* dkv_c, float* dkv_raw,
                              float* dsinks, const DkvWs& w, hipStream_t st);

// Zero n floats on the stream (a fill kernel).
hipError_t launch_zero_f32(float* p, size_t n, hipStream_t st);

}  // namespace csa
