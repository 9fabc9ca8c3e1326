// Internal launcher interface between the C-ABI host code and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "csa.h"

namespace csa {

enum MqaMode : int32_t { MQA_SELECTED = 0, MQA_DENSE = 1, MQA_WINDOW_ONLY = 2 };

hipError_t launch_compress(const csa_params_t& p, const void* va, const void* ga, const void* vb,
                           const void* gb, const float* bias, void* kv_c, hipStream_t st);

hipError_t launch_window_rope(const csa_params_t& p, const void* kv_raw, void* kv_w, hipStream_t st);

hipError_t launch_index_scores(const csa_params_t& p, const void* q_idx, const float* w_idx,
                               const void* k_idx, float* scores, int64_t ld, int32_t t0,
                               int32_t nrows, hipStream_t st);

// Indexer key pass: k_out = round(Hn RoPE(k_idx, pos0 + s*ratio)) (prologue) and/or
// the E4M3 rows (fp8), per p.flags.
hipError_t launch_index_keys(const csa_params_t& p, const void* k_idx, void* k_out, hipStream_t st);

// Indexer scores fused with the top-k selection (topk <= 512); scores stay on chip.
hipError_t launch_index_topk(const csa_params_t& p, const void* q_idx, const float* w_idx,
                             const void* k_idx, int32_t* idx, int32_t* n_visible, hipStream_t st);

hipError_t launch_topk(const csa_params_t& p, const float* scores, int64_t ld, int32_t t0,
                       int32_t nrows, int32_t* idx, int32_t* n_visible, hipStream_t st);

// sinks [H] fp32 or nullptr: per-head softmax-sink logits.  lse [B,S,H] fp32 or
// nullptr: the natural log of each head's softmax denominator (sink included).
hipError_t launch_sparse_mqa(const csa_params_t& p, MqaMode mode, const void* q, const void* kv_c,
                             const void* kv_w, const int32_t* idx, const float* sinks, void* o,
                             float* lse, hipStream_t st);

// Target of the indexer's distillation loss over the selected entries ([B,S,topk] fp32).
hipError_t launch_kl_target(const csa_params_t& p, const void* q, const void* kv_c, const int32_t* idx,
                            float* target, hipStream_t st);

hipError_t launch_debug_layout(const csa_params_t& p, int32_t* comp_pos, int32_t* n_visible,
                               int32_t* win_lo, hipStream_t st);

}  // namespace csa
