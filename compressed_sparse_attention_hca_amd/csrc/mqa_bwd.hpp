// Launcher of the query-side backward of the sparse attention (mqa_bwd.hip).
#pragma once

#include "launch.hpp"

namespace csa {

// dq [B,S,H,D] = dL/dq for the forward of launch_sparse_mqa with the same mode,
// inputs and sinks; o is that forward's output and d_o = dL/do.  kv_w holds the
// rotated window latents (launch_window_rope).
hipError_t launch_mqa_bwd_dq(const csa_params_t& p, MqaMode mode, const void* q, const void* kv_c,
                             const void* kv_w, const int32_t* idx, const float* sinks, const void* o,
                             const void* d_o, void* dq, hipStream_t st);

}  // namespace csa
