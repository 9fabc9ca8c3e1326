// Host-only argument validation and workspace planning for the C-ABI.  No HIP
// headers: this unit also builds with plain g++ for host sanitizer runs.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "csa.h"

namespace csa {

void set_error(const char* fmt, ...);
const char* last_error();

constexpr int32_t kMaxTopk = 2048;
constexpr int32_t kMaxEntries = 32768;  // entries per row the top-k kernel holds
constexpr size_t kScoresTarget = size_t(128) << 20;  // bytes of scores per chunk
constexpr int32_t kFusedTopkMax = 512;  // top-k selected inside the indexer kernel

enum class Need : uint32_t {
  COMPRESS = 1u << 0,
  INDEX = 1u << 1,
  MQA = 1u << 2,
  SELECT = 1u << 3,  // a top-k selection is read (topk range only)
  INDEX_KEYS = 1u << 4,  // the indexer key prologue alone
};
inline uint32_t operator|(Need a, Need b) { return uint32_t(a) | uint32_t(b); }
inline uint32_t operator|(uint32_t a, Need b) { return a | uint32_t(b); }

// Validate the scalar parameters for the stages in `need` (a mask of Need bits).
// `window_only` marks the attention call without compressed entries.
csa_status_t validate_params(const csa_params_t* p, uint32_t need, bool window_only);

// Non-null and 16-byte aligned.
csa_status_t check_ptr(const void* ptr, const char* name);

size_t elem_size(const csa_params_t& p);
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workspace layout of each op.
struct WsPlan {
  size_t kv_c = 0, kv_w = 0, idx = 0, nvis = 0, scores = 0, k_rot = 0;  // offsets
  size_t total = 0;
  int64_t ld = 0;         // scores row stride (floats)
  int32_t chunk_rows = 0; // query rows per indexer/top-k chunk (0: fused, no scores)
};
WsPlan plan_workspace(const csa_params_t& p, int32_t op);

}  // namespace csa
