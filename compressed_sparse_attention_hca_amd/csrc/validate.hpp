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

// Key-side attention backward: the query rows are taken in chunks whose per-pair
// intermediate ([rows, kw, D] in the activation type) stays within a budget.
constexpr int32_t kDkvRowBlock = 64;           // rows per counting block
constexpr int32_t kDkvSeg = 256;               // pairs per summed segment
constexpr int64_t kDkvMaxChunkRows = 8192;     // rows per chunk at most
constexpr size_t kDkvIntermBudget = size_t(4) << 30;
constexpr int32_t kDkvSinkGroups = 256;        // partial sums of the sink gradient
// mode: 0 selected entries (idx), 1 every visible entry, 2 window only.
struct DkvShape {
  int32_t kmax = 0, kw = 0;  // entry slots, all slots per row
  int64_t rows = 0;          // rows per chunk
  int64_t nblk = 0, nkeys = 0, pairs = 0, segs = 0;  // per-chunk bounds
};
DkvShape dkv_shape(const csa_params_t& p, int mode);

// Workspace layout of each op.
struct WsPlan {
  size_t kv_c = 0, kv_w = 0, idx = 0, nvis = 0, scores = 0, k_rot = 0;  // offsets
  // key-side backward (CSA_OP_SPARSE_MQA_BWD)
  size_t interm = 0, ds_row = 0, sink_part = 0, cnt = 0, tot = 0, base = 0, segbase = 0, list = 0,
         partial = 0;
  size_t total = 0;
  int64_t ld = 0;         // scores row stride (floats)
  int32_t chunk_rows = 0; // query rows per indexer/top-k chunk (0: fused, no scores)
};
WsPlan plan_workspace(const csa_params_t& p, int32_t op);

}  // namespace csa
