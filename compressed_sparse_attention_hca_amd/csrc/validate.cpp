// Host-only validation of C-ABI arguments and workspace planning.
#include "validate.hpp"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>

namespace csa {

static thread_local char g_err[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

const char* last_error() { return g_err; }

size_t elem_size(const csa_params_t& p) { return p.dtype == CSA_BF16 ? 2 : 4; }

#define CSA_FAIL(code, ...)  \
  do {                       \
    set_error(__VA_ARGS__);  \
    return code;             \
  } while (0)

csa_status_t check_ptr(const void* ptr, const char* name) {
  if (!ptr) CSA_FAIL(CSA_ERR_INVALID_ARG, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(ptr) % 16)
    CSA_FAIL(CSA_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return CSA_OK;
}

csa_status_t validate_params(const csa_params_t* p, uint32_t need, bool window_only) {
  if (!p) CSA_FAIL(CSA_ERR_INVALID_ARG, "params is NULL");
  if (p->B < 0 || p->S < 0) CSA_FAIL(CSA_ERR_INVALID_ARG, "B=%d S=%d must be >= 0", p->B, p->S);
  if (p->dtype != CSA_F32 && p->dtype != CSA_BF16)
    CSA_FAIL(CSA_ERR_INVALID_ARG, "dtype=%d is not CSA_F32 or CSA_BF16", p->dtype);
  if (p->flags & ~(CSA_FLAG_NORM_WINDOW | CSA_FLAG_INDEX_PROLOGUE | CSA_FLAG_INDEX_FP8))
    CSA_FAIL(CSA_ERR_INVALID_ARG, "unknown flags 0x%x", p->flags);
  const uint32_t index_any = uint32_t(Need::INDEX) | uint32_t(Need::INDEX_KEYS);
  const bool compressed = (need & uint32_t(Need::COMPRESS)) || (need & index_any) ||
                          ((need & uint32_t(Need::MQA)) && !window_only);
  if (need & (uint32_t(Need::COMPRESS) | uint32_t(Need::MQA))) {
    if (p->D <= 0 || p->D % 64 || p->D > 512)
      CSA_FAIL(CSA_ERR_INVALID_ARG, "D=%d must be a multiple of 64 in 64..512", p->D);
    if (p->D != 64 && p->D != 128 && p->D != 256 && p->D != 512)
      CSA_FAIL(CSA_ERR_UNSUPPORTED, "D=%d: compiled for 64, 128, 256, 512", p->D);
    if (p->rope_dim < 0 || p->rope_dim % 2 || p->rope_dim > p->D)
      CSA_FAIL(CSA_ERR_INVALID_ARG, "rope_dim=%d must be even and <= D=%d", p->rope_dim, p->D);
    if (p->rope_dim > 128) CSA_FAIL(CSA_ERR_UNSUPPORTED, "rope_dim=%d > 128", p->rope_dim);
    if (!(p->rope_theta > 0.0) || !isfinite(p->rope_theta))
      CSA_FAIL(CSA_ERR_INVALID_ARG, "rope_theta must be positive and finite");
    if (!(p->rms_eps >= 0.0f) || !isfinite(p->rms_eps))
      CSA_FAIL(CSA_ERR_INVALID_ARG, "rms_eps must be >= 0 and finite");
  }
  if (compressed) {
    if (p->ratio < 1) CSA_FAIL(CSA_ERR_INVALID_ARG, "ratio=%d must be >= 1", p->ratio);
    if (p->S % p->ratio) CSA_FAIL(CSA_ERR_INVALID_ARG, "S=%d is not a multiple of ratio=%d", p->S, p->ratio);
    if (p->overlap != 0 && p->overlap != 1) CSA_FAIL(CSA_ERR_INVALID_ARG, "overlap=%d must be 0 or 1", p->overlap);
  }
  if (need & uint32_t(Need::MQA)) {
    if (p->H < 1 || p->H > 64) CSA_FAIL(CSA_ERR_INVALID_ARG, "H=%d must be in 1..64", p->H);
    if (p->window < 0) CSA_FAIL(CSA_ERR_INVALID_ARG, "window=%d must be >= 0", p->window);
    if (window_only && p->window < 1)
      CSA_FAIL(CSA_ERR_INVALID_ARG, "window=%d must be >= 1 without compressed entries", p->window);
    if (!(p->softmax_scale > 0.0f) || !isfinite(p->softmax_scale))
      CSA_FAIL(CSA_ERR_INVALID_ARG, "softmax_scale must be positive and finite");
  }
  if (need & (uint32_t(Need::INDEX) | uint32_t(Need::SELECT))) {
    if (p->topk < 1 || p->topk > kMaxTopk)
      CSA_FAIL(CSA_ERR_INVALID_ARG, "topk=%d must be in 1..%d", p->topk, kMaxTopk);
  }
  if (need & index_any) {
    if (p->idx_heads < 1 || p->idx_heads > 64)
      CSA_FAIL(CSA_ERR_INVALID_ARG, "idx_heads=%d must be in 1..64", p->idx_heads);
    if (p->idx_dim < 16 || p->idx_dim % 16)
      CSA_FAIL(CSA_ERR_INVALID_ARG, "idx_dim=%d must be a positive multiple of 16", p->idx_dim);
    if (p->idx_dim != 16 && p->idx_dim != 32 && p->idx_dim != 64 && p->idx_dim != 128)
      CSA_FAIL(CSA_ERR_UNSUPPORTED, "idx_dim=%d: compiled for 16, 32, 64, 128", p->idx_dim);
    if (p->S / p->ratio > kMaxEntries)
      CSA_FAIL(CSA_ERR_UNSUPPORTED, "S/ratio=%d entries exceeds %d", p->S / p->ratio, kMaxEntries);
  }
  if (need & uint32_t(Need::INDEX_KEYS)) {
    if (!(p->flags & (CSA_FLAG_INDEX_PROLOGUE | CSA_FLAG_INDEX_FP8)))
      CSA_FAIL(CSA_ERR_INVALID_ARG, "the key pass needs CSA_FLAG_INDEX_PROLOGUE or CSA_FLAG_INDEX_FP8");
  }
  if ((need & index_any) && (p->flags & CSA_FLAG_INDEX_FP8) && p->idx_dim != 64 && p->idx_dim != 128)
    CSA_FAIL(CSA_ERR_UNSUPPORTED, "the FP8 indexer is compiled for idx_dim 64 and 128, not %d", p->idx_dim);
  // the indexer prologue rotates with the layer's RoPE inside the indexer dims
  if ((need & index_any) && (p->flags & CSA_FLAG_INDEX_PROLOGUE)) {
    if (p->rope_dim < 0 || p->rope_dim % 2 || p->rope_dim > p->idx_dim)
      CSA_FAIL(CSA_ERR_INVALID_ARG, "indexer prologue: rope_dim=%d must be even and <= idx_dim=%d",
               p->rope_dim, p->idx_dim);
    if (!(p->rope_theta > 0.0) || !isfinite(p->rope_theta))
      CSA_FAIL(CSA_ERR_INVALID_ARG, "rope_theta must be positive and finite");
  }
  return CSA_OK;
}

DkvShape dkv_shape(const csa_params_t& p, int mode) {
  DkvShape s;
  const int64_t B = p.B > 0 ? p.B : 0, S = p.S > 0 ? p.S : 0, all = B * S;
  const int64_t n = (mode != 2 && p.ratio >= 1) ? S / p.ratio : 0;
  s.kmax = mode == 0 ? p.topk : (mode == 1 ? (int32_t)n : 0);
  s.kw = s.kmax + (p.window > 0 ? p.window : 0);
  const size_t row_bytes = (size_t)s.kw * (size_t)(p.D > 0 ? p.D : 0) * elem_size(p);
  int64_t rows = all < kDkvMaxChunkRows ? all : kDkvMaxChunkRows;
  if (row_bytes) {
    const int64_t fit = (int64_t)(kDkvIntermBudget / row_bytes);
    if (rows > (fit > 0 ? fit : 1)) rows = fit > 0 ? fit : 1;
  }
  if (rows < all && rows >= kDkvRowBlock) rows -= rows % kDkvRowBlock;
  s.rows = rows;
  s.nblk = (rows + kDkvRowBlock - 1) / kDkvRowBlock;
  if (s.kmax > 0 && S > 0) {
    int64_t spans = (rows + S - 1) / S + 1;  // sequences a chunk can touch
    if (spans > B) spans = B;
    s.nkeys = spans * n;
  }
  s.pairs = rows * s.kmax;
  s.segs = s.pairs / kDkvSeg + s.nkeys + 1;
  return s;
}

WsPlan plan_workspace(const csa_params_t& p, int32_t op) {
  WsPlan w;
  const size_t es = elem_size(p);
  const size_t B = (size_t)p.B, S = (size_t)p.S;
  const size_t n = p.ratio > 0 ? S / (size_t)p.ratio : 0;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes, 256);
    return at;
  };
  const bool idx = op == CSA_OP_INDEX_TOPK || op == CSA_OP_CSA_FWD;
  if (op == CSA_OP_CSA_FWD || op == CSA_OP_HCA_FWD) w.kv_c = take(B * n * (size_t)p.D * es);
  if (op == CSA_OP_SPARSE_MQA || op == CSA_OP_CSA_FWD || op == CSA_OP_HCA_FWD || op == CSA_OP_SPARSE_MQA_BWD)
    w.kv_w = take(B * S * (size_t)p.D * es);
  if (op == CSA_OP_SPARSE_MQA_BWD) {  // sized for every mode these params allow
    size_t interm = 0, nblk = 0, nkeys = 0, pairs = 0, segs = 0;
    const bool entries = p.ratio >= 1 && S % (size_t)p.ratio == 0;
    for (int mode = 0; mode < 3; ++mode) {
      if (mode == 0 && !(entries && p.topk >= 1 && p.topk <= kMaxTopk)) continue;
      if (mode == 1 && !entries) continue;
      const DkvShape d = dkv_shape(p, mode);
      const size_t ib = (size_t)d.rows * (size_t)d.kw * (size_t)p.D * es;
      interm = ib > interm ? ib : interm;
      if (d.kmax > 0) {
        nblk = (size_t)d.nblk > nblk ? (size_t)d.nblk : nblk;
        nkeys = (size_t)d.nkeys > nkeys ? (size_t)d.nkeys : nkeys;
        pairs = (size_t)d.pairs > pairs ? (size_t)d.pairs : pairs;
        segs = (size_t)d.segs > segs ? (size_t)d.segs : segs;
      }
    }
    w.interm = take(interm);
    w.ds_row = take(B * S * (size_t)p.H * 4);
    w.sink_part = take((size_t)kDkvSinkGroups * (size_t)p.H * 4);
    w.cnt = take(nblk * nkeys * 4);
    w.tot = take(nkeys * 4);
    w.base = take((nkeys + 1) * 4);
    w.segbase = take((nkeys + 1) * 4);
    w.list = take(pairs * 4);
    w.partial = take(segs * (size_t)p.D * 4);
  }
  if (op == CSA_OP_CSA_FWD) {
    w.idx = take(B * S * (size_t)p.topk * 4);
    w.nvis = take(B * S * 4);
  }
  if (idx && (p.flags & CSA_FLAG_INDEX_FP8)) w.k_rot = take(B * n * (size_t)(p.idx_dim + 16));
  else if (idx && (p.flags & CSA_FLAG_INDEX_PROLOGUE)) w.k_rot = take(B * n * (size_t)p.idx_dim * es);
  if (idx && p.topk > kFusedTopkMax) {  // separate scores + top-k kernels over chunks
    w.ld = (int64_t)align_up(n > 0 ? n : 1, 32);
    const size_t row_bytes = B * (size_t)w.ld * 4;
    size_t rows = row_bytes ? kScoresTarget / row_bytes : S;
    if (rows < 64) rows = 64;
    if (rows > S) rows = S;
    w.chunk_rows = (int32_t)rows;
    w.scores = take(rows * row_bytes);
  }
  w.total = off;
  return w;
}

}  // namespace csa
