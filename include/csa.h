/*
 * csa.h -- C-ABI of the MI355X (gfx950) forward kernels for the DeepSeek-V4-Flash
 * compressed attention layer: compressed sparse attention (CSA), heavily compressed
 * attention (HCA) and the window-only layer.
 *
 * The layer, in four stages, as the pages define it:
 *   1. softmax-gated pooling of per-token KV latents into compressed entries
 *      ("Enabling DeepSeek-V4-Flash Training on AMD Instinct MI355X GPUs with
 *      Primus", subsection "Three attention types, interleaved": a softmax over the
 *      group of gate plus a learnable per-position bias weights the sum; CSA groups
 *      of 4 overlap the previous 4 tokens, HCA groups of 128 are disjoint);
 *   2. RMSNorm of each entry, then RoPE on its last rope_dim dims at the entry's
 *      original-sequence position pos0 + s*ratio ("fix(deepseek-v4): correct
 *      V4-Flash attention math", Part 1 item 2; RMSNorm of entries: item 1);
 *   3. CSA only: lightning-indexer scores I[t,s] = sum_h w[t,h] ReLU(q_I[t,h].k_I[s])
 *      over every causally visible entry, then the top-k entries per query (same
 *      PR, items 4 and 6a; blog, "Three attention types, interleaved");
 *   4. multi-query attention of H heads over one shared D-wide latent that is both
 *      key and value, across the selected entries plus a sliding window of raw
 *      tokens, scale head_dim**-0.5 with no YaRN factor (PR item 1), then the
 *      output's RoPE dims rotated back at -(pos0 + t) (PR item 3).
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers, contiguous row-major, batch-major, and
 *     16-byte aligned.  Activations use params->dtype; bias, indexer head weights and
 *     scores are always fp32; idx and n_visible are int32.  Accumulation is fp32.
 *   - `stream` is a hipStream_t passed as void* (NULL = default stream).  Every call
 *     only enqueues work on that stream and returns; nothing synchronises.
 *   - The library never allocates or frees memory.  The caller owns every buffer,
 *     including the workspace, whose size comes from csa_workspace_bytes(); its
 *     contents are undefined on return.  (csa_fwd_noalloc alone uses a static
 *     workspace that the library holds; see there.)
 *   - Arguments are validated on the host before any launch.  A bad argument
 *     returns a status and enqueues nothing; csa_last_error() then holds a
 *     thread-local message.  No exception crosses the ABI and nothing aborts.
 *     CSA_ERR_HIP reports a launch failure; errors raised while kernels run surface
 *     at the caller's next synchronisation.
 *   - Calls are re-entrant: the library keeps no global mutable state apart from the
 *     thread-local error string (and the static workspace of csa_fwd_noalloc).
 *
 * Integer layout shared by every kernel (bit-exact, see csa_debug_layout):
 *   n_visible(t) = floor((t + 1) / ratio)   entries whose whole group is seen by t
 *   comp_pos(s)  = pos0 + s * ratio         rotation position of entry s
 *   win_lo(t)    = max(0, t - window + 1)   window tokens win_lo(t) .. t
 */
#ifndef CSA_H_
#define CSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA_ABI_VERSION 8

typedef enum {
  CSA_OK = 0,
  CSA_ERR_INVALID_ARG = 1, /* null required pointer, inconsistent shape, misalignment */
  CSA_ERR_WORKSPACE = 2,   /* ws_bytes below csa_workspace_bytes() */
  CSA_ERR_UNSUPPORTED = 3, /* valid but outside the compiled shape set, or no gfx950 */
  CSA_ERR_HIP = 4          /* a HIP launch failed */
} csa_status_t;

typedef enum { CSA_F32 = 0, CSA_BF16 = 1 } csa_dtype_t;

typedef enum {
  CSA_OP_COMPRESS = 0,
  CSA_OP_INDEX_TOPK = 1,
  CSA_OP_SPARSE_MQA = 2,
  CSA_OP_CSA_FWD = 3,
  CSA_OP_HCA_FWD = 4,
  CSA_OP_SPARSE_MQA_BWD = 5 /* csa_sparse_mqa_bwd_dkv */
} csa_op_t;

/* flags */
#define CSA_FLAG_NORM_WINDOW 1u /* RMS-normalise window latents before their RoPE */
/* Indexer prologue ("fix(deepseek-v4): correct V4-Flash attention math", Part 1
 * items 6e and 6a), CSA only.  The indexer scores
 *   I[t,s] = sum_h (T w[t,h]) ReLU(q'[t,h] . k'[s]),   T = (idx_heads * idx_dim)**-0.5,
 *   q'[t,h] = round(Hn RoPE(q_I[t,h], pos0 + t)),  k'[s] = round(Hn RoPE(k_I[s], pos0 + s*ratio)),
 * where RoPE is the layer's (interleaved pairs on the last rope_dim dims, base
 * rope_theta; rope_dim must be <= idx_dim), Hn = H / sqrt(idx_dim) is the normalised
 * Sylvester Hadamard matrix (H[i][j] = (-1)^popcount(i & j)), and round() rounds to the
 * activation dtype.  The top-k is unchanged by T but not by the rotation:
 * csa_index_scores writes the scores with T, while the fused selection of
 * csa_index_topk / csa_fwd (topk <= 512) ranks them without it. */
#define CSA_FLAG_INDEX_PROLOGUE 2u
/* FP8 indexer ("Enabling DeepSeek-V4-Flash Training on AMD Instinct MI355X GPUs with
 * Primus", closing remarks: an E4M3 path for the indexer QK; "fix(deepseek-v4) ...",
 * Part 1 item 4: it changes the selection, so it is opt-in), CSA only, idx_dim 64 or
 * 128.  Each q_I[t,h] and k_I[s] row (after the prologue, when both flags are set) is
 * quantized to OCP E4M3 with its own scale: m = max |x|, codes = E4M3(x * (448 / m)),
 * round to nearest even, scale = m / 448 (both divisions and the product in IEEE
 * fp32; a zero row has codes 0, scale 0); the scores use the decoded operands
 * codes * scale, accumulated in fp32 by the fp8 MFMA. */
#define CSA_FLAG_INDEX_FP8 4u

typedef struct {
  int32_t B;          /* batch */
  int32_t S;          /* tokens per sequence; a multiple of ratio */
  int32_t H;          /* query heads, 1..64 */
  int32_t D;          /* latent width = head dim: 64, 128, 256 or 512 */
  int32_t rope_dim;   /* RoPE on the last rope_dim dims: even, <= D, <= 128 */
  int32_t ratio;      /* compress ratio (4 for CSA, 128 for HCA in V4-Flash) */
  int32_t overlap;    /* 1: CSA groups of 2*ratio (own + previous); 0: disjoint */
  int32_t window;     /* sliding-window length, >= 0 */
  int32_t topk;       /* entries kept per query (CSA), 1..2048 */
  int32_t idx_heads;  /* indexer heads, 1..64 */
  int32_t idx_dim;    /* indexer dim: 16, 32, 64 or 128 */
  int32_t dtype;      /* csa_dtype_t of activations */
  double rope_theta;  /* RoPE base, 40000 for V4-Flash */
  float rms_eps;      /* RMSNorm epsilon (1e-6) */
  float softmax_scale;/* D**-0.5 */
  int64_t pos0;       /* absolute position of token 0 */
  uint32_t flags;     /* CSA_FLAG_* */
} csa_params_t;

/* Device pointers for the fused calls.  Shapes: q [B,S,H,D], kv_raw [B,S,D],
 * va ga vb gb [B,S,D], bias [span,D] fp32 (span = 2*ratio with overlap, else ratio),
 * q_idx [B,S,idx_heads,idx_dim], w_idx [B,S,idx_heads] fp32, k_idx [B,S/ratio,idx_dim].
 * The *_out pointers are optional (NULL = keep in workspace only): kv_c_out
 * [B,S/ratio,D], idx_out [B,S,topk], n_visible_out [B,S].
 * sinks [H] fp32 is optional (NULL = no sink): one softmax-sink logit per head, shared
 * by every batch and token, see csa_sparse_mqa_fwd_sink.  lse_out [B,S,H] fp32 is
 * optional (NULL = not kept): the attention's log-denominators, as
 * csa_sparse_mqa_fwd_lse writes them, for csa_sparse_mqa_bwd_dkv. */
typedef struct {
  const void* q;
  const void* kv_raw;
  const void* va;
  const void* ga;
  const void* vb;
  const void* gb;
  const float* bias;
  const void* q_idx;
  const float* w_idx;
  const void* k_idx;
  void* kv_c_out;
  int32_t* idx_out;
  int32_t* n_visible_out;
  const float* sinks;
  float* lse_out;
} csa_inputs_t;

/* Stages 1-2: gated pooling, RMSNorm and RoPE at pos0 + s*ratio.
 *   va, ga [B,S,D]: value and gate of each entry's own group ("a" projections);
 *   vb, gb [B,S,D]: value and gate read for the previous group ("b" projections);
 *     must be non-NULL iff overlap == 1;
 *   bias [span,D] fp32: row j weights pooling slot j in token order (with overlap,
 *     rows 0..ratio-1 are the previous group, rows ratio..2*ratio-1 the own group);
 *   kv_c [B,S/ratio,D] output.  CSA entry 0 has no previous group: those slots are
 *   left out of its softmax. */
csa_status_t csa_compress(const csa_params_t* p, const void* va, const void* ga,
                          const void* vb, const void* gb, const float* bias, void* kv_c,
                          void* stream);

/* Stage 3, scores only (for checking): rows t0 .. t0+nrows-1 of every batch;
 * scores[b][t - t0][s] for s < n_visible(t), row stride ld floats (ld >= S/ratio);
 * entries s >= n_visible(t) are not written.  With CSA_FLAG_INDEX_PROLOGUE and/or
 * CSA_FLAG_INDEX_FP8 the queries are transformed and the weights scaled inside the
 * kernel, and k_idx must hold the output of csa_index_keys for the same flags. */
csa_status_t csa_index_scores(const csa_params_t* p, const void* q_idx, const float* w_idx,
                              const void* k_idx, float* scores, int64_t ld, int32_t t0,
                              int32_t nrows, void* stream);

/* Indexer key pass for CSA_FLAG_INDEX_PROLOGUE and/or CSA_FLAG_INDEX_FP8 (at least one
 * must be set in p->flags; see both).  k_idx [B,S/ratio,idx_dim] in the activation
 * dtype.  k_out, which must not overlap k_idx:
 *   - prologue only: [B,S/ratio,idx_dim] in the activation dtype,
 *     k_out[b,s] = round(Hn RoPE(k_idx[b,s], pos0 + s*ratio));
 *   - FP8: [B,S/ratio] rows of idx_dim + 16 bytes: the E4M3 codes of the row (after
 *     the prologue, if set) with dim d at byte 64*(d/64) + 32*((d/8)%2) +
 *     8*((d%64)/16) + d%8 (the fp8 MFMA operand order), then the fp32 scale, then 12
 *     zero bytes.
 * The other indexer fields and rope_dim, rope_theta, pos0 are used. */
csa_status_t csa_index_keys(const csa_params_t* p, const void* k_idx, void* k_out, void* stream);

/* Stage 3: indexer scores over visible entries and the top-k per query.
 *   idx [B,S,topk] int32: the min(topk, n_visible(t)) selected entries in ascending
 *   order, then -1 padding; ties at the k-th score go to the smaller entry index.
 *   n_visible [B,S] int32.  ws: csa_workspace_bytes(p, CSA_OP_INDEX_TOPK) bytes (none
 *   when topk <= 512: the selection is made inside the indexer kernel and no score
 *   leaves the chip; larger topk scores query chunks into the workspace, then selects).
 *   With CSA_FLAG_INDEX_PROLOGUE or CSA_FLAG_INDEX_FP8 the key pass's output is also
 *   kept in the workspace. */
csa_status_t csa_index_topk(const csa_params_t* p, const void* q_idx, const float* w_idx,
                            const void* k_idx, int32_t* idx, int32_t* n_visible, void* ws,
                            size_t ws_bytes, void* stream);

/* Stage 4: attention over selected entries plus the window, then de-rotation.
 *   q [B,S,H,D] (RMS-normalised upstream; rotated here at pos0 + t);
 *   kv_c [B,S/ratio,D] rotated entries, or NULL for the window-only layer;
 *   kv_raw [B,S,D] raw latents of the window (rotated here at their positions);
 *   idx [B,S,topk] selection, or NULL to attend to every visible entry (HCA);
 *     an index outside 0..n_visible(t)-1 is ignored;
 *   o [B,S,H,D] output.  ws: csa_workspace_bytes(p, CSA_OP_SPARSE_MQA) bytes. */
csa_status_t csa_sparse_mqa_fwd(const csa_params_t* p, const void* q, const void* kv_c,
                                const void* kv_raw, const int32_t* idx, void* o, void* ws,
                                size_t ws_bytes, void* stream);

/* Stage 4 with a softmax sink ("Enabling DeepSeek-V4-Flash Training on AMD Instinct
 * MI355X GPUs with Primus", section "Kernel fusions", row "SWA / CSA / HCA attention":
 * the attention kernel folds in the softmax sink; "fix(deepseek-v4): correct V4-Flash
 * attention math", Part 1 item 6f: the sink is an FP32 logit that feeds the softmax).
 *   sinks [H] fp32, or NULL for none: head h's softmax also normalises over the logit
 *   sinks[h], which carries no value, so exp(sinks[h]) joins the denominator and a
 *   query with no key gets o = 0.  Other arguments and errors as csa_sparse_mqa_fwd. */
csa_status_t csa_sparse_mqa_fwd_sink(const csa_params_t* p, const void* q, const void* kv_c,
                                     const void* kv_raw, const int32_t* idx, const float* sinks,
                                     void* o, void* ws, size_t ws_bytes, void* stream);

/* Stage 4 as csa_sparse_mqa_fwd_sink, also keeping what its backward needs
 * ("Enabling DeepSeek-V4-Flash Training on AMD Instinct MI355X GPUs with Primus",
 * section "Attention kernels for the three layer types": the backward kernels recompute
 * the softmax of the forward):
 *   lse [B,S,H] fp32 output: lse[b,t,h] = log( sum_k exp(z[h,k]) + exp(sinks[h]) ), the
 *   natural log of head h's softmax denominator over the logits z = (RoPE(q, pos0+t) .
 *   key) * softmax_scale the forward forms (the sink term only with sinks), so that
 *   p[h,k] = exp(z[h,k] - lse[h]); -inf for a head with no valid key and no sink.
 * Other arguments, results and errors as csa_sparse_mqa_fwd_sink, plus
 * CSA_ERR_INVALID_ARG for a NULL lse. */
csa_status_t csa_sparse_mqa_fwd_lse(const csa_params_t* p, const void* q, const void* kv_c,
                                    const void* kv_raw, const int32_t* idx, const float* sinks,
                                    void* o, float* lse, void* ws, size_t ws_bytes, void* stream);

/* Backward of stage 4, query side ("Enabling DeepSeek-V4-Flash Training on AMD
 * Instinct MI355X GPUs with Primus", section "Attention kernels for the three layer
 * types": the dQ kernel, with delta = rowsum(o * do) computed inside it):
 *   dq[b,t,h] = dL/dq[b,t,h] for the forward csa_sparse_mqa_fwd_sink with the same
 *   params, q, kv_c, kv_raw, idx and sinks (NULL alike), given o (that forward's
 *   output [B,S,H,D]) and d_o = dL/do [B,S,H,D].  With P = pos0 + t, du = RoPE(d_o, +P)
 *   and delta[h] = sum_d o[h,d] d_o[h,d]:
 *     dq[h] = RoPE( softmax_scale * sum_k p[h,k] (du[h] . key_k - delta[h]) key_k , -P )
 *   over the same keys and softmax p as the forward (sink in the denominator only).
 *   The selection is held fixed (top-k has no gradient).  dq [B,S,H,D] in the
 *   activation dtype; the gradients of kv_c, kv_raw and the sinks are not computed
 *   here.  ws: csa_workspace_bytes(p, CSA_OP_SPARSE_MQA) bytes.  Errors as
 *   csa_sparse_mqa_fwd_sink, plus CSA_ERR_INVALID_ARG for a NULL o, d_o or dq. */
csa_status_t csa_sparse_mqa_bwd_dq(const csa_params_t* p, const void* q, const void* kv_c,
                                   const void* kv_raw, const int32_t* idx, const float* sinks,
                                   const void* o, const void* d_o, void* dq, void* ws,
                                   size_t ws_bytes, void* stream);

/* Backward of stage 4, key side ("Enabling DeepSeek-V4-Flash Training on AMD Instinct
 * MI355X GPUs with Primus", section "Attention kernels for the three layer types":
 * interm, the contraction over heads that gives each key's gradient, and the scatter of
 * those gradients back to the entries; "fix(deepseek-v4): correct V4-Flash attention
 * math", Part 1 item 6f: the sink is an fp32 logit of the softmax).  For the forward
 * csa_sparse_mqa_fwd_lse with the same params, q, kv_c, kv_raw, idx and sinks, given
 * its o and lse and d_o = dL/do [B,S,H,D], with the selection held fixed:
 *   dkv_c [B,S/ratio,D] fp32 = dL/dkv_c (the rotated entries; a selected entry
 *     collects the key gradient of every query that selected it):
 *       dkey_k = sum_h ( softmax_scale p[h,k] (du[h].key_k - delta[h]) RoPE(q[h], P)
 *                        + p[h,k] du[h] ),  du = RoPE(d_o, P), delta[h] = o[h].d_o[h],
 *     p = exp(z - lse), P = pos0 + t; NULL exactly when kv_c is NULL;
 *   dkv_raw [B,S,D] fp32 = dL/dkv_raw: the key gradients of window token t' over every
 *     query whose window holds it, rotated by -(pos0 + t') and, with
 *     CSA_FLAG_NORM_WINDOW, taken through the RMSNorm;
 *   dsinks [H] fp32 = dL/dsinks[h] = -sum_{b,t} exp(sinks[h] - lse[b,t,h]) delta[b,t,h];
 *     non-NULL exactly when sinks is.
 * The outputs are overwritten (zero where nothing contributes).  Sums are fp32 in an
 * order that does not depend on timing, so two calls give identical results; the
 * per-pair gradients pass through the workspace in the activation dtype.  fp32
 * activations need D <= 256 (CSA_ERR_UNSUPPORTED at 512).  ws:
 * csa_workspace_bytes(p, CSA_OP_SPARSE_MQA_BWD) bytes (at most about 4.2 GiB plus the
 * rotated window latents and per-query terms).  Errors as csa_sparse_mqa_fwd_sink,
 * plus CSA_ERR_INVALID_ARG for a NULL o, lse, d_o or dkv_raw, or a dkv_c or dsinks
 * that does not match kv_c or sinks. */
csa_status_t csa_sparse_mqa_bwd_dkv(const csa_params_t* p, const void* q, const void* kv_c,
                                    const void* kv_raw, const int32_t* idx, const float* sinks,
                                    const void* o, const float* lse, const void* d_o, float* dkv_c,
                                    float* dkv_raw, float* dsinks, void* ws, size_t ws_bytes,
                                    void* stream);

/* Target distribution of the indexer's distillation loss ("fix(deepseek-v4): correct
 * V4-Flash attention math", Part 1 item 5: KL(attention || indexer) over the selected
 * entries, kept in [B, S, K]; item 11: the head sum inside the loop, so the per-head
 * tensor never exists):
 *   target[b,t,k] = (1/H) sum_h softmax_k( (RoPE(q[b,t,h], pos0 + t) . kv_c[b, idx[b,t,k]]) * softmax_scale )
 * for k < min(topk, n_visible(t)), the softmax over those selected entries only (no
 * window), the logits as the attention forms them (activation-dtype operands, fp32
 * accumulation).  q [B,S,H,D], kv_c [B,S/ratio,D] rotated entries, idx [B,S,topk] as
 * csa_index_topk writes it; target [B,S,topk] fp32, 0 past the selection.  An index
 * outside 0..n_visible(t)-1 is left out of the softmax and gets 0. */
csa_status_t csa_kl_target(const csa_params_t* p, const void* q, const void* kv_c,
                           const int32_t* idx, float* target, void* stream);

/* Fused CSA layer (stages 1-4, overlap must be 1). */
csa_status_t csa_fwd(const csa_params_t* p, const csa_inputs_t* in, void* o, void* ws,
                     size_t ws_bytes, void* stream);

/* Fused HCA layer (stages 1, 2 and 4 with every visible entry; overlap must be 0;
 * the indexer fields of `in` are ignored). */
csa_status_t hca_fwd(const csa_params_t* p, const csa_inputs_t* in, void* o, void* ws,
                     size_t ws_bytes, void* stream);

/* csa_fwd without a caller workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, kernels and results as csa_fwd; the workspace is a
 * static device array of CSA_NOALLOC_SCRATCH_BYTES that the library holds on each GPU
 * it runs on until the process ends, on the device of `stream`.  A shape whose
 * workspace (csa_workspace_bytes(p, CSA_OP_CSA_FWD)) exceeds it returns
 * CSA_ERR_WORKSPACE and enqueues nothing; the CSA layer at B = 1, S = 65536,
 * D = 512 bf16, top-512 fits.  Nothing is allocated, freed or cleared.  Every call on
 * one GPU shares that GPU's array, so two calls that overlap in time on one GPU race:
 * keep them on one stream or order them with events.  The first call on a device also
 * looks up the array's device address (hipGetSymbolAddress), which may briefly make
 * that device current on the calling thread. */
#define CSA_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
csa_status_t csa_fwd_noalloc(const csa_params_t* p, const csa_inputs_t* in, void* o, void* stream);

/* Kernels of the fused calls, as reported by the traced variants below. */
typedef enum {
  CSA_KERNEL_COMPRESS = 0,    /* pooling + RMSNorm + RoPE of entries */
  CSA_KERNEL_WINDOW_ROPE = 1, /* rotation of the raw window latents */
  CSA_KERNEL_INDEXER = 2,     /* indexer scores (one launch per query chunk, topk > 512) */
  CSA_KERNEL_TOPK = 3,        /* top-k selection (one launch per query chunk, topk > 512) */
  CSA_KERNEL_ATTENTION = 4,   /* sparse MQA + de-rotation */
  CSA_KERNEL_INDEX_TOPK = 5,  /* indexer scores fused with top-k (topk <= 512) */
  CSA_KERNEL_INDEX_KEYS = 6   /* indexer key pass (CSA_FLAG_INDEX_PROLOGUE / _FP8) */
} csa_kernel_t;

/* Number of events the traced variant of `op` (CSA_OP_CSA_FWD or CSA_OP_HCA_FWD)
 * records for these params: one more than its kernel launches; 0 on invalid params. */
int32_t csa_trace_events(const csa_params_t* p, int32_t op);

/* csa_fwd / hca_fwd that also time each kernel.  `events` are caller-created
 * hipEvent_t handles (as void*); events[0] is recorded on `stream` before the first
 * launch and events[i+1] right after launch i, whose csa_kernel_t is written to
 * kinds[i] (host memory).  n_events must be >= csa_trace_events(p, op).  Recording
 * events allocates nothing.  Work and results are those of the untraced call. */
csa_status_t csa_fwd_traced(const csa_params_t* p, const csa_inputs_t* in, void* o, void* ws,
                            size_t ws_bytes, void* stream, void* const* events, int32_t* kinds,
                            int32_t n_events);
csa_status_t hca_fwd_traced(const csa_params_t* p, const csa_inputs_t* in, void* o, void* ws,
                            size_t ws_bytes, void* stream, void* const* events, int32_t* kinds,
                            int32_t n_events);

/* Workspace bytes an operation needs for these params (0 on invalid params). */
size_t csa_workspace_bytes(const csa_params_t* p, int32_t op);

/* The integer layout the kernels use, written by a kernel from the same helpers:
 * comp_pos [S/ratio] (positions, truncated to int32), n_visible [S], win_lo [S].
 * Any output may be NULL. */
csa_status_t csa_debug_layout(const csa_params_t* p, int32_t* comp_pos, int32_t* n_visible,
                              int32_t* win_lo, void* stream);

const char* csa_status_str(csa_status_t s);
const char* csa_last_error(void);
int32_t csa_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* CSA_H_ */
