// Host test of the C-ABI (abi.cpp + validate.cpp) built with g++ and the address and
// undefined-behaviour sanitizers, against launch_stub.cpp.  Every argument error of
// every entry point must return its status before any launch; valid calls must reach
// the launchers in order, with every output inside the caller's buffers (the stubs
// write each output's full extent, so an undersized workspace plan is an ASan error).
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <string>
#include <vector>

#include "csa.h"

extern std::vector<std::string> g_calls;
extern int g_fail;
extern int g_events;

static int g_bad = 0;
#define EXPECT(cond, ...)                                   \
  do {                                                      \
    if (!(cond)) {                                          \
      ++g_bad;                                              \
      fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__);  \
      fprintf(stderr, __VA_ARGS__);                         \
      fprintf(stderr, " [%s]\n", csa_last_error());        \
    }                                                       \
  } while (0)
#define EXPECT_ST(expr, want) \
  do {                        \
    const int got_ = (int)(expr); \
    EXPECT(got_ == (want), "%s -> %d, expected %d", #expr, got_, (int)(want)); \
  } while (0)

// Exactly sized, 256-byte aligned host buffers (freed at exit).
static std::vector<void*> g_bufs;
static void* buf(size_t n) {
  void* p = nullptr;
  if (posix_memalign(&p, 256, n ? n : 1)) abort();
  memset(p, 0, n ? n : 1);
  g_bufs.push_back(p);
  return p;
}

static csa_params_t small_csa(int dtype = CSA_F32) {
  csa_params_t p{};
  p.B = 2; p.S = 64; p.H = 4; p.D = 64; p.rope_dim = 16; p.ratio = 4; p.overlap = 1;
  p.window = 8; p.topk = 6; p.idx_heads = 4; p.idx_dim = 16; p.dtype = dtype;
  p.rope_theta = 40000.0; p.rms_eps = 1e-6f; p.softmax_scale = 0.125f; p.pos0 = 0; p.flags = 0;
  return p;
}

struct Layer {
  csa_inputs_t in{};
  void* o = nullptr;
};

static size_t es(const csa_params_t& p) { return p.dtype == CSA_BF16 ? 2 : 4; }

static Layer make_layer(const csa_params_t& p, bool csa) {
  Layer L;
  const size_t BS = (size_t)p.B * p.S, n = (size_t)p.B * (p.S / p.ratio);
  L.in.q = buf(BS * p.H * p.D * es(p));
  L.in.kv_raw = buf(BS * p.D * es(p));
  L.in.va = buf(BS * p.D * es(p));
  L.in.ga = buf(BS * p.D * es(p));
  L.in.bias = (const float*)buf((size_t)(csa ? 2 : 1) * p.ratio * p.D * 4);
  if (csa) {
    L.in.vb = buf(BS * p.D * es(p));
    L.in.gb = buf(BS * p.D * es(p));
    L.in.q_idx = buf(BS * p.idx_heads * p.idx_dim * es(p));
    L.in.w_idx = (const float*)buf(BS * p.idx_heads * 4);
    L.in.k_idx = buf(n * p.idx_dim * es(p));
  }
  L.o = buf(BS * p.H * p.D * es(p));
  return L;
}

static void bad_params() {
  // Every scalar validation branch, through the fused CSA call and the workspace query.
  struct Case { const char* what; void (*edit)(csa_params_t&); int want; };
  const Case cases[] = {
      {"B<0", [](csa_params_t& p) { p.B = -1; }, CSA_ERR_INVALID_ARG},
      {"S<0", [](csa_params_t& p) { p.S = -4; }, CSA_ERR_INVALID_ARG},
      {"dtype", [](csa_params_t& p) { p.dtype = 7; }, CSA_ERR_INVALID_ARG},
      {"flags", [](csa_params_t& p) { p.flags = 64; }, CSA_ERR_INVALID_ARG},
      {"D=96", [](csa_params_t& p) { p.D = 96; }, CSA_ERR_INVALID_ARG},
      {"D=576", [](csa_params_t& p) { p.D = 576; }, CSA_ERR_INVALID_ARG},
      {"D=192", [](csa_params_t& p) { p.D = 192; }, CSA_ERR_UNSUPPORTED},
      {"rope odd", [](csa_params_t& p) { p.rope_dim = 15; }, CSA_ERR_INVALID_ARG},
      {"rope>D", [](csa_params_t& p) { p.rope_dim = 80; }, CSA_ERR_INVALID_ARG},
      {"rope>128", [](csa_params_t& p) { p.D = 512; p.rope_dim = 130; }, CSA_ERR_UNSUPPORTED},
      {"theta", [](csa_params_t& p) { p.rope_theta = 0.0; }, CSA_ERR_INVALID_ARG},
      {"theta inf", [](csa_params_t& p) { p.rope_theta = 1.0 / 0.0; }, CSA_ERR_INVALID_ARG},
      {"eps nan", [](csa_params_t& p) { p.rms_eps = 0.0f / 0.0f; }, CSA_ERR_INVALID_ARG},
      {"ratio 0", [](csa_params_t& p) { p.ratio = 0; }, CSA_ERR_INVALID_ARG},
      {"S%ratio", [](csa_params_t& p) { p.S = 66; }, CSA_ERR_INVALID_ARG},
      {"overlap 2", [](csa_params_t& p) { p.overlap = 2; }, CSA_ERR_INVALID_ARG},
      {"H=0", [](csa_params_t& p) { p.H = 0; }, CSA_ERR_INVALID_ARG},
      {"H=65", [](csa_params_t& p) { p.H = 65; }, CSA_ERR_INVALID_ARG},
      {"window<0", [](csa_params_t& p) { p.window = -1; }, CSA_ERR_INVALID_ARG},
      {"scale 0", [](csa_params_t& p) { p.softmax_scale = 0.0f; }, CSA_ERR_INVALID_ARG},
      {"topk 0", [](csa_params_t& p) { p.topk = 0; }, CSA_ERR_INVALID_ARG},
      {"topk 2049", [](csa_params_t& p) { p.topk = 2049; }, CSA_ERR_INVALID_ARG},
      {"idx_heads 0", [](csa_params_t& p) { p.idx_heads = 0; }, CSA_ERR_INVALID_ARG},
      {"idx_heads 65", [](csa_params_t& p) { p.idx_heads = 65; }, CSA_ERR_INVALID_ARG},
      {"idx_dim 24", [](csa_params_t& p) { p.idx_dim = 24; }, CSA_ERR_INVALID_ARG},
      {"idx_dim 48", [](csa_params_t& p) { p.idx_dim = 48; }, CSA_ERR_UNSUPPORTED},
      {"entries", [](csa_params_t& p) { p.S = 4 * 32769; }, CSA_ERR_UNSUPPORTED},
      {"fp8 dim", [](csa_params_t& p) { p.flags = CSA_FLAG_INDEX_FP8; p.idx_dim = 32; }, CSA_ERR_UNSUPPORTED},
      {"prologue rope", [](csa_params_t& p) { p.flags = CSA_FLAG_INDEX_PROLOGUE; p.rope_dim = 18; }, CSA_ERR_INVALID_ARG},
  };
  const csa_params_t base = small_csa();
  Layer L = make_layer(base, true);
  for (const Case& c : cases) {
    csa_params_t p = base;
    c.edit(p);
    g_calls.clear();
    const int st = csa_fwd(&p, &L.in, L.o, nullptr, 0, nullptr);
    EXPECT(st == c.want, "csa_fwd(%s) -> %d, expected %d", c.what, st, c.want);
    EXPECT(g_calls.empty(), "csa_fwd(%s) launched %zu kernels", c.what, g_calls.size());
    EXPECT(csa_workspace_bytes(&p, CSA_OP_CSA_FWD) == 0, "workspace bytes for %s", c.what);
    EXPECT(strlen(csa_last_error()) > 0, "no message for %s", c.what);
  }
  EXPECT_ST(csa_fwd(nullptr, &L.in, L.o, nullptr, 0, nullptr), CSA_ERR_INVALID_ARG);
  EXPECT(csa_workspace_bytes(&base, 99) == 0, "unknown op");
  EXPECT(csa_trace_events(&base, CSA_OP_COMPRESS) == 0, "trace events of a non-fused op");
  csa_params_t w0 = base;
  w0.window = 0;
  EXPECT_ST(csa_sparse_mqa_fwd(&w0, L.in.q, nullptr, L.in.kv_raw, nullptr, L.o, nullptr, 0, nullptr),
            CSA_ERR_INVALID_ARG);  // window-only needs a window
  EXPECT_ST(csa_index_keys(&base, L.in.k_idx, buf(64), nullptr), CSA_ERR_INVALID_ARG);  // no flag
}

static void bad_pointers() {
  const csa_params_t p = small_csa();
  Layer L = make_layer(p, true);
  const size_t wsb = csa_workspace_bytes(&p, CSA_OP_CSA_FWD);
  void* ws = buf(wsb);
  const char* base = static_cast<const char*>(L.in.q);
  // every required pointer NULL, then misaligned
  const char* names[] = {"q", "kv_raw", "va", "ga", "vb", "gb", "bias", "q_idx", "w_idx", "k_idx"};
  for (int i = 0; i < 10; ++i) {
    for (int mis = 0; mis < 2; ++mis) {
      csa_inputs_t in = L.in;
      const void** f = reinterpret_cast<const void**>(&in) + i;
      *f = mis ? static_cast<const void*>(static_cast<const char*>(*f) + 4) : nullptr;
      g_calls.clear();
      const int st = csa_fwd(&p, &in, L.o, ws, wsb, nullptr);
      EXPECT(st == CSA_ERR_INVALID_ARG, "%s %s -> %d", names[i], mis ? "misaligned" : "NULL", st);
      EXPECT(g_calls.empty(), "launch after a bad %s", names[i]);
    }
  }
  (void)base;
  EXPECT_ST(csa_fwd(&p, nullptr, L.o, ws, wsb, nullptr), CSA_ERR_INVALID_ARG);
  {
    csa_inputs_t in = L.in;
    in.lse_out = (float*)((char*)buf(64) + 4);  // misaligned optional output
    g_calls.clear();
    EXPECT_ST(csa_fwd(&p, &in, L.o, ws, wsb, nullptr), CSA_ERR_INVALID_ARG);
    EXPECT(g_calls.empty(), "launch after a misaligned lse_out");
  }
  EXPECT_ST(csa_fwd(&p, &L.in, nullptr, ws, wsb, nullptr), CSA_ERR_INVALID_ARG);
  EXPECT_ST(csa_fwd(&p, &L.in, L.o, ws, wsb - 1, nullptr), CSA_ERR_WORKSPACE);
  EXPECT_ST(csa_fwd(&p, &L.in, L.o, nullptr, wsb, nullptr), CSA_ERR_INVALID_ARG);
  csa_params_t h = p;
  h.overlap = 0;
  EXPECT_ST(csa_fwd(&h, &L.in, L.o, ws, wsb, nullptr), CSA_ERR_INVALID_ARG);  // CSA needs overlap
  EXPECT_ST(hca_fwd(&p, &L.in, L.o, ws, wsb, nullptr), CSA_ERR_INVALID_ARG);  // HCA needs none
  csa_params_t hp = p;
  hp.overlap = 0;
  Layer H = make_layer(hp, false);
  csa_inputs_t hin = H.in;
  hin.vb = L.in.vb;  // vb must be NULL without overlap
  EXPECT_ST(hca_fwd(&hp, &hin, H.o, buf(csa_workspace_bytes(&hp, CSA_OP_HCA_FWD)),
                    csa_workspace_bytes(&hp, CSA_OP_HCA_FWD), nullptr), CSA_ERR_INVALID_ARG);
  // attention: idx without kv_c; misaligned optional pointers
  void* aws = buf(csa_workspace_bytes(&p, CSA_OP_SPARSE_MQA));
  const size_t awsb = csa_workspace_bytes(&p, CSA_OP_SPARSE_MQA);
  int32_t* idx = (int32_t*)buf((size_t)p.B * p.S * p.topk * 4);
  EXPECT_ST(csa_sparse_mqa_fwd(&p, L.in.q, nullptr, L.in.kv_raw, idx, L.o, aws, awsb, nullptr), CSA_ERR_INVALID_ARG);
  EXPECT_ST(csa_sparse_mqa_fwd_sink(&p, L.in.q, L.in.q, L.in.kv_raw, idx, (const float*)((char*)idx + 4), L.o,
                                    aws, awsb, nullptr), CSA_ERR_INVALID_ARG);
  EXPECT_ST(csa_sparse_mqa_bwd_dq(&p, L.in.q, L.in.q, L.in.kv_raw, idx, nullptr, L.o, nullptr, L.o, aws, awsb,
                                  nullptr), CSA_ERR_INVALID_ARG);  // d_o NULL
  EXPECT_ST(csa_kl_target(&p, L.in.q, nullptr, idx, (float*)L.o, nullptr), CSA_ERR_INVALID_ARG);
  EXPECT_ST(csa_sparse_mqa_fwd_lse(&p, L.in.q, L.in.q, L.in.kv_raw, idx, nullptr, L.o, nullptr, aws, awsb, nullptr),
            CSA_ERR_INVALID_ARG);  // lse NULL
  {  // key-side backward: required and matching pointers, dtype limit, workspace size
    const size_t dwsb = csa_workspace_bytes(&p, CSA_OP_SPARSE_MQA_BWD);
    void* dws = buf(dwsb);
    float* f = (float*)buf((size_t)p.B * p.S * p.D * 4);
    float* lse = (float*)buf((size_t)p.B * p.S * p.H * 4);
    const float* sk = (const float*)buf((size_t)p.H * 4);
    float* dsk = (float*)buf((size_t)p.H * 4);
    const void* kv = L.in.q;
    struct Bad { const char* what; int want; int st; };
    g_calls.clear();
    const Bad bads[] = {
        {"lse NULL", CSA_ERR_INVALID_ARG, csa_sparse_mqa_bwd_dkv(&p, L.in.q, kv, L.in.kv_raw, idx, nullptr, L.o,
                                                                  nullptr, L.o, f, f, nullptr, dws, dwsb, nullptr)},
        {"d_o NULL", CSA_ERR_INVALID_ARG, csa_sparse_mqa_bwd_dkv(&p, L.in.q, kv, L.in.kv_raw, idx, nullptr, L.o,
                                                                  lse, nullptr, f, f, nullptr, dws, dwsb, nullptr)},
        {"dkv_raw NULL", CSA_ERR_INVALID_ARG, csa_sparse_mqa_bwd_dkv(&p, L.in.q, kv, L.in.kv_raw, idx, nullptr, L.o,
                                                                      lse, L.o, f, nullptr, nullptr, dws, dwsb, nullptr)},
        {"dkv_c NULL", CSA_ERR_INVALID_ARG, csa_sparse_mqa_bwd_dkv(&p, L.in.q, kv, L.in.kv_raw, idx, nullptr, L.o,
                                                                    lse, L.o, nullptr, f, nullptr, dws, dwsb, nullptr)},
        {"dkv_c without kv_c", CSA_ERR_INVALID_ARG,
         csa_sparse_mqa_bwd_dkv(&p, L.in.q, nullptr, L.in.kv_raw, nullptr, nullptr, L.o, lse, L.o, f, f, nullptr,
                                dws, dwsb, nullptr)},
        {"dsinks NULL", CSA_ERR_INVALID_ARG, csa_sparse_mqa_bwd_dkv(&p, L.in.q, kv, L.in.kv_raw, idx, sk, L.o,
                                                                     lse, L.o, f, f, nullptr, dws, dwsb, nullptr)},
        {"dsinks without sinks", CSA_ERR_INVALID_ARG,
         csa_sparse_mqa_bwd_dkv(&p, L.in.q, kv, L.in.kv_raw, idx, nullptr, L.o, lse, L.o, f, f, dsk, dws, dwsb,
                                nullptr)},
        {"lse misaligned", CSA_ERR_INVALID_ARG,
         csa_sparse_mqa_bwd_dkv(&p, L.in.q, kv, L.in.kv_raw, idx, nullptr, L.o, lse + 1, L.o, f, f, nullptr, dws,
                                dwsb, nullptr)},
        {"ws short", CSA_ERR_WORKSPACE, csa_sparse_mqa_bwd_dkv(&p, L.in.q, kv, L.in.kv_raw, idx, nullptr, L.o, lse,
                                                                L.o, f, f, nullptr, dws, dwsb - 1, nullptr)},
        {"idx without kv_c", CSA_ERR_INVALID_ARG,
         csa_sparse_mqa_bwd_dkv(&p, L.in.q, nullptr, L.in.kv_raw, idx, nullptr, L.o, lse, L.o, nullptr, f, nullptr,
                                dws, dwsb, nullptr)},
    };
    for (const Bad& b : bads) EXPECT(b.st == b.want, "bwd_dkv %s -> %d, expected %d", b.what, b.st, b.want);
    csa_params_t p512 = p;
    p512.D = 512;
    EXPECT_ST(csa_sparse_mqa_bwd_dkv(&p512, L.in.q, kv, L.in.kv_raw, idx, nullptr, L.o, lse, L.o, f, f, nullptr,
                                     dws, dwsb, nullptr), CSA_ERR_UNSUPPORTED);  // fp32 at D = 512
    EXPECT(g_calls.empty(), "bwd_dkv launched after a bad argument");
  }
  // index_scores row range and ld
  float* sc = (float*)buf((size_t)p.B * p.S * 16 * 4);
  EXPECT_ST(csa_index_scores(&p, L.in.q_idx, L.in.w_idx, L.in.k_idx, sc, 16, 60, 8, nullptr), CSA_ERR_INVALID_ARG);
  EXPECT_ST(csa_index_scores(&p, L.in.q_idx, L.in.w_idx, L.in.k_idx, sc, 15, 0, 8, nullptr), CSA_ERR_INVALID_ARG);
  EXPECT_ST(csa_index_scores(&p, L.in.q_idx, L.in.w_idx, L.in.k_idx, sc, 16, -1, 8, nullptr), CSA_ERR_INVALID_ARG);
  // key pass: k_out overlapping k_idx
  csa_params_t pk = p;
  pk.flags = CSA_FLAG_INDEX_PROLOGUE;
  EXPECT_ST(csa_index_keys(&pk, L.in.k_idx, (char*)L.in.k_idx + 16, nullptr), CSA_ERR_INVALID_ARG);
  // traced: too few events, or no kinds array
  void* evs[32] = {};
  int32_t kinds[32];
  const int32_t nev = csa_trace_events(&p, CSA_OP_CSA_FWD);
  EXPECT_ST(csa_fwd_traced(&p, &L.in, L.o, ws, wsb, nullptr, evs, kinds, nev - 1), CSA_ERR_INVALID_ARG);
  EXPECT_ST(csa_fwd_traced(&p, &L.in, L.o, ws, wsb, nullptr, evs, nullptr, nev), CSA_ERR_INVALID_ARG);
  EXPECT_ST(csa_fwd_traced(&p, &L.in, L.o, ws, wsb, nullptr, nullptr, kinds, nev), CSA_ERR_INVALID_ARG);
  EXPECT_ST(csa_debug_layout(nullptr, nullptr, nullptr, nullptr, nullptr), CSA_ERR_INVALID_ARG);
  csa_params_t pr = p;
  pr.ratio = 0;
  EXPECT_ST(csa_debug_layout(&pr, nullptr, nullptr, nullptr, nullptr), CSA_ERR_INVALID_ARG);
}

static std::string joined() {
  std::string s;
  for (auto& c : g_calls) s += (s.empty() ? "" : ",") + c;
  return s;
}

static void run_fused(csa_params_t p, bool csa, const char* want) {
  Layer L = make_layer(p, csa);
  const int op = csa ? CSA_OP_CSA_FWD : CSA_OP_HCA_FWD;
  const size_t wsb = csa_workspace_bytes(&p, op);
  EXPECT(wsb > 0, "workspace of a valid layer");
  void* ws = buf(wsb);
  g_calls.clear();
  EXPECT_ST(csa ? csa_fwd(&p, &L.in, L.o, ws, wsb, nullptr) : hca_fwd(&p, &L.in, L.o, ws, wsb, nullptr), CSA_OK);
  EXPECT(joined() == want, "fused calls %s, expected %s", joined().c_str(), want);
  // traced: one event before the first launch and one after each
  const int32_t nev = csa_trace_events(&p, op);
  std::vector<void*> evs(nev, (void*)0x10);
  std::vector<int32_t> kinds(nev, -1);
  g_calls.clear();
  g_events = 0;
  EXPECT_ST(csa ? csa_fwd_traced(&p, &L.in, L.o, ws, wsb, nullptr, evs.data(), kinds.data(), nev)
                : hca_fwd_traced(&p, &L.in, L.o, ws, wsb, nullptr, evs.data(), kinds.data(), nev), CSA_OK);
  EXPECT(g_events == nev && (int)g_calls.size() == nev - 1, "traced: %d events, %zu launches, expected %d",
         g_events, g_calls.size(), nev);
  // outputs to caller buffers instead of the workspace
  if (csa) {
    csa_inputs_t in = L.in;
    in.kv_c_out = buf((size_t)p.B * (p.S / p.ratio) * p.D * es(p));
    in.idx_out = (int32_t*)buf((size_t)p.B * p.S * p.topk * 4);
    in.n_visible_out = (int32_t*)buf((size_t)p.B * p.S * 4);
    in.lse_out = (float*)buf((size_t)p.B * p.S * p.H * 4);
    EXPECT_ST(csa_fwd(&p, &in, L.o, ws, wsb, nullptr), CSA_OK);
  }
  // a failing launch is reported, not ignored
  g_fail = 719;
  EXPECT_ST(csa ? csa_fwd(&p, &L.in, L.o, ws, wsb, nullptr) : hca_fwd(&p, &L.in, L.o, ws, wsb, nullptr), CSA_ERR_HIP);
  g_fail = 0;
  // an empty batch is a no-op that needs no pointers
  csa_params_t e = p;
  e.B = 0;
  g_calls.clear();
  EXPECT_ST(csa ? csa_fwd(&e, nullptr == &L.in ? nullptr : &L.in, nullptr, nullptr, 0, nullptr)
                : hca_fwd(&e, &L.in, nullptr, nullptr, 0, nullptr), CSA_OK);
  EXPECT(g_calls.empty(), "empty batch launched");
}

static void valid_calls() {
  run_fused(small_csa(), true, "compress,window_rope,index_topk,mqa_selected");
  csa_params_t bf = small_csa(CSA_BF16);
  bf.D = 512; bf.H = 64; bf.rope_dim = 64; bf.idx_heads = 64; bf.idx_dim = 128; bf.S = 256; bf.topk = 32;
  run_fused(bf, true, "compress,window_rope,index_topk,mqa_selected");
  csa_params_t f8 = bf;
  f8.flags = CSA_FLAG_INDEX_FP8 | CSA_FLAG_INDEX_PROLOGUE;
  run_fused(f8, true, "compress,window_rope,index_keys,index_topk,mqa_selected");
  csa_params_t pro = small_csa();
  pro.flags = CSA_FLAG_INDEX_PROLOGUE;
  run_fused(pro, true, "compress,window_rope,index_keys,index_topk,mqa_selected");
  // top-k above the fused limit: scores and top-k per query chunk of the workspace
  csa_params_t big = small_csa();
  big.S = 8192; big.B = 1; big.topk = 1024; big.D = 64; big.H = 1;
  std::string chunks = "compress,window_rope";
  {
    // 128 MB of scores per chunk: rows = 2^27 / (ld * 4) with ld = 2048
    const int rows = (int)((size_t(128) << 20) / (2048 * 4));
    for (int t0 = 0; t0 < big.S; t0 += rows) chunks += ",index_scores,topk";
  }
  chunks += ",mqa_selected";
  run_fused(big, true, chunks.c_str());
  csa_params_t h = small_csa();
  h.overlap = 0; h.ratio = 16; h.S = 128;
  run_fused(h, false, "compress,window_rope,mqa_dense");

  // the separate stages
  const csa_params_t p = small_csa();
  Layer L = make_layer(p, true);
  const size_t awsb = csa_workspace_bytes(&p, CSA_OP_SPARSE_MQA);
  void* aws = buf(awsb);
  void* kv_c = buf((size_t)p.B * (p.S / p.ratio) * p.D * 4);
  int32_t* idx = (int32_t*)buf((size_t)p.B * p.S * p.topk * 4);
  int32_t* nv = (int32_t*)buf((size_t)p.B * p.S * 4);
  const float* sinks = (const float*)buf((size_t)p.H * 4);
  g_calls.clear();
  EXPECT_ST(csa_compress(&p, L.in.va, L.in.ga, L.in.vb, L.in.gb, L.in.bias, kv_c, nullptr), CSA_OK);
  const size_t iwsb = csa_workspace_bytes(&p, CSA_OP_INDEX_TOPK);
  EXPECT_ST(csa_index_topk(&p, L.in.q_idx, L.in.w_idx, L.in.k_idx, idx, nv, iwsb ? buf(iwsb) : nullptr, iwsb,
                           nullptr), CSA_OK);
  EXPECT_ST(csa_index_topk(&p, L.in.q_idx, L.in.w_idx, L.in.k_idx, idx, nullptr, nullptr, 0, nullptr), CSA_OK);
  float* sc = (float*)buf((size_t)p.B * 10 * 16 * 4);
  EXPECT_ST(csa_index_scores(&p, L.in.q_idx, L.in.w_idx, L.in.k_idx, sc, 16, 54, 10, nullptr), CSA_OK);
  EXPECT_ST(csa_sparse_mqa_fwd(&p, L.in.q, kv_c, L.in.kv_raw, idx, L.o, aws, awsb, nullptr), CSA_OK);
  EXPECT_ST(csa_sparse_mqa_fwd(&p, L.in.q, kv_c, L.in.kv_raw, nullptr, L.o, aws, awsb, nullptr), CSA_OK);
  EXPECT_ST(csa_sparse_mqa_fwd_sink(&p, L.in.q, nullptr, L.in.kv_raw, nullptr, sinks, L.o, aws, awsb, nullptr),
            CSA_OK);
  void* dq = buf((size_t)p.B * p.S * p.H * p.D * 4);
  EXPECT_ST(csa_sparse_mqa_bwd_dq(&p, L.in.q, kv_c, L.in.kv_raw, idx, sinks, L.o, L.o, dq, aws, awsb, nullptr),
            CSA_OK);
  EXPECT_ST(csa_kl_target(&p, L.in.q, kv_c, idx, (float*)buf((size_t)p.B * p.S * p.topk * 4), nullptr), CSA_OK);
  float* lse = (float*)buf((size_t)p.B * p.S * p.H * 4);
  EXPECT_ST(csa_sparse_mqa_fwd_lse(&p, L.in.q, kv_c, L.in.kv_raw, idx, sinks, L.o, lse, aws, awsb, nullptr), CSA_OK);
  {  // key-side backward in its three modes, with and without sinks
    const size_t dwsb = csa_workspace_bytes(&p, CSA_OP_SPARSE_MQA_BWD);
    EXPECT(dwsb > awsb, "key-side workspace %zu", dwsb);
    void* dws = buf(dwsb);
    float* dkv_c = (float*)buf((size_t)p.B * (p.S / p.ratio) * p.D * 4);
    float* dkv_raw = (float*)buf((size_t)p.B * p.S * p.D * 4);
    float* dsk = (float*)buf((size_t)p.H * 4);
    EXPECT_ST(csa_sparse_mqa_bwd_dkv(&p, L.in.q, kv_c, L.in.kv_raw, idx, sinks, L.o, lse, L.o, dkv_c, dkv_raw, dsk,
                                     dws, dwsb, nullptr), CSA_OK);
    EXPECT_ST(csa_sparse_mqa_bwd_dkv(&p, L.in.q, kv_c, L.in.kv_raw, nullptr, nullptr, L.o, lse, L.o, dkv_c, dkv_raw,
                                     nullptr, dws, dwsb, nullptr), CSA_OK);
    EXPECT_ST(csa_sparse_mqa_bwd_dkv(&p, L.in.q, nullptr, L.in.kv_raw, nullptr, sinks, L.o, lse, L.o, nullptr,
                                     dkv_raw, dsk, dws, dwsb, nullptr), CSA_OK);
  }
  csa_params_t pk = p;
  pk.flags = CSA_FLAG_INDEX_FP8;
  pk.idx_dim = 64;
  void* kin = buf((size_t)p.B * (p.S / p.ratio) * 64 * 4);
  EXPECT_ST(csa_index_keys(&pk, kin, buf((size_t)p.B * (p.S / p.ratio) * (64 + 16)), nullptr), CSA_OK);
  EXPECT_ST(csa_debug_layout(&p, (int32_t*)buf(16 * 4), (int32_t*)buf(64 * 4), (int32_t*)buf(64 * 4), nullptr),
            CSA_OK);
  const char* want = "compress,index_topk,index_topk,index_scores,window_rope,mqa_selected,window_rope,mqa_dense,"
                     "window_rope,mqa_window,window_rope,bwd_dq,kl_target,window_rope,mqa_selected,"
                     "window_rope,bwd_dkv,window_rope,bwd_dkv,window_rope,bwd_dkv,index_keys,debug_layout";
  EXPECT(joined() == want, "stage calls %s", joined().c_str());
  EXPECT(csa_abi_version() == CSA_ABI_VERSION, "abi version");
  EXPECT(strcmp(csa_status_str((csa_status_t)42), "CSA_ERR_UNKNOWN") == 0, "unknown status string");
}

int main() {
  bad_params();
  bad_pointers();
  valid_calls();
  for (void* p : g_bufs) free(p);
  if (g_bad) {
    fprintf(stderr, "%d check(s) failed\n", g_bad);
    return 1;
  }
  printf("host ABI checks passed\n");
  return 0;
}
