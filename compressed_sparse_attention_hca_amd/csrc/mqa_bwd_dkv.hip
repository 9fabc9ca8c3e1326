// Backward of stage 4, key side, on gfx950: the gradients of the rotated compressed
// entries (dkv_c), of the raw window latents (dkv_raw) and of the softmax sinks.
//
// Sources: "Enabling DeepSeek-V4-Flash Training on AMD Instinct MI355X GPUs with
// Primus", section "Attention kernels for the three layer types": the backward has a
// dQ kernel, "interm" (a contraction over the head dimension that gives each key's
// gradient) and delta folded into dQ, and sparse attention pays a gather/scatter tax,
// two passes over an intermediate tensor: the gather of the selected keys and the
// scatter of their gradients back to the entries.  "fix(deepseek-v4): correct
// V4-Flash attention math", Part 1 item 6f: the sink is an fp32 logit of the softmax.
//
// The forward (sparse_mqa.hip), with P = pos0 + t:
//   z[h,k] = (q~[h] . key_k) * scale,  q~[h] = RoPE(q[h], P),  u[h] = sum_k p[h,k] key_k
// where p = exp(z - lse) and lse is the log of each head's denominator (sink included),
// kept by the forward.  K = V, so with du = RoPE(do, +P), dP[h,k] = du[h] . key_k and
// delta[h] = do[h] . o[h], each key of a query gets
//   dkey_k = sum_h ( scale * p[h,k] (dP[h,k] - delta[h]) * q~[h]  +  p[h,k] * du[h] ),
// a contraction over 2H values per (query, key) pair.  The sink gets
//   dsink[h] = -sum over queries of exp(sink[h] - lse[h]) * delta[h].
//
// Three steps, the query rows taken in chunks so the intermediate stays bounded:
//  1. interm (mqa_bwd_dkv_kernel), one workgroup per query: the key tiles stream
//     through LDS as in the dQ kernel; per 32-key tile the logits and dP come from the
//     same K fragments on MFMA, p and ds = scale p (dP - delta) are rounded to the
//     activation type and swapped through LDS so that every wave holds them for all
//     heads, and wave w contracts them against q~ and du (held in registers, dims
//     w*D/NW .. +D/NW) on MFMA.  Each pair's gradient row is stored to the
//     intermediate [rows, slots, D] in the activation type: entry slots 0..kmax-1 in
//     selection order, then window slots kmax.. for tokens win_lo(t)...
//  2. entries: a counting sort of the chunk's (row, slot) pairs by entry (per block of
//     64 rows, rows in order, so each entry's list is in row order and the sums are
//     deterministic), then a key-major sum of each entry's rows in segments of 256
//     pairs, segment partials added in order, into dkv_c (fp32).
//  3. window tokens: token t' is in the windows of rows t' .. t'+W-1, at slot
//     kmax + t' - win_lo(t), so each token sums its band of rows directly into an fp32
//     accumulator.  After the last chunk the accumulator is rotated back by -(pos0+t')
//     and, with the window norm, taken through the RMSNorm: dkv_raw.
#include "common.hpp"
#include "mqa_bwd_dkv.hpp"
#include "validate.hpp"

#include <type_traits>

namespace csa {
namespace {

constexpr int kMaxTopk = 2048;
constexpr float kLog2e = 1.4426950408889634f;

struct DkvArgs {
  const void* q;
  const void* kv_c;
  const void* kv_w;
  const int32_t* idx;
  const float* sinks;  // [H] or nullptr
  const void* o;       // forward output [B,S,H,D]
  const float* lse;    // forward log-denominators [B,S,H]
  const void* d_o;     // dL/do [B,S,H,D]
  void* interm;        // [nrows, kw, D] activation type
  float* ds_row;       // [B,S,H] per-query sink terms, or nullptr
  int32_t B, S, H, R, ratio, window, topk, n_entries, mode;
  int32_t kmax, kw;  // entry slots per row, all slots per row
  int64_t r0;        // first row (b*S + t) of the chunk
  int32_t nrows;
  float scale_log2, scale;
  double theta;
  int64_t pos0;
};

template <int N> __device__ inline void vm_wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Mapping: wave w owns heads 16w .. 16w+15 for the logits and dP (keys on M, its heads
// on N, v_mfma_f32_16x16x32, q~ and du as register B operands, as in the dQ kernel),
// and dims w*D/NW .. +D/NW for the key gradient (dims on M, keys on N, the 2*HP values
// h' = 2 head + {0: ds, 1: p} on K).  The A operand of the second product, qu, holds at
// k-slot h' = 32j + 8g + e the value (e even: q~, e odd: du) of head 16j + 4g + e/2 at
// the lane's dim; the exchange rows hold ds and p of one key in the same h' order.
//
// Pipeline (one workgroup per CU, one wave per SIMD): per tile t, the softmax of t
// writes its exchange buffer (two, alternating), then one barrier is both the exchange
// barrier of t and the arrival of tile t+1; after it the key gradients of t and the
// logits and dP of t+1 are issued interleaved, so the MFMA pipe has work while the
// LDS reads of either wait.  After that barrier tile t+NS is requested into tile t's
// stage (its logits were formed in the step before), so NS-1 tiles stay in flight
// beyond the one being waited for.  The gradient rows of t are stored right after the
// next barrier: the arrival wait counts stores and loads together (gfx9 vmcnt), and
// stores issued a whole tile earlier have completed by then.
template <typename T, int D, int NW>
__global__ __launch_bounds__(NW * 64, 1) void mqa_bwd_dkv_kernel(DkvArgs a) {
  constexpr int NT = NW * 64;
  constexpr int HP = NW * 16;
  constexpr int ES = (int)sizeof(T);
  constexpr int KT = 32;
  constexpr int ROWB = D * ES;
  constexpr int NCH = ROWB / 16;
  // key tile layout of the dQ kernel: 1 KB lines, one direct-to-LDS wave load each,
  // a 1 KB bf16 row XOR-swizzled by 16-byte chunk, other row sizes padded
  constexpr int RPL = ROWB < 1024 ? 1024 / ROWB : 1;
  constexpr int LPR = ROWB > 1024 ? ROWB / 1024 : 1;
  constexpr int NL = KT * LPR / RPL;
  constexpr bool SWZ = ROWB == 1024 && ES == 2;
  constexpr int LSTRIDE = SWZ ? 1024 : 1024 + 48;
  constexpr int QROWB = ROWB + 16;
  constexpr int TILEB = NL * LSTRIDE;
  constexpr int SB = TILEB > (HP / 2) * QROWB ? TILEB : (HP / 2) * QROWB;
  constexpr int XS = 2 * HP * ES + 16;  // exchange row (one key) stride, padded
  constexpr int XB = KT * XS;
  constexpr int DW = D / NW;            // dims of the key gradient per wave
  constexpr int DBW = DW / 16;
  constexpr int KS = D / 32;            // k-steps of the logit products
  static_assert(NL % NW == 0, "every wave issues the same number of line loads");
  static_assert(DBW * NW * 2 == 4 * KS, "four key-gradient MFMAs per logit k-step");
  constexpr int LPT = NL / NW;
  constexpr int NS = (4 * SB + 2 * XB + 10 * 1024 <= 160 * 1024 && 3 * LPT <= 63) ? 4 : 2;
  constexpr int SB2 = NS == 4 ? SB : 16;
  __shared__ __attribute__((aligned(16))) unsigned char st0[SB];
  __shared__ __attribute__((aligned(16))) unsigned char st1[SB];
  __shared__ __attribute__((aligned(16))) unsigned char st2[SB2];
  __shared__ __attribute__((aligned(16))) unsigned char st3[SB2];
  __shared__ __attribute__((aligned(16))) unsigned char xs0[XB];
  __shared__ __attribute__((aligned(16))) unsigned char xs1[XB];
  __shared__ int kv0[KT], kv1[KT], kv2[KT], kv3[KT];
  __shared__ int sidx[kMaxTopk];
  __shared__ float2 cs[64];
  __shared__ float sdelta[HP];

  // workgroup -> row of the chunk: 32 consecutive rows per XCD visit, latest first
  const int total = a.nrows;
  int gi = blockIdx.x;
  const int nfull = total & ~255;
  if (gi < nfull) {
    const int xcd = gi & 7, j = gi >> 3;
    gi = (((j >> 5) << 3) + xcd) * 32 + (j & 31);
  }
  gi = total - 1 - gi;
  const int64_t r = a.r0 + gi;  // global row b*S + t
  const int b = (int)(r / a.S);
  const int t = (int)(r % a.S);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hl = lane & 15;
  const int g = lane >> 4;
  const int h = 16 * wave + hl;
  const int n_t = a.mode == MQA_WINDOW_ONLY ? 0 : visible_entries(t, a.ratio);
  const int nsel = a.mode == MQA_SELECTED ? min(a.topk, n_t) : n_t;
  const int nwin = window_count(t, a.window);
  const int wlo = window_lo(t, a.window);
  const int nk = nsel + nwin;
  const int64_t P = a.pos0 + t;
  const int rlo = D - a.R;

  if (threadIdx.x < a.R / 2) {
    float c, s;
    rope_cos_sin(P, rope_inv_freq(threadIdx.x, a.R, a.theta), &c, &s);
    cs[threadIdx.x] = make_float2(c, s);
  }
  if (a.mode == MQA_SELECTED) {
    const int32_t* irow = a.idx + r * a.topk;
    for (int i = threadIdx.x; i < nsel; i += NT) sidx[i] = irow[i];
  }

  const int64_t row0 = r * a.H * ROWB;
  const unsigned char* qg = reinterpret_cast<const unsigned char*>(a.q) + row0;
  const unsigned char* dog = reinterpret_cast<const unsigned char*>(a.d_o) + row0;
  const unsigned char* og = reinterpret_cast<const unsigned char*>(a.o) + row0;

  // rows of heads 0..HP/2-1 in stage lo, the rest in stage hi (heads >= H zero)
  constexpr int SCH = HP * NCH / NT;  // 16-byte chunks per thread
  auto stage_rows = [&](const unsigned char* src, unsigned char* lo, unsigned char* hi) {
    uint4 v[SCH];
#pragma unroll
    for (int i = 0; i < SCH; ++i) {
      const int c = threadIdx.x + i * NT;
      const int row = c / NCH, col = (c % NCH) * 16;
      v[i] = row < a.H ? *reinterpret_cast<const uint4*>(src + (int64_t)row * ROWB + col) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < SCH; ++i) {
      const int c = threadIdx.x + i * NT;
      const int row = c / NCH, col = (c % NCH) * 16;
      *reinterpret_cast<uint4*>((row < HP / 2 ? lo : hi) + (row % (HP / 2)) * QROWB + col) = v[i];
    }
  };
  // do rows staged as stage_rows does, with delta[row] = o[row] . do[row] from the o
  // chunks loaded beside them (NCH lanes hold one row: a segmented lane sum)
  static_assert(NCH <= 64 && 64 % NCH == 0, "a row's chunks sit in one wave");
  auto stage_rows_delta = [&](const unsigned char* src, const unsigned char* osrc, unsigned char* lo,
                              unsigned char* hi) {
    uint4 v[SCH], w[SCH];
#pragma unroll
    for (int i = 0; i < SCH; ++i) {
      const int c = threadIdx.x + i * NT;
      const int row = c / NCH, col = (c % NCH) * 16;
      const bool in = row < a.H;
      v[i] = in ? *reinterpret_cast<const uint4*>(src + (int64_t)row * ROWB + col) : make_uint4(0, 0, 0, 0);
      w[i] = in ? *reinterpret_cast<const uint4*>(osrc + (int64_t)row * ROWB + col) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < SCH; ++i) {
      const int c = threadIdx.x + i * NT;
      const int row = c / NCH, col = (c % NCH) * 16;
      *reinterpret_cast<uint4*>((row < HP / 2 ? lo : hi) + (row % (HP / 2)) * QROWB + col) = v[i];
      const T* dv = reinterpret_cast<const T*>(&v[i]);
      const T* ov = reinterpret_cast<const T*>(&w[i]);
      float x = 0.f;
#pragma unroll
      for (int e = 0; e < 16 / ES; ++e) x = fmaf(to_f32(dv[e]), to_f32(ov[e]), x);
#pragma unroll
      for (int m = NCH / 2; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
      if (c % NCH == 0) sdelta[row] = x;
    }
  };
  auto row_in = [&](unsigned char* lo, unsigned char* hi, int hh) -> unsigned char* {
    return (hh < HP / 2 ? lo : hi) + (hh % (HP / 2)) * QROWB;
  };
  auto rotate_frag = [&](Frag<T>& f, int d0) {
    if (d0 + 8 > rlo) {
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        const int d = d0 + i;
        if (d >= rlo) {
          const float2 rr = cs[(d - rlo) >> 1];
          const float x0 = to_f32(f.v[i]), x1 = to_f32(f.v[i + 1]);
          f.v[i] = from_f32<T>(x0 * rr.x - x1 * rr.y);
          f.v[i + 1] = from_f32<T>(x0 * rr.y + x1 * rr.x);
        }
      }
    }
  };
  auto store_frag = [&](unsigned char* p, const Frag<T>& f) {
    *reinterpret_cast<uint4*>(p) = *reinterpret_cast<const uint4*>(f.v);
    if constexpr (ES == 4) *reinterpret_cast<uint4*>(p + 16) = *reinterpret_cast<const uint4*>(f.v + 4);
  };
  // k-slots e = kind (0: q~, 1: du) .. of the key-gradient operand, from rotated rows:
  // head 16j + 4g + e/2 at dim wave*DW + 16db + hl
  Frag<T> qu[DBW][NW];
  auto read_qu = [&](int kind, unsigned char* lo, unsigned char* hi) {
#pragma unroll
    for (int db = 0; db < DBW; ++db)
#pragma unroll
      for (int j = 0; j < NW; ++j)
#pragma unroll
        for (int e = kind; e < 8; e += 2) {
          const int hh = 16 * j + 4 * g + (e >> 1);
          qu[db][j].v[e] = reinterpret_cast<const T*>(row_in(lo, hi, hh))[wave * DW + 16 * db + hl];
        }
  };

  // ---- operands: q~ and du as register fragments (lane: head h, dims 32k + 8g ..),
  // written back rotated so the key-gradient operand can be read from the same rows;
  // delta = o . do from the unrotated rows.  With four stages q and do are staged
  // together (st0/st1 and st2/st3), else one after the other.
  Frag<T> qf[KS], uf[KS];
  unsigned char* ulo = NS == 4 ? st2 : st0;
  unsigned char* uhi = NS == 4 ? st3 : st1;
  auto build_q = [&]() {
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      qf[k] = load_frag(reinterpret_cast<const T*>(row_in(st0, st1, h)) + 32 * k + 8 * g);
      rotate_frag(qf[k], 32 * k + 8 * g);
      store_frag(row_in(st0, st1, h) + (32 * k + 8 * g) * ES, qf[k]);
    }
  };
  auto build_u = [&]() {
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      const int d0 = 32 * k + 8 * g;
      uf[k] = load_frag(reinterpret_cast<const T*>(row_in(ulo, uhi, h)) + d0);
      rotate_frag(uf[k], d0);
      store_frag(row_in(ulo, uhi, h) + d0 * ES, uf[k]);
    }
  };
  if constexpr (NS == 4) {
    stage_rows(qg, st0, st1);
    stage_rows_delta(dog, og, st2, st3);
    __syncthreads();
    build_q();
    build_u();
    __syncthreads();
    read_qu(0, st0, st1);
    read_qu(1, st2, st3);
  } else {
    stage_rows(qg, st0, st1);
    __syncthreads();
    build_q();
    __syncthreads();
    read_qu(0, st0, st1);
    __syncthreads();
    stage_rows_delta(dog, og, st0, st1);
    __syncthreads();
    build_u();
    __syncthreads();
    read_qu(1, st0, st1);
  }
  const float delta = sdelta[h];
  // log2 of the head's denominator; +inf (p = 0) for padded heads and for heads whose
  // forward had no mass (lse = -inf: no valid key and no sink)
  float lse2 = INFINITY;
  if (h < a.H) {
    const float l = a.lse[r * a.H + h];
    lse2 = l == -INFINITY ? INFINITY : l * kLog2e;
  }
  if (a.ds_row && g == 0 && h < a.H)
    a.ds_row[r * a.H + h] = -__builtin_amdgcn_exp2f(a.sinks[h] * kLog2e - lse2) * delta;
  __syncthreads();  // the staging area becomes the key tiles

  const unsigned char* kv_c = reinterpret_cast<const unsigned char*>(a.kv_c);
  const unsigned char* kv_w = reinterpret_cast<const unsigned char*>(a.kv_w);
  auto swz = [](int rr) -> int { return ((rr & 3) << 1) | ((rr >> 2) & 1); };
  auto eoff = [&](int rr, int d) -> int {
    const int byte = d * ES;
    if constexpr (SWZ) return rr * 1024 + ((((byte >> 4) ^ swz(rr)) << 4) | (byte & 15));
    return ((rr / RPL) * LPR + byte / 1024) * LSTRIDE + (rr % RPL) * ROWB + (byte % 1024);
  };
  // source row of key kk (entry s when kk < nsel); masked keys read this query's q row
  auto key_src = [&](int kk, int s, int* ok) -> const unsigned char* {
    if (kk < nsel) {
      if (s >= 0 && s < n_t) {
        *ok = 1;
        return kv_c + ((int64_t)b * a.n_entries + s) * ROWB;
      }
    } else if (kk < nk) {
      *ok = 1;
      return kv_w + ((int64_t)b * a.S + wlo + (kk - nsel)) * ROWB;
    }
    *ok = 0;
    return qg;
  };
  auto issue = [&](int tile, unsigned char* sb, int* kv) {
    if constexpr (ROWB == 1024) {
      // one 1 KB line per key row: lane l < 32 resolves key tile*32 + l (branch-free),
      // each line takes its row base by v_readlane and copies with a fixed per-lane
      // swizzled offset
      const int kk = tile * KT + (lane & 31);
      const unsigned char* src = qg;  // masked keys read finite data that is never used
      bool ok = false;
      if (kk < nsel) {
        const int sv = a.mode == MQA_SELECTED ? sidx[kk] : kk;
        ok = sv >= 0 && sv < n_t;
        src = ok ? kv_c + ((int64_t)b * a.n_entries + sv) * ROWB : qg;
      } else if (kk < nk) {
        ok = true;
        src = kv_w + ((int64_t)b * a.S + wlo + (kk - nsel)) * ROWB;
      }
      if (wave == 0 && lane < KT) kv[lane] = ok;
      const uint64_t sp = reinterpret_cast<uint64_t>(src);
      const uint32_t sp_lo = (uint32_t)sp, sp_hi = (uint32_t)(sp >> 32);
      const uint32_t lds0 = (uint32_t)(uintptr_t)(CSA_LDS unsigned char*)sb;
#pragma unroll
      for (int m = 0; m < LPT; ++m) {
        const int rr = wave + NW * m;
        const uint64_t row = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)sp_hi, rr) << 32) |
                             (uint32_t)__builtin_amdgcn_readlane((int)sp_lo, rr);
        const uint32_t off = (uint32_t)((SWZ ? (lane ^ swz(rr)) : lane) << 4);
        const uint32_t lds = __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)rr * LSTRIDE);
        // The row base was just written to SGPRs by v_readlane (a VALU op), and M0
        // just set: a vector-memory instruction may read such SGPRs only 5 wait states
        // later, and the compiler does not pad for an instruction inside inline
        // assembly.  As assembly the copy is also invisible to the compiler's wait-count
        // tracking, which would otherwise drain every copy in flight before each LDS
        // write it cannot tell apart from the stages; this kernel's own waits
        // (vm_wait_barrier) order the copies.
        asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(row), "{m0}"(lds) : "memory");
      }
    } else {
      int sv = 0;
      if constexpr (RPL == 1) {
        const int kk = tile * KT + (lane % KT);
        sv = a.mode == MQA_SELECTED ? (kk < nsel ? sidx[kk] : -1) : kk;
      }
#pragma unroll
      for (int L = wave; L < NL; L += NW) {
        int rr, byte;
        if constexpr (RPL > 1) {
          rr = L * RPL + lane / NCH;
          byte = (lane % NCH) * 16;
        } else {
          rr = L / LPR;
          byte = (L % LPR) * 1024 + lane * 16;
        }
        int ok, s;
        const int kk = tile * KT + rr;
        if constexpr (RPL == 1) s = __builtin_amdgcn_readlane(sv, rr);
        else s = a.mode == MQA_SELECTED ? (kk < nsel ? sidx[kk] : -1) : kk;
        const unsigned char* src = key_src(kk, s, &ok) + byte;
        // as above: invisible to the compiler's wait counting, padded for M0
        const uint32_t lds =
            __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(CSA_LDS unsigned char*)(sb + L * LSTRIDE));
        asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds) : "memory");
        if (byte == 0) kv[rr] = ok;
      }
    }
  };

  int qk_base[2];
  if constexpr (SWZ) {
    const int s = swz(hl), s2 = s >> 2;
    const int lo = hl * 1024 + (((g ^ s) & 3) << 4);
    qk_base[0] = lo + (s2 ? 64 : 0);
    qk_base[1] = lo - (s2 ? 64 : 0);
  } else {
    qk_base[0] = qk_base[1] = eoff(hl, 8 * g);
  }
  unsigned char* const interm = reinterpret_cast<unsigned char*>(a.interm);
  const int64_t prow = (int64_t)(r - a.r0) * a.kw;  // first slot row of this query

  typedef f32x4 Acc[4];  // logits (keys 4g+i, 16+4g+i) and dP of one tile, this wave's heads
  auto ld_k = [&](const CSA_LDS unsigned char* lb, int row16, int k) {
    Frag<T> f;
    const CSA_LDS unsigned char* p =
        lb + qk_base[k & 1] + (SWZ ? row16 * 1024 + 64 * k : eoff(row16, 32 * k) - eoff(0, 0));
    *reinterpret_cast<u32x4*>(f.v) = *(const CSA_LDS u32x4*)p;
    if constexpr (ES == 4) *reinterpret_cast<u32x4*>(f.v + 4) = *(const CSA_LDS u32x4*)(p + 16);
    return f;
  };
  auto qk_only = [&](const unsigned char* sb, Acc& acc) {
    const CSA_LDS unsigned char* lb = (const CSA_LDS unsigned char*)sb;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      const Frag<T> a0 = ld_k(lb, 0, k), a1 = ld_k(lb, 16, k);
      acc[0] = mfma16x16x32(a0, qf[k], acc[0]);
      acc[1] = mfma16x16x32(a1, qf[k], acc[1]);
      acc[2] = mfma16x16x32(a0, uf[k], acc[2]);
      acc[3] = mfma16x16x32(a1, uf[k], acc[3]);
    }
  };
  // p = exp(z - lse), ds = scale p (dP - delta), both rounded to T, into the exchange
  // rows at h' = 2h (ds) and 2h + 1 (p)
  auto softmax = [&](const Acc& acc, const int* kv, unsigned char* xb) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int key = i < 4 ? 4 * g + i : 12 + 4 * g + i;
      const float z = i < 4 ? acc[0][i] : acc[1][i - 4];
      const float dp = i < 4 ? acc[2][i] : acc[3][i - 4];
      const float pr = kv[key] ? __builtin_amdgcn_exp2f(z * a.scale_log2 - lse2) : 0.f;
      const float2 pd = make_float2(a.scale * pr * (dp - delta), pr);
      unsigned char* xp = xb + key * XS + 2 * h * ES;
      if constexpr (ES == 2) {
        typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
        typedef float f32x2_t __attribute__((ext_vector_type(2)));
        *reinterpret_cast<uint32_t*>(xp) =
            __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{pd.x, pd.y}, bf16x2_t));
      } else {
        *reinterpret_cast<float2*>(xp) = pd;
      }
    }
  };
  // key gradients of a tile, rounded to T: lane (dims 4g..4g+3 of block db, key 16kb + hl)
  typedef typename std::conditional<ES == 2, uint2, uint4>::type Pack;
  // deferred stores need the tile's rows in registers; where that is too many (one
  // wave holding every dim) each dim block is stored as soon as it is formed
  constexpr bool DEFER = DBW * 2 * (int)sizeof(Pack) / 4 <= 32;
  Pack pend[DEFER ? DBW : 1][2];
  auto pack = [&](const f32x4& c) -> Pack {
    if constexpr (ES == 2) {
      typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
      return __builtin_bit_cast(Pack, __builtin_convertvector(c, bf16x4_t));
    } else {
      return __builtin_bit_cast(Pack, c);
    }
  };
  auto row_dst = [&](int tile, int kb) -> unsigned char* {
    const int kk = tile * KT + 16 * kb + hl;
    if (kk >= nk) return nullptr;
    const int slot = kk < nsel ? kk : a.kmax + (kk - nsel);
    return interm + ((prow + slot) * D + wave * DW + 4 * g) * ES;
  };
  // the gradient rows of tile `tile` (in pend) to their slot rows (nothing to do when
  // they were stored as formed)
  auto store_tile = [&](int tile) {
    if constexpr (DEFER) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        unsigned char* dst = row_dst(tile, kb);
        if (dst) {
#pragma unroll
          for (int db = 0; db < DBW; ++db) *reinterpret_cast<Pack*>(dst + 16 * db * ES) = pend[db][kb];
        }
      }
    }
  };
  // key gradients of the tile whose exchange rows are in xb (into pend), interleaved
  // with the logits and dP of the tile in nsb (into nacc): per logit k-step, four
  // MFMAs of each
  auto grad_and_qk = [&](const unsigned char* xb, const unsigned char* nsb, Acc& nacc, int tile) {
    const CSA_LDS unsigned char* lb = (const CSA_LDS unsigned char*)nsb;
    unsigned char* dst0 = DEFER ? nullptr : row_dst(tile, 0);
    unsigned char* dst1 = DEFER ? nullptr : row_dst(tile, 1);
    Frag<T> xf[NW][2];
#pragma unroll
    for (int j = 0; j < NW; ++j)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const unsigned char* p = xb + (16 * kb + hl) * XS + (32 * j + 8 * g) * ES;
        *reinterpret_cast<uint4*>(xf[j][kb].v) = *reinterpret_cast<const uint4*>(p);
        if constexpr (ES == 4) *reinterpret_cast<uint4*>(xf[j][kb].v + 4) = *reinterpret_cast<const uint4*>(p + 16);
      }
#pragma unroll
    for (int i = 0; i < 4; ++i) nacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 c4[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      const Frag<T> a0 = ld_k(lb, 0, k), a1 = ld_k(lb, 16, k);
#pragma unroll
      for (int m = 0; m < 2; ++m) {  // two (db, j) pairs of the key gradient per k-step
        const int f = 2 * k + m;
        const int db = f / NW, j = f % NW;
        c4[0] = mfma16x16x32(qu[db][j], xf[j][0], c4[0]);
        c4[1] = mfma16x16x32(qu[db][j], xf[j][1], c4[1]);
        if (j == NW - 1) {
          if constexpr (DEFER) {
            pend[db][0] = pack(c4[0]);
            pend[db][1] = pack(c4[1]);
          } else {
            if (dst0) *reinterpret_cast<Pack*>(dst0 + 16 * db * ES) = pack(c4[0]);
            if (dst1) *reinterpret_cast<Pack*>(dst1 + 16 * db * ES) = pack(c4[1]);
          }
          c4[0] = c4[1] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
      nacc[0] = mfma16x16x32(a0, qf[k], nacc[0]);
      nacc[1] = mfma16x16x32(a1, qf[k], nacc[1]);
      nacc[2] = mfma16x16x32(a0, uf[k], nacc[2]);
      nacc[3] = mfma16x16x32(a1, uf[k], nacc[3]);
    }
  };

  const int ntiles = (nk + KT - 1) / KT;
  // all stages filled up front; tile t+NS then goes to tile t's stage once tile t's
  // logits (formed in the step before) are done with it
  if (ntiles > 0) issue(0, st0, kv0);
  if (ntiles > 1) issue(1, st1, kv1);
  if (NS == 4 && ntiles > 2) issue(2, st2, kv2);
  if (NS == 4 && ntiles > 3) issue(3, st3, kv3);
  // barrier once this wave's copies of every tile up to tile `need` have landed; the
  // copies of later tiles (up to tile `last`, the last requested) stay in flight.
  // Stores issued in between count too, so the wait may also cover some of them.
  auto wait_tile = [&](int need, int last) {
    const int ahead = min(ntiles - 1, last) - need;
    if (ahead <= 0) vm_wait_barrier<0>();
    else if (ahead == 1) vm_wait_barrier<LPT>();
    else if (ahead == 2) vm_wait_barrier<2 * LPT>();
    else vm_wait_barrier<3 * LPT>();
  };
  Acc accA, accB;
  if (ntiles > 0) {
    wait_tile(0, NS - 1);
    qk_only(st0, accA);
  }
  // tile tl: its logits are in cur; after the barrier its gradients and the next tile's
  // logits (into nxt, from nsb) are formed, the previous tile's gradient rows stored,
  // and tile tl+NS requested into tile tl's stage (isb)
  auto iter = [&](int tl, int* kvc, unsigned char* xb, const Acc& cur, Acc& nxt, const unsigned char* nsb,
                  unsigned char* isb) {
    softmax(cur, kvc, xb);
    wait_tile(tl + 1, tl + NS - 1);  // also: every exchange row of tile tl is written
    if (tl > 0) store_tile(tl - 1);
    if (tl + NS < ntiles) issue(tl + NS, isb, kvc);
    grad_and_qk(xb, nsb, nxt, tl);  // at the last tile the logits of a stale stage are not used
  };
  for (int tile = 0; tile < ntiles; tile += NS) {
    if constexpr (NS == 4) {
      iter(tile, kv0, xs0, accA, accB, st1, st0);
      if (tile + 1 < ntiles) iter(tile + 1, kv1, xs1, accB, accA, st2, st1);
      if (tile + 2 < ntiles) iter(tile + 2, kv2, xs0, accA, accB, st3, st2);
      if (tile + 3 < ntiles) iter(tile + 3, kv3, xs1, accB, accA, st0, st3);
    } else {
      iter(tile, kv0, xs0, accA, accB, st1, st0);
      if (tile + 1 < ntiles) iter(tile + 1, kv1, xs1, accB, accA, st0, st1);
    }
  }
  if (ntiles > 0) store_tile(ntiles - 1);
}

// ---------------------------------------------------------------------------------
// Inverse index of the chunk's entry pairs and the key-major sums.
// ---------------------------------------------------------------------------------
struct RedArgs {
  const int32_t* idx;
  int32_t S, ratio, topk, n_entries, mode, kmax, kw, D;
  int64_t r0;
  int32_t nrows;
  int32_t key_lo, nkeys;  // entry keys b*n + s of the chunk: key_lo .. key_lo + nkeys - 1
  int32_t* cnt;           // [nblk][nkeys] counts, then running positions
  int32_t* tot;           // [nkeys]
  int32_t* base;          // [nkeys + 1] first list position of each key; base[nkeys] = pairs
  int32_t* segbase;       // [nkeys + 1] first segment of each key; segbase[nkeys] = segments
  int32_t* list;          // [pairs] slot rows (row - r0) * kw + slot, per key in row order
  const void* interm;
  float* partial;         // [segments][D]
  float* dkv_c;           // [B, n, D]
};

constexpr int kRowBlock = 64;  // rows per counting block (validate.hpp: kDkvRowBlock)
constexpr int kSeg = 256;      // pairs per summed segment (validate.hpp: kDkvSeg)
static_assert(kRowBlock == kDkvRowBlock && kSeg == kDkvSeg, "host plan and kernels agree");

// Entry j of chunk row rr: its key relative to key_lo, or -1 when masked.
__device__ inline int pair_key(const RedArgs& a, int rr, int j) {
  const int64_t r = a.r0 + rr;
  const int b = (int)(r / a.S), t = (int)(r % a.S);
  const int n_t = visible_entries(t, a.ratio);
  int s;
  if (a.mode == MQA_SELECTED) {
    if (j >= min(a.topk, n_t)) return -1;
    s = a.idx[r * a.topk + j];
  } else {
    if (j >= n_t) return -1;
    s = j;
  }
  if (s < 0 || s >= n_t) return -1;
  return b * a.n_entries + s - a.key_lo;
}

// n 4-byte words from a 16-byte aligned p: whole 16-byte chunks, then the tail words
__global__ __launch_bounds__(256) void fill_zero_kernel(uint32_t* p, int64_t n) {
  const int64_t n16 = n >> 2;
  const int64_t i0 = (int64_t)blockIdx.x * 256 + threadIdx.x, step = (int64_t)gridDim.x * 256;
  for (int64_t i = i0; i < n16; i += step) reinterpret_cast<uint4*>(p)[i] = make_uint4(0, 0, 0, 0);
  if (i0 < (n & 3)) p[4 * n16 + i0] = 0u;
}

__global__ __launch_bounds__(256) void pair_count_kernel(RedArgs a) {
  const int blk = blockIdx.x;
  const int rend = min(a.nrows, (blk + 1) * kRowBlock);
  for (int rr = blk * kRowBlock; rr < rend; ++rr)
    for (int j = threadIdx.x; j < a.kmax; j += 256) {
      const int key = pair_key(a, rr, j);
      if (key >= 0) atomicAdd(&a.cnt[(int64_t)blk * a.nkeys + key], 1);
    }
}

// per key: counts of the blocks -> the blocks' exclusive offsets within the key
__global__ __launch_bounds__(256) void pair_scan_blocks_kernel(RedArgs a, int nblk) {
  const int key = blockIdx.x * 256 + threadIdx.x;
  if (key >= a.nkeys) return;
  int run = 0;
  for (int blk = 0; blk < nblk; ++blk) {
    int32_t* c = a.cnt + (int64_t)blk * a.nkeys + key;
    const int v = *c;
    *c = run;
    run += v;
  }
  a.tot[key] = run;
}

// exclusive scans over keys of the pair counts and of the segment counts (one workgroup)
__global__ __launch_bounds__(1024) void pair_scan_keys_kernel(RedArgs a) {
  __shared__ int sp[1024], ss[1024];
  __shared__ int carry_p, carry_s;
  if (threadIdx.x == 0) carry_p = carry_s = 0;
  __syncthreads();
  for (int k0 = 0; k0 < a.nkeys; k0 += 1024) {
    const int key = k0 + threadIdx.x;
    const int c = key < a.nkeys ? a.tot[key] : 0;
    int vp = c, vs = (c + kSeg - 1) / kSeg;
    sp[threadIdx.x] = vp;
    ss[threadIdx.x] = vs;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {  // inclusive Hillis-Steele scan
      const int ap = threadIdx.x >= d ? sp[threadIdx.x - d] : 0;
      const int as = threadIdx.x >= d ? ss[threadIdx.x - d] : 0;
      __syncthreads();
      sp[threadIdx.x] += ap;
      ss[threadIdx.x] += as;
      __syncthreads();
    }
    if (key < a.nkeys) {
      a.base[key] = carry_p + sp[threadIdx.x] - vp;
      a.segbase[key] = carry_s + ss[threadIdx.x] - vs;
    }
    __syncthreads();
    if (threadIdx.x == 1023) {
      carry_p += sp[1023];
      carry_s += ss[1023];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    a.base[a.nkeys] = carry_p;
    a.segbase[a.nkeys] = carry_s;
  }
}

// rows of a block in order; within a row every key is taken once (atomics only keep a
// repeated entry of one row from colliding)
__global__ __launch_bounds__(256) void pair_fill_kernel(RedArgs a) {
  const int blk = blockIdx.x;
  const int rend = min(a.nrows, (blk + 1) * kRowBlock);
  for (int rr = blk * kRowBlock; rr < rend; ++rr) {
    for (int j = threadIdx.x; j < a.kmax; j += 256) {
      const int key = pair_key(a, rr, j);
      if (key >= 0) {
        const int pos = a.base[key] + atomicAdd(&a.cnt[(int64_t)blk * a.nkeys + key], 1);
        a.list[pos] = rr * a.kw + j;
      }
    }
    __syncthreads();
  }
}

// One wave per segment of up to kSeg pairs of one key: the sum of their gradient rows.
// A key with one segment adds it to dkv_c here; longer keys leave partials.
template <typename T, int D>
__global__ __launch_bounds__(256) void pair_reduce_kernel(RedArgs a, int max_segs) {
  constexpr int V = D / 64;  // dims per lane
  const int lane = threadIdx.x & 63;
  const int seg = (int)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (seg >= max_segs || seg >= a.segbase[a.nkeys]) return;
  int lo = 0, hi = a.nkeys - 1;  // last key whose first segment is <= seg
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.segbase[mid] <= seg) lo = mid;
    else hi = mid - 1;
  }
  const int key = lo;
  const int p0 = a.base[key] + (seg - a.segbase[key]) * kSeg;
  const int p1 = min(p0 + kSeg, a.base[key + 1]);
  float acc[V];
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0.f;
  const T* src = reinterpret_cast<const T*>(a.interm);
  // The pair indices of up to 64 rows come in one load (a lane each) and go to the row
  // loads through v_readlane, and the rows are loaded RB at a time, kept in their storage
  // type, before they are added (in list order, as one at a time would): RB rows in
  // flight per wave instead of one dependent index-then-row chain per row.
  constexpr int RB = sizeof(T) == 2 ? 16 : 8;
  for (int pb = p0; pb < p1; pb += 64) {
    const int n = min(64, p1 - pb);
    const int lidx = a.list[pb + min(lane, n - 1)];
    int j = 0;
    for (; j + RB <= n; j += RB) {
      T r[RB][V];
#pragma unroll
      for (int u = 0; u < RB; ++u) {
        const T* row = src + (int64_t)__builtin_amdgcn_readlane(lidx, j + u) * D + lane * V;
#pragma unroll
        for (int i = 0; i < V; ++i) r[u][i] = row[i];
      }
#pragma unroll
      for (int u = 0; u < RB; ++u)
#pragma unroll
        for (int i = 0; i < V; ++i) acc[i] += to_f32(r[u][i]);
    }
    for (; j < n; ++j) {
      const T* row = src + (int64_t)__builtin_amdgcn_readlane(lidx, j) * D + lane * V;
#pragma unroll
      for (int i = 0; i < V; ++i) acc[i] += to_f32(row[i]);
    }
  }
  const int ns = a.segbase[key + 1] - a.segbase[key];
  float* dst = ns == 1 ? a.dkv_c + ((int64_t)a.key_lo + key) * D : a.partial + (int64_t)seg * D;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    if (ns == 1) dst[lane * V + i] += acc[i];
    else dst[lane * V + i] = acc[i];
  }
}

// keys with several segments: their partials added in segment order
template <int D>
__global__ __launch_bounds__(256) void pair_combine_kernel(RedArgs a) {
  constexpr int V = D / 64;
  const int lane = threadIdx.x & 63;
  const int key = (int)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (key >= a.nkeys) return;
  const int s0 = a.segbase[key], ns = a.segbase[key + 1] - s0;
  if (ns <= 1) return;
  float acc[V];
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0.f;
  for (int s = 0; s < ns; ++s)
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] += a.partial[(int64_t)(s0 + s) * D + lane * V + i];
  float* dst = a.dkv_c + ((int64_t)a.key_lo + key) * D + lane * V;
#pragma unroll
  for (int i = 0; i < V; ++i) dst[i] += acc[i];
}

// One wave per window token x = b*S + t' of the chunk's reach: the sum of its slot rows
// over the chunk's rows t' .. t'+W-1 of the same sequence, added to the fp32 accumulator.
struct WinArgs {
  const void* interm;
  float* acc;  // [B,S,D]
  int32_t S, window, kmax, kw;
  int64_t r0, x0;
  int32_t nrows, ntok;
};
template <typename T, int D>
__global__ __launch_bounds__(256) void window_reduce_kernel(WinArgs a) {
  constexpr int V = D / 64;
  const int lane = threadIdx.x & 63;
  const int w = (int)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= a.ntok) return;
  const int64_t x = a.x0 + w;
  const int64_t bS = x - x % a.S;  // b*S
  const int tp = (int)(x % a.S);
  const int64_t rlo = max(x, a.r0);
  const int64_t rhi = min(min(bS + a.S, x + a.window), a.r0 + a.nrows);  // exclusive
  if (rlo >= rhi) return;
  float acc[V];
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0.f;
  const T* src = reinterpret_cast<const T*>(a.interm);
  auto row_of = [&](int64_t r) -> const T* {
    const int t = (int)(r - bS);
    const int slot = a.kmax + tp - window_lo(t, a.window);
    return src + ((r - a.r0) * a.kw + slot) * D + lane * V;
  };
  int64_t r = rlo;
  for (; r + 8 <= rhi; r += 8) {  // eight rows in flight, added in row order
    float v[8][V];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const T* row = row_of(r + u);
#pragma unroll
      for (int i = 0; i < V; ++i) v[u][i] = to_f32(row[i]);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int i = 0; i < V; ++i) acc[i] += v[u][i];
  }
  for (; r < rhi; ++r) {
    const T* row = row_of(r);
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] += to_f32(row[i]);
  }
  float* dst = a.acc + x * D + lane * V;
#pragma unroll
  for (int i = 0; i < V; ++i) dst[i] += acc[i];
}

// dkv_raw = RMSNorm'( RoPE(acc, -(pos0 + t')) ) in place, one wave per token, lane dims
// 8*lane .. (the window latents' rotation and optional norm, transposed).
struct WinFinArgs {
  float* acc;
  const void* kv_raw;
  int32_t B, S, D, R, norm;
  float eps;
  double theta;
  int64_t pos0;
};
template <typename T>
__global__ __launch_bounds__(256) void window_finish_kernel(WinFinArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t x = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (x >= (int64_t)a.B * a.S) return;
  const int t = (int)(x % a.S);
  const int c0 = lane * 8;
  const bool own = c0 < a.D;
  float gv[8], xv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) gv[i] = xv[i] = 0.f;
  float* gp = a.acc + x * a.D + c0;
  if (own) {
#pragma unroll
    for (int i = 0; i < 8; ++i) gv[i] = gp[i];
    const int lo = a.D - a.R;
    const int64_t P = a.pos0 + t;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = c0 + 2 * k;
      if (c >= lo) {  // transpose of the rotation by +P
        float cs, sn;
        rope_cos_sin(P, rope_inv_freq((c - lo) >> 1, a.R, a.theta), &cs, &sn);
        const float g0 = gv[2 * k], g1 = gv[2 * k + 1];
        gv[2 * k] = g0 * cs + g1 * sn;
        gv[2 * k + 1] = -g0 * sn + g1 * cs;
      }
    }
  }
  if (a.norm) {  // y = x r, r = (mean x^2 + eps)^-1/2: dx = r (dy - y mean(dy y))
    if (own) {
      const T* xp = reinterpret_cast<const T*>(a.kv_raw) + x * a.D + c0;
#pragma unroll
      for (int i = 0; i < 8; ++i) xv[i] = to_f32(xp[i]);
    }
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ss += xv[i] * xv[i];
    ss = wave_sum(ss);
    const float rr = 1.0f / sqrtf(ss / (float)a.D + a.eps);
    float gy = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) gy += gv[i] * xv[i] * rr;
    gy = wave_sum(gy) / (float)a.D;
#pragma unroll
    for (int i = 0; i < 8; ++i) gv[i] = rr * (gv[i] - xv[i] * rr * gy);
  }
  if (own) {
#pragma unroll
    for (int i = 0; i < 8; ++i) gp[i] = gv[i];
  }
}

// dsinks[h] = sum over rows of ds_row[row, h], in a fixed order: workgroup g sums rows
// g, g + G, ... (4 row phases per workgroup), then one workgroup adds the G partials.
constexpr int kSinkGroups = 256;
__global__ __launch_bounds__(256) void sink_partial_kernel(const float* ds_row, int64_t rows, int H,
                                                           float* part) {
  __shared__ float red[4][64];
  const int hh = threadIdx.x & 63, ph = threadIdx.x >> 6;
  float s = 0.f;
  if (hh < H)
    for (int64_t r = (int64_t)blockIdx.x * 4 + ph; r < rows; r += (int64_t)gridDim.x * 4) s += ds_row[r * H + hh];
  red[ph][hh] = s;
  __syncthreads();
  if (ph == 0 && hh < H) part[(int64_t)blockIdx.x * H + hh] = ((red[0][hh] + red[1][hh]) + red[2][hh]) + red[3][hh];
}
__global__ __launch_bounds__(64) void sink_sum_kernel(const float* part, int groups, int H, float* dsinks) {
  const int hh = threadIdx.x;
  if (hh >= H) return;
  float s = 0.f;
  for (int gi = 0; gi < groups; ++gi) s += part[(int64_t)gi * H + hh];
  dsinks[hh] = s;
}

// bytes: a multiple of 4 (every region cleared here holds 4-byte words)
hipError_t zero(void* p, size_t bytes, hipStream_t st) {
  const int64_t n = (int64_t)(bytes / 4);
  if (n == 0) return hipSuccess;
  const int64_t blocks = (n / 4 + 255) / 256;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)(blocks < 1 ? 1 : (blocks < 4096 ? blocks : 4096))),
                     dim3(256), 0, st, static_cast<uint32_t*>(p), n);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t run_chunks(const csa_params_t& p, MqaMode mode, DkvArgs a, const DkvWs& w, float* dkv_c,
                      float* dkv_raw, hipStream_t st) {
  const DkvShape sh = dkv_shape(p, mode == MQA_SELECTED ? 0 : (mode == MQA_DENSE ? 1 : 2));
  const int64_t rows = (int64_t)p.B * p.S;
  const int n = a.n_entries;
  a.kmax = sh.kmax;
  a.kw = sh.kw;
  for (int64_t r0 = 0; r0 < rows; r0 += sh.rows) {
    const int nr = (int)(rows - r0 < sh.rows ? rows - r0 : sh.rows);
    a.r0 = r0;
    a.nrows = nr;
    // waves of 16 heads; one wave holding all 512 dims of the key-gradient operand would
    // run out of registers, so up to 32 heads take two waves there
    bool done = false;
    if constexpr (D <= 256) {
      if (p.H <= 16) {
        hipLaunchKernelGGL((mqa_bwd_dkv_kernel<T, D, 1>), dim3(nr), dim3(64), 0, st, a);
        done = true;
      }
    }
    if (!done) {
      if (p.H <= 32) hipLaunchKernelGGL((mqa_bwd_dkv_kernel<T, D, 2>), dim3(nr), dim3(128), 0, st, a);
      else hipLaunchKernelGGL((mqa_bwd_dkv_kernel<T, D, 4>), dim3(nr), dim3(256), 0, st, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (sh.kmax > 0) {
      RedArgs ra{};
      ra.idx = a.idx;
      ra.S = p.S;
      ra.ratio = p.ratio;
      ra.topk = p.topk;
      ra.n_entries = n;
      ra.mode = mode;
      ra.kmax = sh.kmax;
      ra.kw = sh.kw;
      ra.D = D;
      ra.r0 = r0;
      ra.nrows = nr;
      const int b_lo = (int)(r0 / p.S), b_hi = (int)((r0 + nr - 1) / p.S);
      ra.key_lo = b_lo * n;
      ra.nkeys = (b_hi - b_lo + 1) * n;
      ra.cnt = w.cnt;
      ra.tot = w.tot;
      ra.base = w.base;
      ra.segbase = w.segbase;
      ra.list = w.list;
      ra.interm = a.interm;
      ra.partial = w.partial;
      ra.dkv_c = dkv_c;
      const int nblk = (nr + kRowBlock - 1) / kRowBlock;
      if ((e = zero(w.cnt, (size_t)nblk * ra.nkeys * 4, st)) != hipSuccess) return e;
      hipLaunchKernelGGL(pair_count_kernel, dim3(nblk), dim3(256), 0, st, ra);
      hipLaunchKernelGGL(pair_scan_blocks_kernel, dim3((ra.nkeys + 255) / 256), dim3(256), 0, st, ra, nblk);
      hipLaunchKernelGGL(pair_scan_keys_kernel, dim3(1), dim3(1024), 0, st, ra);
      hipLaunchKernelGGL(pair_fill_kernel, dim3(nblk), dim3(256), 0, st, ra);
      const int64_t max_segs = (int64_t)nr * sh.kmax / kSeg + ra.nkeys + 1;
      hipLaunchKernelGGL((pair_reduce_kernel<T, D>), dim3((unsigned)((max_segs + 3) / 4)), dim3(256), 0, st, ra,
                         (int)max_segs);
      hipLaunchKernelGGL((pair_combine_kernel<D>), dim3((ra.nkeys + 3) / 4), dim3(256), 0, st, ra);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (p.window > 0) {
      WinArgs wa{};
      wa.interm = a.interm;
      wa.acc = dkv_raw;
      wa.S = p.S;
      wa.window = p.window;
      wa.kmax = sh.kmax;
      wa.kw = sh.kw;
      wa.r0 = r0;
      wa.x0 = r0 - (p.window - 1) > 0 ? r0 - (p.window - 1) : 0;
      wa.nrows = nr;
      wa.ntok = (int)(r0 + nr - wa.x0);
      hipLaunchKernelGGL((window_reduce_kernel<T, D>), dim3((wa.ntok + 3) / 4), dim3(256), 0, st, wa);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

template <typename T>
hipError_t run_t(const csa_params_t& p, MqaMode mode, const DkvArgs& a, const DkvWs& w, float* dkv_c,
                 float* dkv_raw, hipStream_t st) {
  switch (p.D) {
    case 64: return run_chunks<T, 64>(p, mode, a, w, dkv_c, dkv_raw, st);
    case 128: return run_chunks<T, 128>(p, mode, a, w, dkv_c, dkv_raw, st);
    case 256: return run_chunks<T, 256>(p, mode, a, w, dkv_c, dkv_raw, st);
    case 512:
      if constexpr (sizeof(T) == 2) return run_chunks<T, 512>(p, mode, a, w, dkv_c, dkv_raw, st);
      else return hipErrorInvalidValue;  // fp32 at D = 512 is refused by the caller
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_zero_f32(float* p, size_t n, hipStream_t st) { return zero(p, n * 4, st); }

hipError_t launch_mqa_bwd_dkv(const csa_params_t& p, MqaMode mode, const void* q, const void* kv_c,
                              const void* kv_w, const void* kv_raw, const int32_t* idx, const float* sinks,
                              const void* o, const float* lse, const void* d_o, float* dkv_c, float* dkv_raw,
                              float* dsinks, const DkvWs& w, hipStream_t st) {
  const int64_t rows = (int64_t)p.B * p.S;
  const int n = mode == MQA_WINDOW_ONLY ? 0 : p.S / p.ratio;
  hipError_t e;
  if (dkv_c && (e = zero(dkv_c, (size_t)p.B * n * p.D * 4, st)) != hipSuccess) return e;
  if ((e = zero(dkv_raw, (size_t)rows * p.D * 4, st)) != hipSuccess) return e;
  if (rows == 0) return dsinks ? zero(dsinks, (size_t)p.H * 4, st) : hipSuccess;
  DkvArgs a{};
  a.q = q;
  a.kv_c = kv_c;
  a.kv_w = kv_w;
  a.idx = idx;
  a.sinks = sinks;
  a.o = o;
  a.lse = lse;
  a.d_o = d_o;
  a.interm = w.interm;
  a.ds_row = sinks ? w.ds_row : nullptr;
  a.B = p.B;
  a.S = p.S;
  a.H = p.H;
  a.R = p.rope_dim;
  a.ratio = p.ratio;
  a.window = p.window;
  a.topk = p.topk;
  a.n_entries = n;
  a.mode = mode;
  a.scale_log2 = p.softmax_scale * kLog2e;
  a.scale = p.softmax_scale;
  a.theta = p.rope_theta;
  a.pos0 = p.pos0;
  e = p.dtype == CSA_BF16 ? run_t<bf16>(p, mode, a, w, dkv_c, dkv_raw, st)
                          : run_t<float>(p, mode, a, w, dkv_c, dkv_raw, st);
  if (e != hipSuccess) return e;
  const bool norm = (p.flags & CSA_FLAG_NORM_WINDOW) != 0;
  if (p.window > 0 && (p.rope_dim > 0 || norm)) {
    WinFinArgs f{dkv_raw, kv_raw, p.B, p.S, p.D, p.rope_dim, norm ? 1 : 0, p.rms_eps, p.rope_theta, p.pos0};
    const dim3 grid((unsigned)((rows + 3) / 4));
    if (p.dtype == CSA_BF16) hipLaunchKernelGGL(window_finish_kernel<bf16>, grid, dim3(256), 0, st, f);
    else hipLaunchKernelGGL(window_finish_kernel<float>, grid, dim3(256), 0, st, f);
  }
  if (sinks) {
    const int groups = (int)(rows < kSinkGroups * 4 ? (rows + 3) / 4 : kSinkGroups);
    hipLaunchKernelGGL(sink_partial_kernel, dim3(groups), dim3(256), 0, st, w.ds_row, rows, p.H, w.sink_part);
    hipLaunchKernelGGL(sink_sum_kernel, dim3(1), dim3(64), 0, st, w.sink_part, groups, p.H, dsinks);
  }
  return hipGetLastError();
}

}  // namespace csa
