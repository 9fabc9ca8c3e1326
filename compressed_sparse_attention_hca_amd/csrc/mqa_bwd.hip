// Backward of stage 4, query side, on gfx950: dL/dq of the sparse multi-query
// attention, with delta = rowsum(o * do) computed inside the same kernel.
//
// Sources: "Enabling DeepSeek-V4-Flash Training on AMD Instinct MI355X GPUs with
// Primus", section "Attention kernels for the three layer types": the backward splits
// into dQ, interm (the key-side head contraction) and delta, and delta is folded into
// dQ; dQ runs at one wave per SIMD (its register set is large) and hides the latency
// of the key gather by keeping the per-tile chain of products interleaved.  The
// forward it differentiates is the one of sparse_mqa.hip:
//   z[h,k] = (RoPE(q[h], P) . key_k) * scale,  u[h] = sum_k softmax_k(z) key_k,
//   o[h]   = RoPE(u[h], -P)                     (P = pos0 + t)
// With du = RoPE(do, +P) (the transpose of the de-rotation), dP[h,k] = du[h] . key_k,
// delta[h] = du[h] . u[h] = do[h] . o[h] (a rotation preserves the dot product) and
// dz = P_hk (dP - delta):
//   dq[h] = RoPE( scale * sum_k dz[h,k] key_k , -P ).
//
// One pass over the keys.  P = e / l with e = exp2(z*log2e - m_ref) against a fixed
// reference m_ref (the first tile's max, exact by shift invariance, with a second pass
// when a later logit could overflow, as in the forward) and delta known before the
// loop, so the kernel accumulates sum_k e_k (dP_k - delta) key_k and divides by l at
// the end: no statistics pass.  A sink only joins l.
//
// Mapping (as the forward's 16-head kernel): one workgroup per query, wave w owns heads
// 16w .. 16w+15 and all D dims.  Keys stream through LDS in tiles of 32 rows, staged by
// direct-to-LDS loads into two stages.  Per tile, from the same K fragments:
//   S^T[key, head]  = K . Q^T     and   dP^T[key, head] = K . dU^T
//   (v_mfma_f32_16x16x32_bf16, keys on M, heads on N with q and du in registers)
//   dz^T = e (dP - delta) in registers, rounded to the activation type
//   dQ^T[dim, head] += K^T . dz^T  (K^T by transposing LDS reads, dz^T as B operand)
// The accumulator layout of S^T gives lane (head, g) exactly the keys that are its
// B-operand k-slots in the last product, so dz never leaves registers.
#include "common.hpp"
#include "mqa_bwd.hpp"

namespace csa {
namespace {

struct DqArgs {
  const void* q;
  const void* kv_c;
  const void* kv_w;
  const int32_t* idx;
  const float* sinks;  // [H] softmax-sink logits, or nullptr
  const void* o;       // forward output [B,S,H,D]
  const void* d_o;     // dL/do [B,S,H,D]
  void* dq;            // dL/dq [B,S,H,D]
  int32_t B, S, H, R, ratio, window, topk, n_entries, mode;
  float scale_log2;  // softmax_scale * log2(e)
  float scale;       // softmax_scale
  double theta;
  int64_t pos0;
};

constexpr int kMaxTopk = 2048;
constexpr float kLog2e = 1.4426950408889634f;

// Key slot (within a tile of 32) held at k-slot i of lane group g: the rows of the
// S^T accumulator that lane group g holds (4g..4g+3, then 16+4g..16+4g+3).
__device__ constexpr int dz_slot_key(int g, int i) { return i < 4 ? 4 * g + i : 12 + 4 * g + i; }

// Wait until at most N of this wave's vector-memory loads are outstanding and its LDS
// operations are done, then barrier.  Unlike __syncthreads this leaves the N youngest
// direct-to-LDS loads in flight; the memory clobber keeps the compiler from moving LDS
// accesses across it.
template <int N> __device__ inline void vm_wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

template <typename T, int D, int NW>
__global__ __launch_bounds__(NW * 64, 1) void mqa_bwd_dq_kernel(DqArgs a) {
  constexpr int NT = NW * 64;
  constexpr int HP = NW * 16;
  constexpr int ES = (int)sizeof(T);
  constexpr int KT = 32;
  constexpr int ROWB = D * ES;
  constexpr int NCH = ROWB / 16;
  // Tile layout as in the forward: 1 KB lines, one direct-to-LDS wave load each; a
  // 1 KB row (D = 512 bf16) is XOR-swizzled by 16-byte chunk so that the row reads and
  // the transposing reads are free of bank conflicts; other row sizes pad the lines.
  constexpr int RPL = ROWB < 1024 ? 1024 / ROWB : 1;
  constexpr int LPR = ROWB > 1024 ? ROWB / 1024 : 1;
  constexpr int NL = KT * LPR / RPL;
  constexpr bool SWZ = ROWB == 1024 && ES == 2;
  constexpr int LSTRIDE = SWZ ? 1024 : 1024 + 48;
  constexpr int QROWB = ROWB + 16;
  constexpr int TILEB = NL * LSTRIDE;
  constexpr int SB = TILEB > (HP / 2) * QROWB ? TILEB : (HP / 2) * QROWB;
  // Direct-to-LDS loads per wave per tile, and the pipeline depth: NS stages, tile t+NS-1
  // in flight while tile t is used (the gather's latency is what this kernel waits on
  // at one workgroup per CU).  Four stages where the LDS holds them and the wait count
  // fits the 6-bit vmcnt field, else two.
  static_assert(NL % NW == 0, "every wave issues the same number of line loads");
  constexpr int LPT = NL / NW;
  constexpr int NS = (4 * SB + 12 * 1024 <= 160 * 1024 && 2 * LPT <= 63) ? 4 : 2;
  constexpr int SB2 = NS == 4 ? SB : 16;
  // Each stage is its own array: the compiler then sees that the loads in flight into
  // one stage do not alias the reads of another.
  __shared__ __attribute__((aligned(16))) unsigned char st0[SB];
  __shared__ __attribute__((aligned(16))) unsigned char st1[SB];
  __shared__ __attribute__((aligned(16))) unsigned char st2[SB2];
  __shared__ __attribute__((aligned(16))) unsigned char st3[SB2];
  __shared__ int kv0[KT], kv1[KT], kv2[KT], kv3[KT];
  __shared__ int sidx[kMaxTopk];
  __shared__ float2 cs[64];
  __shared__ int overflow;

  // workgroup -> query: 32 consecutive queries per XCD visit, XCDs interleaved across
  // the sequence, latest (heaviest) queries first.
  const int total = a.B * a.S;
  int gi = blockIdx.x;
  const int nfull = total & ~255;
  if (gi < nfull) {
    const int xcd = gi & 7, j = gi >> 3;
    gi = (((j >> 5) << 3) + xcd) * 32 + (j & 31);
  }
  gi = total - 1 - gi;
  const int b = gi / a.S;
  const int t = gi % a.S;

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

  if (threadIdx.x == 0) overflow = 0;
  if (threadIdx.x < a.R / 2) {
    float c, s;
    rope_cos_sin(P, rope_inv_freq(threadIdx.x, a.R, a.theta), &c, &s);
    cs[threadIdx.x] = make_float2(c, s);
  }
  if (a.mode == MQA_SELECTED) {
    const int32_t* irow = a.idx + ((int64_t)b * a.S + t) * a.topk;
    for (int i = threadIdx.x; i < nsel; i += NT) sidx[i] = irow[i];
  }

  const int64_t row0 = ((int64_t)b * a.S + t) * a.H * ROWB;  // byte offset of [b,t,0,0]
  const unsigned char* qg = reinterpret_cast<const unsigned char*>(a.q) + row0;
  const unsigned char* dog = reinterpret_cast<const unsigned char*>(a.d_o) + row0;
  const unsigned char* og = reinterpret_cast<const unsigned char*>(a.o) + row0;

  // H rows of D elements (heads >= H zero) -> LDS, heads 0..HP/2-1 in st0.
  auto stage_rows = [&](const unsigned char* src) {
    for (int c = threadIdx.x; c < HP * NCH; c += NT) {
      const int row = c / NCH, col = (c % NCH) * 16;
      const uint4 v = row < a.H ? *reinterpret_cast<const uint4*>(src + (int64_t)row * ROWB + col)
                                : make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>((row < HP / 2 ? st0 : st1) + (row % (HP / 2)) * QROWB + col) = v;
    }
  };
  auto my_row = [&]() -> const unsigned char* {
    return (h < HP / 2 ? st0 : st1) + (h % (HP / 2)) * QROWB;
  };
  // Rotate the pairs of a fragment (dims d0 .. d0+7) that fall in the last R dims by +P.
  auto rotate_frag = [&](Frag<T>& f, int d0) {
    if (d0 + 8 > rlo) {
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        const int d = d0 + i;
        if (d >= rlo) {
          const float2 r = cs[(d - rlo) >> 1];
          const float x0 = to_f32(f.v[i]), x1 = to_f32(f.v[i + 1]);
          f.v[i] = from_f32<T>(x0 * r.x - x1 * r.y);
          f.v[i + 1] = from_f32<T>(x0 * r.y + x1 * r.x);
        }
      }
    }
  };

  // ---- B operands: lane (head h, group g), k-step k holds dims 32k + 8g .. +7.
  Frag<T> qf[D / 32], uf[D / 32];
  stage_rows(qg);
  __syncthreads();
  {
    const unsigned char* r = my_row();
#pragma unroll
    for (int k = 0; k < D / 32; ++k) {
      qf[k] = load_frag(reinterpret_cast<const T*>(r) + 32 * k + 8 * g);
      rotate_frag(qf[k], 32 * k + 8 * g);
    }
  }
  __syncthreads();
  stage_rows(dog);
  __syncthreads();
  float delta = 0.f;
  {
    const unsigned char* r = my_row();
#pragma unroll
    for (int k = 0; k < D / 32; ++k) {
      const int d0 = 32 * k + 8 * g;
      uf[k] = load_frag(reinterpret_cast<const T*>(r) + d0);
      if (h < a.H) {
        const Frag<T> of = load_frag(reinterpret_cast<const T*>(og + (int64_t)h * ROWB) + d0);
#pragma unroll
        for (int i = 0; i < 8; ++i) delta = fmaf(to_f32(uf[k].v[i]), to_f32(of.v[i]), delta);
      }
      rotate_frag(uf[k], d0);
    }
  }
  delta += __shfl_xor(delta, 16, 64);
  delta += __shfl_xor(delta, 32, 64);
  __syncthreads();  // the staging area becomes the key tiles

  const unsigned char* kv_c = reinterpret_cast<const unsigned char*>(a.kv_c);
  const unsigned char* kv_w = reinterpret_cast<const unsigned char*>(a.kv_w);
  auto swz = [](int r) -> int { return ((r & 3) << 1) | ((r >> 2) & 1); };
  auto eoff = [&](int r, int d) -> int {
    const int byte = d * ES;
    if constexpr (SWZ) return r * 1024 + ((((byte >> 4) ^ swz(r)) << 4) | (byte & 15));
    return ((r / RPL) * LPR + byte / 1024) * LSTRIDE + (r % RPL) * ROWB + (byte % 1024);
  };
  // Source row of key kk; masked keys read this query's own q row (finite data whose
  // weight e is 0).
  // `s` is the entry index of key kk when kk < nsel.
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
    // With one key row per line the row, hence its entry index, is wave-uniform: the
    // tile's indices come from one LDS read (lane j: key tile*KT + j % KT) and are
    // picked per line with v_readlane, so no line waits on its own LDS read.
    int sv = 0;
    if constexpr (RPL == 1) {
      const int kk = tile * KT + (lane % KT);
      sv = a.mode == MQA_SELECTED ? (kk < nsel ? sidx[kk] : -1) : kk;
    }
#pragma unroll
    for (int L = wave; L < NL; L += NW) {
      int r, byte;
      if constexpr (RPL > 1) {
        r = L * RPL + lane / NCH;
        byte = (lane % NCH) * 16;
      } else if constexpr (SWZ) {
        r = L;
        byte = (lane ^ swz(r)) * 16;
      } else {
        r = L / LPR;
        byte = (L % LPR) * 1024 + lane * 16;
      }
      int ok, s;
      const int kk = tile * KT + r;
      if constexpr (RPL == 1) s = __builtin_amdgcn_readlane(sv, r);
      else s = a.mode == MQA_SELECTED ? (kk < nsel ? sidx[kk] : -1) : kk;
      const unsigned char* src = key_src(kk, s, &ok);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src + byte),
                                       (CSA_LDS void*)(sb + L * LSTRIDE), 16, 0, 0);
      if (byte == 0) kv[r] = ok;
    }
  };

  float m_seen = -INFINITY, m_ref = -INFINITY, l_run = 0.f;
  f32x4 acc[D / 16];

  // Per-lane LDS offsets of the K (row) and K^T (transposing) fragments, as in the
  // forward's 16-head kernel.
  int qk_base[2], tr_base[4];
  if constexpr (SWZ) {
    const int s = swz(hl), s2 = s >> 2;
    const int lo = hl * 1024 + (((g ^ s) & 3) << 4);
    qk_base[0] = lo + (s2 ? 64 : 0);
    qk_base[1] = lo - (s2 ? 64 : 0);
    const int a4 = hl >> 2, c = g & 1, hb = (hl >> 1) & 1;
    const int row = 4 * g + a4;
#pragma unroll
    for (int m = 0; m < 4; ++m)
      tr_base[m] = row * 1024 + ((m ^ a4) - m) * 32 + ((hb ^ c) << 4) + ((hl & 1) << 3);
  } else {
    qk_base[0] = qk_base[1] = eoff(hl, 8 * g);
#pragma unroll
    for (int m = 0; m < 4; ++m) tr_base[m] = eoff(4 * g + (hl >> 2), 4 * (hl & 3));
  }
  typedef short i16x4 __attribute__((ext_vector_type(4)));

  auto compute = [&](const unsigned char* sb, const int* kv) {
    const CSA_LDS unsigned char* lb = (const CSA_LDS unsigned char*)sb;
    auto ld_k = [&](int row16, int k) {
      Frag<T> f;
      const CSA_LDS unsigned char* p =
          lb + qk_base[k & 1] + (SWZ ? row16 * 1024 + 64 * k : eoff(row16, 32 * k) - eoff(0, 0));
      *reinterpret_cast<u32x4*>(f.v) = *(const CSA_LDS u32x4*)p;
      if constexpr (ES == 4) *reinterpret_cast<u32x4*>(f.v + 4) = *(const CSA_LDS u32x4*)(p + 16);
      return f;
    };
    // One wave per SIMD leaves no other wave to cover LDS latency, so the fragment
    // reads run PQ k-steps (QK) and PT dim blocks (the transposed product) ahead.
    constexpr int KS = D / 32, PQ = KS < 3 ? KS : 3;
    constexpr int DB = D / 16, PT = DB < 6 ? DB : 6;
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0, p0 = s0, p1 = s0;
    Frag<T> ka[PQ], kb[PQ];
#pragma unroll
    for (int k = 0; k < PQ; ++k) {
      ka[k] = ld_k(0, k);
      kb[k] = ld_k(16, k);
    }
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      const Frag<T> a0 = ka[k % PQ], a1 = kb[k % PQ];
      if (k + PQ < KS) {
        ka[k % PQ] = ld_k(0, k + PQ);
        kb[k % PQ] = ld_k(16, k + PQ);
      }
      s0 = mfma16x16x32(a0, qf[k], s0);
      s1 = mfma16x16x32(a1, qf[k], s1);
      p0 = mfma16x16x32(a0, uf[k], p0);
      p1 = mfma16x16x32(a1, uf[k], p1);
    }
    // dQ^T += K^T . dz^T: lane (dim 16db+hl, group g) takes keys dz_slot_key(g, 0..7)
    // of that dim from two transposing 8-byte reads.
    auto ld_t = [&](int db) {
      Frag<T> f;
      if constexpr (ES == 2) {
        const CSA_LDS unsigned char* p =
            lb + tr_base[db & 3] + (SWZ ? 32 * db : eoff(0, 16 * db) - eoff(0, 0));
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((CSA_LDS i16x4*)p);
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (CSA_LDS i16x4*)(p + (SWZ ? 16 * 1024 : eoff(16, 0) - eoff(0, 0))));
        typedef short i16x8 __attribute__((ext_vector_type(8)));
        const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        *reinterpret_cast<i16x8*>(f.v) = v;
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          f.v[i] = *(const CSA_LDS T*)(lb + eoff(dz_slot_key(g, i), 16 * db + hl));
      }
      return f;
    };
    Frag<T> tv[PT];
#pragma unroll
    for (int i = 0; i < PT; ++i) tv[i] = ld_t(i);  // independent of dz: issued before the softmax
    float z[8], dp[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      z[i] = kv[4 * g + i] ? s0[i] * a.scale_log2 : -INFINITY;
      z[4 + i] = kv[16 + 4 * g + i] ? s1[i] * a.scale_log2 : -INFINITY;
      dp[i] = p0[i];
      dp[4 + i] = p1[i];
    }
    float mt = z[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mt = fmaxf(mt, z[i]);
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    m_seen = fmaxf(m_seen, mt);
    if (m_ref == -INFINITY) m_ref = mt;  // acc and l are still zero
    const float mref = (m_ref == -INFINITY) ? 0.f : m_ref;
    Frag<T> dzf;
    float ls = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float e = __builtin_amdgcn_exp2f(z[i] - mref);
      ls += e;
      dzf.v[i] = from_f32<T>(e * (dp[i] - delta));
    }
    l_run += ls;

#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const Frag<T> av = tv[db % PT];
      if (db + PT < DB) tv[db % PT] = ld_t(db + PT);
      acc[db] = mfma16x16x32(av, dzf, acc[db]);
    }
  };

  const int ntiles = (nk + KT - 1) / KT;
  // One pipeline step: wait until this wave's loads of tile t have landed (at most
  // `after` younger tiles, LPT loads each, may still be in flight), barrier (every
  // wave's part of tile t is in LDS, every wave is done with tile t-1), refill the
  // stage of tile t-1 with tile t+NS-1, then use tile t.
  auto step = [&](int t, const unsigned char* cur, const int* kvc, unsigned char* nxt, int* kvn) {
    const int after = min(ntiles - 1, t + NS - 2) - t;
    if (after <= 0) vm_wait_barrier<0>();
    else if (after == 1) vm_wait_barrier<LPT>();
    else vm_wait_barrier<2 * LPT>();
    if (t + NS - 1 < ntiles) issue(t + NS - 1, nxt, kvn);
    compute(cur, kvc);
  };
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int db = 0; db < D / 16; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    l_run = 0.f;
    for (int i = 0; i < NS - 1 && i < ntiles; ++i) {
      if (i == 0) issue(0, st0, kv0);
      else if (i == 1) issue(1, st1, kv1);
      else issue(2, st2, kv2);
    }
    for (int tile = 0; tile < ntiles; tile += NS) {
      if constexpr (NS == 4) {
        step(tile, st0, kv0, st3, kv3);
        if (tile + 1 < ntiles) step(tile + 1, st1, kv1, st0, kv0);
        if (tile + 2 < ntiles) step(tile + 2, st2, kv2, st1, kv1);
        if (tile + 3 < ntiles) step(tile + 3, st3, kv3, st2, kv2);
      } else {
        step(tile, st0, kv0, st1, kv1);
        if (tile + 1 < ntiles) step(tile + 1, st1, kv1, st0, kv0);
      }
    }
    __syncthreads();  // every wave is done with the stages
    if (__any(m_seen > m_ref + 64.0f) && lane == 0) atomicOr(&overflow, 1);
    __syncthreads();
    if (!overflow || pass == 1) break;
    m_ref = m_seen;
  }

  // ---- dq = RoPE(scale / l * acc, -P), staged through LDS, written coalesced.
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (a.sinks && h < a.H) l_run += __builtin_amdgcn_exp2f(a.sinks[h] * kLog2e - m_ref);
  const float f = l_run > 0.f ? a.scale / l_run : 0.f;
  {
    unsigned char* orow = (h < HP / 2 ? st0 : st1) + (h % (HP / 2)) * QROWB;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      const int d0 = 16 * db + 4 * g;
      float x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = acc[db][i] * f;
      if (d0 >= rlo) {
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          const float2 r = cs[(d0 + i - rlo) >> 1];
          const float x0 = x[i], x1 = x[i + 1];
          x[i] = x0 * r.x + x1 * r.y;
          x[i + 1] = -x0 * r.y + x1 * r.x;
        }
      }
      T* dst = reinterpret_cast<T*>(orow) + d0;
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i] = from_f32<T>(x[i]);
    }
  }
  __syncthreads();
  unsigned char* dqg = reinterpret_cast<unsigned char*>(a.dq) + row0;
  for (int c = threadIdx.x; c < a.H * NCH; c += NT) {
    const int row = c / NCH, col = (c % NCH) * 16;
    const unsigned char* src = (row < HP / 2 ? st0 : st1) + (row % (HP / 2)) * QROWB + col;
    *reinterpret_cast<uint4*>(dqg + (int64_t)row * ROWB + col) = *reinterpret_cast<const uint4*>(src);
  }
}

// ---------------------------------------------------------------------------------
// bf16 fast path for D = 512 and up to 64 heads, on the forward's head-group x
// latent-half mapping: wave w owns heads 32(w/2) .. +31 (hg) and dims 256(w%2) .. +255
// (dh), so every LDS fragment feeds 32 heads on v_mfma_f32_32x32x16_bf16 and each wave
// reads only its half of every key row: per 32-key tile a wave reads 16 KB for the two
// logit-side products and 16 KB for the transposed one, half of the 16-head mapping.
// Per tile:
//   partial S^T and dP^T [32 keys, 32 heads] over the wave's 256 dims (32 MFMAs, one
//     K fragment per k-step feeding both); rows r hold key r ^ 16dh, so rows 0..15 are
//     the wave's own half of the keys
//   send the partner wave (same heads, other half) its keys' partials of both, add the
//     partner's partials of this wave's keys (through LDS)
//   e = exp2 against the fixed reference, dz = e (dP - delta) for the wave's 16 keys,
//     rounded to bf16; swap dz with the partner (through LDS)
//   dQ^T[256 dims, 32 heads] += K^T . dz^T over all 32 keys (16 MFMAs)
// Delta of a head is summed over the lane halves (v_permlane32_swap) and the partner.
// Keys stream through four stages as in the generic kernel; the entry indices sit in
// LDS.  The tiles are software-pipelined: the partial products of tile t+1 are issued
// while tile t's exchange, softmax and dz run, and one barrier per tile is both tile
// t's exchange barrier and tile t+1's arrival, so a tile costs two barriers, not three.  One workgroup per CU (q, du and the accumulator take about 256 registers).
// ---------------------------------------------------------------------------------
__device__ inline float halves_sum2(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ inline float halves_max2(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// Workgroup barrier for the LDS exchange: this wave's LDS operations are done, the
// direct-to-LDS copies in flight stay in flight (a workgroup fence would wait for them
// too, since they write LDS).
__device__ inline void lds_barrier2() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__global__ __launch_bounds__(256, 1) void mqa_bwd_dq_hd_kernel(DqArgs a) {
  constexpr int D = 512, ROWB = 1024, KT = 32, NT = 256, LPT = 8;
  // Key rows padded to RP = 1040 bytes and key x of each 16-key half in row slot
  // 4(x&3) + (x>>2), as in the forward's head-group kernel: the 16-byte K reads and the
  // transposing reads are then free of bank conflicts on gfx950's 64 banks.
  constexpr int RP = ROWB + 16;
  auto slot = [](int key) -> int { return (key & 16) | ((key & 3) << 2) | ((key >> 2) & 3); };
  __shared__ __attribute__((aligned(16))) unsigned char st0[KT * RP];
  __shared__ __attribute__((aligned(16))) unsigned char st1[KT * RP];
  __shared__ __attribute__((aligned(16))) unsigned char st2[KT * RP];
  __shared__ __attribute__((aligned(16))) unsigned char st3[KT * RP];
  // exchange: partial logits xh (8 KB), partial dP xd (8 KB), dz xp (4 KB), per-head
  // values xm (1 KB); then the RoPE table, the sink logits and the overflow flag
  __shared__ __attribute__((aligned(16))) unsigned char xbuf[22304];
  f32x4 (*xh)[2][64] = reinterpret_cast<f32x4 (*)[2][64]>(xbuf);
  f32x4 (*xd)[2][64] = reinterpret_cast<f32x4 (*)[2][64]>(xbuf + 8192);
  u32x4 (*xp)[64] = reinterpret_cast<u32x4 (*)[64]>(xbuf + 16384);
  float (*xm)[64] = reinterpret_cast<float (*)[64]>(xbuf + 20480);
  float2* cs = reinterpret_cast<float2*>(xbuf + 21504);
  float* sk = reinterpret_cast<float*>(xbuf + 22016);
  int* ovf = reinterpret_cast<int*>(xbuf + 22272);
  __shared__ int sidx[kMaxTopk];

  const int total = a.B * a.S;
  int gi = blockIdx.x;
  const int nfull = total & ~255;
  if (gi < nfull) {
    const int xcd = gi & 7, j = gi >> 3;
    gi = (((j >> 5) << 3) + xcd) * 32 + (j & 31);
  }
  gi = total - 1 - gi;
  const int b = gi / a.S;
  const int t = gi % a.S;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hg = wave >> 1, dh = wave & 1;
  const int l32 = lane & 31;
  const int g = lane >> 5;
  const int h = 32 * hg + l32;
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
  if (threadIdx.x == 0) *ovf = 0;
  if (a.sinks && threadIdx.x < a.H) sk[threadIdx.x] = a.sinks[threadIdx.x];
  if (a.mode == MQA_SELECTED) {
    const int32_t* irow = a.idx + ((int64_t)b * a.S + t) * a.topk;
    for (int i = threadIdx.x; i < nsel; i += NT) sidx[i] = irow[i];
  }
  const int64_t row0 = ((int64_t)b * a.S + t) * a.H * ROWB;
  const unsigned char* qg = reinterpret_cast<const unsigned char*>(a.q) + row0;
  const unsigned char* dog = reinterpret_cast<const unsigned char*>(a.d_o) + row0;
  const unsigned char* og = reinterpret_cast<const unsigned char*>(a.o) + row0;
  const unsigned char* kv_c = reinterpret_cast<const unsigned char*>(a.kv_c);
  const unsigned char* kv_w = reinterpret_cast<const unsigned char*>(a.kv_w);
  __syncthreads();  // table, sinks, indices and flag are in LDS

  const uint32_t dma_off = (uint32_t)lane << 4;
  // Direct-to-LDS copy of tile `tile`: lane l < 32 resolves key tile*32 + l, wave w
  // loads keys w, w+4, ... (one 1 KB wave load per key, LPT per wave; key w + 4m into
  // slot 16(m>>2) + 4w + (m&3)); returns the tile's key-validity bits.
  auto issue = [&](int tile, unsigned char* sb) -> uint32_t {
    const int kk = tile * KT + l32;
    const unsigned char* src = qg;  // masked keys read finite data that is never used
    bool ok = false;
    if (kk < nsel) {
      const int sv = a.mode == MQA_SELECTED ? sidx[kk] : kk;
      if (sv >= 0 && sv < n_t) {
        ok = true;
        src = kv_c + ((int64_t)b * a.n_entries + sv) * ROWB;
      }
    } else if (kk < nk) {
      ok = true;
      src = kv_w + ((int64_t)b * a.S + wlo + (kk - nsel)) * ROWB;
    }
    const uint32_t bits = (uint32_t)__ballot(ok && lane < 32);
    const uint64_t sp = reinterpret_cast<uint64_t>(src);
    const uint32_t sp_lo = (uint32_t)sp, sp_hi = (uint32_t)(sp >> 32);
    const uint32_t lds0 = (uint32_t)(uintptr_t)(CSA_LDS unsigned char*)sb;
#pragma unroll
    for (int m = 0; m < KT / 4; ++m) {
      const int r = wave + 4 * m;
      const uint64_t row = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)sp_hi, r) << 32) |
                           (uint32_t)__builtin_amdgcn_readlane((int)sp_lo, r);
      const uint32_t lds = __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)slot(r) * RP);
      // In assembly, so the compiler does not track the copies: it cannot tell their LDS
      // destinations from the exchange slots and would otherwise wait for every copy in
      // flight before each exchange write and fragment read, draining the four-stage
      // ring; the explicit vm_wait_barrier waits are the only ones.  s_nop 4: the row
      // base was just written to SGPRs by v_readlane, which a vector memory instruction
      // may read only 5 wait states later (and M0 needs 1).
      asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(dma_off), "s"(row), "{m0}"(lds) : "memory");
    }
    return bits;
  };

  const int ntiles = (nk + KT - 1) / KT;
  uint32_t km0 = 0u, km1 = 0u, km2 = 0u, km3 = 0u;
  auto prologue_issue = [&]() {
    if (ntiles > 0) km0 = issue(0, st0);
    if (ntiles > 1) km1 = issue(1, st1);
    if (ntiles > 2) km2 = issue(2, st2);
  };
  prologue_issue();  // the first tiles are requested before q, du and o

  // ---- B operands straight from global memory: lane (head h, g), k-step k holds dims
  // 256dh + 16k + 8g .. +7; q and du rotated at +P in the last R dims; delta partials.
  bf16x8 qf[16], uf[16];
  float delta = 0.f;
  auto rot = [&](bf16x8& v, int d0) {
    if (d0 + 8 > rlo) {
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        const int d = d0 + i;
        if (d >= rlo) {
          const float2 r = cs[(d - rlo) >> 1];
          const float x0 = (float)v[i], x1 = (float)v[i + 1];
          v[i] = (bf16)(x0 * r.x - x1 * r.y);
          v[i + 1] = (bf16)(x0 * r.y + x1 * r.x);
        }
      }
    }
  };
  // Every lane loads, with no branch, so all 48 loads are in flight together (a head
  // test around them made the compiler wait for each k-step's loads before the next,
  // sixteen memory round trips per query).  Lanes of heads past H load head H-1: their
  // logits, probabilities and accumulator columns copy that head's, and their dq rows
  // are never written.
  {
    const int64_t hrow = (int64_t)min(h, a.H - 1) * ROWB;
    u32x4 ov[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int64_t eo = hrow + 2 * (256 * dh + 16 * k + 8 * g);
      qf[k] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qg + eo));
      uf[k] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(dog + eo));
      ov[k] = *reinterpret_cast<const u32x4*>(og + eo);
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const bf16x8 o8 = __builtin_bit_cast(bf16x8, ov[k]);
#pragma unroll
      for (int i = 0; i < 8; ++i) delta = fmaf((float)uf[k][i], (float)o8[i], delta);
    }
  }
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int d0 = 256 * dh + 16 * k + 8 * g;
    rot(qf[k], d0);
    rot(uf[k], d0);
  }
  delta = halves_sum2(delta);
  xm[wave][lane] = delta;
  lds_barrier2();
  delta += xm[wave ^ 1][lane];
  lds_barrier2();  // xm is free again
  // q, du and o have landed (and with them the first tiles, requested before them); the
  // explicit wait tells the compiler so: otherwise it keeps waits for the registers that
  // the divergent head test and rotation left untouched on some path, before the first
  // product of every tile, and in hardware those waits drain the ring
  __builtin_amdgcn_s_waitcnt(0x0F70);  // gfx9 encoding of vmcnt(0), expcnt and lgkmcnt not waited

  // Per-lane LDS offsets, as in the forward's head-group kernel.
  const int kr = l32 ^ (16 * dh);
  const int qk_base = slot(kr) * RP + 512 * dh + 16 * g;  // + 32k for k-step k
  // transposing reads: key 4g + a4 of a half in slot 4a4 + g, key 8 + 4g + a4 in slot
  // 4a4 + 2 + g; dims 256dh + 32db + 16hh + 4(hj&3)
  const int hj = lane & 15, hh = (lane >> 4) & 1, a4 = hj >> 2;
  const int pv_base = (4 * a4 + g) * RP + 512 * dh + 32 * hh + 8 * (hj & 3);
  typedef short i16x4 __attribute__((ext_vector_type(4)));
  const int pv_mine = 16 * RP * dh, pv_other = 16 * RP * (dh ^ 1);

  float m_seen = -INFINITY, m_ref = -INFINITY, l_run = 0.f;
  f32x16 O[8];

  // Partial S^T and dP^T of the tile in `sb` over this wave's 256 dims.
  auto qk = [&](const unsigned char* sb, f32x16& s, f32x16& dp) {
    const CSA_LDS unsigned char* lb = (const CSA_LDS unsigned char*)sb;
    s = f32x16{};
    dp = f32x16{};
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const bf16x8 ka = __builtin_bit_cast(bf16x8, *(const CSA_LDS u32x4*)(lb + qk_base + 32 * k));
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[k], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, uf[k], dp, 0, 0, 0);
    }
  };
  // The rest of a tile once its partials are in xh / xd and the exchange barrier is
  // passed; `nxt` (may be null): the next tile, whose partial products are issued
  // here so that the MFMA pipe works while this tile's softmax and exchange run.
  auto rest = [&](const unsigned char* sb, uint32_t kmask, bool first, const f32x16& s, const f32x16& dp,
                  const unsigned char* nxt, f32x16& sn, f32x16& dpn) {
    const CSA_LDS unsigned char* lb = (const CSA_LDS unsigned char*)sb;
    if (nxt) qk(nxt, sn, dpn);
    float z[8], dv[8];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const f32x4 o4 = xh[wave ^ 1][q][lane], d4 = xd[wave ^ 1][q][lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        z[4 * q + i] = s[4 * q + i] + o4[i];
        dv[4 * q + i] = dp[4 * q + i] + d4[i];
      }
    }
    if (kmask != 0xffffffffu) {
      const uint32_t kml = kmask >> (4 * g + 16 * dh);  // bit 8q + i: key 16dh + 8q + 4g + i
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (!((kml >> (8 * (e >> 2) + (e & 3))) & 1u)) z[e] = -INFINITY;
    }
    float mt = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) mt = fmaxf(mt, z[e]);
    mt = halves_max2(mt);
    m_seen = fmaxf(m_seen, mt);
    if (first) {  // workgroup-uniform: the pair agrees on the reference
      xm[wave][lane] = mt;
      lds_barrier2();
      const float m0 = fmaxf(mt, xm[wave ^ 1][lane]);
      m_ref = m0 == -INFINITY ? 0.f : m0;
      // a reference forced to 0 may lie far above every logit: the end of the pass
      // then takes the exact maximum and runs again
      if (__any(m0 == -INFINITY) && lane == 0) *ovf = 1;
    }
    const float nbias = -m_ref * a.scale_log2;
    bf16x8 dzm;
    float ls = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = __builtin_amdgcn_exp2f(fmaf(z[e], a.scale_log2, nbias));
      ls += p;
      dzm[e] = (bf16)(p * (dv[e] - delta));
    }
    l_run += ls;
    xp[wave][lane] = __builtin_bit_cast(u32x4, dzm);
    lds_barrier2();
    const bf16x8 dzo = __builtin_bit_cast(bf16x8, xp[wave ^ 1][lane]);
#pragma unroll
    for (int db = 0; db < 8; ++db) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const CSA_LDS unsigned char* p = lb + pv_base + 64 * db + (ks ? pv_other : pv_mine);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((CSA_LDS i16x4*)p);
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((CSA_LDS i16x4*)(p + 2 * RP));
        const bf16x8 av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        O[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, ks ? dzo : dzm, O[db], 0, 0, 0);
      }
      if (db & 1) __builtin_amdgcn_sched_barrier(0);
    }
  };

  auto send = [&](const f32x16& s, const f32x16& dp) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      xh[wave][q][lane] = f32x4{s[8 + 4 * q], s[9 + 4 * q], s[10 + 4 * q], s[11 + 4 * q]};
      xd[wave][q][lane] = f32x4{dp[8 + 4 * q], dp[9 + 4 * q], dp[10 + 4 * q], dp[11 + 4 * q]};
    }
  };
  // Tile t, its partials (s, dp) already formed: send them, then one barrier that is
  // both the exchange barrier of tile t and the arrival of tile t+1 (at most tile t+2
  // may still be in flight); refill the stage of tile t-1 with tile t+3; form tile t+1's
  // partials while finishing tile t.
  f32x16 sA, dA, sB, dB;
  auto iter = [&](int tt, const unsigned char* cur, uint32_t kmc, const unsigned char* n1, unsigned char* n3,
                  uint32_t& km3r, bool first, f32x16& s, f32x16& dp, f32x16& sn, f32x16& dpn) {
    send(s, dp);
    if (tt + 2 < ntiles) vm_wait_barrier<LPT>();
    else vm_wait_barrier<0>();
    if (tt + 3 < ntiles) km3r = issue(tt + 3, n3);
    rest(cur, kmc, first, s, dp, tt + 1 < ntiles ? n1 : nullptr, sn, dpn);
  };
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) O[db][i] = 0.f;
    l_run = 0.f;
    if (pass > 0) prologue_issue();
    if (ntiles > 0) {
      if (ntiles > 2) vm_wait_barrier<2 * LPT>();
      else if (ntiles > 1) vm_wait_barrier<LPT>();
      else vm_wait_barrier<0>();
      qk(st0, sA, dA);
    }
    for (int tile = 0; tile < ntiles; tile += 4) {
      iter(tile, st0, km0, st1, st3, km3, pass == 0 && tile == 0, sA, dA, sB, dB);
      if (tile + 1 < ntiles) iter(tile + 1, st1, km1, st2, st0, km0, false, sB, dB, sA, dA);
      if (tile + 2 < ntiles) iter(tile + 2, st2, km2, st3, st1, km1, false, sA, dA, sB, dB);
      if (tile + 3 < ntiles) iter(tile + 3, st3, km3, st0, st2, km2, false, sB, dB, sA, dA);
    }
    // Run again with the pair's exact maximum as the reference if some probability could
    // have overflowed, or (reference forced to 0 after an all-masked first tile, flagged
    // there) underflowed.  The reference is the maximum over a subset of the head's
    // keys, so otherwise only overflow is possible, and the lane's own maximum tells.
    if (pass == 1) break;
    if (__any(m_seen != -INFINITY && (m_seen - m_ref) * a.scale_log2 > 64.0f) && lane == 0) *ovf = 1;
    __syncthreads();  // every wave is done with the stages and the exchange area
    if (!*ovf) break;
    xm[wave][lane] = m_seen;
    __syncthreads();
    const float mall = fmaxf(m_seen, xm[wave ^ 1][lane]);
    m_ref = mall == -INFINITY ? 0.f : mall;  // exact reference for the second pass
    __syncthreads();  // xm is read
  }

  // ---- dq = RoPE(scale / l * acc, -P), staged by head rows, written coalesced
  xm[wave][lane] = l_run;
  __syncthreads();
  l_run = halves_sum2(l_run + xm[wave ^ 1][lane]);
  if (a.sinks && h < a.H) l_run += __builtin_amdgcn_exp2f(sk[h] * kLog2e - m_ref * a.scale_log2);
  const float f = l_run > 0.f ? a.scale / l_run : 0.f;
  {
    unsigned char* os = hg == 0 ? st0 : st1;
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d0 = 256 * dh + 32 * db + 8 * j + 4 * g;
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = O[db][4 * j + i] * f;
        if (d0 >= rlo) {
#pragma unroll
          for (int i = 0; i < 4; i += 2) {
            const float2 r = cs[(d0 + i - rlo) >> 1];
            const float x0 = x[i], x1 = x[i + 1];
            x[i] = x0 * r.x + x1 * r.y;
            x[i + 1] = -x0 * r.y + x1 * r.x;
          }
        }
        bf16 y[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) y[i] = (bf16)x[i];
        *reinterpret_cast<uint2*>(os + l32 * RP + 2 * d0) = *reinterpret_cast<const uint2*>(y);
      }
  }
  __syncthreads();
  unsigned char* dqg = reinterpret_cast<unsigned char*>(a.dq) + row0;
  for (int c = threadIdx.x; c < a.H * (ROWB / 16); c += NT) {
    const int row = c >> 6, col = (c & 63) * 16;
    *reinterpret_cast<uint4*>(dqg + (int64_t)row * ROWB + col) =
        *reinterpret_cast<const uint4*>((row < 32 ? st0 : st1) + (row & 31) * RP + col);
  }
}

template <typename T, int D>
void launch_d(const DqArgs& a, int H, hipStream_t st) {
  const dim3 grid(a.B * a.S);
  if constexpr (D == 512 && sizeof(T) == 2) {
    if (H > 16) {
      hipLaunchKernelGGL(mqa_bwd_dq_hd_kernel, grid, dim3(256), 0, st, a);
      return;
    }
  }
  if (H <= 16) hipLaunchKernelGGL((mqa_bwd_dq_kernel<T, D, 1>), grid, dim3(64), 0, st, a);
  else hipLaunchKernelGGL((mqa_bwd_dq_kernel<T, D, 4>), grid, dim3(256), 0, st, a);
}

template <typename T>
hipError_t launch_t(const DqArgs& a, int D, int H, hipStream_t st) {
  switch (D) {
    case 64: launch_d<T, 64>(a, H, st); break;
    case 128: launch_d<T, 128>(a, H, st); break;
    case 256: launch_d<T, 256>(a, H, st); break;
    case 512: launch_d<T, 512>(a, H, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mqa_bwd_dq(const csa_params_t& p, MqaMode mode, const void* q, const void* kv_c,
                             const void* kv_w, const int32_t* idx, const float* sinks, const void* o,
                             const void* d_o, void* dq, hipStream_t st) {
  DqArgs a{};
  a.q = q;
  a.kv_c = kv_c;
  a.kv_w = kv_w;
  a.idx = idx;
  a.sinks = sinks;
  a.o = o;
  a.d_o = d_o;
  a.dq = dq;
  a.B = p.B;
  a.S = p.S;
  a.H = p.H;
  a.R = p.rope_dim;
  a.ratio = p.ratio;
  a.window = p.window;
  a.topk = p.topk;
  a.n_entries = mode == MQA_WINDOW_ONLY ? 0 : p.S / p.ratio;
  a.mode = mode;
  a.scale_log2 = p.softmax_scale * kLog2e;
  a.scale = p.softmax_scale;
  a.theta = p.rope_theta;
  a.pos0 = p.pos0;
  if (p.B * p.S == 0) return hipSuccess;
  return p.dtype == CSA_BF16 ? launch_t<bf16>(a, p.D, p.H, st) : launch_t<float>(a, p.D, p.H, st);
}

}  // namespace csa
