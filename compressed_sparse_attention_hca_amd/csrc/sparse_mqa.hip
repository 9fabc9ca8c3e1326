// Stage 4 on gfx950: multi-query attention of H heads over one shared D-wide latent
// that is both key and value, across a query's selected compressed entries plus a
// sliding window of raw tokens, then the output's RoPE dims rotated back.
//
//   keys(t)  = kv_c[Sel_t] ++ RoPE(kv_raw[t'], pos0 + t'),  t' = max(0, t-W+1) .. t
//   z        = (RoPE(q[t,h], pos0 + t) . key) * D**-0.5          (no YaRN factor)
//   o[t,h]   = RoPE(sum_k softmax_k(z) key_k, -(pos0 + t))
//
// Sources: "Enabling DeepSeek-V4-Flash Training on AMD Instinct MI355X GPUs with
// Primus", "The DeepSeek-V4-Flash architecture" (64 heads read one 512-d latent as K
// and V), "Three attention types, interleaved" (selected entries plus the 128-token
// window, HCA attends to all entries) and "Attention kernels for the three layer
// types" (one single-latent kernel gathering selected entries in-kernel with the
// window folded into the same softmax); "fix(deepseek-v4): correct V4-Flash attention
// math", Part 1 items 1 (scale) and 3 (de-rotation at -i on the last dims before the
// output leaves; item 6g: done in-kernel).
//
// Mapping: one workgroup per query; wave w owns heads 16w .. 16w+15 and all D output
// dims.  Keys stream through LDS in tiles of 32 rows, shared by every head, staged by
// direct-to-LDS loads (one 1 KB wave load per line) into two stages while the other
// stage is being used.  Per tile:
//   S^T[key, head] = K_tile . Q^T     v_mfma_f32_16x16x32_bf16, keys on M (A from the
//                                     row-major tile), heads on N (B = rotated q in regs)
//   softmax in registers, base-2, against a fixed reference (the first tile's max;
//   exact by shift invariance, with a second pass if later logits could overflow)
//   O^T[dim, head] += V^T . P^T       dims on M (A read from the same row-major tile with
//                                     ds_read_b64_tr_b16), heads on N (B = P from S^T)
// The S^T accumulator gives lane (head, g) keys 4g..4g+3 and 16+4g..16+4g+3; those 8
// are that lane's B-operand k-slots for PV, and the two transposing reads fetch V for
// exactly those keys, so P never leaves registers.
#include "common.hpp"
#include "launch.hpp"

namespace csa {

struct MqaArgs {
  const void* q;
  const void* kv_c;
  const void* kv_w;
  const int32_t* idx;
  const float* sinks;  // [H] softmax-sink logits, or nullptr
  void* o;
  float* lse;          // [B,S,H] log of each head's softmax denominator, or nullptr
  int32_t B, S, H, R, ratio, window, topk, n_entries, mode;
  float scale_log2;  // softmax_scale * log2(e)
  double theta;
  int64_t pos0;
};

// Key slot (within a tile of 32) held at k-slot i of lane group g.
__device__ __host__ constexpr int slot_key(int g, int i) { return i < 4 ? 4 * g + i : 12 + 4 * g + i; }

constexpr int MQA_MAX_TOPK = 2048;
constexpr float kLog2e = 1.4426950408889634f;

// Natural log of a head's softmax denominator, the statistic a training forward keeps
// for its backward: ln(2^m2 * l + e^sink), from the keys' mass l against the log2
// reference m2 and the sink logit (if any).  No key and no sink: -inf.
__device__ inline float head_lse(float m2, float l, const float* sinks, int h) {
  const float a2 = l > 0.f ? m2 + log2f(l) : -INFINITY;
  const float b2 = sinks ? sinks[h] * kLog2e : -INFINITY;
  const float hi = fmaxf(a2, b2), lo = fminf(a2, b2);
  const float r = lo == -INFINITY ? hi : hi + log2f(1.0f + exp2f(lo - hi));
  return r * 0.69314718055994531f;
}

template <typename T, int D, int NW>
__global__ __launch_bounds__(NW * 64, 2) void sparse_mqa_kernel(MqaArgs a) {
  constexpr int NT = NW * 64;
  constexpr int HP = NW * 16;                       // heads handled (padded)
  constexpr int ES = (int)sizeof(T);
  constexpr int KT = 32;                            // keys per tile
  constexpr int ROWB = D * ES;                      // bytes per latent row
  constexpr int NCH = ROWB / 16;                    // 16-byte pieces per row
  // A key tile is a sequence of 1 KB lines, one direct-to-LDS wave load each.  When a
  // latent row is exactly one line (D = 512 bf16) the 16-byte chunks of row r are
  // stored XOR-swizzled, chunk c at position c ^ swz(r) with swz(r) = 2(r&3) | (r>>2 &1):
  // then the 8 rows read together by ds_read_b128 and the 4-row x 32-byte blocks read
  // by ds_read_b64_tr_b16 both cover the 32 LDS banks without conflicts.  Other row
  // sizes use lines padded to 1072 B.
  constexpr int RPL = ROWB < 1024 ? 1024 / ROWB : 1;  // rows per line
  constexpr int LPR = ROWB > 1024 ? ROWB / 1024 : 1;  // lines per row
  constexpr int NL = KT * LPR / RPL;                  // lines per tile
  constexpr bool SWZ = ROWB == 1024 && ES == 2;
  constexpr int LSTRIDE = SWZ ? 1024 : 1024 + 48;
  constexpr int QROWB = ROWB + 16;                    // q / o staging row
  constexpr int TILEB = NL * LSTRIDE;
  constexpr int SB = TILEB > (HP / 2) * QROWB ? TILEB : (HP / 2) * QROWB;
  // Two stages in two distinct arrays: the compiler then sees that the loads in
  // flight into one stage do not alias the reads of the other.
  __shared__ __attribute__((aligned(16))) unsigned char st0[SB];
  __shared__ __attribute__((aligned(16))) unsigned char st1[SB];
  __shared__ int kv0[KT], kv1[KT];
  __shared__ int sidx[MQA_MAX_TOPK];
  __shared__ float2 cs[64];

  // workgroup -> query: 32 consecutive queries per XCD visit (window keys stay in that
  // XCD's L2), XCDs interleaved across the sequence, latest (heaviest) queries first.
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
  const int wave = threadIdx.x >> 6;
  const int hl = lane & 15;
  const int g = lane >> 4;
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
    const int32_t* irow = a.idx + ((int64_t)b * a.S + t) * a.topk;
    for (int i = threadIdx.x; i < nsel; i += NT) sidx[i] = irow[i];
  }

  // ---- q[b,t] (H x D, contiguous) -> LDS (heads 0..HP/2-1 in st0, the rest in st1)
  const unsigned char* qg =
      reinterpret_cast<const unsigned char*>(a.q) + ((int64_t)b * a.S + t) * a.H * ROWB;
  for (int c = threadIdx.x; c < HP * NCH; c += NT) {
    const int row = c / NCH, col = (c % NCH) * 16;
    const uint4 v = row < a.H ? *reinterpret_cast<const uint4*>(qg + (int64_t)row * ROWB + col)
                              : make_uint4(0, 0, 0, 0);
    unsigned char* dst = (row < HP / 2 ? st0 : st1) + (row % (HP / 2)) * QROWB + col;
    *reinterpret_cast<uint4*>(dst) = v;
  }
  __syncthreads();

  // ---- Q^T fragments (B operand): lane (head 16w+hl, group g), k-step k holds dims
  // 32k + 8g .. +7, rotated at +P where they fall in the last R dims.
  Frag<T> qf[D / 32];
  {
    const int h = 16 * wave + hl;
    const unsigned char* qrow = (h < HP / 2 ? st0 : st1) + (h % (HP / 2)) * QROWB;
#pragma unroll
    for (int k = 0; k < D / 32; ++k) {
      const int d0 = 32 * k + 8 * g;
      qf[k] = load_frag(reinterpret_cast<const T*>(qrow) + d0);
      if (d0 + 8 > rlo) {
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
          const int d = d0 + i;
          if (d >= rlo) {
            const float2 r = cs[(d - rlo) >> 1];
            const float x0 = to_f32(qf[k].v[i]), x1 = to_f32(qf[k].v[i + 1]);
            qf[k].v[i] = from_f32<T>(x0 * r.x - x1 * r.y);
            qf[k].v[i + 1] = from_f32<T>(x0 * r.y + x1 * r.x);
          }
        }
      }
    }
  }
  __syncthreads();  // the staging area becomes the key tiles

  const unsigned char* kv_c = reinterpret_cast<const unsigned char*>(a.kv_c);
  const unsigned char* kv_w = reinterpret_cast<const unsigned char*>(a.kv_w);

  // Byte offset of (key row r, dim d) inside a tile.
  auto swz = [](int r) -> int { return ((r & 3) << 1) | ((r >> 2) & 1); };
  auto eoff = [&](int r, int d) -> int {
    const int byte = d * ES;
    if constexpr (SWZ) return r * 1024 + ((((byte >> 4) ^ swz(r)) << 4) | (byte & 15));
    return ((r / RPL) * LPR + byte / 1024) * LSTRIDE + (r % RPL) * ROWB + (byte % 1024);
  };
  // Source row of key kk of this query's list; masked keys read this query's own q
  // row instead (finite data, never used: their probability is 0).
  auto key_src = [&](int kk, int* ok) -> const unsigned char* {
    if (kk < nsel) {
      const int s = a.mode == MQA_SELECTED ? sidx[kk] : kk;
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
  // Direct-to-LDS loads of tile `tile`: wave w loads lines w, w+NW, ...; one 16-byte
  // piece per lane lands at line base + 16 * lane.
  auto issue = [&](int tile, unsigned char* sb, int* kv) {
#pragma unroll
    for (int L = wave; L < NL; L += NW) {
      int r, byte;
      if constexpr (RPL > 1) {
        r = L * RPL + lane / NCH;
        byte = (lane % NCH) * 16;
      } else if constexpr (SWZ) {
        r = L;
        byte = (lane ^ swz(r)) * 16;  // LDS position `lane` holds chunk lane ^ swz(r)
      } else {
        r = L / LPR;
        byte = (L % LPR) * 1024 + lane * 16;
      }
      int ok;
      const unsigned char* src = key_src(tile * KT + r, &ok);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src + byte),
                                       (CSA_LDS void*)(sb + L * LSTRIDE), 16, 0, 0);
      if (byte == 0) kv[r] = ok;
    }
  };

  // Softmax with a fixed reference (shift invariance): the first tile's max per head,
  // so the accumulator is never rescaled inside the loop.  If a later tile's max
  // exceeds the reference by more than 2^64 (not reachable with RMS-normalised inputs,
  // possible in general), the workgroup runs the tiles again with the largest max
  // seen as the reference, so every exp2 argument is <= 0 and nothing can overflow.
  __shared__ int overflow;
  float m_seen = -INFINITY, m_ref = -INFINITY, l_run = 0.f;
  f32x4 O[D / 16];

  // Per-lane LDS byte offsets of the fragments this lane reads (constant across tiles).
  // QK: rows hl and 16+hl, dims 32k+8g..+7 (chunk 4k+g).  With the swizzle the chunk
  // position is (4k+g) ^ swz = 4(k ^ s2) + ((g ^ s) & 3), s = swz(hl), s2 = s >> 2, so
  // even and odd k use two bases and 64k stays an immediate.
  // PV: rows 4g+hl/4 (+16), bytes 32db + 8(hl&3): chunk 2db + hb, hb = (hl>>1)&1;
  // position (2db+hb) ^ swz = 2(db ^ a) + (hb ^ c), a = hl>>2, c = g&1, so four bases
  // (by db mod 4) and 128 (db>>2) stays an immediate.
  int qk_base[2], pv_base[4];
  if constexpr (SWZ) {
    const int s = swz(hl), s2 = s >> 2;
    const int lo = hl * 1024 + (((g ^ s) & 3) << 4);
    qk_base[0] = lo + (s2 ? 64 : 0);   // k even: 4(k ^ s2) = 4k + 4 s2
    qk_base[1] = lo - (s2 ? 64 : 0);   // k odd:  4(k ^ s2) = 4k - 4 s2
    const int a4 = hl >> 2, c = g & 1, hb = (hl >> 1) & 1;
    const int row = 4 * g + a4;
#pragma unroll
    for (int m = 0; m < 4; ++m)
      pv_base[m] = row * 1024 + ((m ^ a4) - m) * 32 + ((hb ^ c) << 4) + ((hl & 1) << 3);
  } else {
    qk_base[0] = qk_base[1] = eoff(hl, 8 * g);
#pragma unroll
    for (int m = 0; m < 4; ++m) pv_base[m] = eoff(4 * g + (hl >> 2), 4 * (hl & 3));
  }
  typedef short i16x4 __attribute__((ext_vector_type(4)));

  auto compute = [&](const unsigned char* sb, const int* kv) {
    const CSA_LDS unsigned char* lb = (const CSA_LDS unsigned char*)sb;
    auto ld_k = [&](int row16, int k) {  // QK A fragment: rows row16+hl, dims 32k+8g..
      Frag<T> f;
      const CSA_LDS unsigned char* p =
          lb + qk_base[k & 1] + (SWZ ? row16 * 1024 + 64 * k : eoff(row16, 32 * k) - eoff(0, 0));
      *reinterpret_cast<u32x4*>(f.v) = *(const CSA_LDS u32x4*)p;
      if constexpr (ES == 4) *reinterpret_cast<u32x4*>(f.v + 4) = *(const CSA_LDS u32x4*)(p + 16);
      return f;
    };
    // S^T = K . Q^T : keys 0..15 and 16..31, one fragment pair ahead
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    Frag<T> n0 = ld_k(0, 0), n1 = ld_k(16, 0);
#pragma unroll
    for (int k = 0; k < D / 32; ++k) {
      const Frag<T> a0 = n0, a1 = n1;
      if (k + 1 < D / 32) {
        n0 = ld_k(0, k + 1);
        n1 = ld_k(16, k + 1);
      }
      s0 = mfma16x16x32(a0, qf[k], s0);
      s1 = mfma16x16x32(a1, qf[k], s1);
    }
    float z[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      z[i] = kv[4 * g + i] ? s0[i] * a.scale_log2 : -INFINITY;
      z[4 + i] = kv[16 + 4 * g + i] ? s1[i] * a.scale_log2 : -INFINITY;
    }
    float mt = z[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mt = fmaxf(mt, z[i]);
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    m_seen = fmaxf(m_seen, mt);
    if (m_ref == -INFINITY) m_ref = mt;  // O and l are still zero
    const float mref = (m_ref == -INFINITY) ? 0.f : m_ref;
    Frag<T> pfr;
    float ls = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p = __builtin_amdgcn_exp2f(z[i] - mref);
      ls += p;
      pfr.v[i] = from_f32<T>(p);
    }
    l_run += ls;

    // O^T += V^T . P^T.  The V^T fragment of lane (dim 16db+hl, group g) is keys
    // sigma(g, 0..7) of that dim: two transposing 8-byte LDS reads (keys 4g..4g+3 and
    // 16+4g..16+4g+3), each lane addressing key 4g+hl/4 (+16), dims 16db+4(hl%4)..+3.
    auto ld_v = [&](int db) {
      Frag<T> f;
      if constexpr (ES == 2) {
        const CSA_LDS unsigned char* p =
            lb + pv_base[db & 3] + (SWZ ? 32 * db : eoff(0, 16 * db) - eoff(0, 0));
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((CSA_LDS i16x4*)p);
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (CSA_LDS i16x4*)(p + (SWZ ? 16 * 1024 : eoff(16, 0) - eoff(0, 0))));
        typedef short i16x8 __attribute__((ext_vector_type(8)));
        const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        *reinterpret_cast<i16x8*>(f.v) = v;
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          f.v[i] = *(const CSA_LDS T*)(lb + eoff(slot_key(g, i), 16 * db + hl));
      }
      return f;
    };
    Frag<T> nv = ld_v(0);
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      const Frag<T> av = nv;
      if (db + 1 < D / 16) nv = ld_v(db + 1);
      O[db] = mfma16x16x32(av, pfr, O[db]);
    }
  };

  const int ntiles = (nk + KT - 1) / KT;
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int db = 0; db < D / 16; ++db) O[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    l_run = 0.f;
    if (threadIdx.x == 0) overflow = 0;
    if (ntiles > 0) issue(0, st0, kv0);
    __syncthreads();
    for (int tile = 0; tile < ntiles; tile += 2) {
      if (tile + 1 < ntiles) issue(tile + 1, st1, kv1);
      compute(st0, kv0);
      __syncthreads();  // tile+1 landed in st1; every wave is done with st0
      if (tile + 1 < ntiles) {
        if (tile + 2 < ntiles) issue(tile + 2, st0, kv0);
        compute(st1, kv1);
        __syncthreads();
      }
    }
    if (__any(m_seen > m_ref + 64.0f) && lane == 0) atomicOr(&overflow, 1);
    __syncthreads();
    if (!overflow) break;
    m_ref = m_seen;  // exact reference for the second pass
  }

  // ---- normalise, de-rotate at -P, stage through LDS, write o[b,t] coalesced
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (a.lse && g == 0) {
    const int h = 16 * wave + hl;
    if (h < a.H)
      a.lse[((int64_t)b * a.S + t) * a.H + h] = head_lse(m_ref == -INFINITY ? 0.f : m_ref, l_run, a.sinks, h);
  }
  if (a.sinks) {  // the sink joins the denominator against the same reference
    const int h = 16 * wave + hl;
    if (h < a.H) l_run += __builtin_amdgcn_exp2f(a.sinks[h] * kLog2e - m_ref);
  }
  const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
  {
    const int h = 16 * wave + hl;
    unsigned char* orow = (h < HP / 2 ? st0 : st1) + (h % (HP / 2)) * QROWB;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      const int d0 = 16 * db + 4 * g;
      float x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = O[db][i] * inv;
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
  unsigned char* og = reinterpret_cast<unsigned char*>(a.o) + ((int64_t)b * a.S + t) * a.H * ROWB;
  for (int c = threadIdx.x; c < a.H * NCH; c += NT) {
    const int row = c / NCH, col = (c % NCH) * 16;
    const unsigned char* src = (row < HP / 2 ? st0 : st1) + (row % (HP / 2)) * QROWB + col;
    *reinterpret_cast<uint4*>(og + (int64_t)row * ROWB + col) = *reinterpret_cast<const uint4*>(src);
  }
}

// ---------------------------------------------------------------------------------
// bf16 fast path for D = 512 and up to 64 heads: four waves per query, wave w owning
// head group hg = w/2 (32 heads) and latent half dh = w%2 (dims 256dh .. 256dh+255).
// Every LDS fragment then feeds 32 heads on v_mfma_f32_32x32x16_bf16, and each wave
// reads only its half of every key row, so a 32-key tile costs 160 KB of LDS reads and
// writes per workgroup instead of the 256 KB of the 16-head mapping.  Per tile:
//   partial S^T[32 keys, 32 heads] over the wave's 256 dims      (16 MFMAs)
//     lane (head l%32, g = l/32) holds accumulator rows 8j + 4g + i, j, i = 0..3;
//     row r is key r ^ 16dh, so rows 0..15 are the wave's own half of the keys
//   send the partner wave (same heads, other latent half) the partials of its keys and
//   add the partner's partials of this wave's keys (through LDS)
//   softmax of the wave's 16 keys against a fixed reference, P^T to bf16; swap the
//   bf16 probabilities with the partner (through LDS)
//   O^T[256 dims, 32 heads] += V^T . P^T over all 32 keys        (16 MFMAs)
//     k-step 0 takes the wave's own keys, k-step 1 the partner's: keys {4g..4g+3,
//     8+4g..8+4g+3} of that half; V^T for them comes from two transposing LDS reads.
// Splitting the softmax halves its exponentials and VALU work per wave, for one more
// barrier per tile.  LDS is exactly two 32.5 KB key stages (rows padded to 1040 B for
// conflict-free reads) plus a 15 KB exchange area (two workgroups per CU); the RoPE
// table and the overflow flag borrow the exchange area outside the key loop, and the
// key indices are read from global memory one tile ahead.
// ---------------------------------------------------------------------------------
// Combine lane l with lane l ^ 32 (v_permlane32_swap: no LDS traffic, no address
// register).  The swap yields both halves' values in every lane, in the same order in
// both halves, so the two halves get bit-identical results.
__device__ inline uint2 swap_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return make_uint2(r[0], r[1]);
}
__device__ inline float halves_max(float x) {
  const uint2 r = swap_halves(x);
  return fmaxf(__uint_as_float(r.x), __uint_as_float(r.y));
}
__device__ inline float halves_sum(float x) {
  const uint2 r = swap_halves(x);
  return __uint_as_float(r.x) + __uint_as_float(r.y);
}

// Barrier after this wave's LDS accesses have completed; copies in flight stay in
// flight.  The memory clobber keeps the compiler from moving memory accesses across it,
// and as inline assembly it also bounds the scheduling regions.
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
// Barrier after every vector-memory load of this wave (the direct-to-LDS copies of the
// next tile included) and its LDS accesses have completed.  The compiler does not see
// inside the assembly, so the trailing s_waitcnt vmcnt(0) (free: the counter is already
// 0) tells it that no load is outstanding; otherwise it keeps waits for loads it thinks
// are pending, and in hardware those waits drain the next tile's copies.
__device__ inline void copies_barrier() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0F70);  // gfx9 encoding of vmcnt(0), expcnt and lgkmcnt not waited
}

// The lane's index within the wave, formed by instructions the compiler cannot merge with
// an earlier copy, so a value needed only after a long loop is formed again there instead
// of being kept in (or spilled from) a register across it.
__device__ inline int lane_id_fresh() {
  int v;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(v));
  return v;
}

// Scheduling groups (LLVM's AMDGPU sched_group_barrier masks): MFMA, LDS read.
constexpr int kSgMfma = 0x008, kSgDsRead = 0x100;

__global__ __launch_bounds__(256, 2) void sparse_mqa_hd_kernel(MqaArgs a) {
  typedef bf16 T;
  constexpr int D = 512, ROWB = 1024, KT = 32, NT = 256;
  // LDS rows are padded to RP = 1040 bytes, so row r starts 4r banks (mod 64) further
  // on, and key x of each 16-key half of a tile sits in row slot pi(x) = 4(x&3) + (x>>2)
  // of that half.  On gfx950 a 16-byte read serves 16 lanes a cycle from 64 banks:
  // the QK reads (16 lanes = 16 consecutive keys at one chunk) then meet 16 distinct
  // bank quads, and the transposing PV reads (16 lanes = keys 4g..4g+3, 32 bytes each,
  // in slots 4a+g) meet 4 disjoint 8-bank runs.  (An XOR swizzle of 3 bits left every
  // QK read 2-way conflicted; a 4-bit one would need 8 base registers.)
  constexpr int RP = ROWB + 16;
  auto slot = [](int key) -> int { return (key & 16) | ((key & 3) << 2) | ((key >> 2) & 3); };
  __shared__ __attribute__((aligned(16))) unsigned char st0[KT * RP];
  __shared__ __attribute__((aligned(16))) unsigned char st1[KT * RP];
  // exchange area, 1 KB per wave and block: partial logits xh[q][wave][lane] at
  // 4096q + 1024 wave + 16 lane (8 KB), probabilities xp[wave][lane] at 8192 + 1024 wave
  // + 16 lane (4 KB), per-head maxima and sums xm (1 KB); past them the overflow flag,
  // the sink logits [H] and the RoPE table, which the loop leaves alone (a table of
  // more than 192 pairs borrows the start of the area and is formed again for the
  // output).  A wave's own exchange slots and its partner's (wave ^ 1) differ by 1024,
  // so two address registers cover them all.  Stages and exchange area fill 80 KB, so two
  // workgroups share a CU.
  __shared__ __attribute__((aligned(16))) unsigned char xbuf[15360];
  static_assert(2 * KT * RP + 15360 == 80 * 1024, "two workgroups per CU");
  float (*xm)[64] = reinterpret_cast<float (*)[64]>(xbuf + 12288);
  float (*mr)[64] = reinterpret_cast<float (*)[64]>(xbuf + 4096);  // references, after the loop
  int* ovf = reinterpret_cast<int*>(xbuf + 13312);  // overflow flag
  float* sk = reinterpret_cast<float*>(xbuf + 13568);  // softmax-sink logits [H]
  const bool cs_kept = a.R / 2 <= 192;
  float2* cs = reinterpret_cast<float2*>(xbuf + (cs_kept ? 13824 : 0));  // RoPE table

  // workgroup -> query: as sparse_mqa_kernel (32 consecutive queries per XCD visit)
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
  const int h = 32 * hg + l32;  // this lane's head
  const int n_t = a.mode == MQA_WINDOW_ONLY ? 0 : visible_entries(t, a.ratio);
  const int nsel = a.mode == MQA_SELECTED ? min(a.topk, n_t) : n_t;
  const int nwin = window_count(t, a.window);
  const int wlo = window_lo(t, a.window);
  const int nk = nsel + nwin;
  const int64_t P = a.pos0 + t;
  const int rlo = D - a.R;

  auto rope_table = [&]() {
    if (threadIdx.x < a.R / 2) {
      float c, sn;
      rope_cos_sin(P, rope_inv_freq(threadIdx.x, a.R, a.theta), &c, &sn);
      cs[threadIdx.x] = make_float2(c, sn);
    }
  };

  const unsigned char* qg =
      reinterpret_cast<const unsigned char*>(a.q) + ((int64_t)b * a.S + t) * a.H * ROWB;

  // Key sources, one tile ahead: lane l < 32 resolves key tile*32 + l.
  const unsigned char* kv_c = reinterpret_cast<const unsigned char*>(a.kv_c);
  const unsigned char* kv_w = reinterpret_cast<const unsigned char*>(a.kv_w);
  // Entry index of key tile*32 + l32.  Every lane loads, always (from a clamped
  // position, or from the query's q row when no entry is gathered), so the value
  // arrives in the same register on every path: a register merge of a load's result
  // would make the compiler wait for it, and that wait drains the copies in flight.  The
  // value is only inspected at the next tile's issue.
  const bool gather = a.mode == MQA_SELECTED && nsel > 0;
  const int32_t* irow = gather ? a.idx + ((int64_t)b * a.S + t) * a.topk : reinterpret_cast<const int32_t*>(qg);
  const int ilast = gather ? nsel - 1 : 0;
  // The lane index inside the per-tile address arithmetic is formed afresh at each use:
  // otherwise the compiler precomputes the first tiles' per-lane addresses at the start
  // and spills them across the key loop (each spill a scratch store and a reload per
  // query).
  auto load_idx = [&](int tile) -> int { return irow[min(tile * KT + (lane_id_fresh() & 31), ilast)]; };
  // The lane's 16-byte piece of a key row lands at byte 16 lane of the row's slot.
  const uint32_t dma_off = (uint32_t)lane << 4;
  // Direct-to-LDS copy of tile `tile` (index values `sv` from load_idx): wave w loads
  // keys w, w+4, ..., one 1 KB wave load per key (scalar row base, 32-bit lane offset),
  // key w + 4m into slot 16(m>>2) + 4w + (m&3); returns the tile's key-validity bits.
  // The copies are written in assembly, so the compiler adds no waits for them;
  // copies_barrier() is the only wait.
  auto issue = [&](int tile, int sv, unsigned char* sb) -> uint32_t {
    const int kk = tile * KT + (lane_id_fresh() & 31);
    const unsigned char* src = qg;  // masked keys read finite data that is never used
    bool ok = false;
    if (kk < nsel) {
      if (!gather) sv = kk;
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
      // The row base was just written to SGPRs by v_readlane (a VALU op); a vector-memory
      // instruction may read such an SGPR only 5 wait states later, and the compiler
      // does not pad for an instruction inside inline assembly: s_nop 4 gives the 5 (and
      // the 1 that the M0 write needs before the copy).
      asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(dma_off), "s"(row), "{m0}"(lds) : "memory");
    }
    return bits;
  };

  // Q^T fragments straight from global memory: lane (head 32hg + l32, g), k-step k
  // holds dims 256dh + 16k + 8g .. +7 (bf16x8 vectors: two values per register).  Lanes
  // of heads past H load head H-1 (no branch): their logits copy that head's, and their
  // output rows are never written.
  bf16x8 qf[16];
  auto load_q = [&]() {
    const unsigned char* q0 = qg + (int64_t)min(h, a.H - 1) * ROWB + 2 * (256 * dh + 8 * g);
#pragma unroll
    for (int k = 0; k < 16; ++k) qf[k] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(q0 + 32 * k));
  };
  // rotate q at +P where its dims fall in the last R
  auto rotate_q = [&]() {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int d0 = 256 * dh + 16 * k + 8 * g;
      if (d0 + 8 > rlo) {
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
          const int d = d0 + i;
          if (d >= rlo) {
            const float2 r = cs[(d - rlo) >> 1];
            const float x0 = (float)qf[k][i], x1 = (float)qf[k][i + 1];
            qf[k][i] = (bf16)(x0 * r.x - x1 * r.y);
            qf[k][i + 1] = (bf16)(x0 * r.y + x1 * r.x);
          }
        }
      }
    }
  };

  // Pass 0's first tile is requested before q, so both latencies overlap, and the RoPE
  // table (a chain of fp64 operations in the first wave) is formed while they are in
  // flight.
  const int ntiles = (nk + KT - 1) / KT;
  uint32_t km0 = 0u, km1 = 0u;
  int sv = 0;
  {
    // Without a gather the first copies need no index: they are issued without waiting
    // for one (the dense and window-only layers then pay one memory latency per query
    // before their first tile instead of two).
    if (gather) {
      // The index load goes out first (the empty asm keeps the compiler from moving the
      // q loads ahead of it), so the copies wait for it alone, not for q as well.
      const int sv0 = load_idx(0);
      asm volatile("" ::: "memory");
      load_q();
      if (ntiles > 0) km0 = issue(0, sv0, st0);
    } else {
      load_q();
      if (ntiles > 0) km0 = issue(0, 0, st0);
    }
    sv = load_idx(1);
    const float skv = a.sinks && threadIdx.x < a.H ? a.sinks[threadIdx.x] : 0.f;
    rope_table();
    if (a.sinks && threadIdx.x < a.H) sk[threadIdx.x] = skv;
    if (threadIdx.x == 0) *ovf = 0;
  }
  copies_barrier();  // the RoPE table and sinks are written; q and key tile 0 have landed
  rotate_q();
  // A table of more than 224 pairs sits where the loop exchanges partial logits: every
  // wave must have read it first.
  if (!cs_kept) lds_barrier();

  // Per-lane LDS offsets.  QK: lane row l32 holds key kr = l32 ^ 16dh (this wave's own
  // keys 16dh .. 16dh+15 become accumulator rows 0..15, the partner's rows 16..31);
  // dims 256dh + 16k + 8g .. +7 of key kr sit at slot(kr) RP + 512dh + 16g + 32k: one
  // base, 32k an immediate.
  const int kr = l32 ^ (16 * dh);
  const int qk_base = slot(kr) * RP + 512 * dh + 16 * g;
  // PV: 16-lane group hq = lane/16 covers dims 128 wave + 32db + 16(hq&1) .. +15; lane j of
  // the group addresses key 16kh + 4g + j/4 (and +8), dims + 4(j%4).  Key 4g + a (a =
  // j/4) of a half sits in slot 4a + g and key 8 + 4g + a in slot 4a + 2 + g: one base,
  // 64db, 16 RP for key half kh and 2 RP for the +8 keys are immediates.
  const int hj = lane & 15, hh = (lane >> 4) & 1, a4 = hj >> 2;
  const int pv_base = (4 * a4 + g) * RP + 256 * wave + 32 * hh + 8 * (hj & 3);
  const int xo = 1024 * wave + 16 * lane;  // this wave's exchange slot (its partner's: xo ^ 1024)
  typedef short i16x4 __attribute__((ext_vector_type(4)));

  // Softmax with a fixed reference (shift invariance), as in sparse_mqa_kernel.
  float m_seen = -INFINITY, m_ref = -INFINITY, l_run = 0.f;
  f32x16 O[8];

  // The partner waves (same heads, other latent half) split the softmax: wave dh owns
  // keys 16dh .. 16dh+15 of each tile (its accumulator rows 0..15).  Each sends the
  // partner its partial logits of the partner's keys, forms the full logits of its own,
  // and the two swap their bf16 probabilities for PV.  Both use the same per-head
  // reference: the maximum of the pass's first tile, agreed through xm (0 if that tile
  // has no valid key; the end-of-pass check then catches any under- or overflow).
  //
  // The LDS fragment reads of both products run ahead of the MFMAs that consume them
  // (KA fragments ahead for QK, VA for PV), and sched_group_barrier pins that order, so
  // an MFMA waits for a read issued KA (VA) MFMAs earlier, not for a full LDS round trip.
  // The look-ahead is what the 256 registers leave: QK also holds the logits (16).
  constexpr int KA = 1, VA = 2;
  auto compute = [&](const unsigned char* sb, uint32_t kmask, bool first) {
    const CSA_LDS unsigned char* lb = (const CSA_LDS unsigned char*)sb;
    CSA_LDS unsigned char* xb = (CSA_LDS unsigned char*)xbuf;
    auto ld_k = [&](int k) {
      return __builtin_bit_cast(bf16x8, *(const CSA_LDS u32x4*)(lb + qk_base + 32 * k));
    };
    f32x16 s = {};
    {
      bf16x8 kb[KA + 1];
#pragma unroll
      for (int k = 0; k < KA; ++k) kb[k] = ld_k(k);
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        if (k + KA < 16) kb[(k + KA) % (KA + 1)] = ld_k(k + KA);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb[k % (KA + 1)], qf[k], s, 0, 0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(kSgDsRead, KA, 0);
#pragma unroll
      for (int k = 0; k < 16 - KA; ++k) {
        __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(kSgMfma, KA, 0);
    }
    // send the partner's keys (rows 16..31), receive this wave's
#pragma unroll
    for (int q = 0; q < 2; ++q)
      *(CSA_LDS f32x4*)(xb + xo + 4096 * q) = f32x4{s[8 + 4 * q], s[9 + 4 * q], s[10 + 4 * q], s[11 + 4 * q]};
    lds_barrier();
    // logits in unscaled units; the base-2 scale is folded into the exponent's FMA
    float z[8];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const f32x4 o4 = *(const CSA_LDS f32x4*)(xb + (xo ^ 1024) + 4096 * q);
#pragma unroll
      for (int i = 0; i < 4; ++i) z[4 * q + i] = s[4 * q + i] + o4[i];
    }
    if (kmask != 0xffffffffu) {  // wave-uniform: only partial or masked tiles pay for the mask
      const uint32_t kml = kmask >> (4 * g + 16 * dh);  // bit 8q + i: key 16dh + 8q + 4g + i
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (!((kml >> (8 * (e >> 2) + (e & 3))) & 1u)) z[e] = -INFINITY;
    }
    float mt = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) mt = fmaxf(mt, z[e]);
    mt = halves_max(mt);
    m_seen = fmaxf(m_seen, mt);
    if (first) {  // workgroup-uniform: agree on the reference
      xm[wave][lane] = mt;
      lds_barrier();
      const float m0 = fmaxf(mt, xm[wave ^ 1][lane]);
      m_ref = m0 == -INFINITY ? 0.f : m0;
      // a reference forced to 0 may lie far above every logit: the end of the pass
      // then takes the exact maximum and runs again
      if (__any(m0 == -INFINITY) && lane == 0) *ovf = 1;
    }
    const float nbias = -m_ref * a.scale_log2;
    bf16x8 pm;
    float ls = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = __builtin_amdgcn_exp2f(fmaf(z[e], a.scale_log2, nbias));
      ls += p;
      pm[e] = (bf16)p;
    }
    l_run += ls;
    *(CSA_LDS u32x4*)(xb + xo + 8192) = __builtin_bit_cast(u32x4, pm);
    lds_barrier();
    // O^T[dims of quarter `wave`, heads 32hb ..] += V^T . P^T: V^T fragment (db, key
    // half kh) feeds both head groups, so each transposing read serves two MFMAs.  The
    // probabilities of head group hb and key half kh are wave 2hb + kh's (this wave's
    // own read back like the others).  Step jj = 0, 1 takes key half jj ^ (wave >> 1):
    // the accumulation order of a dims half is that of the waves that owned it whole.
    const int kfirst = wave >> 1;
    bf16x8 pf[2][2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
        pf[hb][jj] = __builtin_bit_cast(
            bf16x8, *(const CSA_LDS u32x4*)(xb + 8192 + 1024 * (2 * hb + (jj ^ kfirst)) + 16 * lane));
    {
      // fragment j: dims block j & 3 of the quarter, key half (j >> 2) ^ kfirst; two
      // transposing reads (keys 16kh + 4g + j/4 and +8)
      auto ld_v = [&](int j) {
        const CSA_LDS unsigned char* p = lb + pv_base + 64 * (j & 3) + 16 * RP * ((j >> 2) ^ kfirst);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((CSA_LDS i16x4*)p);
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((CSA_LDS i16x4*)(p + 2 * RP));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      bf16x8 vb[VA + 1];
#pragma unroll
      for (int j = 0; j < VA; ++j) vb[j] = ld_v(j);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j + VA < 8) vb[(j + VA) % (VA + 1)] = ld_v(j + VA);
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
          O[4 * hb + (j & 3)] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(vb[j % (VA + 1)], pf[hb][j >> 2], O[4 * hb + (j & 3)], 0, 0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(kSgDsRead, 4 + 2 * VA, 0);
#pragma unroll
      for (int j = 0; j < 8 - VA; ++j) {
        __builtin_amdgcn_sched_group_barrier(kSgDsRead, 2, 0);
        __builtin_amdgcn_sched_group_barrier(kSgMfma, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(kSgMfma, 2 * VA, 0);
    }
  };

  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) O[db][i] = 0.f;
    l_run = 0.f;
    if (pass > 0) {
      if (ntiles > 0) km0 = issue(0, load_idx(0), st0);
      sv = load_idx(1);
      copies_barrier();
    }
    for (int tile = 0; tile < ntiles; tile += 2) {
      if (tile + 1 < ntiles) km1 = issue(tile + 1, sv, st1);
      sv = load_idx(tile + 2);
      compute(st0, km0, pass == 0 && tile == 0);
      copies_barrier();  // tile+1 landed in st1; every wave is done with st0 and the exchange area
      if (tile + 1 < ntiles) {
        if (tile + 2 < ntiles) km0 = issue(tile + 2, sv, st0);
        sv = load_idx(tile + 3);
        compute(st1, km1, false);
        copies_barrier();
      }
    }
    // Run again with the pair's exact maximum as the reference if some probability could
    // have overflowed, or (reference forced to 0 after an all-masked first tile, flagged
    // there) underflowed.  The reference is the maximum over a subset of the head's
    // keys, so otherwise only overflow is possible, and the lane's own maximum tells.
    // The pass's row sums go out with the overflow flag behind one barrier; the partner
    // adds them unless the pass runs again.
    xm[wave][lane] = l_run;
    mr[wave][lane] = m_ref;  // the epilogue normalises both head groups
    if (pass == 0 && __any(m_seen != -INFINITY && (m_seen - m_ref) * a.scale_log2 > 64.0f) && lane == 0)
      *ovf = 1;
    lds_barrier();
    if (pass == 1 || !*ovf) break;
    xm[wave][lane] = m_seen;  // every wave takes this path, so no wave reads the row sums
    lds_barrier();
    const float mall = fmaxf(m_seen, xm[wave ^ 1][lane]);
    m_ref = mall == -INFINITY ? 0.f : mall;  // exact reference for the second pass
    lds_barrier();  // xm is read
  }

  // normalise, de-rotate at -P, stage by head rows, write o[b,t] coalesced.  The lane's
  // indices are formed again here rather than kept (or spilled) across the key loop.
  // Head h's denominator sums both lane halves of both key-half waves of its group;
  // its reference is that group's (published with the sums).
  const int ln = lane_id_fresh();
  const int l32e = ln & 31, ge = ln >> 5;
  float inv[2];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const int he = 32 * hb + l32e;
    const float l = halves_sum(xm[2 * hb][ln] + xm[2 * hb + 1][ln]);
    const float mh = mr[2 * hb][ln];
    if (a.lse && wave == hb && ge == 0 && he < a.H)
      a.lse[((int64_t)b * a.S + t) * a.H + he] = head_lse(mh * a.scale_log2, l, a.sinks, he);
    float lt = l;
    if (a.sinks && he < a.H)  // the sink joins the denominator, same reference
      lt += __builtin_amdgcn_exp2f(sk[he] * kLog2e - mh * a.scale_log2);
    inv[hb] = lt > 0.f ? __builtin_amdgcn_rcpf(lt) : 0.f;
  }
  if (!cs_kept) {
    lds_barrier();
    rope_table();
    lds_barrier();
  }
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    unsigned char* os = hb == 0 ? st0 : st1;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int dbase = 128 * wave + 32 * db;
      // the table entries of a rotated dims block are read together: one LDS round trip
      const bool rot = dbase + 32 > rlo;  // wave-uniform
      float2 r[8];
      if (rot) {
#pragma unroll
        for (int e = 0; e < 8; ++e) r[e] = cs[max(dbase + 8 * (e >> 1) + 4 * ge + 2 * (e & 1) - rlo, 0) >> 1];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d0 = dbase + 8 * j + 4 * ge;
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = O[4 * hb + db][4 * j + i] * inv[hb];
        if (rot && d0 >= rlo) {
#pragma unroll
          for (int i = 0; i < 4; i += 2) {
            const float2 c = r[2 * j + (i >> 1)];
            const float x0 = x[i], x1 = x[i + 1];
            x[i] = x0 * c.x + x1 * c.y;
            x[i + 1] = -x0 * c.y + x1 * c.x;
          }
        }
        T y[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) y[i] = from_f32<T>(x[i]);
        *reinterpret_cast<uint2*>(os + l32e * RP + 2 * d0) = *reinterpret_cast<const uint2*>(y);
      }
    }
  }
  lds_barrier();
  unsigned char* og = reinterpret_cast<unsigned char*>(a.o) + ((int64_t)b * a.S + t) * a.H * ROWB;
  for (int c = 64 * wave + ln; c < a.H * (ROWB / 16); c += NT) {
    const int row = c >> 6, col = (c & 63) * 16;
    *reinterpret_cast<uint4*>(og + (int64_t)row * ROWB + col) =
        *reinterpret_cast<const uint4*>((row < 32 ? st0 : st1) + (row & 31) * RP + col);
  }
}

template <typename T, int D>
static void launch_d(const MqaArgs& a, int H, hipStream_t st) {
  dim3 grid(a.B * a.S);
  if constexpr (D == 512 && sizeof(T) == 2) {
    if (H > 16) {
      hipLaunchKernelGGL(sparse_mqa_hd_kernel, grid, dim3(256), 0, st, a);
      return;
    }
  }
  if (H <= 16) hipLaunchKernelGGL((sparse_mqa_kernel<T, D, 1>), grid, dim3(64), 0, st, a);
  else hipLaunchKernelGGL((sparse_mqa_kernel<T, D, 4>), grid, dim3(256), 0, st, a);
}

template <typename T>
static hipError_t launch_t(const MqaArgs& a, int D, int H, hipStream_t st) {
  switch (D) {
    case 64: launch_d<T, 64>(a, H, st); break;
    case 128: launch_d<T, 128>(a, H, st); break;
    case 256: launch_d<T, 256>(a, H, st); break;
    case 512: launch_d<T, 512>(a, H, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_sparse_mqa(const csa_params_t& p, MqaMode mode, const void* q, const void* kv_c,
                             const void* kv_w, const int32_t* idx, const float* sinks, void* o,
                             float* lse, hipStream_t st) {
  MqaArgs a{};
  a.q = q;
  a.kv_c = kv_c;
  a.kv_w = kv_w;
  a.idx = idx;
  a.sinks = sinks;
  a.o = o;
  a.lse = lse;
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
  a.theta = p.rope_theta;
  a.pos0 = p.pos0;
  if (p.B * p.S == 0) return hipSuccess;
  return p.dtype == CSA_BF16 ? launch_t<bf16>(a, p.D, p.H, st) : launch_t<float>(a, p.D, p.H, st);
}

}  // namespace csa
