// Stage 3a on gfx950: lightning-indexer scores of every causally visible entry,
//   I[t,s] = sum_h w[t,h] * ReLU(q_I[t,h,:] . k_I[s,:]),
// computed from bf16 inputs with fp32 MFMA accumulation ("fix(deepseek-v4): correct
// V4-Flash attention math", Part 1 item 4 keeps this product in high precision; the
// formula is "Enabling DeepSeek-V4-Flash Training on AMD Instinct MI355X GPUs with
// Primus", "Three attention types, interleaved").  The scoring tail (ReLU, per-head
// weight, head sum, causal mask) is fused into the MFMA epilogue, as the "Indexer
// scoring tail" row of that blog's "Kernel fusions" table describes for one kernel.
//
// Mapping: a workgroup of 8 waves owns 8 consecutive queries of one batch and a chunk
// of entries.  Each wave keeps its query's q_I (64 heads x D_I) in registers as the A
// operand of v_mfma_f32_32x32x16_bf16 with heads on M, so the head sum of the
// epilogue is 16 in-lane terms plus one cross-half shuffle.  Entry tiles of 64 rows of
// k_I are staged once per workgroup in double-buffered LDS and read by all 8 waves.
#include "common.hpp"
#include "launch.hpp"

namespace csa {

constexpr int IDX_WAVES = 8;      // queries per workgroup
constexpr int IDX_TILE = 64;      // entries per LDS tile
constexpr int IDX_CHUNK = 1024;   // entries per workgroup
constexpr int IDX_MAX_CHUNKS = 64;

// The indexer prologue's parameters ("fix(deepseek-v4): correct V4-Flash attention
// math", Part 1 items 6a and 6e).  on = 0: plain scores (w_scale = 1 exactly).
struct IndexPrologue {
  double theta;     // RoPE base
  int64_t pos0;     // position of token 0
  int32_t on;       // rotate the queries (the keys arrive rotated)
  int32_t rope_dim; // rotated dims: the last rope_dim of the indexer dims
  float w_scale;    // (idx_heads * idx_dim)^-1/2 with the prologue, else 1
  int32_t fp8;      // E4M3 operands: queries quantized in-kernel, keys arrive as fp8 rows
};

__host__ inline IndexPrologue index_prologue_args(const csa_params_t& p) {
  IndexPrologue r{p.rope_theta, p.pos0, 0, p.rope_dim, 1.0f, (p.flags & CSA_FLAG_INDEX_FP8) ? 1 : 0};
  if (p.flags & CSA_FLAG_INDEX_PROLOGUE) {
    r.on = 1;
    r.w_scale = (float)(1.0 / sqrt((double)p.idx_heads * (double)p.idx_dim));
  }
  return r;
}

struct IndexArgs {
  const void* q_idx;
  const float* w_idx;
  const void* k_idx;
  float* scores;
  int64_t ld;
  int32_t B, S, HI, ratio, n_entries, t0, nrows, qblocks;  // qblocks per batch
  int32_t n_chunks;
  IndexPrologue pro;
  int32_t chunk_wg_off[IDX_MAX_CHUNKS + 1];  // prefix sums of workgroups per chunk
  int32_t chunk_qb_min[IDX_MAX_CHUNKS];      // first query block that needs the chunk
};

// ReLU as one integer max on the bit pattern: every negative float (and -0) is a
// negative int32, every positive float a positive one.  fmaxf(x, 0) would cost two
// instructions on MFMA results, which the compiler cannot prove NaN-canonical.
__device__ inline float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// 32x32 fragment: lane l holds row/col (l % 32) and k-slots 8*(l/32) .. +7.  bf16 is
// one v_mfma_f32_32x32x16_bf16; fp32 issues eight v_mfma_f32_32x32x2_f32 (instruction
// i consumes element i), summing the same 16 k-slots.
__device__ inline f32x16 mfma32x32x16(const Frag<bf16>& a, const Frag<bf16>& b, f32x16 c) {
  bf16x8 av, bv;
#pragma unroll
  for (int i = 0; i < 8; ++i) { av[i] = a.v[i]; bv[i] = b.v[i]; }
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, c, 0, 0, 0);
}
__device__ inline f32x16 mfma32x32x16(const Frag<float>& a, const Frag<float>& b, f32x16 c) {
#pragma unroll
  for (int i = 0; i < 8; ++i) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.v[i], b.v[i], c, 0, 0, 0);
  return c;
}

// ---------------------------------------------------------------------------------
// FP8 (E4M3) indexer operands ("Enabling DeepSeek-V4-Flash Training on AMD Instinct
// MI355X GPUs with Primus", closing remarks: an E4M3 path for the indexer QK).  Each
// q_I[t,h] and k_I[s] row is quantized with its own scale: m = max |x|, codes =
// E4M3(x * (448 / m)) rounded to nearest even by v_cvt_pk_fp8_f32, scale = m / 448
// (both divisions IEEE fp32); a zero row has codes 0 and scale 0.  The scales factor
// out of the ReLU: score = sk[s] * sum_h (w[h] sq[h]) ReLU(codes_q[h] . codes_k[s]).
// The MFMA is v_mfma_f32_32x32x64_f8f6f4: lane (g, l32) holds 32 codes of row l32 in
// k-slot order p = 0..31, p -> dim 64*kk + 16*(p/8) + 8*g + p%8 for k-step kk; this is
// the bf16 fragment layout (fragment ks = 4*kk + p/8, element p%8), so the queries
// convert in place, and the key rows are stored in that order (byte 64*kk + 32*g + p
// of a row), followed by the fp32 scale and 12 bytes of padding: DI + 16 bytes a row.
// ---------------------------------------------------------------------------------
constexpr float kE4M3Max = 448.0f;
typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ inline int key_fp8_pos(int d) {  // byte of dim d in a key row
  return (d & ~63) + 32 * ((d >> 3) & 1) + 8 * ((d & 63) >> 4) + (d & 7);
}

// Four E4M3 codes of x[0..3] * inv packed into one word (byte i = x[i]).
__device__ inline uint32_t pack_fp8x4(float x0, float x1, float x2, float x3, float inv) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0 * inv, x1 * inv, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(x2 * inv, x3 * inv, w, true);
  return (uint32_t)w;
}

__device__ inline f32x16 mfma32x32x64_fp8(const i32x8& a, const i32x8& b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// A pointer the wave holds in every lane, moved to scalar registers (a global_load_lds
// base operand).  readfirstlane works on 32-bit ints: each half is widened as an
// unsigned value, so a low half with bit 31 set is not sign-extended into the high one.
__device__ inline const float* wave_uniform(const float* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return (const float*)(((uint64_t)hi << 32) | (uint64_t)lo);
}

// Two neighbouring fragment elements as fp32, and back (round to nearest even): bf16
// pairs are one 32-bit word, unpacked with a shift and a mask and packed with one
// v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ inline void frag_get2(const Frag<float>& f, int i, float& a, float& b) {
  a = f.v[i];
  b = f.v[i + 1];
}
__device__ inline void frag_get2(const Frag<bf16>& f, int i, float& a, float& b) {
  const uint32_t w = reinterpret_cast<const uint32_t*>(f.v)[i >> 1];
  a = __uint_as_float(w << 16);
  b = __uint_as_float(w & 0xffff0000u);
}
__device__ inline void frag_set2(Frag<float>& f, int i, float a, float b) {
  f.v[i] = a;
  f.v[i + 1] = b;
}
__device__ inline void frag_set2(Frag<bf16>& f, int i, float a, float b) {
  reinterpret_cast<uint32_t*>(f.v)[i >> 1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// Indexer prologue of one wave's query, on its A fragments in registers: RoPE on the
// last R of the DI dims at position P, then the normalised Sylvester Hadamard
// Hn = H / sqrt(DI), H[i][j] = (-1)^popcount(i & j) ("fix(deepseek-v4): correct
// V4-Flash attention math", Part 1 item 6e), in fp32 and rounded once to T.  Lane
// (g, l32) holds dims 16*ks + 8*g + i (i = 0..7) of head hb*32 + l32, so the Hadamard's
// dim bits 0-2 are within a fragment, bits 4.. index the fragments and bit 3 is the
// lane half.
//   * The rotation of pair (x0, x1) by (c, s), the butterfly of dim bit 0 and the
//     1/sqrt(DI) scale fold into h0 = x0 a + x1 b, h1 = x0 b - x1 a with
//     a = (c + s) / sqrt(DI), b = (c - s) / sqrt(DI) (c = 1, s = 0 outside the rope
//     dims).  `tab` is DI words of this wave's LDS: lane q writes (a, b) of dim pair q
//     and every lane reads the four pairs of a fragment with two 16-byte loads.
//   * Dim bit 3 goes last, two registers at a time through v_permlane32_swap (a swap
//     between the lane halves, no trip through the LDS crossbar): swapping (u, v) puts
//     both halves of u in the lower lanes and both halves of v in the upper lanes, one
//     add and one subtract make the butterfly, and a second swap puts them back.
// Every lane of the wave must call it.
template <typename T, int DI>
__device__ void index_query_prologue(Frag<T> (&qa)[2][DI / 16], int64_t P, int R, double theta,
                                     uint32_t* tab) {
  constexpr int KS = DI / 16;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 5;
  const int lo = DI - R;  // first rotated dim
  if (lane < DI / 2) {
    float c = 1.f, sn = 0.f;
    if (2 * lane >= lo) rope_cos_sin(P, rope_inv_freq((2 * lane - lo) >> 1, R, theta), &c, &sn);
    const float scale = 1.0f / __builtin_sqrtf((float)DI);
    CSA_LDS uint32_t* tp = (CSA_LDS uint32_t*)tab + 2 * lane;
    tp[0] = __float_as_uint((c + sn) * scale);
    tp[1] = __float_as_uint((c - sn) * scale);
  }
  // the wave's own LDS writes are seen by its later reads (in-order LDS queue)
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    __builtin_amdgcn_sched_barrier(0);  // one head block's vector live at a time
    float x[KS][8];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      // pairs 8ks + 4g .. +3: (a, b) interleaved, 32 bytes
      const CSA_LDS u32x4* tp = (const CSA_LDS u32x4*)((CSA_LDS uint32_t*)tab + 2 * (8 * ks + 4 * g));
      const u32x4 t0 = tp[0], t1 = tp[1];
      const float ca[4] = {__uint_as_float(t0[0]), __uint_as_float(t0[2]), __uint_as_float(t1[0]), __uint_as_float(t1[2])};
      const float cb[4] = {__uint_as_float(t0[1]), __uint_as_float(t0[3]), __uint_as_float(t1[1]), __uint_as_float(t1[3])};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float x0, x1;
        frag_get2(qa[hb][ks], 2 * j, x0, x1);
        x[ks][2 * j] = fmaf(x0, ca[j], x1 * cb[j]);
        x[ks][2 * j + 1] = fmaf(x0, cb[j], -(x1 * ca[j]));
      }
    }
    // dim bits 1-2: within a fragment
#pragma unroll
    for (int m = 2; m < 8; m <<= 1)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (!(i & m)) {
            const float u = x[ks][i], v = x[ks][i | m];
            x[ks][i] = u + v;
            x[ks][i | m] = u - v;
          }
    // dim bits 4..: across fragments
#pragma unroll
    for (int m = 1; m < KS; m <<= 1)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        if (!(ks & m)) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float u = x[ks][i], v = x[ks | m][i];
            x[ks][i] = u + v;
            x[ks | m][i] = u - v;
          }
        }
    // dim bit 3, registers i and i+1 of each fragment as one swap pair
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[ks][i]), __float_as_uint(x[ks][i + 1]),
                                                        false, false);
        const float lo_v = __uint_as_float(r[0]), hi_v = __uint_as_float(r[1]);
        const auto back = __builtin_amdgcn_permlane32_swap(__float_as_uint(lo_v + hi_v),
                                                           __float_as_uint(lo_v - hi_v), false, false);
        frag_set2(qa[hb][ks], i, __uint_as_float(back[0]), __uint_as_float(back[1]));
      }
  }
}

// E4M3 codes of one wave's query fragments (after the prologue, if any), in the MFMA
// k-slot order described above.  Per head row: the maximum of the lane's 8*KS values
// and of the partner half's (v_permlane32_swap), the multiplier 448 / max, the codes.
// The lower-half lane of head hb*32 + l32 writes the row's scale max / 448 to tab[h].
// Every lane of the wave must call it.
template <typename T, int DI>
__device__ void index_query_fp8(const Frag<T> (&qa)[2][DI / 16], i32x8 (&q8)[2][DI / 64], uint32_t* tab) {
  constexpr int KS = DI / 16;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 5;
  const int l32 = lane & 31;
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    float m = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        float x0, x1;
        frag_get2(qa[hb][ks], i, x0, x1);
        m = fmaxf(m, fmaxf(fabsf(x0), fabsf(x1)));
      }
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    m = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    const float inv = m > 0.f ? kE4M3Max / m : 0.f;
    if (g == 0) ((CSA_LDS uint32_t*)tab)[hb * 32 + l32] = __float_as_uint(m / kE4M3Max);
#pragma unroll
    for (int kk = 0; kk < DI / 64; ++kk)
#pragma unroll
      for (int m4 = 0; m4 < 4; ++m4) {
        float x[8];
#pragma unroll
        for (int i = 0; i < 8; i += 2) frag_get2(qa[hb][4 * kk + m4], i, x[i], x[i + 1]);
        q8[hb][kk][2 * m4] = (int)pack_fp8x4(x[0], x[1], x[2], x[3], inv);
        q8[hb][kk][2 * m4 + 1] = (int)pack_fp8x4(x[4], x[5], x[6], x[7], inv);
      }
  }
}

template <typename T, int DI, bool PRO, bool F8>
__global__ __launch_bounds__(IDX_WAVES * 64) void index_scores_kernel(IndexArgs a) {
  constexpr int KS = DI / 16;                    // k-steps of 16
  constexpr int VEC = 16 / sizeof(T);            // elements per 16-byte load
  constexpr int ROW = DI + 16 / sizeof(T);       // padded LDS row (elements)
  constexpr int HB = 2;                          // head blocks of 32 (up to 64 heads)
  __shared__ __attribute__((aligned(16))) T tile[F8 ? 1 : 2][F8 ? 8 : IDX_TILE * ROW];
  __shared__ __attribute__((aligned(16))) uint32_t pro_tab[(PRO || F8) ? IDX_WAVES : 1][(PRO || F8) ? DI : 1];
  // fp8 key rows: DI codes, the scale and padding (RB8 bytes), one pad chunk in LDS
  constexpr int RB8 = DI + 16, RP8 = RB8 + 16, KK = F8 ? DI / 64 : 1;
  __shared__ __attribute__((aligned(16))) unsigned char tile8[F8 ? 2 : 1][F8 ? IDX_TILE * RP8 : 16];

  // workgroup -> (chunk, batch, query block)
  const int wg = blockIdx.x;
  int chunk = 0;
  while (chunk + 1 < a.n_chunks && wg >= a.chunk_wg_off[chunk + 1]) ++chunk;
  const int within = wg - a.chunk_wg_off[chunk];
  const int nqb = a.qblocks - a.chunk_qb_min[chunk];
  const int b = within / nqb;
  const int qb = a.chunk_qb_min[chunk] + within % nqb;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 5;      // k-slot half
  const int l32 = lane & 31;
  const int trow0 = qb * IDX_WAVES;                  // first row of this block (rel. t0)
  const int t_last = a.t0 + min(a.nrows, trow0 + IDX_WAVES) - 1;
  const int n_blk = visible_entries(t_last, a.ratio);
  const int e_begin = chunk * IDX_CHUNK;
  const int e_end = min(e_begin + IDX_CHUNK, n_blk);

  const int trow = trow0 + wave;
  const bool q_ok = trow < a.nrows;
  const int t = a.t0 + trow;
  const int n_t = q_ok ? visible_entries(t, a.ratio) : 0;

  // A operand: q_I[b, t, h, :] with h = hb*32 + l32; zero for h >= HI.
  Frag<T> qa[HB][KS];
  i32x8 q8[HB][KK];  // E4M3 codes (F8)
  float w[HB][16];
  const T* qrow = static_cast<const T*>(a.q_idx) + ((int64_t)b * a.S + t) * a.HI * DI;
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const int h = hb * 32 + l32;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (q_ok && h < a.HI) qa[hb][ks] = load_frag(qrow + (int64_t)h * DI + ks * 16 + g * 8);
      else {
#pragma unroll
        for (int i = 0; i < 8; ++i) qa[hb][ks].v[i] = from_f32<T>(0.f);
      }
    }
  }
  // (a.pro.on is always set in the PRO instance; the runtime test keeps the compiler
  // from folding the fragment loads into the prologue, which needs 40-140 more VGPRs)
  if constexpr (PRO)
    if (a.pro.on) index_query_prologue<T, DI>(qa, a.pro.pos0 + t, a.pro.rope_dim, a.pro.theta, pro_tab[wave]);
  if constexpr (F8)
    if (a.pro.fp8) index_query_fp8<T, DI>(qa, q8, pro_tab[wave]);  // head scales -> pro_tab[wave][0..63]
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    // accumulator element 4j+i is head hb*32 + 8j + 4g + i
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hh = hb * 32 + 8 * j + 4 * g + i;
        float wv = (q_ok && hh < a.HI) ? a.w_idx[((int64_t)b * a.S + t) * a.HI + hh] : 0.f;
        if constexpr (PRO) wv *= a.pro.w_scale;
        if constexpr (F8) wv *= __uint_as_float(pro_tab[wave][hh]);
        w[hb][4 * j + i] = wv;
      }
  }

  const T* kbase = static_cast<const T*>(a.k_idx) + (int64_t)b * a.n_entries * DI;
  // k_I tiles go global -> registers -> LDS; the next tile's loads are in flight
  // while the current tile is multiplied.
  constexpr int NT = IDX_WAVES * 64;
  constexpr int CHUNKS_PER_TILE = IDX_TILE * DI / VEC;   // 16-byte pieces per tile
  constexpr int PER_THREAD = (CHUNKS_PER_TILE + NT - 1) / NT;
  uint4 pf[PER_THREAD];
  constexpr int CH8 = IDX_TILE * RB8 / 16;                  // 16-byte pieces per fp8 tile
  constexpr int PER8 = (CH8 + NT - 1) / NT;
  uint4 pf8[PER8];
  const unsigned char* kbase8 = static_cast<const unsigned char*>(a.k_idx) + (int64_t)b * a.n_entries * RB8;
  auto fetch8 = [&](int e0) {
#pragma unroll
    for (int k = 0; k < PER8; ++k) {
      const int c = threadIdx.x + k * NT;
      const int row = c / (RB8 / 16);
      pf8[k] = (c < CH8 && e0 + row < e_end)
                   ? *reinterpret_cast<const uint4*>(kbase8 + (int64_t)(e0 + row) * RB8 + (c % (RB8 / 16)) * 16)
                   : make_uint4(0, 0, 0, 0);
    }
  };
  auto commit8 = [&](int buf) {
#pragma unroll
    for (int k = 0; k < PER8; ++k) {
      const int c = threadIdx.x + k * NT;
      if (c < CH8) *reinterpret_cast<uint4*>(&tile8[buf][(c / (RB8 / 16)) * RP8 + (c % (RB8 / 16)) * 16]) = pf8[k];
    }
  };
  auto fetch = [&](int e0) {
#pragma unroll
    for (int k = 0; k < PER_THREAD; ++k) {
      const int c = threadIdx.x + k * NT;
      const int row = c / (DI / VEC);
      const int col = (c % (DI / VEC)) * VEC;
      pf[k] = (c < CHUNKS_PER_TILE && e0 + row < e_end)
                  ? *reinterpret_cast<const uint4*>(kbase + (int64_t)(e0 + row) * DI + col)
                  : make_uint4(0, 0, 0, 0);
    }
  };
  auto commit = [&](int buf) {
#pragma unroll
    for (int k = 0; k < PER_THREAD; ++k) {
      const int c = threadIdx.x + k * NT;
      if (c < CHUNKS_PER_TILE) {
        const int row = c / (DI / VEC);
        const int col = (c % (DI / VEC)) * VEC;
        *reinterpret_cast<uint4*>(&tile[buf][row * ROW + col]) = pf[k];
      }
    }
  };

  float* srow = a.scores + ((int64_t)b * a.nrows + trow) * a.ld;
  const int ntiles = (e_end - e_begin + IDX_TILE - 1) / IDX_TILE;
  if (ntiles > 0) {
    if constexpr (F8) {
      fetch8(e_begin);
      commit8(0);
    } else {
      fetch(e_begin);
      commit(0);
    }
  }
  __syncthreads();
  for (int it = 0; it < ntiles; ++it) {
    const int e0 = e_begin + it * IDX_TILE;
    if (it + 1 < ntiles) {
      if constexpr (F8) fetch8(e0 + IDX_TILE);
      else fetch(e0 + IDX_TILE);
    }
    const T* tb = tile[F8 ? 0 : (it & 1)];
    const unsigned char* tb8 = tile8[F8 ? (it & 1) : 0];
#pragma unroll
    for (int nb = 0; nb < IDX_TILE / 32; ++nb) {
      const int eb = e0 + nb * 32;
      if (eb >= n_t) break;  // wave-uniform: n_t is per wave
      f32x16 acc[HB];
#pragma unroll
      for (int hb = 0; hb < HB; ++hb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[hb][i] = 0.f;
      float sk = 1.f;
      if constexpr (F8) {
        const unsigned char* rp = tb8 + (nb * 32 + l32) * RP8;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const uint4 lo4 = *reinterpret_cast<const uint4*>(rp + kk * 64 + g * 32);
          const uint4 hi4 = *reinterpret_cast<const uint4*>(rp + kk * 64 + g * 32 + 16);
          const i32x8 kb = {(int)lo4.x, (int)lo4.y, (int)lo4.z, (int)lo4.w,
                            (int)hi4.x, (int)hi4.y, (int)hi4.z, (int)hi4.w};
#pragma unroll
          for (int hb = 0; hb < HB; ++hb) acc[hb] = mfma32x32x64_fp8(q8[hb][kk], kb, acc[hb]);
        }
        sk = *reinterpret_cast<const float*>(rp + DI);
      } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const Frag<T> kb = load_frag(tb + (nb * 32 + l32) * ROW + ks * 16 + g * 8);
#pragma unroll
          for (int hb = 0; hb < HB; ++hb) acc[hb] = mfma32x32x16(qa[hb][ks], kb, acc[hb]);
        }
      }
      float v = 0.f;
#pragma unroll
      for (int hb = 0; hb < HB; ++hb)
#pragma unroll
        for (int i = 0; i < 16; ++i) v = fmaf(w[hb][i], relu(acc[hb][i]), v);
      v += __shfl_xor(v, 32, 64);
      if constexpr (F8) v *= sk;  // the entry's scale (sq is folded into w)
      const int e = eb + l32;
      if (g == 0 && e < n_t) srow[e] = v;
    }
    if (it + 1 < ntiles) {
      if constexpr (F8) commit8((it + 1) & 1);
      else commit((it + 1) & 1);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------
// Indexer scores fused with the top-k selection (top-k up to FT_MAXK).
//
// A workgroup of 8 waves owns 8 consecutive queries of one batch and sweeps every
// visible entry, so the scores never leave the chip.  Each wave scores its query with
// the same MFMA tiles and epilogue as index_scores_kernel and keeps a streaming
// selection in LDS: a score whose order-preserving key exceeds the wave's threshold is
// appended (entries arrive in ascending order, so the buffer stays sorted by index).
// When the buffer is nearly full the wave prunes it with one radix pass to the keys
// at or above a bound that at least k buffered keys reach, and the bound becomes the
// new threshold; at the end an exact radix select keeps the top-k by (key desc, index
// asc).  A dropped or refused entry always has at least k buffered entries that beat
// it (a higher key, or an equal key and a smaller index), so the final set is exact.
//
// Entry tiles of k_I (64 rows) go straight from global memory into a three-stage LDS
// ring (global_load_lds), two tiles ahead of the one being multiplied.  Rows are
// padded by 16 bytes, so the fragment reads are free of bank conflicts and their
// addresses are one base plus immediate offsets; the DMA simply also fills the pads.
// Each wave issues the MFMAs of its next 32-entry block next to the ReLU-weighted head
// sums of the previous one, so the scoring VALU work overlaps the matrix core, and
// admits a tile's two blocks in one step: the low lane half scores one block and the
// high half the other, so the key and admission bookkeeping (branch-free) runs once
// per 64 entries.
// ---------------------------------------------------------------------------------
constexpr int FT_WAVES = 8;
constexpr int FT_TILE = 64;    // entries per LDS stage (two 32-entry MFMA blocks)
constexpr int FT_MAXK = 512;   // largest top-k of the fused path
constexpr int FT_LDS = 160 * 1024;
constexpr int FT_COPIERS = 4;  // waves 0..3 issue a tile's copies

template <typename T, int DI, bool F8> struct FtShape {
  // bytes per k_I row: DI elements, or DI E4M3 codes then the fp32 scale (16 bytes)
  static constexpr int ROWB = F8 ? DI + 16 : DI * (int)sizeof(T);
  static constexpr int CPR = ROWB / 16;                  // 16-byte chunks per row
  static constexpr int SPR = CPR + 1;                    // LDS slots per row (one pad)
  static constexpr int ROWP = SPR * 16;                  // padded row pitch in LDS
  static constexpr int STAGE = FT_TILE * ROWP;           // bytes per ring stage
  static constexpr int NI = STAGE / 1024;                // 1 KB DMA instructions per stage
  static constexpr int LPW = (NI + FT_COPIERS - 1) / FT_COPIERS;  // DMA lines per copying wave (max)
  static constexpr int CAP_FIT = (FT_LDS - 3 * STAGE - FT_WAVES * 1024 - 256) / (FT_WAVES * 8) / 64 * 64;
  static constexpr int CAP = CAP_FIT < 2048 ? CAP_FIT : 2048;  // candidates per query
  static_assert(STAGE % 1024 == 0, "a stage is whole 1 KB DMA lines");
  static_assert(CAP >= FT_MAXK + 2 * FT_TILE + 2, "candidate buffer too small");
  static_assert(CAP % 4 == 0, "16-byte candidate accesses");
};

struct IndexTopkArgs {
  const void* q_idx;
  const float* w_idx;
  const void* k_idx;
  int32_t* idx;
  int32_t* n_visible;
  int32_t B, S, HI, ratio, n_entries, topk, qblocks;  // query blocks per batch
  IndexPrologue pro;
};

// Order-preserving key of a score: negative floats have every bit flipped, the others
// only the sign bit.  The epilogue's scores are never -0 (each is a round-to-nearest sum
// that starts from +0, and such a sum is -0 only when every term is -0), so +0 and -0
// need no merging here.
__device__ inline uint32_t score_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

// Wave-wide scan and reductions without LDS round trips.  Exclusive prefix sum:
// Hillis-Steele steps over row_shr 1, 2, 4, 8 within each 16-lane row (lanes with no
// source add 0), then the last lane of row 0 / 2 is broadcast into rows 1 / 3
// (row_bcast:15) and lane 31 into rows 2 and 3 (row_bcast:31).
__device__ inline int wave_excl_scan(int v) {
  int x = v;
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 -> rows 2, 3
  return x - v;
}

// Minimum / maximum over the wave, in every lane: DPP swaps within quads, the 8-lane
// and 16-lane mirrors, then v_permlane16_swap (row pairs) and v_permlane32_swap (halves).
template <bool MAX>
__device__ inline uint32_t wave_minmax(uint32_t x) {
  auto f = [](uint32_t a, uint32_t b) { return MAX ? max(a, b) : min(a, b); };
  x = f(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false));   // quad xor 1
  x = f(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false));   // quad xor 2
  x = f(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x141, 0xF, 0xF, false));  // half-row mirror
  x = f(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x140, 0xF, 0xF, false));  // row mirror
  const auto r16 = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = f(r16[0], r16[1]);
  const auto r32 = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return f(r32[0], r32[1]);
}
__device__ inline uint32_t wave_min(uint32_t x) { return wave_minmax<false>(x); }
__device__ inline uint32_t wave_max(uint32_t x) { return wave_minmax<true>(x); }

#define CSA_WAVE_FENCE() __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront")

// s_waitcnt on the vector-memory counter only (gfx9 encoding: vmcnt in bits 3:0 and
// 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their "no wait" maxima), optionally also
// draining this wave's LDS operations.
template <int N, bool LGKM0>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((LGKM0 ? 0 : 15) << 8) | ((N >> 4) << 14));
}

// Barrier after this wave's LDS accesses have completed; the copies in flight are
// waited for separately (wait_vmcnt), and the memory clobber keeps the compiler from
// moving LDS accesses across it.
__device__ inline void lds_only_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

struct Pruned {
  int c;              // keys kept
  uint32_t theta;     // admit later keys strictly above this
  uint32_t kept_min;  // smallest kept key
};

// Shrink the candidates ckey/cidx[0..c) of one wave, in place and in buffer order.
// kmin <= every key <= kmax (wave-uniform).  An 8-bit radix pass at a time narrows
// the prefix of the k-th largest key.  EXACT keeps exactly the top K by (key desc,
// buffer position asc); otherwise the wave may stop as soon as the keys at or above
// the current prefix number at most `target` (>= K), and keeps all of them.
// Lane l handles buffer positions 4(l + 64j) .. +3 of batch j (one 16-byte LDS access
// each for keys and indices, made only when the first of them is below c; the buffers
// are 16-byte aligned and their capacity is a multiple of 4, so such an access stays in
// the buffer).  Positions >= c are ignored.  Each batch's reads are issued one batch
// ahead, so their latency overlaps the previous batch's atomics or stores.
template <bool EXACT>
__device__ __forceinline__ Pruned wave_select(uint32_t* ckey, int* cidx, int* hist, int c, int K, int target,
                                              uint32_t kmin, uint32_t kmax) {
  const int lane = threadIdx.x & 63;
  const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  const uint32_t diff = kmin ^ kmax;
  int shift = diff ? 32 - __clz(diff) : 0;  // bits below `shift` are still undecided
  // the decided bits: key & hmask == pbits (hmask = 0 while shift == 32)
  uint32_t hmask = shift >= 32 ? 0u : (~0u << shift);
  uint32_t pbits = kmin & hmask;
  int rem = K;           // slots left among keys matching the decided bits
  bool keep_eq = false;  // keep every matching key (no tie cut needed)
  const int nb = (c + 255) >> 8;  // 256-key batches (wave-uniform)
  while (shift > 0) {
    const int w = shift >= 8 ? 8 : shift;
    const int lo = shift - w;
    const uint32_t dmask = (1u << w) - 1u;
    *reinterpret_cast<int4*>(&hist[4 * lane]) = make_int4(0, 0, 0, 0);
    CSA_WAVE_FENCE();
    uint4 kn = 4 * lane < c ? *reinterpret_cast<const uint4*>(&ckey[4 * lane]) : make_uint4(0, 0, 0, 0);
    for (int jb = 0; jb < nb; ++jb) {
      const int base = 4 * (lane + 64 * jb);
      const uint32_t kk[4] = {kn.x, kn.y, kn.z, kn.w};
      if (base + 256 < c) kn = *reinterpret_cast<const uint4*>(&ckey[base + 256]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool m = base + u < c && (kk[u] & hmask) == pbits;
        atomicAdd(&hist[(kk[u] >> lo) & dmask], m ? 1 : 0);
      }
    }
    CSA_WAVE_FENCE();
    // lane l holds digits 255-4l .. 252-4l (top digits first)
    const int4 h4 = *reinterpret_cast<const int4*>(&hist[252 - 4 * lane]);
    const int cnt[4] = {h4.w, h4.z, h4.y, h4.x};
    const int sum = cnt[0] + cnt[1] + cnt[2] + cnt[3];
    int above = wave_excl_scan(sum);
    int sel = -1, sel_above = 0, sel_cnt = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (sel < 0 && cnt[j] > 0 && above < rem && rem <= above + cnt[j]) {
        sel = 255 - 4 * lane - j;
        sel_above = above;
        sel_cnt = cnt[j];
      }
      above += cnt[j];
    }
    const uint64_t who = __ballot(sel >= 0);
    const int src = __ffsll((unsigned long long)who) - 1;  // wave-uniform
    sel = __builtin_amdgcn_readlane(sel, src);
    sel_above = __builtin_amdgcn_readlane(sel_above, src);
    sel_cnt = __builtin_amdgcn_readlane(sel_cnt, src);
    rem -= sel_above;
    pbits |= (uint32_t)sel << lo;
    hmask = ~0u << lo;
    if (lo == 0) hmask = ~0u;
    shift = lo;
    CSA_WAVE_FENCE();
    if (sel_cnt == rem || (!EXACT && K - rem + sel_cnt <= target)) {
      keep_eq = true;
      break;
    }
  }
  if (shift == 0) hmask = ~0u;
  // stable in-place compaction; track the smallest kept key.  A batch's kept entries
  // land below the batch's end, so the next batch, read before they are stored, is
  // still intact.
  int out = 0, eq_seen = 0;
  uint32_t nmin = 0xffffffffu;
  uint4 kn = make_uint4(0, 0, 0, 0);
  int4 in4 = make_int4(0, 0, 0, 0);
  if (4 * lane < c) {
    kn = *reinterpret_cast<const uint4*>(&ckey[4 * lane]);
    in4 = *reinterpret_cast<const int4*>(&cidx[4 * lane]);
  }
  for (int jb = 0; jb < nb; ++jb) {
    const int base = 4 * (lane + 64 * jb);
    const uint32_t kk[4] = {kn.x, kn.y, kn.z, kn.w};
    const int ii[4] = {in4.x, in4.y, in4.z, in4.w};
    if (base + 256 < c) {
      kn = *reinterpret_cast<const uint4*>(&ckey[base + 256]);
      in4 = *reinterpret_cast<const int4*>(&cidx[base + 256]);
    }
    bool gt[4], eq[4];
    uint64_t be[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool valid = base + u < c;
      const uint32_t hk = kk[u] & hmask;
      gt[u] = valid && hk > pbits;
      eq[u] = valid && hk == pbits;
      be[u] = __ballot(eq[u]);
    }
    // rank among equal keys in buffer order: lanes below, then this lane's earlier slots
    int eq_rank = eq_seen;
#pragma unroll
    for (int u = 0; u < 4; ++u) eq_rank += __popcll(be[u] & lt);
    bool keep[4];
    uint64_t bk[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      keep[u] = gt[u] || (eq[u] && (keep_eq || eq_rank < rem));
      eq_rank += eq[u] ? 1 : 0;
      bk[u] = __ballot(keep[u]);
    }
    int pos = out;
#pragma unroll
    for (int u = 0; u < 4; ++u) pos += __popcll(bk[u] & lt);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (keep[u]) {
        ckey[pos] = kk[u];
        cidx[pos] = ii[u];
        nmin = min(nmin, kk[u]);
        ++pos;
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      out += __popcll(bk[u]);
      eq_seen += __popcll(be[u]);
    }
  }
  CSA_WAVE_FENCE();
  Pruned r;
  r.c = out;
  // keep_eq: every kept key is >= pbits and at least K of them are kept, so a later key
  // below pbits is beaten K times.  Otherwise the kept set is exactly the top K and a
  // later key equal to the smallest kept one loses on index.
  r.kept_min = wave_min(nmin);
  r.theta = (keep_eq && out > K) ? (pbits ? pbits - 1u : 0u) : r.kept_min;
  return r;
}

template <typename T, int DI, bool PRO, bool F8>
__global__ __launch_bounds__(FT_WAVES * 64) void index_topk_kernel(IndexTopkArgs a) {
  using SH = FtShape<T, DI, F8>;
  constexpr int KK = F8 ? DI / 64 : 1;  // fp8 k-steps of 64
  constexpr int KS = DI / 16;
  constexpr int HB = 2;
  constexpr int CAP = SH::CAP;
  // two blocks admitted per step (see admit_pair) except with fp32 query fragments
  constexpr bool PAIR = sizeof(T) == 2 || F8;
  // three distinct arrays, so the compiler can tell a stage being read from the
  // stages that DMA writes are still in flight to
  __shared__ __attribute__((aligned(1024))) unsigned char st0[SH::STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char st1[SH::STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char st2[SH::STAGE];
  __shared__ __attribute__((aligned(16))) uint32_t ckey[FT_WAVES][CAP];
  __shared__ __attribute__((aligned(16))) int cidx[FT_WAVES][CAP];
  __shared__ __attribute__((aligned(16))) int hist[FT_WAVES][256];
  __shared__ int vote;  // latest tile at which some wave asked for a prune (LDS max)

  // latest (heaviest) query blocks first
  const int id = a.B * a.qblocks - 1 - (int)blockIdx.x;
  const int b = id / a.qblocks;
  const int qb = id % a.qblocks;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: SGPR arithmetic
  const int g = lane >> 5;
  const int l32 = lane & 31;
  const int t = qb * FT_WAVES + wave;
  const bool q_ok = t < a.S;
  const int n_t = q_ok ? visible_entries(t, a.ratio) : 0;
  const int n_blk = visible_entries(min(qb * FT_WAVES + FT_WAVES - 1, a.S - 1), a.ratio);
  const int K = a.topk;
  const bool select_all = n_t <= K;

  Frag<T> qa[HB][KS];
  i32x8 q8[HB][KK];  // E4M3 codes (F8)
  float w[HB][16];
  const T* qrow = static_cast<const T*>(a.q_idx) + ((int64_t)b * a.S + t) * a.HI * DI;
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const int h = hb * 32 + l32;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (q_ok && h < a.HI) qa[hb][ks] = load_frag(qrow + (int64_t)h * DI + ks * 16 + g * 8);
      else {
#pragma unroll
        for (int i = 0; i < 8; ++i) qa[hb][ks].v[i] = from_f32<T>(0.f);
      }
    }
  }
  if constexpr (!PRO && !F8) {
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      // accumulator element 4j+i is head hb*32 + 8j + 4g + i
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int hh = hb * 32 + 8 * j + 4 * g + i;
          w[hb][4 * j + i] = (q_ok && hh < a.HI) ? a.w_idx[((int64_t)b * a.S + t) * a.HI + hh] : 0.f;
        }
    }
  } else {
    // With the prologue or fp8 operands the head weights go straight to LDS (this
    // wave's index buffer, unused until the first tile): their latency overlaps the q
    // loads and no register holds them while the query is transformed.  Lane l copies w[h = min(l, HI-1)];
    // heads past HI are zeroed when read back.
    const float* wrow = wave_uniform(a.w_idx + ((int64_t)b * a.S + min(t, a.S - 1)) * a.HI);
    const uint32_t voff = (uint32_t)min(lane, a.HI - 1) * 4u;
    const uint32_t lds = (uint32_t)(uintptr_t)(CSA_LDS int*)cidx[wave];
    asm volatile("s_nop 4\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(wrow), "{m0}"(lds) : "memory");
  }

  // Stage layout: row r at r * ROWP, chunk c of the row at slot r * SPR + c; the DMA
  // line L of a stage covers slots 64L .. 64L+63, one per lane.  A lane's row and
  // chunk do not depend on the tile, so they are worked out once.  Only waves 0..3 (one
  // on each SIMD) copy: each stalls at the copy issue while the texture path drains the
  // tile's lines, and meanwhile the other wave of its SIMD (4..7) is already multiplying
  // (7.21 -> 7.04 ms at S=65536 against every wave copying its share).
  const unsigned char* kbase =
      static_cast<const unsigned char*>(a.k_idx) + (int64_t)b * a.n_entries * SH::ROWB;
  int dma_row[SH::LPW], dma_off[SH::LPW];
  uint32_t lane_off[SH::LPW];  // the lane's byte offset within a tile's rows
#pragma unroll
  for (int j = 0; j < SH::LPW; ++j) {
    const int slot = (wave + j * FT_COPIERS) * 64 + lane;
    const int ch = slot % SH::SPR;
    dma_row[j] = slot / SH::SPR;
    dma_off[j] = ch < SH::CPR ? ch * 16 : 0;  // a pad slot reloads chunk 0
    lane_off[j] = (uint32_t)dma_row[j] * SH::ROWB + dma_off[j];
  }
  // Copies of tile `tile`, written in assembly (the compiler adds no conservative waits
  // for the LDS writes; the waits are the explicit vmcnt waits before each tile's
  // barrier).  A vector-memory instruction may read an SGPR only 5 wait states after a
  // VALU instruction wrote it (v_readfirstlane, or v_readlane restoring a spilled SGPR),
  // and the compiler pads for its own instructions but not for assembly: s_nop 4.  A
  // tile wholly inside the visible entries takes its row base in the scalar address
  // (scalar arithmetic) and the lane's fixed offset; the last tile clamps each row past
  // the end to a valid one.
  auto issue = [&](int tile, unsigned char* st) {
    const bool whole = (tile + 1) * FT_TILE <= n_blk;  // wave-uniform
    const unsigned char* tbase = kbase + (int64_t)tile * FT_TILE * SH::ROWB;
#pragma unroll
    for (int j = 0; j < SH::LPW; ++j) {
      const int L = wave + j * FT_COPIERS;
      if (wave < FT_COPIERS && L < SH::NI) {  // wave-uniform
        const uint32_t lds = (uint32_t)(uintptr_t)(CSA_LDS unsigned char*)(st + L * 1024);
        if (whole) {
          asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(lane_off[j]), "s"(tbase), "{m0}"(lds) : "memory");
        } else {
          const int row = min(tile * FT_TILE + dma_row[j], n_blk - 1);  // past the end: a valid row
          const uint32_t voff = (uint32_t)row * SH::ROWB + dma_off[j];
          asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(kbase), "{m0}"(lds) : "memory");
        }
      }
    }
  };
  // B fragment of block nb, k-step ks: row nb*32 + l32, elements ks*16 + 8g .. +7
  auto frag = [&](const unsigned char* st, int nb, int ks) -> Frag<T> {
    const CSA_LDS unsigned char* p = (const CSA_LDS unsigned char*)st + (nb * 32 + l32) * SH::ROWP +
                                     (ks * 16 + g * 8) * (int)sizeof(T);
    Frag<T> f;
    *reinterpret_cast<u32x4*>(f.v) = *(const CSA_LDS u32x4*)p;
    if constexpr (sizeof(T) == 4) *reinterpret_cast<u32x4*>(f.v + 4) = *(const CSA_LDS u32x4*)(p + 16);
    return f;
  };
  // The fragment reads run two k-steps ahead of the MFMAs that consume them, so the
  // LDS latency hides behind the matrix work of the same wave.
  constexpr int LA = KS < 3 ? KS : 3;
  // fp8: B fragment of block nb, k-step kk: 32 codes of row nb*32 + l32 at byte
  // 64kk + 32g (two 16-byte reads); the row's scale sits at byte DI.
  auto frag8 = [&](const unsigned char* st, int nb, int kk) -> i32x8 {
    const CSA_LDS unsigned char* p = (const CSA_LDS unsigned char*)st + (nb * 32 + l32) * SH::ROWP + kk * 64 + g * 32;
    const u32x4 lo4 = *(const CSA_LDS u32x4*)p, hi4 = *(const CSA_LDS u32x4*)(p + 16);
    i32x8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r[i] = (int)lo4[i];
      r[4 + i] = (int)hi4[i];
    }
    return r;
  };
  auto mfma_block8 = [&](const unsigned char* st, int nb, f32x16* acc, float& sk) {
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[hb][i] = 0.f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const i32x8 kb = frag8(st, nb, kk);
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) acc[hb] = mfma32x32x64_fp8(q8[hb][kk], kb, acc[hb]);
    }
    sk = __uint_as_float(*(const CSA_LDS uint32_t*)((const CSA_LDS unsigned char*)st + (nb * 32 + l32) * SH::ROWP + DI));
  };
  auto mfma_block = [&](const unsigned char* st, int nb, f32x16* acc) {
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[hb][i] = 0.f;
    Frag<T> kb[LA];
#pragma unroll
    for (int ks = 0; ks < LA - 1; ++ks) kb[ks] = frag(st, nb, ks);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + LA - 1 < KS) kb[(ks + LA - 1) % LA] = frag(st, nb, ks + LA - 1);
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) acc[hb] = mfma32x32x16(qa[hb][ks], kb[ks % LA], acc[hb]);
    }
  };

  uint32_t* my_key = ckey[wave];
  int* my_idx = cidx[wave];
  int* my_hist = hist[wave];
  uint32_t theta = 0u;                      // admit keys strictly above
  // Bounds of the buffered keys for the radix select: the smallest key kept by the
  // last prune, and per lane the smallest and largest key admitted since (largest:
  // ever).  Tight bounds make the first radix digit discriminate.
  uint32_t kept_lo = 0xffffffffu, kmn_l = 0xffffffffu, kmax_l = 0u;
  int c = 0;

  // ReLU(.) * w summed over the lane's 16 heads of a block (four independent partial
  // sums); the two lane halves hold the two 16-head halves of each entry.
  auto partial = [&](const f32x16* acc) -> float {
    float v4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
      for (int i = 0; i < 16; ++i) v4[i & 3] = fmaf(w[hb][i], relu(acc[hb][i]), v4[i & 3]);
    return (v4[0] + v4[1]) + (v4[2] + v4[3]);
  };
  // Admit two blocks at once: vlo holds the partials of entries elo + 0..31, vhi those
  // of ehi + 0..31 (elo's block comes first in entry order).  One v_permlane32_swap
  // gives the low lanes vlo's two halves and the high lanes vhi's, so lane l scores
  // entry elo + l (l < 32) or ehi + l - 32 and the key and admission bookkeeping run
  // once for 64 entries, in entry order across the lanes.
  // One block alone (fp32 activations without fp8, whose query fragments leave no
  // registers for the paired order): the two lane halves' sums meet in both halves
  // and the low half admits.
  auto admit_one = [&](float v, int eb, float sk) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    float s = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    if constexpr (F8) s *= sk;
    const int e = eb + l32;
    const uint32_t key = score_key(s);
    const bool admit = g == 0 && e >= 0 && e < n_t && key > theta;
    const uint64_t bm = __ballot(admit);
    const int nadm = __popcll(bm);
    const int pos = c + (admit ? (int)__builtin_amdgcn_mbcnt_lo((uint32_t)bm, 0u) : nadm);
    my_key[pos] = key;
    my_idx[pos] = e;
    kmax_l = admit ? max(kmax_l, key) : kmax_l;
    kmn_l = admit ? min(kmn_l, key) : kmn_l;
    c += nadm;
  };
  auto admit_pair = [&](float vlo, float vhi, int elo, int ehi, float sklo, float skhi) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(vlo), __float_as_uint(vhi), false, false);
    float s = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    if constexpr (F8) s *= g ? skhi : sklo;  // the entry's scale (sq is folded into w)
    const int e = (g ? ehi : elo) + l32;
    const uint32_t key = score_key(s);
    const bool admit = e >= 0 && e < n_t && key > theta;
    const uint64_t bm = __ballot(admit);
    const int nadm = __popcll(bm);
    // branch-free append: an admitted lane writes after the admitted lanes below it;
    // refused lanes all write the first free slot (c + 64 < CAP holds here, see
    // make_room)
    const int below = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bm, 0u));
    const int pos = c + (admit ? below : nadm);
    my_key[pos] = key;
    my_idx[pos] = e;
    kmax_l = admit ? max(kmax_l, key) : kmax_l;
    kmn_l = admit ? min(kmn_l, key) : kmn_l;
    c += nadm;
  };

  const int ntiles = (n_blk + FT_TILE - 1) / FT_TILE;
  wait_vmcnt<0, false>();  // q and w have arrived before any copy is counted
  if (ntiles > 0) issue(0, st0);
  if (ntiles > 1) issue(1, st1);
  if constexpr (PRO || F8) {
    // the query transforms run while the first two tiles are in flight.  (a.pro.on /
    // a.pro.fp8 are always set in these instances; the runtime tests keep the compiler
    // from folding the fragment loads into the transforms, which takes 40-140 more
    // VGPRs.)
    if constexpr (PRO)
      if (a.pro.on) index_query_prologue<T, DI>(qa, a.pro.pos0 + t, a.pro.rope_dim, a.pro.theta, ckey[wave]);
    if constexpr (F8)
      if (a.pro.fp8) index_query_fp8<T, DI>(qa, q8, ckey[wave]);  // head scales -> ckey[wave][0..63]
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 v = *(const CSA_LDS f32x4*)((CSA_LDS int*)cidx[wave] + hb * 32 + 8 * j + 4 * g);
        f32x4 sq = {1.f, 1.f, 1.f, 1.f};
        if constexpr (F8) sq = *(const CSA_LDS f32x4*)((CSA_LDS uint32_t*)ckey[wave] + hb * 32 + 8 * j + 4 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int hh = hb * 32 + 8 * j + 4 * g + i;
          // The prologue's temperature is left out here: it scales every score of the
          // query by one positive constant, which leaves the top-k unchanged, and this
          // kernel writes only the selection.  (The selection's work depends on the
          // scores' bit patterns: at C3 a scale of 1/90.5 costs 0.5 ms more than any
          // power of two.)  index_scores_kernel, whose scores are its output, applies it.
          float wv = v[i];
          if constexpr (F8) wv *= sq[i];
          w[hb][4 * j + i] = (q_ok && hh < a.HI) ? wv : 0.f;
        }
      }
  }

  // Prune when fewer than `need` + 1 slots are free (each admission step admits up to
  // 64 keys and may write one spare slot past them), or, with `early`, once the buffer
  // is more than half way from K to full.  A prune stalls the whole workgroup at the
  // next barrier, so the waves announce an upcoming prune two tiles ahead (vote) and
  // then prune together: the stalls overlap instead of adding up.
  constexpr int PRUNE_EARLY = (FT_MAXK + CAP) / 2;
  auto make_room = [&](int need, bool early) __attribute__((always_inline)) {
    if (c > CAP - need - 1 || (early && c > max(K, PRUNE_EARLY))) {
      CSA_WAVE_FENCE();
      const Pruned pr = wave_select<false>(my_key, my_idx, my_hist, c, K, (K + CAP) / 2,
                                           min(kept_lo, wave_min(kmn_l)), wave_max(kmax_l));
      c = pr.c;
      theta = pr.theta;
      kept_lo = pr.kept_min;
      kmn_l = 0xffffffffu;
    }
  };

  f32x16 accA[HB], accB[HB];
  float skA = 0.f, skB = 0.f;  // fp8: scales of the entries of the blocks in accA / accB
#pragma unroll
  for (int hb = 0; hb < HB; ++hb)
#pragma unroll
    for (int i = 0; i < 16; ++i) accB[hb][i] = 0.f;
  // One tile: wait for its stage, refill the stage read two tiles ago, then
  // MFMA(block 0) | partial sums of block 1 of the previous tile | MFMA(block 1) |
  // partial sums of block 0, and both blocks admitted together.  Blocks past n_t are
  // multiplied too (their rows are valid data) and refused by the admission mask; at
  // it == 0 there is no previous block (its entries are negative).
  // The votes are read after a tile's barrier and acted on at the next tile, so the
  // read's latency hides behind this tile's copies and products: a vote cast at the end
  // of tile it-1 prunes every wave at tile it+1.
  if (threadIdx.x == 0) vote = -4;
  int vseen = -4;
  auto step = [&](int it, const unsigned char* cur, unsigned char* refill) {
    // A copying wave issues floor(NI/4) or ceil(NI/4) copies a tile, in order: with at
    // most floor(NI/4) left in flight, all of this tile's have landed.
    if (it + 1 < ntiles) wait_vmcnt<SH::NI / FT_COPIERS, false>();
    else wait_vmcnt<0, false>();
    lds_only_barrier();
    // prune before the refill is issued: the prune's LDS atomics wait for every copy in
    // flight, and the older one has likely landed
    if (!select_all) make_room(64, vseen >= it - 2);
    if (it + 2 < ntiles) issue(it + 2, refill);
    if (select_all) return;
    const int vnow = vote;
    const int e0 = it * FT_TILE;
    if constexpr (PAIR) {
      if constexpr (F8) mfma_block8(cur, 0, accA, skA);
      else mfma_block(cur, 0, accA);
      const float vb = partial(accB);
      const float skb = skB;
      if constexpr (F8) mfma_block8(cur, 1, accB, skB);
      else mfma_block(cur, 1, accB);
      admit_pair(vb, partial(accA), e0 - 32, e0, skb, skA);
    } else {
      mfma_block(cur, 0, accA);
      admit_one(partial(accB), e0 - 32, 0.f);
      mfma_block(cur, 1, accB);
      admit_one(partial(accA), e0, 0.f);
    }
    vseen = vnow;
    // three more tiles could fill the buffer: ask every wave to prune (two tiles on)
    if (c > CAP - 4 * FT_TILE - 1 && lane == 0) atomicMax(&vote, it);
  };
  for (int it = 0; it < ntiles; it += 3) {
    step(it, st0, st2);
    if (it + 1 < ntiles) step(it + 1, st1, st0);
    if (it + 2 < ntiles) step(it + 2, st2, st1);
  }
  if (!select_all && ntiles > 0) {  // block 1 of the last tile, alone (the high lanes' entries are negative)
    make_room(64, false);
    if constexpr (PAIR) admit_pair(partial(accB), 0.f, ntiles * FT_TILE - 32, -64, skB, 0.f);
    else admit_one(partial(accB), ntiles * FT_TILE - 32, 0.f);
  }

  if (!q_ok) return;
  int32_t* out = a.idx + ((int64_t)b * a.S + t) * K;
  if (lane == 0 && a.n_visible) a.n_visible[(int64_t)b * a.S + t] = n_t;
  if (select_all) {
    for (int j = lane; j < K; j += 64) out[j] = j < n_t ? j : -1;
    return;
  }
  CSA_WAVE_FENCE();
  if (c > K) wave_select<true>(my_key, my_idx, my_hist, c, K, K, min(kept_lo, wave_min(kmn_l)), wave_max(kmax_l));
  for (int j = lane; j < K; j += 64) out[j] = my_idx[j];
}

// ---------------------------------------------------------------------------------
// Indexer key pass, for the prologue and/or fp8 operands: k'[s] = round(Hn RoPE(k_I[s],
// pos0 + s*ratio)) ("fix(deepseek-v4): correct V4-Flash attention math", Part 1 item
// 6e: keys rotate at s * compress_ratio), then, with fp8, the row's E4M3 codes in the
// MFMA k-slot order and its fp32 scale (DI + 16 bytes a row).  DI/2 lanes per row, each
// holding the pair of dims (2j, 2j+1): the Hadamard's dim bit 0 is within the lane and
// bits 1.. are lane bits of the row's group, exchanged by shuffles, as is the row's
// maximum.  Streaming, HBM-bound.
// ---------------------------------------------------------------------------------
struct IndexKeysArgs {
  const void* k_idx;
  void* k_out;
  int64_t rows;      // B * n_entries
  int32_t n_entries, ratio;
  IndexPrologue pro;
};

constexpr int IK_THREADS = 256;

template <typename T, int DI, bool PRO, bool F8>
__global__ __launch_bounds__(IK_THREADS) void index_keys_kernel(IndexKeysArgs a) {
  constexpr int LPR = DI / 2;  // lanes per row (divides 64)
  const int64_t gid = (int64_t)blockIdx.x * IK_THREADS + threadIdx.x;
  const int64_t row = gid / LPR;
  const int j = (int)(gid % LPR);
  const bool ok = row < a.rows;
  float x0 = 0.f, x1 = 0.f;
  const T* src = static_cast<const T*>(a.k_idx) + row * DI + 2 * j;
  if (ok) {
    x0 = to_f32(src[0]);
    x1 = to_f32(src[1]);
  }
  if constexpr (PRO) {
    const int R = a.pro.rope_dim;
    const int lo = DI - R;
    if (ok && 2 * j >= lo) {
      const int s = (int)(row % a.n_entries);
      float c, sn;
      rope_cos_sin(entry_position(a.pro.pos0, s, a.ratio), rope_inv_freq((2 * j - lo) >> 1, R, a.pro.theta), &c, &sn);
      const float r0 = x0 * c - x1 * sn, r1 = x0 * sn + x1 * c;
      x0 = r0;
      x1 = r1;
    }
    float h0 = x0 + x1, h1 = x0 - x1;  // dim bit 0
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) {  // dim bit k = lane bit k-1
      const float sg = (j & m) ? -1.f : 1.f;
      h0 = fmaf(sg, h0, __shfl_xor(h0, m, 64));
      h1 = fmaf(sg, h1, __shfl_xor(h1, m, 64));
    }
    const float scale = 1.0f / __builtin_sqrtf((float)DI);
    x0 = to_f32(from_f32<T>(h0 * scale));  // the prologue's output is in the activation dtype
    x1 = to_f32(from_f32<T>(h1 * scale));
  }
  if constexpr (!F8) {
    if (ok) {
      T* dst = static_cast<T*>(a.k_out) + row * DI + 2 * j;
      dst[0] = from_f32<T>(x0);
      dst[1] = from_f32<T>(x1);
    }
  } else {
    float m = fmaxf(fabsf(x0), fabsf(x1));
#pragma unroll
    for (int k = 1; k < LPR; k <<= 1) m = fmaxf(m, __shfl_xor(m, k, 64));
    const float inv = m > 0.f ? kE4M3Max / m : 0.f;
    if (ok) {
      unsigned char* dst = static_cast<unsigned char*>(a.k_out) + row * (DI + 16);
      const int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0 * inv, x1 * inv, 0, false);
      *reinterpret_cast<uint16_t*>(dst + key_fp8_pos(2 * j)) = (uint16_t)(w & 0xffff);
      if (j == 0) *reinterpret_cast<uint4*>(dst + DI) = make_uint4(__float_as_uint(m / kE4M3Max), 0u, 0u, 0u);
    }
  }
}

hipError_t launch_index_keys(const csa_params_t& p, const void* k_idx, void* k_out, hipStream_t st) {
  IndexKeysArgs a{k_idx, k_out, (int64_t)p.B * (p.S / p.ratio), p.S / p.ratio, p.ratio, index_prologue_args(p)};
  if (a.rows == 0) return hipSuccess;
  const bool pro = (p.flags & CSA_FLAG_INDEX_PROLOGUE) != 0, f8 = (p.flags & CSA_FLAG_INDEX_FP8) != 0;
  if (!pro && !f8) return hipErrorInvalidValue;
  if (f8 && p.idx_dim != 64 && p.idx_dim != 128) return hipErrorInvalidValue;
  const int64_t threads = a.rows * (p.idx_dim / 2);
  const dim3 grid((unsigned)((threads + IK_THREADS - 1) / IK_THREADS));
#define CSA_IK_LAUNCH(T, DI, PRO, F8) hipLaunchKernelGGL((index_keys_kernel<T, DI, PRO, F8>), grid, dim3(IK_THREADS), 0, st, a)
#define CSA_IK_CASE(T, DI)                      \
  do {                                          \
    if (!f8) CSA_IK_LAUNCH(T, DI, true, false); \
    else if (pro) CSA_IK_LAUNCH(T, DI, true, true); \
    else CSA_IK_LAUNCH(T, DI, false, true);     \
  } while (0)
#define CSA_IK_CASE_NO8(T, DI) CSA_IK_LAUNCH(T, DI, true, false)
  const bool bf = p.dtype == CSA_BF16;
  switch (p.idx_dim) {
    case 16: if (bf) CSA_IK_CASE_NO8(bf16, 16); else CSA_IK_CASE_NO8(float, 16); break;
    case 32: if (bf) CSA_IK_CASE_NO8(bf16, 32); else CSA_IK_CASE_NO8(float, 32); break;
    case 64: if (bf) CSA_IK_CASE(bf16, 64); else CSA_IK_CASE(float, 64); break;
    case 128: if (bf) CSA_IK_CASE(bf16, 128); else CSA_IK_CASE(float, 128); break;
    default: return hipErrorInvalidValue;
  }
#undef CSA_IK_CASE
#undef CSA_IK_CASE_NO8
#undef CSA_IK_LAUNCH
  return hipGetLastError();
}

hipError_t launch_index_topk(const csa_params_t& p, const void* q_idx, const float* w_idx,
                             const void* k_idx, int32_t* idx, int32_t* n_visible, hipStream_t st) {
  if (p.topk > FT_MAXK) return hipErrorInvalidValue;
  IndexTopkArgs a{q_idx, w_idx, k_idx, idx, n_visible, p.B, p.S, p.idx_heads, p.ratio,
                  p.S / p.ratio, p.topk, (p.S + FT_WAVES - 1) / FT_WAVES, index_prologue_args(p)};
  const int grid = p.B * a.qblocks;
  if (grid == 0) return hipSuccess;
  if (a.pro.fp8 && p.idx_dim != 64 && p.idx_dim != 128) return hipErrorInvalidValue;
#define CSA_FT_LAUNCH(T, DI, PRO, F8) \
  hipLaunchKernelGGL((index_topk_kernel<T, DI, PRO, F8>), dim3(grid), dim3(FT_WAVES * 64), 0, st, a)
#define CSA_FT_CASE(T, DI)                          \
  do {                                              \
    if (a.pro.fp8) {                                \
      if (a.pro.on) CSA_FT_LAUNCH(T, DI, true, true); \
      else CSA_FT_LAUNCH(T, DI, false, true);       \
    } else if (a.pro.on) CSA_FT_LAUNCH(T, DI, true, false); \
    else CSA_FT_LAUNCH(T, DI, false, false);        \
  } while (0)
#define CSA_FT_CASE_NO8(T, DI)                      \
  do {                                              \
    if (a.pro.on) CSA_FT_LAUNCH(T, DI, true, false); \
    else CSA_FT_LAUNCH(T, DI, false, false);        \
  } while (0)
  const bool bf = p.dtype == CSA_BF16;
  switch (p.idx_dim) {
    case 16: if (bf) CSA_FT_CASE_NO8(bf16, 16); else CSA_FT_CASE_NO8(float, 16); break;
    case 32: if (bf) CSA_FT_CASE_NO8(bf16, 32); else CSA_FT_CASE_NO8(float, 32); break;
    case 64: if (bf) CSA_FT_CASE(bf16, 64); else CSA_FT_CASE(float, 64); break;
    case 128: if (bf) CSA_FT_CASE(bf16, 128); else CSA_FT_CASE(float, 128); break;
    default: return hipErrorInvalidValue;
  }
#undef CSA_FT_CASE
#undef CSA_FT_CASE_NO8
#undef CSA_FT_LAUNCH
  return hipGetLastError();
}

hipError_t launch_index_scores(const csa_params_t& p, const void* q_idx, const float* w_idx,
                               const void* k_idx, float* scores, int64_t ld, int32_t t0,
                               int32_t nrows, hipStream_t st) {
  IndexArgs a{};
  a.q_idx = q_idx;
  a.w_idx = w_idx;
  a.k_idx = k_idx;
  a.scores = scores;
  a.ld = ld;
  a.B = p.B;
  a.S = p.S;
  a.HI = p.idx_heads;
  a.ratio = p.ratio;
  a.n_entries = p.S / p.ratio;
  a.t0 = t0;
  a.nrows = nrows;
  a.qblocks = (nrows + IDX_WAVES - 1) / IDX_WAVES;
  a.pro = index_prologue_args(p);
  const int n_max = visible_entries(t0 + nrows - 1, p.ratio);
  a.n_chunks = (n_max + IDX_CHUNK - 1) / IDX_CHUNK;
  if (a.n_chunks == 0 || nrows == 0) return hipSuccess;
  if (a.n_chunks > IDX_MAX_CHUNKS) return hipErrorInvalidValue;
  int off = 0;
  for (int c = 0; c < a.n_chunks; ++c) {
    // first query block whose last row sees entry c*CHUNK: visible_entries(t) > c*CHUNK
    int qmin = 0;
    const int need_t = (c * IDX_CHUNK + 1) * p.ratio - 1;  // smallest t with n_t > c*CHUNK
    if (need_t > t0) {
      const int rel = need_t - t0;                         // row index relative to t0
      qmin = rel / IDX_WAVES;                              // block containing that row
    }
    a.chunk_qb_min[c] = qmin;
    a.chunk_wg_off[c] = off;
    off += p.B * (a.qblocks - qmin);
  }
  a.chunk_wg_off[a.n_chunks] = off;
  if (off == 0) return hipSuccess;
  dim3 grid(off), block(IDX_WAVES * 64);
  if (a.pro.fp8 && p.idx_dim != 64 && p.idx_dim != 128) return hipErrorInvalidValue;
#define CSA_IDX_LAUNCH(T, DI, PRO, F8) hipLaunchKernelGGL((index_scores_kernel<T, DI, PRO, F8>), grid, block, 0, st, a)
#define CSA_IDX_CASE(T, DI)                          \
  do {                                               \
    if (a.pro.fp8) {                                 \
      if (a.pro.on) CSA_IDX_LAUNCH(T, DI, true, true); \
      else CSA_IDX_LAUNCH(T, DI, false, true);       \
    } else if (a.pro.on) CSA_IDX_LAUNCH(T, DI, true, false); \
    else CSA_IDX_LAUNCH(T, DI, false, false);        \
  } while (0)
#define CSA_IDX_CASE_NO8(T, DI)                      \
  do {                                               \
    if (a.pro.on) CSA_IDX_LAUNCH(T, DI, true, false); \
    else CSA_IDX_LAUNCH(T, DI, false, false);        \
  } while (0)
  const bool bf = p.dtype == CSA_BF16;
  switch (p.idx_dim) {
    case 16: if (bf) CSA_IDX_CASE_NO8(bf16, 16); else CSA_IDX_CASE_NO8(float, 16); break;
    case 32: if (bf) CSA_IDX_CASE_NO8(bf16, 32); else CSA_IDX_CASE_NO8(float, 32); break;
    case 64: if (bf) CSA_IDX_CASE(bf16, 64); else CSA_IDX_CASE(float, 64); break;
    case 128: if (bf) CSA_IDX_CASE(bf16, 128); else CSA_IDX_CASE(float, 128); break;
    default: return hipErrorInvalidValue;
  }
#undef CSA_IDX_CASE
#undef CSA_IDX_CASE_NO8
#undef CSA_IDX_LAUNCH
  return hipGetLastError();
}

}  // namespace csa
