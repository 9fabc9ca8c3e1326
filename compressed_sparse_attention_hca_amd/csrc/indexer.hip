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

struct IndexArgs {
  const void* q_idx;
  const float* w_idx;
  const void* k_idx;
  float* scores;
  int64_t ld;
  int32_t B, S, HI, ratio, n_entries, t0, nrows, qblocks;  // qblocks per batch
  int32_t n_chunks;
  int32_t chunk_wg_off[IDX_MAX_CHUNKS + 1];  // prefix sums of workgroups per chunk
  int32_t chunk_qb_min[IDX_MAX_CHUNKS];      // first query block that needs the chunk
};

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

template <typename T, int DI>
__global__ __launch_bounds__(IDX_WAVES * 64) void index_scores_kernel(IndexArgs a) {
  constexpr int KS = DI / 16;                    // k-steps of 16
  constexpr int VEC = 16 / sizeof(T);            // elements per 16-byte load
  constexpr int ROW = DI + 16 / sizeof(T);       // padded LDS row (elements)
  constexpr int HB = 2;                          // head blocks of 32 (up to 64 heads)
  __shared__ __attribute__((aligned(16))) T tile[2][IDX_TILE * ROW];

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
    // accumulator element 4j+i is head hb*32 + 8j + 4g + i
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hh = hb * 32 + 8 * j + 4 * g + i;
        w[hb][4 * j + i] = (q_ok && hh < a.HI) ? a.w_idx[((int64_t)b * a.S + t) * a.HI + hh] : 0.f;
      }
  }

  const T* kbase = static_cast<const T*>(a.k_idx) + (int64_t)b * a.n_entries * DI;
  // k_I tiles go global -> registers -> LDS; the next tile's loads are in flight
  // while the current tile is multiplied.
  constexpr int NT = IDX_WAVES * 64;
  constexpr int CHUNKS_PER_TILE = IDX_TILE * DI / VEC;   // 16-byte pieces per tile
  constexpr int PER_THREAD = (CHUNKS_PER_TILE + NT - 1) / NT;
  uint4 pf[PER_THREAD];
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
    fetch(e_begin);
    commit(0);
  }
  __syncthreads();
  for (int it = 0; it < ntiles; ++it) {
    const int e0 = e_begin + it * IDX_TILE;
    if (it + 1 < ntiles) fetch(e0 + IDX_TILE);
    const T* tb = tile[it & 1];
#pragma unroll
    for (int nb = 0; nb < IDX_TILE / 32; ++nb) {
      const int eb = e0 + nb * 32;
      if (eb >= n_t) break;  // wave-uniform: n_t is per wave
      f32x16 acc[HB];
#pragma unroll
      for (int hb = 0; hb < HB; ++hb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[hb][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const Frag<T> kb = load_frag(tb + (nb * 32 + l32) * ROW + ks * 16 + g * 8);
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) acc[hb] = mfma32x32x16(qa[hb][ks], kb, acc[hb]);
      }
      float v = 0.f;
#pragma unroll
      for (int hb = 0; hb < HB; ++hb)
#pragma unroll
        for (int i = 0; i < 16; ++i) v = fmaf(w[hb][i], fmaxf(acc[hb][i], 0.f), v);
      v += __shfl_xor(v, 32, 64);
      const int e = eb + l32;
      if (g == 0 && e < n_t) srow[e] = v;
    }
    if (it + 1 < ntiles) commit((it + 1) & 1);
    __syncthreads();
  }
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
#define CSA_IDX_CASE(T, DI) hipLaunchKernelGGL((index_scores_kernel<T, DI>), grid, block, 0, st, a)
  const bool bf = p.dtype == CSA_BF16;
  switch (p.idx_dim) {
    case 16: if (bf) CSA_IDX_CASE(bf16, 16); else CSA_IDX_CASE(float, 16); break;
    case 32: if (bf) CSA_IDX_CASE(bf16, 32); else CSA_IDX_CASE(float, 32); break;
    case 64: if (bf) CSA_IDX_CASE(bf16, 64); else CSA_IDX_CASE(float, 64); break;
    case 128: if (bf) CSA_IDX_CASE(bf16, 128); else CSA_IDX_CASE(float, 128); break;
    default: return hipErrorInvalidValue;
  }
#undef CSA_IDX_CASE
  return hipGetLastError();
}

}  // namespace csa
