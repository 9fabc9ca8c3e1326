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

// ---------------------------------------------------------------------------------
// Indexer scores fused with the top-k selection (top-k up to FT_MAXK).
//
// A workgroup of 8 waves owns 8 consecutive queries of one batch and sweeps every
// visible entry, so the scores never leave the chip.  Each wave scores its query with
// the same MFMA tiles and epilogue as index_scores_kernel and keeps a streaming
// selection in LDS: a score whose order-preserving key exceeds the wave's threshold is
// appended (entries arrive in ascending order, so the buffer stays sorted by index).
// When the buffer is nearly full the wave compacts it to exactly the top-k by (key
// desc, index asc) with a wave-local radix select, and the k-th key becomes the new
// threshold.  An entry at or below the threshold has at least k entries that beat it
// (a higher key, or an equal key with a smaller index), so the final set is exact.
// ---------------------------------------------------------------------------------
constexpr int FT_WAVES = 8;
constexpr int FT_TILE = 64;
constexpr int FT_CAP = 1024;   // candidates per query
constexpr int FT_MAXK = 512;   // largest top-k of the fused path

struct IndexTopkArgs {
  const void* q_idx;
  const float* w_idx;
  const void* k_idx;
  int32_t* idx;
  int32_t* n_visible;
  int32_t B, S, HI, ratio, n_entries, topk, qblocks;  // query blocks per batch
};

__device__ inline uint32_t score_key(float f) {
  const uint32_t u = __float_as_uint(f == 0.0f ? 0.0f : f);  // -0 and +0 tie
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ inline int wave_excl_scan(int v) {
  const int lane = threadIdx.x & 63;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  return x - v;
}

#define CSA_WAVE_FENCE() __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront")

// Keep exactly the top `K` of ckey/cidx[0..c) in place (in buffer order); returns the
// k-th key.  Wave-local: every lane of the wave calls it.
__device__ inline uint32_t wave_compact(uint32_t* ckey, int* cidx, int* hist, int c, int K) {
  const int lane = threadIdx.x & 63;
  const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  // common high bits of the buffered keys
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  for (int i = lane; i < c; i += 64) {
    const uint32_t k = ckey[i];
    kmin = min(kmin, k);
    kmax = max(kmax, k);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, m, 64));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, m, 64));
  }
  const uint32_t diff = kmin ^ kmax;
  int shift = diff ? 32 - __clz(diff) : 0;
  uint64_t prefix = (uint64_t)kmin >> shift;
  int rem = K;  // slots left among keys whose bits above `shift` equal `prefix`
  while (shift > 0) {
    const int w = shift >= 8 ? 8 : shift;
    const int lo = shift - w;
#pragma unroll
    for (int j = 0; j < 4; ++j) hist[4 * lane + j] = 0;
    CSA_WAVE_FENCE();
    for (int i = lane; i < c; i += 64) {
      const uint32_t k = ckey[i];
      if (((uint64_t)k >> shift) == prefix) atomicAdd(&hist[(k >> lo) & ((1u << w) - 1u)], 1);
    }
    CSA_WAVE_FENCE();
    // lane l holds digits 255-4l .. 252-4l (top digits first)
    int cnt[4], sum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = 255 - 4 * lane - j;
      cnt[j] = d < (1 << w) ? hist[d] : 0;
      sum += cnt[j];
    }
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
    const int src = __ffsll((unsigned long long)who) - 1;
    sel = __shfl(sel, src, 64);
    sel_above = __shfl(sel_above, src, 64);
    sel_cnt = __shfl(sel_cnt, src, 64);
    rem -= sel_above;
    prefix = (prefix << w) | (uint64_t)sel;
    shift = lo;
    CSA_WAVE_FENCE();
    if (sel_cnt == rem) break;  // every key with this prefix is kept
  }
  // stable in-place compaction: key above the prefix, or equal and among the first rem
  int out = 0, eq_seen = 0;
  for (int base = 0; base < c; base += 64) {
    const int i = base + lane;
    uint32_t k = 0;
    int id = 0;
    if (i < c) {
      k = ckey[i];
      id = cidx[i];
    }
    const uint64_t kp = (uint64_t)k >> shift;
    const bool gt = i < c && kp > prefix;
    const bool eq = i < c && kp == prefix;
    const uint64_t be = __ballot(eq);
    const bool keep = gt || (eq && eq_seen + __popcll(be & lt) < rem);
    const uint64_t bk = __ballot(keep);
    CSA_WAVE_FENCE();  // all reads of this chunk precede the writes below
    if (keep) {
      const int pos = out + __popcll(bk & lt);
      ckey[pos] = k;
      cidx[pos] = id;
    }
    out += __popcll(bk);
    eq_seen += __popcll(be);
    CSA_WAVE_FENCE();
  }
  // the k-th key: smallest kept key (prefix padded with zeros bounds it from below)
  uint32_t kth = 0xffffffffu;
  for (int i = lane; i < K; i += 64) kth = min(kth, ckey[i]);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) kth = min(kth, (uint32_t)__shfl_xor((int)kth, m, 64));
  CSA_WAVE_FENCE();
  return kth;
}

template <typename T, int DI>
__global__ __launch_bounds__(FT_WAVES * 64) void index_topk_kernel(IndexTopkArgs a) {
  constexpr int KS = DI / 16;
  constexpr int VEC = 16 / sizeof(T);
  constexpr int ROW = DI + 16 / sizeof(T);
  constexpr int HB = 2;
  constexpr int NT = FT_WAVES * 64;
  constexpr int CHUNKS_PER_TILE = FT_TILE * DI / VEC;
  constexpr int PER_THREAD = (CHUNKS_PER_TILE + NT - 1) / NT;
  __shared__ __attribute__((aligned(16))) T tile[2][FT_TILE * ROW];
  __shared__ uint32_t ckey[FT_WAVES][FT_CAP];
  __shared__ int cidx[FT_WAVES][FT_CAP];
  __shared__ int hist[FT_WAVES][256];

  // latest (heaviest) query blocks first
  const int id = a.B * a.qblocks - 1 - (int)blockIdx.x;
  const int b = id / a.qblocks;
  const int qb = id % a.qblocks;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 5;
  const int l32 = lane & 31;
  const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  const int t = qb * FT_WAVES + wave;
  const bool q_ok = t < a.S;
  const int n_t = q_ok ? visible_entries(t, a.ratio) : 0;
  const int n_blk = visible_entries(min(qb * FT_WAVES + FT_WAVES - 1, a.S - 1), a.ratio);
  const int K = a.topk;
  const bool select_all = n_t <= K;

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
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hh = hb * 32 + 8 * j + 4 * g + i;
        w[hb][4 * j + i] = (q_ok && hh < a.HI) ? a.w_idx[((int64_t)b * a.S + t) * a.HI + hh] : 0.f;
      }
  }

  const T* kbase = static_cast<const T*>(a.k_idx) + (int64_t)b * a.n_entries * DI;
  uint4 pf[PER_THREAD];
  auto fetch = [&](int e0) {
#pragma unroll
    for (int k = 0; k < PER_THREAD; ++k) {
      const int cI = threadIdx.x + k * NT;
      const int row = cI / (DI / VEC);
      const int col = (cI % (DI / VEC)) * VEC;
      pf[k] = (cI < CHUNKS_PER_TILE && e0 + row < n_blk)
                  ? *reinterpret_cast<const uint4*>(kbase + (int64_t)(e0 + row) * DI + col)
                  : make_uint4(0, 0, 0, 0);
    }
  };
  auto commit = [&](int buf) {
#pragma unroll
    for (int k = 0; k < PER_THREAD; ++k) {
      const int cI = threadIdx.x + k * NT;
      if (cI < CHUNKS_PER_TILE) {
        const int row = cI / (DI / VEC);
        const int col = (cI % (DI / VEC)) * VEC;
        *reinterpret_cast<uint4*>(&tile[buf][row * ROW + col]) = pf[k];
      }
    }
  };

  uint32_t theta = 0u;  // admit keys strictly above (every real score's key is > 0)
  int c = 0;
  uint32_t* my_key = ckey[wave];
  int* my_idx = cidx[wave];
  int* my_hist = hist[wave];

  const int ntiles = (n_blk + FT_TILE - 1) / FT_TILE;
  if (ntiles > 0) {
    fetch(0);
    commit(0);
  }
  __syncthreads();
  for (int it = 0; it < ntiles; ++it) {
    const int e0 = it * FT_TILE;
    if (it + 1 < ntiles) fetch(e0 + FT_TILE);
    const T* tb = tile[it & 1];
    if (!select_all) {
#pragma unroll
      for (int nb = 0; nb < FT_TILE / 32; ++nb) {
        const int eb = e0 + nb * 32;
        if (eb < n_t) {  // wave-uniform
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
          // ReLU(.) * w summed over the lane's 16 heads of each block, as four
          // independent partial sums, then across the two lane halves
          float v4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int hb = 0; hb < HB; ++hb)
#pragma unroll
            for (int i = 0; i < 16; ++i) v4[i & 3] = fmaf(w[hb][i], fmaxf(acc[hb][i], 0.f), v4[i & 3]);
          float v = (v4[0] + v4[1]) + (v4[2] + v4[3]);
          v += __shfl_xor(v, 32, 64);
          const int e = eb + l32;
          const uint32_t key = score_key(v);
          const bool admit = g == 0 && e < n_t && key > theta;
          const uint64_t bm = __ballot(admit);
          if (admit) {
            const int pos = c + __popcll(bm & lt);
            my_key[pos] = key;
            my_idx[pos] = e;
          }
          c += __popcll(bm);
          if (c > FT_CAP - 32) {
            CSA_WAVE_FENCE();
            theta = wave_compact(my_key, my_idx, my_hist, c, K);
            c = K;
          }
        }
      }
    }
    if (it + 1 < ntiles) commit((it + 1) & 1);
    __syncthreads();
  }

  if (!q_ok) return;
  int32_t* out = a.idx + ((int64_t)b * a.S + t) * K;
  if (lane == 0 && a.n_visible) a.n_visible[(int64_t)b * a.S + t] = n_t;
  if (select_all) {
    for (int j = lane; j < K; j += 64) out[j] = j < n_t ? j : -1;
    return;
  }
  CSA_WAVE_FENCE();
  if (c > K) wave_compact(my_key, my_idx, my_hist, c, K);
  for (int j = lane; j < K; j += 64) out[j] = my_idx[j];
}

hipError_t launch_index_topk(const csa_params_t& p, const void* q_idx, const float* w_idx,
                             const void* k_idx, int32_t* idx, int32_t* n_visible, hipStream_t st) {
  if (p.topk > FT_MAXK) return hipErrorInvalidValue;
  IndexTopkArgs a{q_idx, w_idx, k_idx, idx, n_visible, p.B, p.S, p.idx_heads, p.ratio,
                  p.S / p.ratio, p.topk, (p.S + FT_WAVES - 1) / FT_WAVES};
  const int grid = p.B * a.qblocks;
  if (grid == 0) return hipSuccess;
#define CSA_FT_CASE(T, DI) hipLaunchKernelGGL((index_topk_kernel<T, DI>), dim3(grid), dim3(FT_WAVES * 64), 0, st, a)
  const bool bf = p.dtype == CSA_BF16;
  switch (p.idx_dim) {
    case 16: if (bf) CSA_FT_CASE(bf16, 16); else CSA_FT_CASE(float, 16); break;
    case 32: if (bf) CSA_FT_CASE(bf16, 32); else CSA_FT_CASE(float, 32); break;
    case 64: if (bf) CSA_FT_CASE(bf16, 64); else CSA_FT_CASE(float, 64); break;
    case 128: if (bf) CSA_FT_CASE(bf16, 128); else CSA_FT_CASE(float, 128); break;
    default: return hipErrorInvalidValue;
  }
#undef CSA_FT_CASE
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
