// Target distribution of the indexer's distillation loss on gfx950:
//   T[t,k] = (1/H) sum_h softmax_k( (RoPE(q[t,h], pos0 + t) . kv_c[Sel_t[k]]) * scale )
// over the selected entries only ("fix(deepseek-v4): correct V4-Flash attention
// math", Part 1 item 5: KL(attention || indexer) over the selected entries, kept in
// [B, S, K]; item 11: the head sum inside the loop, so the per-head [B, H, S, K] tensor
// never exists).
//
// Mapping: one workgroup per query, four waves; wave w owns heads 16w .. 16w+15.
// The selected rows of kv_c are gathered 32 at a time into LDS; the logits are
// S^T[key, head] = K_tile . Q^T on v_mfma_f32_16x16x32 (keys on M from the tile, heads
// on N from the rotated query in registers).  Pass 1 keeps a running maximum and sum
// per head; pass 2 recomputes the logits, turns them into probabilities and sums them
// over the wave's heads in registers and over the four waves in LDS.
#include "common.hpp"
#include "launch.hpp"

namespace csa {

struct KlArgs {
  const void* q;
  const void* kv_c;
  const int32_t* idx;
  float* target;
  int32_t B, S, H, R, ratio, topk, n_entries;
  double theta;
  int64_t pos0;
  float scale_log2;  // softmax_scale * log2(e)
};

constexpr int KL_WAVES = 4;
constexpr int KL_KT = 32;  // keys per tile

template <typename T, int D>
__global__ __launch_bounds__(KL_WAVES * 64) void kl_target_kernel(KlArgs a) {
  constexpr int KS = D / 32;                   // k-steps of the 16x16x32 product
  constexpr int ES = (int)sizeof(T);
  constexpr int ROWE = D + 16 / ES;            // padded LDS row (elements)
  constexpr int CPR = D * ES / 16;             // 16-byte chunks per row
  __shared__ __attribute__((aligned(16))) T tile[KL_KT * ROWE];
  __shared__ int sel[KL_KT];
  __shared__ float2 cs[64];
  __shared__ float part[KL_WAVES][KL_KT];

  const int gi = a.B * a.S - 1 - (int)blockIdx.x;  // latest queries first
  const int b = gi / a.S, t = gi % a.S;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hl = lane & 15, g = lane >> 4;
  const int h = 16 * wave + hl;
  const int n_t = visible_entries(t, a.ratio);
  const int nsel = min(a.topk, n_t);
  const int32_t* irow = a.idx + ((int64_t)b * a.S + t) * a.topk;
  float* orow = a.target + ((int64_t)b * a.S + t) * a.topk;

  if (threadIdx.x < a.R / 2) {
    float c, s;
    rope_cos_sin(a.pos0 + t, rope_inv_freq(threadIdx.x, a.R, a.theta), &c, &s);
    cs[threadIdx.x] = make_float2(c, s);
  }
  __syncthreads();

  // B operand: rotated q[b, t, h], dims 32ks + 8g + i; zero for padded heads
  Frag<T> qf[KS];
  const T* qrow = static_cast<const T*>(a.q) + (((int64_t)b * a.S + t) * a.H + min(h, a.H - 1)) * D;
  const int rlo = D - a.R;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    Frag<T> f = load_frag(qrow + 32 * ks + 8 * g);
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      const int d = 32 * ks + 8 * g + i;
      float x0 = to_f32(f.v[i]), x1 = to_f32(f.v[i + 1]);
      if (d >= rlo) {
        const float2 r = cs[(d - rlo) >> 1];
        const float y0 = x0 * r.x - x1 * r.y, y1 = x0 * r.y + x1 * r.x;
        x0 = y0;
        x1 = y1;
      }
      if (h >= a.H) x0 = x1 = 0.f;
      f.v[i] = from_f32<T>(x0);
      f.v[i + 1] = from_f32<T>(x1);
    }
    qf[ks] = f;
  }

  // Gather the selected rows of tile `it` (an index outside 0 .. n_t-1 is masked).
  const T* kbase = static_cast<const T*>(a.kv_c) + (int64_t)b * a.n_entries * D;
  auto gather = [&](int it) {
    __syncthreads();  // every wave is done with the previous tile
    if (threadIdx.x < KL_KT) {
      const int k = it * KL_KT + threadIdx.x;
      const int s = k < nsel ? irow[k] : -1;
      sel[threadIdx.x] = (s >= 0 && s < n_t) ? s : -1;
    }
    __syncthreads();
    for (int c = threadIdx.x; c < KL_KT * CPR; c += KL_WAVES * 64) {
      const int r = c / CPR, ch = c % CPR;
      const int s = sel[r];
      const uint4 v = s >= 0 ? *reinterpret_cast<const uint4*>(kbase + (int64_t)s * D + ch * (16 / ES))
                             : make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(&tile[r * ROWE + ch * (16 / ES)]) = v;
    }
    __syncthreads();
  };
  // Logits (base-2 units) of tile keys 16*blk + 4g + i for head h; -inf when masked.
  auto logits = [&](float (&z)[2][4]) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const Frag<T> ka = load_frag(&tile[(16 * blk + hl) * ROWE + 32 * ks + 8 * g]);
        acc = mfma16x16x32(ka, qf[ks], acc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) z[blk][i] = sel[16 * blk + 4 * g + i] >= 0 ? acc[i] * a.scale_log2 : -INFINITY;
    }
  };

  const int ntiles = (nsel + KL_KT - 1) / KL_KT;
  // pass 1: running maximum and sum per head, per lane, then over the four lanes of h
  float m = -INFINITY, l = 0.f;
  for (int it = 0; it < ntiles; ++it) {
    gather(it);
    float z[2][4];
    logits(z);
    float mt = m;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int i = 0; i < 4; ++i) mt = fmaxf(mt, z[blk][i]);
    if (mt != -INFINITY) {
      l *= __builtin_amdgcn_exp2f(m - mt);
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int i = 0; i < 4; ++i) l += __builtin_amdgcn_exp2f(z[blk][i] - mt);
      m = mt;
    }
  }
#pragma unroll
  for (int x = 16; x <= 32; x <<= 1) {
    const float mo = __shfl_xor(m, x, 64), lo = __shfl_xor(l, x, 64);
    const float mn = fmaxf(m, mo);
    if (mn != -INFINITY) {
      l = l * __builtin_amdgcn_exp2f(m - mn) + lo * __builtin_amdgcn_exp2f(mo - mn);
      m = mn;
    }
  }
  const float inv_l = (h < a.H && l > 0.f) ? 1.f / l : 0.f;  // padded heads add nothing
  const float inv_h = 1.f / (float)a.H;

  // pass 2: probabilities, summed over the wave's heads, then over the waves
  for (int it = 0; it < ntiles; ++it) {
    gather(it);
    float z[2][4];
    logits(z);
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float p = z[blk][i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(z[blk][i] - m) * inv_l;
#pragma unroll
        for (int x = 1; x < 16; x <<= 1) p += __shfl_xor(p, x, 64);
        if (hl == 0) part[wave][16 * blk + 4 * g + i] = p;
      }
    __syncthreads();
    if (threadIdx.x < KL_KT) {
      const int k = it * KL_KT + threadIdx.x;
      if (k < nsel) orow[k] = (part[0][threadIdx.x] + part[1][threadIdx.x] + part[2][threadIdx.x] + part[3][threadIdx.x]) * inv_h;
    }
  }
  for (int k = nsel + (int)threadIdx.x; k < a.topk; k += KL_WAVES * 64) orow[k] = 0.f;
}

// ---------------------------------------------------------------------------------
// bf16 fast path for D = 512 and up to 64 heads.  Tiles of 64 selected rows are copied
// straight into LDS (one 1 KB wave load per row, 16-byte chunk c of row r at chunk
// position c ^ swz(r), so the 32 rows read together hit 8 distinct chunk columns).
// Wave w = (hg, kh) multiplies keys 32kh .. 32kh+31 of the tile by heads 32hg ..
// 32hg+31 on v_mfma_f32_32x32x16_bf16 (keys on M from LDS, heads on N from the
// rotated query in registers), so each fragment read feeds 32 heads.  Pass 2 writes
// the probabilities [64 keys x 64 heads] over the tile it has finished with, and one
// thread per key sums its row of heads.  64 KB of LDS: two workgroups per CU.
// ---------------------------------------------------------------------------------
__global__ __launch_bounds__(256, 2) void kl_target_hd_kernel(KlArgs a) {
  constexpr int D = 512, ROWB = 1024, KT = 64;
  __shared__ __attribute__((aligned(1024))) unsigned char tile[KT * ROWB];
  __shared__ float2 cs[64];
  __shared__ float stat[2][2][32][2];  // [hg][kh][head][m, l]
  auto swz = [](int r) -> int { return ((r & 3) << 1) | ((r >> 2) & 1); };

  const int gi = a.B * a.S - 1 - (int)blockIdx.x;  // latest queries first
  const int b = gi / a.S, t = gi % a.S;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hg = wave >> 1, kh = wave & 1;
  const int l32 = lane & 31, g = lane >> 5;
  const int h = 32 * hg + l32;
  const int n_t = visible_entries(t, a.ratio);
  const int nsel = min(a.topk, n_t);
  const int32_t* irow = a.idx + ((int64_t)b * a.S + t) * a.topk;
  float* orow = a.target + ((int64_t)b * a.S + t) * a.topk;
  const unsigned char* kvb = static_cast<const unsigned char*>(a.kv_c) + (int64_t)b * a.n_entries * ROWB;

  if (threadIdx.x < a.R / 2) {
    float c, s;
    rope_cos_sin(a.pos0 + t, rope_inv_freq(threadIdx.x, a.R, a.theta), &c, &s);
    cs[threadIdx.x] = make_float2(c, s);
  }
  __syncthreads();

  // B operand: rotated q[b, t, h], k-step ks holds dims 16ks + 8g .. +7; a 32-bit word
  // holds one rope pair (x0 low, x1 high), rotated in fp32 and packed back with one
  // round-to-nearest-even conversion
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  bf16x8 qf[32];
  {
    const bf16* qrow = static_cast<const bf16*>(a.q) + (((int64_t)b * a.S + t) * a.H + min(h, a.H - 1)) * D;
    const int rlo = D - a.R;
    const bool live = h < a.H;
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) {
      u32x4 w = *reinterpret_cast<const u32x4*>(qrow + 16 * ks + 8 * g);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 16 * ks + 8 * g + 2 * j;
        float x0 = __uint_as_float(w[j] << 16), x1 = __uint_as_float(w[j] & 0xffff0000u);
        if (d >= rlo) {
          const float2 r = cs[(d - rlo) >> 1];
          const float y0 = x0 * r.x - x1 * r.y, y1 = x0 * r.y + x1 * r.x;
          w[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{y0, y1}, bf16x2_t));
        }
        if (!live) w[j] = 0u;
      }
      qf[ks] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // Direct-to-LDS copy of tile `it`: lane l holds key it*64 + l; wave w copies rows
  // w, w+4, ...; returns the keys' validity bits (an index outside 0 .. n_t-1 is
  // masked and its row address replaced by a valid one).
  auto issue = [&](int it) -> uint64_t {
    const int k = it * KT + lane;
    int s = k < nsel ? irow[k] : -1;
    const bool ok = s >= 0 && s < n_t;
    if (!ok) s = 0;
    const uint64_t sp = reinterpret_cast<uint64_t>(kvb + (int64_t)s * ROWB);
    const uint32_t sp_lo = (uint32_t)sp, sp_hi = (uint32_t)(sp >> 32);
#pragma unroll
    for (int m = 0; m < KT / 4; ++m) {
      const int r = wave + 4 * m;
      const uint64_t row = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)sp_hi, r) << 32) |
                           (uint32_t)__builtin_amdgcn_readlane((int)sp_lo, r);
      const unsigned char* gp = reinterpret_cast<const unsigned char*>(row) + ((lane ^ swz(r)) << 4);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(gp), (CSA_LDS void*)(tile + r * ROWB), 16, 0, 0);
    }
    return __ballot(ok);
  };
  // logits (base-2 units) of keys 32kh + 8j + 4g + i for head h; -inf when masked
  auto logits = [&](uint64_t kmask, float (&z)[16]) {
    const int r = 32 * kh + l32;
    const CSA_LDS unsigned char* lb = (const CSA_LDS unsigned char*)tile + r * ROWB;
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) {
      const bf16x8 ka = __builtin_bit_cast(bf16x8, *(const CSA_LDS u32x4*)(lb + (((2 * ks + g) ^ swz(r)) << 4)));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], acc, 0, 0, 0);
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = 32 * kh + 8 * (e >> 2) + 4 * g + (e & 3);
      z[e] = ((kmask >> key) & 1ull) ? acc[e] * a.scale_log2 : -INFINITY;
    }
  };

  const int ntiles = (nsel + KT - 1) / KT;
  // pass 1: running maximum and sum per head
  float m = -INFINITY, l = 0.f;
  for (int it = 0; it < ntiles; ++it) {
    const uint64_t km = issue(it);
    __syncthreads();  // the copies have landed (each wave waits for its own first)
    float z[16];
    logits(km, z);
    float mt = m;
#pragma unroll
    for (int e = 0; e < 16; ++e) mt = fmaxf(mt, z[e]);
    if (mt != -INFINITY) {
      l *= __builtin_amdgcn_exp2f(m - mt);
#pragma unroll
      for (int e = 0; e < 16; ++e) l += __builtin_amdgcn_exp2f(z[e] - mt);
      m = mt;
    }
    __syncthreads();  // every wave is done with the tile
  }
  // combine the two lane halves, then the two key halves (waves kh = 0, 1)
  {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    const auto rl = __builtin_amdgcn_permlane32_swap(__float_as_uint(l), __float_as_uint(l), false, false);
    const float m0 = __uint_as_float(r[0]), m1 = __uint_as_float(r[1]);
    const float l0 = __uint_as_float(rl[0]), l1 = __uint_as_float(rl[1]);
    const float mn = fmaxf(m0, m1);
    m = mn;
    l = mn == -INFINITY ? 0.f : l0 * __builtin_amdgcn_exp2f(m0 - mn) + l1 * __builtin_amdgcn_exp2f(m1 - mn);
  }
  if (g == 0) {
    stat[hg][kh][l32][0] = m;
    stat[hg][kh][l32][1] = l;
  }
  __syncthreads();
  {
    const float mo = stat[hg][kh ^ 1][l32][0], lo = stat[hg][kh ^ 1][l32][1];
    const float mn = fmaxf(m, mo);
    if (mn != -INFINITY) {
      l = l * __builtin_amdgcn_exp2f(m - mn) + lo * __builtin_amdgcn_exp2f(mo - mn);
      m = mn;
    }
  }
  const float inv_l = (h < a.H && l > 0.f) ? 1.f / l : 0.f;  // padded heads add nothing
  const float inv_h = 1.f / (float)a.H;

  // pass 2: probabilities over the finished tile as P[key][head], then a sum per key
  float* pb = reinterpret_cast<float*>(tile);
  for (int it = 0; it < ntiles; ++it) {
    const uint64_t km = issue(it);
    __syncthreads();
    float z[16];
    logits(km, z);
    __syncthreads();  // every wave is done reading the tile
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = 32 * kh + 8 * (e >> 2) + 4 * g + (e & 3);
      pb[key * 64 + h] = z[e] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(z[e] - m) * inv_l;
    }
    __syncthreads();
    if (threadIdx.x < KT) {
      const int k = it * KT + threadIdx.x;
      const f32x4* row = reinterpret_cast<const f32x4*>(pb + threadIdx.x * 64);
      f32x4 acc4 = row[0];
#pragma unroll
      for (int c = 1; c < 16; ++c) acc4 += row[c];
      if (k < nsel) orow[k] = ((acc4[0] + acc4[1]) + (acc4[2] + acc4[3])) * inv_h;
    }
    __syncthreads();  // the sums are read before the next tile lands
  }
  for (int k = nsel + (int)threadIdx.x; k < a.topk; k += 256) orow[k] = 0.f;
}

hipError_t launch_kl_target(const csa_params_t& p, const void* q, const void* kv_c, const int32_t* idx,
                            float* target, hipStream_t st) {
  KlArgs a{q, kv_c, idx, target, p.B, p.S, p.H, p.rope_dim, p.ratio, p.topk, p.S / p.ratio,
           p.rope_theta, p.pos0, p.softmax_scale * 1.4426950408889634f};
  const int grid = p.B * p.S;
  if (grid == 0) return hipSuccess;
  if (p.dtype == CSA_BF16 && p.D == 512) {
    hipLaunchKernelGGL(kl_target_hd_kernel, dim3(grid), dim3(256), 0, st, a);
    return hipGetLastError();
  }
#define CSA_KL_CASE(T, D) hipLaunchKernelGGL((kl_target_kernel<T, D>), dim3(grid), dim3(KL_WAVES * 64), 0, st, a)
  const bool bf = p.dtype == CSA_BF16;
  switch (p.D) {
    case 64: if (bf) CSA_KL_CASE(bf16, 64); else CSA_KL_CASE(float, 64); break;
    case 128: if (bf) CSA_KL_CASE(bf16, 128); else CSA_KL_CASE(float, 128); break;
    case 256: if (bf) CSA_KL_CASE(bf16, 256); else CSA_KL_CASE(float, 256); break;
    case 512: if (bf) CSA_KL_CASE(bf16, 512); else CSA_KL_CASE(float, 512); break;
    default: return hipErrorInvalidValue;
  }
#undef CSA_KL_CASE
  return hipGetLastError();
}

}  // namespace csa
