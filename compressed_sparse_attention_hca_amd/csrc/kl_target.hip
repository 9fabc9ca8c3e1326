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

hipError_t launch_kl_target(const csa_params_t& p, const void* q, const void* kv_c, const int32_t* idx,
                            float* target, hipStream_t st) {
  KlArgs a{q, kv_c, idx, target, p.B, p.S, p.H, p.rope_dim, p.ratio, p.topk, p.S / p.ratio,
           p.rope_theta, p.pos0, p.softmax_scale * 1.4426950408889634f};
  const int grid = p.B * p.S;
  if (grid == 0) return hipSuccess;
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
