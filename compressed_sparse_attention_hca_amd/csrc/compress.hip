// Stages 1-2 of the compressed attention layer on gfx950: softmax-gated pooling of
// per-token latents into compressed entries, RMSNorm, and RoPE at the entry's
// original-sequence position; plus the rotation of the raw window latents that the
// attention kernel reads as keys.
//
// Pooling: "Enabling DeepSeek-V4-Flash Training on AMD Instinct MI355X GPUs with
// Primus", subsection "Three attention types, interleaved" (softmax over the group of
// gate + per-position bias, weighting the values; CSA entries also cover the previous
// 4 tokens) and section "Kernel fusions", row "Compressor pooling" (one kernel that
// reduces in fp32 for both the window of 8 and of 128).  Norm and rotation: "fix(
// deepseek-v4): correct V4-Flash attention math", Part 1 items 1-2.
//
// Memory-bound streaming: each lane owns 8 channels (16 B of bf16 per load), a wave
// covers a 512-wide row, and every input byte is read once.  CSA (8 slots) uses one
// wave per entry, with all 8 slots in registers and a two-pass softmax per channel;
// HCA (128 slots) splits the slots over the 4 waves of a workgroup, runs the softmax
// online in registers and merges the waves through LDS.
#include "common.hpp"
#include "launch.hpp"

namespace csa {

struct CompressArgs {
  const void* va;
  const void* ga;
  const void* vb;
  const void* gb;
  const float* bias;
  void* kv_c;
  int32_t B, S, D, R, ratio, overlap, n_entries;
  float eps;
  double theta;
  int64_t pos0;
};

template <typename T>
__device__ inline void load8(const T* p, float (&x)[8]) {
  if constexpr (sizeof(T) == 2) {
    Vec16<T> v = load16(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = to_f32(v.v[i]);
  } else {
    Vec16<T> a = load16(p), b = load16(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) { x[i] = a.v[i]; x[4 + i] = b.v[i]; }
  }
}

template <typename T>
__device__ inline void store8(T* p, const float (&x)[8]) {
  if constexpr (sizeof(T) == 2) {
    Vec16<T> v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v.v[i] = from_f32<T>(x[i]);
    store16(p, v);
  } else {
    Vec16<T> a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) { a.v[i] = x[i]; b.v[i] = x[4 + i]; }
    store16(p, a);
    store16(p + 4, b);
  }
}

// Inverse frequencies of this lane's 4 channel pairs c0..c0+7 (0 outside the last R dims).
__device__ inline void rope8_freq(double (&f)[4], int c0, int D, int R, double theta) {
  const int lo = D - R;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int c = c0 + 2 * k;
    f[k] = c >= lo ? rope_inv_freq((c - lo) >> 1, R, theta) : 0.0;
  }
}

// Rotate this lane's 8 channels c0..c0+7 in place where they fall in the last R dims,
// with the inverse frequencies from rope8_freq.
__device__ inline void rope8(float (&x)[8], int c0, int D, int R, int64_t P, const double (&f)[4], bool inverse) {
  const int lo = D - R;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int c = c0 + 2 * k;
    if (c >= lo) {
      float cs, sn;
      rope_cos_sin(P, f[k], &cs, &sn);
      if (inverse) sn = -sn;
      const float x0 = x[2 * k], x1 = x[2 * k + 1];
      x[2 * k] = x0 * cs - x1 * sn;
      x[2 * k + 1] = x0 * sn + x1 * cs;
    }
  }
}

// e^x as one v_exp_f32 of x * log2(e): its error (about 1e-6 relative for the
// arguments here, all <= 0) is far below the activations' bf16 rounding, and the
// pooling is otherwise bound by the accurate expf's instruction count.
__device__ inline float exp_fast(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

// WPE = waves per entry (1: one entry per wave; 4: the workgroup splits one entry).
template <typename T, int WPE>
__global__ __launch_bounds__(256) void compress_kernel(CompressArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int total = a.B * a.n_entries;
  const int e = (WPE == 1) ? (int)blockIdx.x * 4 + wave : (int)blockIdx.x;
  const bool entry_ok = e < total;
  const int b = entry_ok ? e / a.n_entries : 0;
  const int s = entry_ok ? e % a.n_entries : 0;
  const int c0 = lane * 8;
  const bool lane_ok = entry_ok && c0 < a.D;
  const int r = a.ratio;
  const int span = a.overlap ? 2 * r : r;
  int j0 = 0, j1 = span;
  if (WPE > 1) {
    const int per = (span + WPE - 1) / WPE;
    j0 = wave * per;
    j1 = min(span, j0 + per);
  }
  const T* va = static_cast<const T*>(a.va);
  const T* ga = static_cast<const T*>(a.ga);
  const T* vb = static_cast<const T*>(a.vb);
  const T* gb = static_cast<const T*>(a.gb);

  float m[8], l[8], acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) { m[i] = -INFINITY; l[i] = 0.f; acc[i] = 0.f; }

  if (WPE == 1 && span == 8) {
    // 8 slots (CSA at ratio 4): every load is issued first, then a two-pass softmax
    // per channel (one exponential per slot instead of the online form's two)
    if (lane_ok) {
      float lg[8][8], v[8][8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int tok = a.overlap ? s * r - r + j : s * r + j;  // wave-uniform
        if (tok >= 0) {
          const bool prev = a.overlap && j < r;
          const int64_t off = ((int64_t)b * a.S + tok) * a.D + c0;
          float g[8], bias[8];
          load8<T>((prev ? gb : ga) + off, g);
          load8<T>((prev ? vb : va) + off, v[j]);
          load8<float>(a.bias + (int64_t)j * a.D + c0, bias);
#pragma unroll
          for (int i = 0; i < 8; ++i) lg[j][i] = g[i] + bias[i];
        } else {  // CSA entry 0: no previous group
#pragma unroll
          for (int i = 0; i < 8; ++i) { lg[j][i] = -INFINITY; v[j][i] = 0.f; }
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float mx = lg[0][i];
#pragma unroll
        for (int j = 1; j < 8; ++j) mx = fmaxf(mx, lg[j][i]);
        float li = 0.f, ai = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float ex = exp_fast(lg[j][i] - mx);
          li += ex;
          ai += ex * v[j][i];
        }
        l[i] = li;
        acc[i] = ai;
      }
    }
  } else if (lane_ok) {
    for (int j = j0; j < j1; ++j) {
      const int tok = a.overlap ? s * r - r + j : s * r + j;
      if (tok < 0) continue;  // CSA entry 0: no previous group
      const bool prev = a.overlap && j < r;
      const int64_t off = ((int64_t)b * a.S + tok) * a.D + c0;
      float g[8], v[8], bias[8];
      load8<T>((prev ? gb : ga) + off, g);
      load8<T>((prev ? vb : va) + off, v);
      load8<float>(a.bias + (int64_t)j * a.D + c0, bias);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float lg = g[i] + bias[i];
        const float mn = fmaxf(m[i], lg);
        const float sc = exp_fast(m[i] - mn);
        const float ex = exp_fast(lg - mn);
        l[i] = l[i] * sc + ex;
        acc[i] = acc[i] * sc + ex * v[i];
        m[i] = mn;
      }
    }
  }

  if constexpr (WPE > 1) {
    __shared__ float part[WPE][3][8][64];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      part[wave][0][i][lane] = m[i];
      part[wave][1][i][lane] = l[i];
      part[wave][2][i][lane] = acc[i];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < WPE; ++w) M = fmaxf(M, part[w][0][i][lane]);
      float L = 0.f, A = 0.f;
#pragma unroll
      for (int w = 0; w < WPE; ++w) {
        const float mw = part[w][0][i][lane];
        const float f = (mw == -INFINITY) ? 0.f : exp_fast(mw - M);
        L += part[w][1][i][lane] * f;
        A += part[w][2][i][lane] * f;
      }
      l[i] = L;
      acc[i] = A;
    }
  }

  // pooled value, RMSNorm over the row (weight 1), RoPE at pos0 + s * ratio
  float p[8];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    p[i] = lane_ok ? acc[i] / l[i] : 0.f;
    ss += p[i] * p[i];
  }
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / (float)a.D + a.eps);
#pragma unroll
  for (int i = 0; i < 8; ++i) p[i] *= inv;
  if (!lane_ok) return;
  double f[4];
  rope8_freq(f, c0, a.D, a.R, a.theta);
  rope8(p, c0, a.D, a.R, entry_position(a.pos0, s, r), f, false);
  store8<T>(static_cast<T*>(a.kv_c) + ((int64_t)b * a.n_entries + s) * a.D + c0, p);
}

struct WindowArgs {
  const void* kv_raw;
  void* kv_w;
  int32_t B, S, D, R, norm;
  float eps;
  double theta;
  int64_t pos0;
};

// Raw window latents rotated at their own positions pos0 + t (optionally normalised
// first).  One wave rotates WR_TOKENS consecutive tokens (one 16-byte chunk per lane per
// token), so the inverse frequencies (an fp64 pow each) are worked out once per wave.
constexpr int WR_TOKENS = 8;
template <typename T>
__global__ __launch_bounds__(256) void window_rope_kernel(WindowArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t tok0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * WR_TOKENS;
  const int64_t total = (int64_t)a.B * a.S;
  if (tok0 >= total) return;
  const int c0 = lane * 8;
  const bool lane_ok = c0 < a.D;
  double f[4];
  rope8_freq(f, c0, a.D, a.R, a.theta);
  for (int j = 0; j < WR_TOKENS; ++j) {
    const int64_t tok = tok0 + j;
    if (tok >= total) break;  // wave-uniform
    const int t = (int)(tok % a.S);
    float x[8];
    const int64_t off = tok * a.D + c0;
    if (lane_ok) load8<T>(static_cast<const T*>(a.kv_raw) + off, x);
    else {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = 0.f;
    }
    if (a.norm) {
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) ss += x[i] * x[i];
      ss = wave_sum(ss);
      const float inv = 1.0f / sqrtf(ss / (float)a.D + a.eps);
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] *= inv;
    }
    if (lane_ok) {
      rope8(x, c0, a.D, a.R, a.pos0 + t, f, false);
      store8<T>(static_cast<T*>(a.kv_w) + off, x);
    }
  }
}

hipError_t launch_compress(const csa_params_t& p, const void* va, const void* ga, const void* vb,
                           const void* gb, const float* bias, void* kv_c, hipStream_t st) {
  CompressArgs a{va, ga, vb, gb, bias, kv_c, p.B, p.S, p.D, p.rope_dim, p.ratio, p.overlap,
                 p.S / p.ratio, p.rms_eps, p.rope_theta, p.pos0};
  const int total = p.B * a.n_entries;
  if (total == 0) return hipSuccess;
  const int span = p.overlap ? 2 * p.ratio : p.ratio;
  const bool split = span > 16;
  dim3 grid(split ? total : (total + 3) / 4), block(256);
  if (p.dtype == CSA_BF16) {
    if (split) hipLaunchKernelGGL((compress_kernel<bf16, 4>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((compress_kernel<bf16, 1>), grid, block, 0, st, a);
  } else {
    if (split) hipLaunchKernelGGL((compress_kernel<float, 4>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((compress_kernel<float, 1>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_window_rope(const csa_params_t& p, const void* kv_raw, void* kv_w, hipStream_t st) {
  WindowArgs a{kv_raw, kv_w, p.B, p.S, p.D, p.rope_dim, (p.flags & CSA_FLAG_NORM_WINDOW) ? 1 : 0,
               p.rms_eps, p.rope_theta, p.pos0};
  const int total = p.B * p.S;
  if (total == 0) return hipSuccess;
  const int64_t waves = ((int64_t)total + WR_TOKENS - 1) / WR_TOKENS;
  dim3 grid((unsigned)((waves + 3) / 4)), block(256);
  if (p.dtype == CSA_BF16) hipLaunchKernelGGL((window_rope_kernel<bf16>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((window_rope_kernel<float>), grid, block, 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------
// Integer layout export, from the same helpers the kernels use.
// ---------------------------------------------------------------------------------
__global__ void debug_layout_kernel(int32_t S, int32_t ratio, int32_t window, int64_t pos0,
                                    int32_t* comp_pos, int32_t* n_vis, int32_t* win_lo) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= S) return;
  if (n_vis) n_vis[t] = visible_entries(t, ratio);
  if (win_lo) win_lo[t] = window_lo(t, window);
  if (comp_pos && t < S / ratio) comp_pos[t] = (int32_t)entry_position(pos0, t, ratio);
}

hipError_t launch_debug_layout(const csa_params_t& p, int32_t* comp_pos, int32_t* n_visible,
                               int32_t* win_lo, hipStream_t st) {
  if (p.S == 0) return hipSuccess;
  hipLaunchKernelGGL(debug_layout_kernel, dim3((p.S + 255) / 256), dim3(256), 0, st, p.S, p.ratio,
                     p.window, p.pos0, comp_pos, n_visible, win_lo);
  return hipGetLastError();
}

}  // namespace csa
