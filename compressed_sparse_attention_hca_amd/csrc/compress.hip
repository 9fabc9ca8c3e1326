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

// Lowest finite float: the online softmax's starting maximum.
constexpr float kLowest = -3.40282346638528859812e+38f;

// WPE = waves per entry (1: one entry per wave; 4: the workgroup splits one entry).
template <typename T, int WPE>
__global__ __launch_bounds__(256) void compress_kernel(CompressArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));  // uniform
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

  // m starts at the lowest finite float rather than -inf, so a slot with logit -inf leaves the online
  // update below unchanged (scale 1, weight 0) instead of producing a NaN; for a real
  // logit the first update gives the same values as from -inf (scale exactly 0).
  float m[8], l[8], acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) { m[i] = kLowest; l[i] = 0.f; acc[i] = 0.f; }

  if (WPE == 1 && span == 8) {
    // 8 slots (CSA at ratio 4): every load is issued first, then a two-pass softmax
    // per channel (one exponential per slot instead of the online form's two).  The
    // loads take no branch, so all of them are in flight together instead of one slot
    // at a time: a slot before token 0 (CSA entry 0's missing previous group) reads
    // token 0 and gets logit -inf, i.e. weight exactly 0 (its finite values then add 0;
    // they are left unmasked, or the compiler would skip, and branch around, their load).
    if (lane_ok) {
      float lg[8][8], v[8][8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int tok = a.overlap ? s * r - r + j : s * r + j;  // wave-uniform
        const bool prev = a.overlap && j < r;
        const int64_t off = ((int64_t)b * a.S + max(tok, 0)) * a.D + c0;
        const float pen = tok >= 0 ? 0.f : -INFINITY;
        float g[8], bias[8];
        load8<T>((prev ? gb : ga) + off, g);
        load8<T>((prev ? vb : va) + off, v[j]);
        load8<float>(a.bias + (int64_t)j * a.D + c0, bias);
#pragma unroll
        for (int i = 0; i < 8; ++i) lg[j][i] = g[i] + bias[i] + pen;
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
    // Online softmax over the wave's slots, branch-free as above (a slot before token 0
    // reads token 0 with logit -inf), unrolled so that several slots' loads are in flight.
#pragma unroll 4
    for (int j = j0; j < j1; ++j) {
      const int tok = a.overlap ? s * r - r + j : s * r + j;
      const bool prev = a.overlap && j < r;
      const int64_t off = ((int64_t)b * a.S + max(tok, 0)) * a.D + c0;
      const float pen = tok >= 0 ? 0.f : -INFINITY;
      float g[8], v[8], bias[8];
      load8<T>((prev ? gb : ga) + off, g);
      load8<T>((prev ? vb : va) + off, v);
      load8<float>(a.bias + (int64_t)j * a.D + c0, bias);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float lg = g[i] + bias[i] + pen;
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
        const float f = (mw == kLowest) ? 0.f : exp_fast(mw - M);  // a wave with no slot: 0
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
  const int64_t P = entry_position(a.pos0, s, r);
  if (a.D == 512 && a.R == 64) {
    // The V4 shape: every lane is here (lane_ok is the wave's entry_ok).  Lanes 0..31
    // form the 32 pairs' cos / sin once into LDS, and the 8 lanes holding the last 64
    // channels read theirs, instead of those 8 lanes forming 4 each (an fp64 pow and a
    // sincosf apiece) while the rest of the wave waits.
    __shared__ float2 ctab[4][32];
    if (lane < 32) {
      float c, sn;
      rope_cos_sin(P, rope_inv_freq(lane, 64, a.theta), &c, &sn);
      ctab[wave][lane] = make_float2(c, sn);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");  // the table is read by other lanes
    if (lane >= 56) {  // channels 448 + 8(lane - 56) ..: pairs 4(lane - 56) .. +3
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float2 cs = ctab[wave][4 * (lane - 56) + k];
        const float x0 = p[2 * k], x1 = p[2 * k + 1];
        p[2 * k] = x0 * cs.x - x1 * cs.y;
        p[2 * k + 1] = x0 * cs.y + x1 * cs.x;
      }
    }
  } else {
    double f[4];
    rope8_freq(f, c0, a.D, a.R, a.theta);
    rope8(p, c0, a.D, a.R, P, f, false);
  }
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

// Eight elements as loaded (one 16-byte vector for bf16, two for fp32), converted only
// when used, so a load can stay in flight past the code that follows it.
template <typename T>
struct Raw8 {
  Vec16<T> v[sizeof(T) / 2];
};
template <typename T>
__device__ inline Raw8<T> load_raw8(const T* p) {
  Raw8<T> r;
#pragma unroll
  for (int k = 0; k < (int)(sizeof(T) / 2); ++k) r.v[k] = load16(p + k * (16 / (int)sizeof(T)));
  return r;
}
template <typename T>
__device__ inline void unpack8(const Raw8<T>& r, float (&x)[8]) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = to_f32(r.v[0].v[i]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) { x[i] = r.v[0].v[i]; x[4 + i] = r.v[1].v[i]; }
  }
}

// Raw window latents rotated at their own positions pos0 + t (optionally normalised
// first).  One wave rotates WR_TOKENS consecutive tokens (one 16-byte chunk per lane per
// token), so the inverse frequencies (an fp64 pow each) are worked out once per wave.
// Rows are loaded one token ahead, into two alternating registers: a row is in flight
// while the wave rotates and stores the one before (the compiler itself would not move
// a load above a store to memory that may alias it).
// FULL: D == 512 and R == 64 (the V4 layer shape).  Every lane holds 8 channels, so no
// store is masked (a masked store sits behind a branch, and the compiler's wait for the
// next row then also waits for it); and the wave's WR_TOKENS x 32 rotation angles are
// formed once, four per lane with every lane busy, into an LDS table that the 8 lanes
// holding the last 64 channels read, instead of those 8 lanes forming 32 each while
// the rest of the wave waits.
constexpr int WR_TOKENS = 8;
template <typename T, bool FULL>
__global__ __launch_bounds__(256) void window_rope_kernel(WindowArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));  // uniform
  const int64_t tok0 = ((int64_t)blockIdx.x * 4 + wave) * WR_TOKENS;
  const int64_t total = (int64_t)a.B * a.S;
  if (tok0 >= total) return;
  const int c0 = lane * 8;
  const bool lane_ok = FULL || c0 < a.D;
  const int nt = (int)min((int64_t)WR_TOKENS, total - tok0);  // at least 1
  // lanes past D read channel 0 of the row (their values are never stored); a token
  // past nt reads token nt - 1 again
  const T* src = static_cast<const T*>(a.kv_raw) + tok0 * a.D + (lane_ok ? c0 : 0);
  T* dst = static_cast<T*>(a.kv_w) + tok0 * a.D + c0;
  auto load_tok = [&](int j) { return load_raw8(src + (int64_t)min(j, nt - 1) * a.D); };
  Raw8<T> ra = load_tok(0);
  __shared__ float2 tab[4][FULL ? WR_TOKENS * 32 : 1];
  double f[4];
  if constexpr (FULL) {
    // entry 32 j + p: token j's cos / sin of pair p (lane l forms pair l % 32 of tokens
    // l / 32 + 2m; a token past nt repeats token nt - 1)
    const double fp = rope_inv_freq(lane & 31, 64, a.theta);
#pragma unroll
    for (int m = 0; m < WR_TOKENS / 2; ++m) {
      const int j = (lane >> 5) + 2 * m;
      float c, sn;
      rope_cos_sin(a.pos0 + (tok0 + min(j, nt - 1)) % a.S, fp, &c, &sn);
      tab[wave][32 * j + (lane & 31)] = make_float2(c, sn);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");  // the table is read by other lanes
  } else {
    rope8_freq(f, c0, a.D, a.R, a.theta);
  }
  auto rotate_store = [&](const Raw8<T>& r, int j) {
    const int t = (int)((tok0 + j) % a.S);
    float x[8];
    unpack8(r, x);
    if (!lane_ok) {
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
    if constexpr (FULL) {
      if (lane >= 56) {  // channels 448 + 8(lane - 56) ..: pairs 4(lane - 56) .. +3
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float2 r = tab[wave][32 * j + 4 * (lane - 56) + k];
          const float x0 = x[2 * k], x1 = x[2 * k + 1];
          x[2 * k] = x0 * r.x - x1 * r.y;
          x[2 * k + 1] = x0 * r.y + x1 * r.x;
        }
      }
    } else {
      // every lane rotates (lanes past D hold zeros), so only the store is masked
      rope8(x, c0, a.D, a.R, a.pos0 + t, f, false);
    }
    if (lane_ok) store8<T>(dst + (int64_t)j * a.D, x);
  };
  for (int j = 0; j < nt; j += 2) {
    const Raw8<T> rb = load_tok(j + 1);
    rotate_store(ra, j);
    if (j + 1 >= nt) break;
    ra = load_tok(j + 2);
    rotate_store(rb, j + 1);
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
  const bool full = p.D == 512 && p.rope_dim == 64;
  if (p.dtype == CSA_BF16) {
    if (full) hipLaunchKernelGGL((window_rope_kernel<bf16, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((window_rope_kernel<bf16, false>), grid, block, 0, st, a);
  } else {
    if (full) hipLaunchKernelGGL((window_rope_kernel<float, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((window_rope_kernel<float, false>), grid, block, 0, st, a);
  }
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
