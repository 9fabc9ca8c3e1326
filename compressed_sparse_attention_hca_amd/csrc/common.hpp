// Device-side helpers shared by the gfx950 kernels: the integer layout of the
// compressed attention layer, element types, RoPE angles and MFMA fragments.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

// ---------------------------------------------------------------------------------
// Integer layout ("Enabling DeepSeek-V4-Flash Training ...", "Three attention types,
// interleaved"; "fix(deepseek-v4) ...", Part 1 item 2).  Every kernel and the
// debug-layout export use exactly these.
// ---------------------------------------------------------------------------------
__host__ __device__ inline int visible_entries(int t, int ratio) { return (t + 1) / ratio; }
__host__ __device__ inline int64_t entry_position(int64_t pos0, int s, int ratio) {
  return pos0 + (int64_t)s * ratio;
}
__host__ __device__ inline int window_lo(int t, int window) {
  return t - window + 1 > 0 ? t - window + 1 : 0;
}
// Number of window keys of query t (tokens window_lo(t)..t; none if window == 0).
__host__ __device__ inline int window_count(int t, int window) {
  return window <= 0 ? 0 : t - window_lo(t, window) + 1;
}

// ---------------------------------------------------------------------------------
// Element types.  Activations are fp32 or bf16; bf16 is stored as raw 16-bit words.
// ---------------------------------------------------------------------------------
typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Pointer qualifier for LDS (address space 3): reads through it compile to ds_* ops.
#define CSA_LDS __attribute__((address_space(3)))

__device__ inline float to_f32(float x) { return x; }
__device__ inline float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ inline T from_f32(float x);
template <> __device__ inline float from_f32<float>(float x) { return x; }
template <> __device__ inline bf16 from_f32<bf16>(float x) { return (bf16)x; }

// 16 bytes of T: 8 bf16 or 4 fp32.
template <typename T> struct Vec16 {
  static constexpr int N = 16 / sizeof(T);
  T v[N];
};

template <typename T> __device__ inline Vec16<T> load16(const T* p) {
  Vec16<T> r;
  *reinterpret_cast<uint4*>(r.v) = *reinterpret_cast<const uint4*>(p);
  return r;
}
template <typename T> __device__ inline void store16(T* p, const Vec16<T>& r) {
  *reinterpret_cast<uint4*>(p) = *reinterpret_cast<const uint4*>(r.v);
}

// ---------------------------------------------------------------------------------
// RoPE angles.  angle = P * theta^(-2i/R).  The product and its reduction modulo 2*pi
// are done in fp64 (an fp32 inverse frequency times a position near 65536 would be off
// by ~4e-3 rad); only the reduced angle goes through fp32 sincos.
// ---------------------------------------------------------------------------------
__device__ inline double rope_inv_freq(int i, int rope_dim, double theta) {
  return pow(theta, -2.0 * (double)i / (double)rope_dim);
}

__device__ inline void rope_cos_sin(int64_t P, double inv_freq, float* c, float* s) {
  const double two_pi_hi = 6.28318530717958623200e+00;   // 2*pi rounded to double
  const double two_pi_lo = 2.44929359829470635446e-16;   // 2*pi - two_pi_hi
  double a = (double)P * inv_freq;
  double k = rint(a * 0.15915494309189533577);            // a / (2*pi)
  double r = fma(-k, two_pi_hi, a);
  r = fma(-k, two_pi_lo, r);
  sincosf((float)r, s, c);
}

// ---------------------------------------------------------------------------------
// Wave helpers (wave64).
// ---------------------------------------------------------------------------------
__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

// ---------------------------------------------------------------------------------
// MFMA 16x16x32 fragments.  A fragment is 8 elements per lane: for the A operand lane l
// holds row (l % 16) and k-slots 8*(l/16) .. 8*(l/16)+7; for B, column (l % 16) and the
// same k-slots.  The accumulator (f32x4) holds rows 4*(l/16) + i, column l % 16.
// bf16 uses one v_mfma_f32_16x16x32_bf16; fp32 issues eight v_mfma_f32_16x16x4_f32,
// instruction i consuming element i, which sums over the same 32 k-slots.  Because
// A and B use one common lane -> k-slot assignment the product does not depend on how
// the hardware orders k inside an instruction.
// ---------------------------------------------------------------------------------
template <typename T> struct Frag { T v[8]; };

__device__ inline f32x4 mfma16x16x32(const Frag<bf16>& a, const Frag<bf16>& b, f32x4 c) {
  bf16x8 av, bv;
#pragma unroll
  for (int i = 0; i < 8; ++i) { av[i] = a.v[i]; bv[i] = b.v[i]; }
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, c, 0, 0, 0);
}
__device__ inline f32x4 mfma16x16x32(const Frag<float>& a, const Frag<float>& b, f32x4 c) {
#pragma unroll
  for (int i = 0; i < 8; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[i], b.v[i], c, 0, 0, 0);
  return c;
}

// Load 8 consecutive elements (one fragment's k-slots) from LDS or global memory.
template <typename T> __device__ inline Frag<T> load_frag(const T* p) {
  Frag<T> f;
  if constexpr (sizeof(T) == 2) {
    *reinterpret_cast<uint4*>(f.v) = *reinterpret_cast<const uint4*>(p);
  } else {
    *reinterpret_cast<uint4*>(f.v) = *reinterpret_cast<const uint4*>(p);
    *reinterpret_cast<uint4*>(f.v + 4) = *reinterpret_cast<const uint4*>(p + 4);
  }
  return f;
}

}  // namespace csa
