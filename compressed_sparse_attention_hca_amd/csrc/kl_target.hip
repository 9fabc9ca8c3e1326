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
// The lane's index within the wave, formed by instructions the compiler cannot merge with
// an earlier copy (so a value needed only after the key loop is formed there instead of
// being kept in, or spilled from, a register across the loop).
__device__ inline int lane_id_fresh() {
  int v;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(v));
  return v;
}

__global__ __launch_bounds__(256, 2) void kl_target_hd_kernel(KlArgs a) {
  constexpr int D = 512, ROWB = 1024, KT = 64;
  __shared__ __attribute__((aligned(1024))) unsigned char tile[KT * ROWB];
  __shared__ float2 cs[64];
  __shared__ float stat[2][2][32][2];  // [hg][kh][head][m, l]
  auto swz = [](int r) -> int { return ((r & 3) << 1) | ((r >> 2) & 1); };

  const int gi = a.B * a.S - 1 - (int)blockIdx.x;  // latest queries first
  const int b = gi / a.S, t = gi % a.S;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
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
  for (int k = nsel + 64 * wave_u + lane_id_fresh(); k < a.topk; k += 256) orow[k] = 0.f;
}

// ---------------------------------------------------------------------------------
// bf16 fast path for D = 512, up to 64 heads and at most 512 selected entries: one pass
// over the keys, one workgroup per CU.  Wave w = (hg, dh) owns heads 32hg .. 32hg+31
// and latent half dh (dims 256dh .. 256dh+255), as in the attention forward; the
// logits are S[head, key] = Q . K^T on v_mfma_f32_32x32x16_bf16 with the rotated
// query's head rows as A (head row r is head 32hg + (r ^ 16dh), so rows 0..15 are
// the wave's own 16 heads) and the tile's key rows as B (key = column = lane % 32).
// The partner waves (same hg, other dh) swap the partial sums of each other's heads
// through LDS, so each wave ends a tile with the full logits of its own 16 heads for
// all 32 keys: 8 per lane, keys across lanes.
//
// Every probability is kept until the end of the query: e = 2^(z - m_ref) with the
// first tile's per-head maximum as the reference (shift invariance; the exact
// maximum and a second pass take over when a later logit is more than 64 log2 units
// away), 8 registers per tile, 128 for 512 keys.  At the end each head's sum l is
// reduced across the lanes, and T[key] = (1/H) sum_h e[h, key] / l_h is summed over
// the lane's 8 heads, the two lane halves (v_permlane32_swap) and the four waves (LDS).
// So the keys are gathered and multiplied once, with no statistics pass.
//
// The selected rows are copied straight into a four-stage LDS ring (32 rows of 1 KB
// per stage, chunks XOR-swizzled as in the attention forward) by assembly
// global_load_lds copies: three tiles are in flight while one is multiplied.  One
// barrier per tile serves as the partner exchange of tile t, the arrival of tile t+1
// and the release of tile t's stage; tile t+1's products are issued before tile t's
// exponentials, so the two overlap.
// ---------------------------------------------------------------------------------
constexpr int KLP_KT = 32;       // keys per tile
constexpr int KLP_STAGES = 4;
constexpr int KLP_MAX_TILES = 16;  // 512 selected entries

// Reductions over the 32 lanes of each lane half (lanes 0..31 and 32..63), the result
// in every lane of the half, with no LDS round trip: DPP swaps within quads, the
// 8-lane and 16-lane mirrors, then v_permlane16_swap exchanges the two 16-lane rows of
// the half (each operand copy comes back holding one row's values in both rows).
__device__ inline float klp_dpp(float x, int ctrl) {
  switch (ctrl) {  // the control must be an immediate
    case 0xB1: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
    case 0x4E: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));
    case 0x141: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, false));
    default: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, false));
  }
}
template <bool MAX> __device__ inline void klp_reduce32(float (&x)[8]) {
  constexpr int ctrl[4] = {0xB1, 0x4E, 0x141, 0x140};  // xor 1, xor 2, half-row mirror, row mirror
#pragma unroll
  for (int st = 0; st < 4; ++st)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float y = klp_dpp(x[i], ctrl[st]);
      x[i] = MAX ? fmaxf(x[i], y) : x[i] + y;
    }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x[i]), __float_as_uint(x[i]), false, false);
    const float a0 = __uint_as_float(r[0]), a1 = __uint_as_float(r[1]);
    x[i] = MAX ? fmaxf(a0, a1) : a0 + a1;
  }
}
// Values kept in AGPRs for the whole key loop (the probabilities of every tile), so the
// VGPRs stay free for the fragment read-ahead.  The value usually comes straight from
// v_exp_f32: a VALU instruction may read a transcendental's result only after one wait
// state, and the compiler does not pad for an instruction inside inline assembly (without
// the s_nop the write picks up the exponential's argument), so the assembly pads itself.
__device__ inline float klp_to_agpr(float v) {
  float a;
  asm volatile("s_nop 1\n\tv_accvgpr_write_b32 %0, %1" : "=a"(a) : "v"(v));
  return a;
}
__device__ inline float klp_from_agpr(float a) {
  float v;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
  return v;
}

// Wait until at most n of this wave's vector-memory operations are outstanding, then
// for every wave (LDS accesses completed too).
template <int N> __device__ inline void klp_wait_barrier() {
  static_assert(N == 0 || N == 8 || N == 16 || N == 24, "vmcnt values used by the ring");
  if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 8) asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 16) asm volatile("s_waitcnt vmcnt(16) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(24) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__global__ __launch_bounds__(256, 1) void kl_target_pipe_kernel(KlArgs a) {
  constexpr int D = 512, ROWB = 1024, KT = KLP_KT, NS = KLP_STAGES;
  // Key rows padded to RP = 1040 bytes and key x of each 16-key half in row slot
  // 4(x&3) + (x>>2): the 16-byte B-operand reads (16 lanes = 16 consecutive keys at one
  // chunk) then meet 16 distinct bank groups of gfx950's 64 banks.
  constexpr int RP = ROWB + 16, STG = KT * RP;
  auto slot = [](int key) -> int { return (key & 16) | ((key & 3) << 2) | ((key >> 2) & 3); };
  __shared__ __attribute__((aligned(16))) unsigned char ring[NS * STG];
  // partner exchange, [parity][wave][lane] x 8 floats; the RoPE table borrows it
  __shared__ __attribute__((aligned(16))) unsigned char xbuf[2 * 4 * 64 * 32];
  __shared__ int ovf;
  float2* cs = reinterpret_cast<float2*>(xbuf);

  const int gi = a.B * a.S - 1 - (int)blockIdx.x;  // latest queries first
  const int b = gi / a.S, t = gi % a.S;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hg = wave >> 1, dh = wave & 1;
  const int l32 = lane & 31, g = lane >> 5;
  const int n_t = visible_entries(t, a.ratio);
  const int nsel = min(a.topk, n_t);
  const int ntiles = (nsel + KT - 1) / KT;
  float* orow = a.target + ((int64_t)b * a.S + t) * a.topk;
  if (ntiles == 0) {
    for (int k = threadIdx.x; k < a.topk; k += 256) orow[k] = 0.f;
    return;
  }
  const int32_t* irow = a.idx + ((int64_t)b * a.S + t) * a.topk;
  const unsigned char* qg = static_cast<const unsigned char*>(a.q) + ((int64_t)b * a.S + t) * a.H * ROWB;
  const unsigned char* kvb = static_cast<const unsigned char*>(a.kv_c) + (int64_t)b * a.n_entries * ROWB;

  if (threadIdx.x < a.R / 2) {
    float c, s;
    rope_cos_sin(a.pos0 + t, rope_inv_freq(threadIdx.x, a.R, a.theta), &c, &s);
    cs[threadIdx.x] = make_float2(c, s);
  }

  // Entry indices: lane (l32, g) holds key l32 of tile 2m + g in sidx[m] (-1 past the
  // selection).  Every lane loads (from a clamped position), with no branch, so the
  // loads are in flight together.
  int sidx[KLP_MAX_TILES / 2];
#pragma unroll
  for (int m = 0; m < KLP_MAX_TILES / 2; ++m) sidx[m] = irow[min((2 * m + g) * KT + l32, nsel - 1)];
#pragma unroll
  for (int m = 0; m < KLP_MAX_TILES / 2; ++m)
    if ((2 * m + g) * KT + l32 >= nsel) sidx[m] = -1;
  // A operand: head row l32 is head 32hg + (l32 ^ 16dh); k-step k holds dims
  // 256dh + 16k + 8g .. +7.  Heads past H load head H-1 (their sums are never used).
  const int hrow = 32 * hg + (l32 ^ (16 * dh));
  bf16x8 qf[16];
  {
    const unsigned char* q0 = qg + (int64_t)min(hrow, a.H - 1) * ROWB + 2 * (256 * dh + 8 * g);
#pragma unroll
    for (int k = 0; k < 16; ++k) qf[k] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(q0 + 32 * k));
  }
  __syncthreads();  // the RoPE table is written; q and the indices have arrived
  {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    const int rlo = D - a.R;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int d0 = 256 * dh + 16 * k + 8 * g;
      if (d0 + 8 > rlo) {
        u32x4 w = __builtin_bit_cast(u32x4, qf[k]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = d0 + 2 * j;
          if (d >= rlo) {
            const float2 r = cs[(d - rlo) >> 1];
            const float x0 = __uint_as_float(w[j] << 16), x1 = __uint_as_float(w[j] & 0xffff0000u);
            const float y0 = x0 * r.x - x1 * r.y, y1 = x0 * r.y + x1 * r.x;
            w[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{y0, y1}, bf16x2_t));
          }
        }
        qf[k] = __builtin_bit_cast(bf16x8, w);
      }
    }
  }
  // q and the indices have landed; the explicit wait tells the compiler so, since
  // otherwise it keeps waits for them in the first products, and in hardware those
  // waits would drain the copies issued after them
  __builtin_amdgcn_s_waitcnt(0x0F70);  // gfx9 encoding of vmcnt(0), expcnt and lgkmcnt not waited

  // Row addresses of tiles 2m (lanes 0..31) and 2m+1 (lanes 32..63); an index outside
  // 0 .. n_t-1 reads the query's own q row instead (finite data, masked out).
  auto row_src = [&](int m, uint32_t* lo, uint32_t* hi) -> uint64_t {
    const int s = sidx[m];
    const bool ok = s >= 0 && s < n_t;
    const uint64_t sp = reinterpret_cast<uint64_t>(ok ? kvb + (int64_t)s * ROWB : qg);
    *lo = (uint32_t)sp;
    *hi = (uint32_t)(sp >> 32);
    return __ballot(ok);
  };
  const uint32_t dma_off = (uint32_t)lane << 4;
  uint32_t kmask[KLP_MAX_TILES];
  // Copy tile `tile` into stage tile % NS: wave w copies keys w, w+4, ... (8 rows, one
  // 1 KB wave load each; key w + 4m into slot 16(m>>2) + 4w + (m&3)); the compiler does
  // not see these loads, so it adds no waits for them; klp_wait_barrier is the only
  // wait.
  auto issue = [&](int tile) {
    uint32_t lo, hi;
    const uint64_t bits = row_src(tile >> 1, &lo, &hi);
    kmask[tile] = (uint32_t)(bits >> (32 * (tile & 1)));
    const uint32_t lds0 = (uint32_t)(uintptr_t)(CSA_LDS unsigned char*)(ring + (tile % NS) * STG);
#pragma unroll
    for (int m = 0; m < KT / 4; ++m) {
      const int r = wave + 4 * m;
      const int src_lane = 32 * (tile & 1) + r;
      const uint64_t row = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)hi, src_lane) << 32) |
                           (uint32_t)__builtin_amdgcn_readlane((int)lo, src_lane);
      const uint32_t lds = __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)slot(r) * RP);
      // s_nop 4: the row base was just written to SGPRs by v_readlane, which a vector
      // memory instruction may read only 5 wait states later (and M0 needs 1).
      asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(dma_off), "s"(row), "{m0}"(lds) : "memory");
    }
  };

  // B operand reads: key l32, dims 256dh + 16k + 8g .. +7 at slot(l32) RP + 512dh + 16g + 32k
  const int kb_base = slot(l32) * RP + 512 * dh + 16 * g;
  // The fragment reads run KA ahead of the MFMAs that consume them, pinned with
  // scheduling groups (the compiler otherwise waits for each read just before its MFMA).
  constexpr int KA = 3;
  auto qk = [&](int tile) -> f32x16 {
    const CSA_LDS unsigned char* lb = (const CSA_LDS unsigned char*)(ring + (tile % NS) * STG);
    auto ld = [&](int k) {
      return __builtin_bit_cast(bf16x8, *(const CSA_LDS u32x4*)(lb + kb_base + 32 * k));
    };
    bf16x8 kf[KA + 1];
#pragma unroll
    for (int k = 0; k < KA; ++k) kf[k] = ld(k);
    f32x16 s = {};
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (k + KA < 16) kf[(k + KA) % (KA + 1)] = ld(k + KA);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[k], kf[k % (KA + 1)], s, 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, KA, 0);
#pragma unroll
    for (int k = 0; k < 16 - KA; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, KA, 0);
    return s;
  };
  // exchange slot of (parity, wave, lane): the partner's is xo ^ 2048
  const int xo = 2048 * wave + 32 * lane;
  auto send = [&](int tile, const f32x16& s) {
    CSA_LDS unsigned char* xb = (CSA_LDS unsigned char*)xbuf + 8192 * (tile & 1) + xo;
    *(CSA_LDS f32x4*)xb = f32x4{s[8], s[9], s[10], s[11]};
    *(CSA_LDS f32x4*)(xb + 16) = f32x4{s[12], s[13], s[14], s[15]};
  };

  const float sl2 = a.scale_log2;
  float e[KLP_MAX_TILES][8];
  float m_ref[8], m_seen[8], l[8];
  bool forced = false;  // some head's reference was taken as 0 (its first tile all masked)
  if (threadIdx.x == 0) ovf = 0;
  float* part = reinterpret_cast<float*>(ring);  // [wave][512], once the ring is idle
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      m_seen[i] = -INFINITY;
      l[i] = 0.f;
    }
    __syncthreads();  // the exchange area (RoPE table) is free; the ring is idle
#pragma unroll
    for (int j = 0; j < NS; ++j)
      if (j < ntiles) issue(j);
    if (ntiles > 3) klp_wait_barrier<24>();  // tile 0 landed; tiles 1..3 in flight
    else if (ntiles == 3) klp_wait_barrier<16>();
    else if (ntiles == 2) klp_wait_barrier<8>();
    else klp_wait_barrier<0>();
    f32x16 s = qk(0);
    send(0, s);
#pragma unroll
    for (int tl = 0; tl < KLP_MAX_TILES; ++tl) {
      if (tl < ntiles) {
        // tile tl+1 landed (tiles up to tl+3 were issued); the partials of tile tl are
        // in LDS; every wave is done reading stage tl % NS
        const int after = min(ntiles - 1, tl + 3) - (tl + 1);
        if (after >= 2) klp_wait_barrier<16>();
        else if (after == 1) klp_wait_barrier<8>();
        else klp_wait_barrier<0>();
        if (tl + NS < ntiles) issue(tl + NS);
        const CSA_LDS unsigned char* xr = (const CSA_LDS unsigned char*)xbuf + 8192 * (tl & 1) + (xo ^ 2048);
        const f32x4 p0 = *(const CSA_LDS f32x4*)xr, p1 = *(const CSA_LDS f32x4*)(xr + 16);
        __builtin_amdgcn_sched_barrier(0);  // the partner's sums are read before the fragments
        f32x16 sn = {};
        if (tl + 1 < ntiles) sn = qk(tl + 1);
        float z[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          z[i] = s[i] + p0[i];
          z[4 + i] = s[4 + i] + p1[i];
        }
        const uint32_t km = kmask[tl];
        if (km != 0xffffffffu) {
          const bool ok = (km >> l32) & 1u;
#pragma unroll
          for (int i = 0; i < 8; ++i) z[i] = ok ? z[i] : -INFINITY;
        }
        if (tl == 0 && pass == 0) {
#pragma unroll
          for (int i = 0; i < 8; ++i) m_ref[i] = z[i];
          klp_reduce32<true>(m_ref);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            forced |= m_ref[i] == -INFINITY;
            m_ref[i] = m_ref[i] == -INFINITY ? 0.f : m_ref[i];
          }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          m_seen[i] = fmaxf(m_seen[i], z[i]);
          const float ev = __builtin_amdgcn_exp2f((z[i] - m_ref[i]) * sl2);
          l[i] += ev;
          e[tl][i] = klp_to_agpr(ev);
        }
        if (tl + 1 < ntiles) send(tl + 1, sn);
        s = sn;
      }
    }
    // A second pass with the exact maximum is needed if some probability could have
    // overflowed or (reference taken as 0 after an all-masked first tile) underflowed.
    // The reference is each head's maximum over a subset of its keys, so unless it was
    // forced to 0 only overflow is possible, and the lane's own maximum tells: no
    // reduction across lanes.  The targets are formed before the decision (and formed
    // again after a second pass), so one barrier serves both.
    bool bad = false;
    if (__any(forced)) {
      float mall[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) mall[i] = m_seen[i];
      klp_reduce32<true>(mall);
#pragma unroll
      for (int i = 0; i < 8; ++i) bad |= mall[i] != -INFINITY && fabsf((mall[i] - m_ref[i]) * sl2) > 64.0f;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) bad |= (m_seen[i] - m_ref[i]) * sl2 > 64.0f;
    }
    if (pass == 0 && __any(bad) && lane == 0) ovf = 1;
    // T[key] = (1/H) sum_h e[h, key] / l_h: the lane's 8 heads, the two lane halves (the
    // wave's 16 heads), then the four waves through LDS (the ring is idle now)
    float inv[8];
    klp_reduce32<false>(l);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int h = 32 * hg + ((8 * (i >> 2) + 4 * g + (i & 3)) ^ (16 * dh));
      inv[i] = (h < a.H && l[i] > 0.f) ? __builtin_amdgcn_rcpf(l[i]) : 0.f;
    }
#pragma unroll
    for (int tl = 0; tl < KLP_MAX_TILES; ++tl) {
      if (tl < ntiles) {
        float v = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) v = fmaf(klp_from_agpr(e[tl][i]), inv[i], v);
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
        if (g == 0) part[wave * 512 + tl * KT + l32] = v;
      }
    }
    __syncthreads();
    if (pass == 1 || !ovf) break;
    klp_reduce32<true>(m_seen);  // the exact maximum
#pragma unroll
    for (int i = 0; i < 8; ++i) m_ref[i] = m_seen[i] == -INFINITY ? 0.f : m_seen[i];
  }

  const float inv_h = __builtin_amdgcn_rcpf((float)a.H);
  for (int k = threadIdx.x; k < a.topk; k += 256) {
    float v = 0.f;
    if (k < nsel) v = ((part[k] + part[512 + k]) + (part[1024 + k] + part[1536 + k])) * inv_h;
    orow[k] = v;
  }
}

hipError_t launch_kl_target(const csa_params_t& p, const void* q, const void* kv_c, const int32_t* idx,
                            float* target, hipStream_t st) {
  KlArgs a{q, kv_c, idx, target, p.B, p.S, p.H, p.rope_dim, p.ratio, p.topk, p.S / p.ratio,
           p.rope_theta, p.pos0, p.softmax_scale * 1.4426950408889634f};
  const int grid = p.B * p.S;
  if (grid == 0) return hipSuccess;
  if (p.dtype == CSA_BF16 && p.D == 512 && p.topk <= KLP_MAX_TILES * KLP_KT) {
    hipLaunchKernelGGL(kl_target_pipe_kernel, dim3(grid), dim3(256), 0, st, a);
    return hipGetLastError();
  }
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
