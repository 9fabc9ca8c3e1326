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
// dims.  Keys stream through LDS in tiles of 32, shared by every head.  Per tile:
//   S^T[key, head] = K_tile . Q^T     v_mfma_f32_16x16x32_bf16, keys on M (A from LDS,
//                                     row-major), heads on N (B = rotated q in regs)
//   online softmax in registers, base-2, max rescale only when the tile max grows by
//   more than 2^8 (exact: the final normalisation uses the same reference)
//   O^T[dim, head] += V^T . P^T       dims on M (A from a transposed LDS copy of the
//                                     tile), heads on N (B = P straight from S^T)
// The S^T accumulator gives lane (head, g) keys 4g..4g+3 and 16+4g..16+4g+3; those 8
// are exactly that lane's B-operand k-slots for PV if the transposed copy stores key
// sigma(g,i) at slot 8g+i, so P never leaves registers.
#include "common.hpp"
#include "launch.hpp"

namespace csa {

struct MqaArgs {
  const void* q;
  const void* kv_c;
  const void* kv_w;
  const int32_t* idx;
  void* o;
  int32_t B, S, H, R, ratio, window, topk, n_entries, mode;
  float scale_log2;  // softmax_scale * log2(e)
  double theta;
  int64_t pos0;
};

// Key slot (within a tile of 32) held at k-slot i of lane group g.
__device__ __host__ constexpr int slot_key(int g, int i) { return i < 4 ? 4 * g + i : 12 + 4 * g + i; }

template <typename T, int D, int NW>
__global__ __launch_bounds__(NW * 64) void sparse_mqa_kernel(MqaArgs a) {
  constexpr int NT = NW * 64;
  constexpr int HP = NW * 16;                 // heads handled (padded)
  constexpr int VEC = 16 / sizeof(T);         // elements per 16-byte piece
  constexpr int KT = 32;                      // keys per tile
  constexpr int QROW = D + VEC;               // padded row of the q / o staging
  constexpr int KROW = D + VEC;               // padded row of the key tile
  constexpr int VROW = KT + VEC;              // padded row of the transposed tile
  constexpr int NCH = D / VEC;                // 16-byte pieces per latent row
  constexpr int NBLK = 4 * NCH;               // staging blocks (8 keys x VEC dims) per tile
  constexpr int BPT = (NBLK + NT - 1) / NT;   // blocks per thread
  constexpr int SZ_Q = HP * QROW * (int)sizeof(T);
  constexpr int SZ_KV = (KT * KROW + D * VROW) * (int)sizeof(T);
  constexpr int SZ = SZ_Q > SZ_KV ? SZ_Q : SZ_KV;
  __shared__ __attribute__((aligned(16))) unsigned char smem[SZ];
  __shared__ int kvalid[KT];
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

  // ---- q[b,t] (H x D, contiguous) -> LDS, coalesced; rows >= H are zero
  T* qs = reinterpret_cast<T*>(smem);
  const T* qg = static_cast<const T*>(a.q) + ((int64_t)b * a.S + t) * a.H * D;
  for (int c = threadIdx.x; c < HP * NCH; c += NT) {
    const int row = c / NCH, col = (c % NCH) * VEC;
    Vec16<T> v;
    if (row < a.H) v = load16(qg + (int64_t)row * D + col);
    else *reinterpret_cast<uint4*>(v.v) = make_uint4(0, 0, 0, 0);
    store16(qs + row * QROW + col, v);
  }
  __syncthreads();

  // ---- Q^T fragments (B operand): lane (head 16w+hl, group g), k-step k holds dims
  // 32k + 8g .. +7, rotated at +P where they fall in the last R dims.
  Frag<T> qf[D / 32];
#pragma unroll
  for (int k = 0; k < D / 32; ++k) {
    const int d0 = 32 * k + 8 * g;
    qf[k] = load_frag(qs + (16 * wave + hl) * QROW + d0);
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
  __syncthreads();  // the q staging area becomes the key tile

  T* krm = reinterpret_cast<T*>(smem);  // [KT][KROW]  key-major
  T* vt = krm + KT * KROW;              // [D][VROW]   dim-major, slot-permuted
  const T* kv_c = static_cast<const T*>(a.kv_c);
  const T* kv_w = static_cast<const T*>(a.kv_w);
  const int32_t* irow = a.mode == MQA_SELECTED ? a.idx + ((int64_t)b * a.S + t) * a.topk : nullptr;

  // Address of key kk of this query's list, or null if it is masked.
  auto key_ptr = [&](int kk) -> const T* {
    if (kk < nsel) {
      const int s = irow ? irow[kk] : kk;
      if (s < 0 || s >= n_t) return nullptr;  // malformed selection: ignored
      return kv_c + ((int64_t)b * a.n_entries + s) * D;
    }
    if (kk < nk) return kv_w + ((int64_t)b * a.S + wlo + (kk - nsel)) * D;
    return nullptr;
  };

  // Staging block bi: key group gq = bi & 3 (keys sigma(gq, 0..7)), dims (bi >> 2)*VEC.
  uint4 pf[BPT][8];
  int pbits[BPT];
  auto fetch = [&](int tile) {
#pragma unroll
    for (int k = 0; k < BPT; ++k) {
      const int bi = threadIdx.x + k * NT;
      int bits = 0;
      if (bi < NBLK) {
        const int gq = bi & 3, col = (bi >> 2) * VEC;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const T* p = key_ptr(tile * KT + slot_key(gq, i));
          pf[k][i] = p ? *reinterpret_cast<const uint4*>(p + col) : make_uint4(0, 0, 0, 0);
          bits |= (p != nullptr) << i;
        }
      }
      pbits[k] = bits;
    }
  };
  auto commit = [&]() {
#pragma unroll
    for (int k = 0; k < BPT; ++k) {
      const int bi = threadIdx.x + k * NT;
      if (bi < NBLK) {
        const int gq = bi & 3, col = (bi >> 2) * VEC;
#pragma unroll
        for (int i = 0; i < 8; ++i)
          *reinterpret_cast<uint4*>(krm + slot_key(gq, i) * KROW + col) = pf[k][i];
        // transpose: for each dim of the piece, the 8 keys in slot order
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
          T col8[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) col8[i] = reinterpret_cast<const T*>(&pf[k][i])[j];
          T* dst = vt + (col + j) * VROW + 8 * gq;
          *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(col8);
          if constexpr (sizeof(T) == 4)
            *reinterpret_cast<uint4*>(dst + 4) = *reinterpret_cast<const uint4*>(col8 + 4);
        }
        if (col == 0) {
#pragma unroll
          for (int i = 0; i < 8; ++i) kvalid[slot_key(gq, i)] = (pbits[k] >> i) & 1;
        }
      }
    }
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 O[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) O[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int ntiles = (nk + KT - 1) / KT;
  if (ntiles > 0) {
    fetch(0);
    commit();
  }
  __syncthreads();
  for (int tile = 0; tile < ntiles; ++tile) {
    if (tile + 1 < ntiles) fetch(tile + 1);

    // S^T = K . Q^T : keys 0..15 and 16..31 of the tile
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < D / 32; ++k) {
      const Frag<T> a0 = load_frag(krm + hl * KROW + 32 * k + 8 * g);
      const Frag<T> a1 = load_frag(krm + (16 + hl) * KROW + 32 * k + 8 * g);
      s0 = mfma16x16x32(a0, qf[k], s0);
      s1 = mfma16x16x32(a1, qf[k], s1);
    }
    float z[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      z[i] = kvalid[4 * g + i] ? s0[i] * a.scale_log2 : -INFINITY;
      z[4 + i] = kvalid[16 + 4 * g + i] ? s1[i] * a.scale_log2 : -INFINITY;
    }
    float mt = z[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mt = fmaxf(mt, z[i]);
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    if (__any(mt > m_run + 8.0f)) {
      const float mn = fmaxf(m_run, mt);
      const float al = (m_run == -INFINITY) ? 0.f : exp2f(m_run - mn);
#pragma unroll
      for (int db = 0; db < D / 16; ++db) O[db] *= al;
      l_run *= al;
      m_run = mn;
    }
    const float mref = (m_run == -INFINITY) ? 0.f : m_run;
    Frag<T> pfr;
    float ls = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p = exp2f(z[i] - mref);
      ls += p;
      pfr.v[i] = from_f32<T>(p);
    }
    l_run += ls;

    // O^T += V^T . P^T
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      const Frag<T> av = load_frag(vt + (16 * db + hl) * VROW + 8 * g);
      O[db] = mfma16x16x32(av, pfr, O[db]);
    }
    __syncthreads();
    if (tile + 1 < ntiles) {
      commit();
      __syncthreads();
    }
  }

  // ---- normalise, de-rotate at -P, stage through LDS, write o[b,t] coalesced
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
  T* os = reinterpret_cast<T*>(smem);
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
    T* dst = os + (16 * wave + hl) * QROW + d0;
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = from_f32<T>(x[i]);
  }
  __syncthreads();
  T* og = static_cast<T*>(a.o) + ((int64_t)b * a.S + t) * a.H * D;
  for (int c = threadIdx.x; c < a.H * NCH; c += NT) {
    const int row = c / NCH, col = (c % NCH) * VEC;
    store16(og + (int64_t)row * D + col, load16(os + row * QROW + col));
  }
}

template <typename T, int D>
static void launch_d(const MqaArgs& a, int H, hipStream_t st) {
  dim3 grid(a.B * a.S);
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
                             const void* kv_w, const int32_t* idx, void* o, hipStream_t st) {
  MqaArgs a{};
  a.q = q;
  a.kv_c = kv_c;
  a.kv_w = kv_w;
  a.idx = idx;
  a.o = o;
  a.B = p.B;
  a.S = p.S;
  a.H = p.H;
  a.R = p.rope_dim;
  a.ratio = p.ratio;
  a.window = p.window;
  a.topk = p.topk;
  a.n_entries = mode == MQA_WINDOW_ONLY ? 0 : p.S / p.ratio;
  a.mode = mode;
  a.scale_log2 = p.softmax_scale * 1.4426950408889634f;
  a.theta = p.rope_theta;
  a.pos0 = p.pos0;
  if (p.B * p.S == 0) return hipSuccess;
  return p.dtype == CSA_BF16 ? launch_t<bf16>(a, p.D, p.H, st) : launch_t<float>(a, p.D, p.H, st);
}

}  // namespace csa
