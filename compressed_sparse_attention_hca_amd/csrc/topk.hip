// Stage 3b on gfx950: top-k selection of indexer scores per query row.
//
// The selection lives in [B, S, K] ("fix(deepseek-v4): correct V4-Flash attention
// math", Part 1 item 5: the computation stays in [B,S,K] and the dense per-head tensor
// is never formed); V4-Flash keeps the best 512 entries ("Enabling DeepSeek-V4-Flash
// Training on AMD Instinct MI355X GPUs with Primus", "Three attention types,
// interleaved").
//
// One workgroup per row.  The row's fp32 scores are read once, coalesced, into
// registers as order-preserving uint32 keys.  A radix select over 8-bit digits (LDS
// histograms, one per wave) finds the exact k-th key, starting below the bits every key
// shares.  The output is the exact set: every key above the threshold plus the
// smallest-index keys equal to it, written in ascending index order through a
// ballot/prefix scan, so results are deterministic and match a stable sort by
// (-score, index).
#include "common.hpp"
#include "launch.hpp"

namespace csa {

struct TopkArgs {
  const float* scores;
  int64_t ld;
  int32_t* idx;
  int32_t* n_visible;
  int32_t B, S, ratio, topk, t0, nrows;
};

__device__ inline uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f == 0.0f ? 0.0f : f);  // -0 and +0 tie
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum over NT values held one per thread; returns this thread's
// prefix and the total.  `buf` holds NT/64 ints.
template <int NT>
__device__ inline int block_excl_scan(int v, int* buf, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) buf[wave] = x;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int s = buf[w];
    if (w < wave) base += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

// NT threads, ITEMS keys per thread: rows of up to NT*ITEMS visible entries.
template <int NT, int ITEMS>
__global__ __launch_bounds__(NT) void topk_kernel(TopkArgs a) {
  constexpr int NW = NT / 64;
  static_assert(ITEMS * NW <= NT, "one scan pass over the (item, wave) counts");
  __shared__ int hist[NW][256];
  __shared__ int scan_buf[NW];
  __shared__ int sel_digit, sel_above;
  __shared__ int cnt_gt[ITEMS * NW], cnt_eq[ITEMS * NW];
  __shared__ uint64_t msk_gt[ITEMS * NW], msk_eq[ITEMS * NW];
  __shared__ uint32_t red_min[NW], red_max[NW];

  const int row = blockIdx.x;  // over B * nrows
  const int b = row / a.nrows;
  const int trow = row % a.nrows;
  const int t = a.t0 + trow;
  const int n = visible_entries(t, a.ratio);
  const int K = a.topk;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int32_t* out = a.idx + ((int64_t)b * a.S + t) * K;
  if (threadIdx.x == 0 && a.n_visible) a.n_visible[(int64_t)b * a.S + t] = n;

  if (n <= K) {  // every visible entry is selected
    for (int j = threadIdx.x; j < K; j += NT) out[j] = j < n ? j : -1;
    return;
  }

  const float* srow = a.scores + ((int64_t)b * a.nrows + trow) * a.ld;
  uint32_t key[ITEMS];
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    const int i = it * NT + threadIdx.x;
    key[it] = i < n ? order_key(srow[i]) : 0u;
    if (i < n) {
      kmin = min(kmin, key[it]);
      kmax = max(kmax, key[it]);
    }
  }
  // bits shared by every key need no histogram pass
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, m, 64));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, m, 64));
  }
  if (lane == 0) { red_min[wave] = kmin; red_max[wave] = kmax; }
  __syncthreads();
  kmin = red_min[0];
  kmax = red_max[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) { kmin = min(kmin, red_min[w]); kmax = max(kmax, red_max[w]); }
  const uint32_t diff = kmin ^ kmax;
  int hi = diff ? 32 - __clz(diff) : 0;  // bits [hi, 32) are common to all keys

  // Radix select: find prefix P (the key bits above `shift`) of the k-th largest key
  // and kRem, how many keys to take among those whose bits above `shift` equal P.
  // 64-bit so that a shift by 32 (no common bits) is defined
  uint64_t prefix = (uint64_t)kmin >> hi;  // common high bits
  int shift = hi;
  int kRem = K;
  while (shift > 0) {
    const int width = shift >= 8 ? 8 : shift;
    const int lo = shift - width;
    for (int i = threadIdx.x; i < NW * 256; i += NT) (&hist[0][0])[i] = 0;
    __syncthreads();
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
      const int i = it * NT + threadIdx.x;
      if (i < n && ((uint64_t)key[it] >> shift) == prefix)
        atomicAdd(&hist[wave][(key[it] >> lo) & ((1u << width) - 1)], 1);
    }
    __syncthreads();
    // one bin per thread, scanned from the top digit down
    int c = 0;
    const int d = 255 - (int)threadIdx.x;  // threads 0.. hold digits 255..
    if (threadIdx.x < 256 && d < (1 << width)) {
#pragma unroll
      for (int w = 0; w < NW; ++w) c += hist[w][d];
    }
    int tot;
    const int above = block_excl_scan<NT>(threadIdx.x < 256 ? c : 0, scan_buf, &tot);
    if (threadIdx.x < 256 && c > 0 && above < kRem && kRem <= above + c) {
      sel_digit = d;
      sel_above = above;
      hist[0][0] = c;  // count in the selected bin (hist no longer needed)
    }
    __syncthreads();
    const int dsel = sel_digit, asel = sel_above, csel = hist[0][0];
    __syncthreads();
    kRem -= asel;
    prefix = (prefix << width) | (uint64_t)dsel;
    shift = lo;
    if (csel == kRem) break;  // every key with this prefix is selected
  }
  // Selected: (key >> shift) > prefix, or == prefix with equal-rank < kRem (equal keys
  // taken in ascending index order).  Positions come from a scan in index order:
  // index i = it * NT + threadIdx.x, i.e. (it, wave, lane) order.
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    const int i = it * NT + threadIdx.x;
    const uint64_t kp = (uint64_t)key[it] >> shift;
    const bool gt = i < n && kp > prefix;
    const bool eq = i < n && kp == prefix;
    const uint64_t bg = __ballot(gt), be = __ballot(eq);
    if (lane == 0) {
      cnt_gt[it * NW + wave] = __popcll(bg);
      cnt_eq[it * NW + wave] = __popcll(be);
      msk_gt[it * NW + wave] = bg;
      msk_eq[it * NW + wave] = be;
    }
  }
  __syncthreads();
  // exclusive scans over the ITEMS*NW (it, wave) counts, in place
  {
    const int j = threadIdx.x;
    const int vg = j < ITEMS * NW ? cnt_gt[j] : 0;
    const int ve = j < ITEMS * NW ? cnt_eq[j] : 0;
    int tg, te;
    const int pg = block_excl_scan<NT>(vg, scan_buf, &tg);
    const int pe = block_excl_scan<NT>(ve, scan_buf, &te);
    if (j < ITEMS * NW) { cnt_gt[j] = pg; cnt_eq[j] = pe; }
    __syncthreads();
  }
  for (int it = 0; it < ITEMS; ++it) {
    const int i = it * NT + threadIdx.x;
    const uint64_t bg = msk_gt[it * NW + wave], be = msk_eq[it * NW + wave];
    const bool gt = (bg >> lane) & 1, eq = (be >> lane) & 1;
    const int gt_before = cnt_gt[it * NW + wave] + __popcll(bg & lt);
    const int eq_before = cnt_eq[it * NW + wave] + __popcll(be & lt);
    const int pos = gt ? gt_before + min(eq_before, kRem) : gt_before + eq_before;
    if ((gt || (eq && eq_before < kRem)) && pos < K) out[pos] = i;
  }
}

hipError_t launch_topk(const csa_params_t& p, const float* scores, int64_t ld, int32_t t0,
                       int32_t nrows, int32_t* idx, int32_t* n_visible, hipStream_t st) {
  TopkArgs a{scores, ld, idx, n_visible, p.B, p.S, p.ratio, p.topk, t0, nrows};
  const int rows = p.B * nrows;
  if (rows == 0) return hipSuccess;
  const int n_max = visible_entries(t0 + nrows - 1, p.ratio);
  dim3 grid(rows);
  if (n_max <= 256 * 16) hipLaunchKernelGGL((topk_kernel<256, 16>), grid, dim3(256), 0, st, a);
  else if (n_max <= 256 * 64) hipLaunchKernelGGL((topk_kernel<256, 64>), grid, dim3(256), 0, st, a);
  else if (n_max <= 512 * 64) hipLaunchKernelGGL((topk_kernel<512, 64>), grid, dim3(512), 0, st, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace csa
