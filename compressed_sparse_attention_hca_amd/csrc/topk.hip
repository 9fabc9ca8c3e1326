// Stage 3b on gfx950: top-k selection of indexer scores per query row.
//
// The selection lives in [B, S, K] ("fix(deepseek-v4): correct V4-Flash attention
// math", Part 1 item 5: the computation stays in [B,S,K] and the dense per-head tensor
// is never formed); V4-Flash keeps the best 512 entries ("Enabling DeepSeek-V4-Flash
// Training on AMD Instinct MI355X GPUs with Primus", "Three attention types,
// interleaved").
//
// One workgroup per row.  The output is the exact set that a stable sort by
// (-score, index) selects, in ascending index order, so results are deterministic.
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
//
// 1. Keys (order-preserving uint32) are read once into registers; the row's min and
//    max give the bits every key shares.
// 2. One histogram pass over the 8-bit digit below the shared bits finds the digit B
//    holding the k-th largest key: keys with digit > B are selected outright, keys with
//    digit == B are candidates for the remaining kRem slots.
// 3. The candidates (a few dozen for realistic rows) are compacted into LDS and ranked
//    exactly by (key desc, index asc); the kRem best are selected.
// 4. Selection is kept as a bitmap, one 64-bit ballot per 64 consecutive indices, and a
//    scan over the bitmap writes the indices in ascending order.
// Rows with more than CAND candidates (many keys crowding one digit) continue with
// further radix passes over all keys instead.
template <int NT, int ITEMS>
__global__ __launch_bounds__(NT) void topk_kernel(TopkArgs a) {
  constexpr int NW = NT / 64;
  constexpr int NWORD = ITEMS * NW;  // 64-bit bitmap words (64 indices each)
  constexpr int CAND = 2048;
  static_assert(NWORD <= NT, "one scan pass over the bitmap words");
  __shared__ int hist[NW][256];
  __shared__ int scan_buf[NW];
  __shared__ int sel_digit, sel_above, sel_count, cand_n;
  __shared__ uint64_t bitmap[NWORD];
  __shared__ uint32_t cand_key[CAND];
  __shared__ int cand_idx[CAND];
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
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, m, 64));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, m, 64));
  }
  if (lane == 0) { red_min[wave] = kmin; red_max[wave] = kmax; }
  for (int i = threadIdx.x; i < NW * 256; i += NT) (&hist[0][0])[i] = 0;
  if (threadIdx.x == 0) cand_n = 0;
  __syncthreads();
  kmin = red_min[0];
  kmax = red_max[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) { kmin = min(kmin, red_min[w]); kmax = max(kmax, red_max[w]); }
  const uint32_t diff = kmin ^ kmax;
  const int hi = diff ? 32 - __clz(diff) : 0;  // bits [hi, 32) are common to all keys
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

  // ---- pass 1: histogram of the digit right below the common bits (all keys take part)
  const int width = hi >= 8 ? 8 : hi;
  const int lo = hi - width;
  const uint32_t dmask = (1u << width) - 1u;
  if (width > 0) {
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
      const int i = it * NT + threadIdx.x;
      if (i < n) atomicAdd(&hist[wave][(key[it] >> lo) & dmask], 1);
    }
  } else if (threadIdx.x == 0) {
    hist[0][0] = n;  // every key is equal: one bin
  }
  __syncthreads();
  {
    int c = 0;
    const int d = 255 - (int)threadIdx.x;  // threads 0.. hold digits 255..
    if (threadIdx.x < 256 && d <= (int)dmask) {
#pragma unroll
      for (int w = 0; w < NW; ++w) c += hist[w][d];
    }
    int tot;
    const int above = block_excl_scan<NT>(threadIdx.x < 256 ? c : 0, scan_buf, &tot);
    if (threadIdx.x < 256 && c > 0 && above < K && K <= above + c) {
      sel_digit = d;
      sel_above = above;
      sel_count = c;
    }
  }
  __syncthreads();
  const uint32_t B = (uint32_t)sel_digit;
  const int kRem = K - sel_above;
  const int cB = sel_count;

  if (cB <= CAND) {
    // ---- selected-outright bitmap and candidate compaction
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
      const int i = it * NT + threadIdx.x;
      const uint32_t dg = width > 0 ? (key[it] >> lo) & dmask : 0u;
      const bool gt = i < n && dg > B;
      const bool eq = i < n && dg == B;
      const uint64_t bg = __ballot(gt), be = __ballot(eq);
      if (lane == 0) bitmap[it * NW + wave] = bg;
      if (be) {
        int base = 0;
        if (lane == 0) base = atomicAdd(&cand_n, __popcll(be));
        base = __shfl(base, 0, 64);
        if (eq) {
          const int pos = base + __popcll(be & lt);
          cand_key[pos] = key[it];
          cand_idx[pos] = i;
        }
      }
    }
    __syncthreads();
    // ---- exact rank of each candidate among the candidates; the kRem best are kept
    const int C = cand_n;
    for (int c = threadIdx.x; c < C; c += NT) {
      const uint32_t kc = cand_key[c];
      const int ic = cand_idx[c];
      int rank = 0;
      for (int j = 0; j < C; ++j) {
        const uint32_t kj = cand_key[j];
        rank += (kj > kc) || (kj == kc && cand_idx[j] < ic);
      }
      if (rank < kRem) atomicOr((unsigned long long*)&bitmap[ic >> 6], 1ull << (ic & 63));
    }
  } else {
    // ---- many keys in one digit: further radix passes over all keys
    uint64_t prefix = ((uint64_t)kmin >> hi << width) | B;
    int shift = lo;
    int rem = kRem;
    bool exact = false;
    while (shift > 0 && !exact) {
      const int w2 = shift >= 8 ? 8 : shift;
      const int lo2 = shift - w2;
      __syncthreads();
      for (int i = threadIdx.x; i < NW * 256; i += NT) (&hist[0][0])[i] = 0;
      __syncthreads();
#pragma unroll
      for (int it = 0; it < ITEMS; ++it) {
        const int i = it * NT + threadIdx.x;
        if (i < n && ((uint64_t)key[it] >> shift) == prefix)
          atomicAdd(&hist[wave][(key[it] >> lo2) & ((1u << w2) - 1u)], 1);
      }
      __syncthreads();
      int c = 0;
      const int d = 255 - (int)threadIdx.x;
      if (threadIdx.x < 256 && d < (1 << w2)) {
#pragma unroll
        for (int w = 0; w < NW; ++w) c += hist[w][d];
      }
      int tot;
      const int above = block_excl_scan<NT>(threadIdx.x < 256 ? c : 0, scan_buf, &tot);
      if (threadIdx.x < 256 && c > 0 && above < rem && rem <= above + c) {
        sel_digit = d;
        sel_above = above;
        sel_count = c;
      }
      __syncthreads();
      rem -= sel_above;
      prefix = (prefix << w2) | (uint64_t)sel_digit;
      shift = lo2;
      exact = sel_count == rem;  // every key with this prefix is selected
    }
    // keys above the prefix are selected; keys equal to it fill `rem` slots in index
    // order (ranks from a scan over (item, wave) ballot counts)
    __syncthreads();
    int* cnt = reinterpret_cast<int*>(cand_key);  // reuse: NWORD counts
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
      const int i = it * NT + threadIdx.x;
      const uint64_t kp = (uint64_t)key[it] >> shift;
      const uint64_t bg = __ballot(i < n && kp > prefix), be = __ballot(i < n && kp == prefix);
      if (lane == 0) {
        bitmap[it * NW + wave] = bg;
        cnt[it * NW + wave] = __popcll(be);
        cand_idx[it * NW + wave] = 0;
      }
    }
    __syncthreads();
    int te;
    const int pe = block_excl_scan<NT>(threadIdx.x < NWORD ? cnt[threadIdx.x] : 0, scan_buf, &te);
    if (threadIdx.x < NWORD) cand_idx[threadIdx.x] = pe;
    __syncthreads();
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
      const int i = it * NT + threadIdx.x;
      const uint64_t kp = (uint64_t)key[it] >> shift;
      const bool eq = i < n && kp == prefix;
      const uint64_t be = __ballot(eq);
      const int r = cand_idx[it * NW + wave] + __popcll(be & lt);
      if (eq && r < rem) atomicOr((unsigned long long*)&bitmap[it * NW + wave], 1ull << lane);
    }
  }
  __syncthreads();

  // ---- write the selected indices in ascending order
  const uint64_t word = threadIdx.x < NWORD ? bitmap[threadIdx.x] : 0ull;
  int tot;
  int pos = block_excl_scan<NT>(__popcll(word), scan_buf, &tot);
  uint64_t wv = word;
  while (wv) {
    const int bit = __ffsll((unsigned long long)wv) - 1;
    wv &= wv - 1;
    if (pos < K) out[pos] = threadIdx.x * 64 + bit;
    ++pos;
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
