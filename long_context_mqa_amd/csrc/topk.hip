// Exact top-k selection of candidate keys by head-summed score, for gfx950.
//
// Method (page title and section): arex-research.com, "Xiaomi MiMo lead Luo Fuli
// publishes the MiMo-V3 core architecture HySparse2", section "Outer KV Bridging, inner
// KV Reuse": besides the 128 most recent tokens, each full-attention layer selects
// 1,024 global tokens from outside that window by score. toolnavs.com (German),
// section "Was HySparse2 tut": selection is token-level.
//
// Order used: a key ranks above another if its score is larger, or the scores are equal
// and its position is smaller. Scores are non-negative, so their fp32 bit patterns
// order like the values; the 64-bit key ((bits << 32) | ~position) is then unique per
// candidate and its k largest values are exactly the selection.
//
// Pipeline per query (the score pass already built a histogram of bits 30..19):
//   filter  (many workgroups per query): from the histogram, find the bin b1 that holds
//           the k-th largest; keys with a larger bin are selected outright, keys in b1
//           are copied to a per-query candidate list (up to kCandCap).
//   finish  (one workgroup per query): radix-select the remaining r keys among the b1
//           candidates in LDS (or, if b1 overflowed the list, by streaming the query's
//           scores again), then sort the k positions ascending and write them.
#include "hs2_internal.h"

namespace hs2 {
namespace {

constexpr int kThreads = 256;

// Exclusive prefix sum over the 256 threads of a workgroup (values in thread order).
__device__ inline uint32_t block_excl_scan(uint32_t v, uint32_t* s_wave, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) s_wave[wave] = x;
  __syncthreads();
  uint32_t before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) {
    const uint32_t c = s_wave[w];
    if (w < wave) before += c;
    total += c;
  }
  __syncthreads();
  return before + x - v;
}

// Finds the histogram bin holding the k-th largest element (bins scanned from the top)
// and the number of elements in higher bins. Called by all 256 threads.
__device__ inline void threshold_bin(const uint32_t* __restrict__ hist, int k, uint32_t* s_wave,
                                     int* s_res, int& bin, int& above) {
  constexpr int kPer = kHistBins / kThreads;  // 16 bins per thread, descending
  uint32_t c[kPer];
  uint32_t tot = 0;
  const int top = kHistBins - 1 - threadIdx.x * kPer;
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    c[r] = hist[top - r];
    tot += c[r];
  }
  uint32_t total;
  const uint32_t excl = block_excl_scan(tot, s_wave, total);
  if (threadIdx.x == 0) {
    s_res[0] = 0;
    s_res[1] = 0;
  }
  __syncthreads();
  if (excl < (uint32_t)k && (uint32_t)k <= excl + tot) {
    uint32_t run = excl;
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      if (run < (uint32_t)k && (uint32_t)k <= run + c[r]) {
        s_res[0] = top - r;
        s_res[1] = (int)run;
      }
      run += c[r];
    }
  }
  __syncthreads();
  bin = s_res[0];
  above = s_res[1];
  __syncthreads();
}

__device__ inline int cand_count(int t, int window) { return max(0, t - window + 1); }

// ------------------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void topk_filter_kernel(TopkArgs a) {
  __shared__ uint32_t s_wave[kThreads / 64];
  __shared__ int s_res[2];
  const int i = blockIdx.x / a.n_split;
  const int split = blockIdx.x - i * a.n_split;
  int64_t base;
  int t;
  if (!query_desc(a.b, i, base, t)) return;
  const int nc = cand_count(t, a.window);
  if (a.top_k == 0 || nc <= a.top_k) return;
  const int k0 = split * a.split_len;
  if (k0 >= nc) return;
  const int k1 = min(nc, k0 + a.split_len);

  int b1, above;
  threshold_bin(a.hist + (size_t)i * kHistBins, a.top_k, s_wave, s_res, b1, above);

  const float* sc = a.scores + (size_t)i * a.score_stride;
  uint32_t* cnt = a.counters + (size_t)i * 4;
  int32_t* abv = a.above + (size_t)i * a.top_k;
  uint2* cand = a.cand + (size_t)i * kCandCap;
  const int lane = threadIdx.x & 63;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int p0 = k0; p0 < k1; p0 += kThreads) {
    const int p = p0 + threadIdx.x;
    uint32_t u = 0;
    int d = -1;
    if (p < k1) {
      u = __float_as_uint(sc[p]);
      d = (int)(u >> kHistShift);
    }
    const bool is_above = d > b1;
    const bool is_bin = d == b1;
    const uint64_t ma = __ballot(is_above);
    const uint64_t mb = __ballot(is_bin);
    uint32_t base_a = 0, base_b = 0;
    if (lane == 0) {
      if (ma) base_a = atomicAdd(&cnt[0], (uint32_t)__popcll(ma));
      if (mb) base_b = atomicAdd(&cnt[1], (uint32_t)__popcll(mb));
    }
    base_a = __shfl(base_a, 0);
    base_b = __shfl(base_b, 0);
    if (is_above) {
      const uint32_t slot = base_a + (uint32_t)__popcll(ma & lt_mask);
      if (slot < (uint32_t)a.top_k) abv[slot] = p;
    } else if (is_bin) {
      const uint32_t slot = base_b + (uint32_t)__popcll(mb & lt_mask);
      if (slot < (uint32_t)kCandCap) cand[slot] = make_uint2(u, (uint32_t)p);
    }
  }
}

// ------------------------------------------------------------------------------------
// Radix select of the r largest 64-bit keys among the threshold-bin elements.
// Key of an element: ((u & low bits) << 32) | ~position: 51 significant bits, resolved in
// seven digit passes (8,8,8,8,8,8,3 bits). Exactly r elements have a key >= the result.
constexpr int kSortCap = HS2_MAX_TOP_K;
constexpr uint32_t kLowMask = (1u << kHistShift) - 1u;

struct SelShared {
  uint32_t hist[256];
  uint32_t s_wave[kThreads / 64];
  int res[4];
  uint32_t nsel;
  int32_t sel[kSortCap];
  uint32_t cu[kCandCap];
  uint32_t cp[kCandCap];
};

__device__ inline uint64_t sel_key(uint32_t u_low, uint32_t p) {
  return ((uint64_t)u_low << 32) | (uint64_t)(~p);
}

// Visits the threshold-bin elements: from LDS (n elements) or by streaming the scores.
template <bool kLds, typename F>
__device__ inline void for_each_elem(const SelShared& sh, uint32_t n, const float* __restrict__ sc,
                                     int nc, int b1, F&& f) {
  if (kLds) {
    for (uint32_t e = threadIdx.x; e < n; e += kThreads) f(sh.cu[e], sh.cp[e]);
  } else {
    for (int p = threadIdx.x; p < nc; p += kThreads) {
      const uint32_t u = __float_as_uint(sc[p]);
      if ((int)(u >> kHistShift) == b1) f(u & kLowMask, (uint32_t)p);
    }
  }
}

template <bool kLds>
__device__ void radix_select_append(SelShared& sh, uint32_t n, const float* __restrict__ sc, int nc,
                                    int b1, int r_need) {
  uint64_t prefix = 0;
  int r_rem = r_need;
  for (int pass = 0; pass < 7; ++pass) {
    const int shift = pass < 6 ? 43 - 8 * pass : 0;
    const int width = pass < 6 ? 8 : 3;
    const int hi = shift + width;
    for (int e = threadIdx.x; e < 256; e += kThreads) sh.hist[e] = 0u;
    __syncthreads();
    const uint64_t pre_hi = prefix >> hi;
    for_each_elem<kLds>(sh, n, sc, nc, b1, [&](uint32_t ul, uint32_t p) {
      const uint64_t key = sel_key(ul, p);
      if ((key >> hi) == pre_hi) atomicAdd(&sh.hist[(uint32_t)(key >> shift) & ((1u << width) - 1u)], 1u);
    });
    __syncthreads();
    const int bin = 255 - (int)threadIdx.x;
    const uint32_t c = (bin < (1 << width)) ? sh.hist[bin] : 0u;
    uint32_t total;
    const uint32_t excl = block_excl_scan(c, sh.s_wave, total);
    if (threadIdx.x == 0) { sh.res[0] = 0; sh.res[1] = 0; }
    __syncthreads();
    if (excl < (uint32_t)r_rem && (uint32_t)r_rem <= excl + c) {
      sh.res[0] = bin;
      sh.res[1] = (int)excl;
    }
    __syncthreads();
    prefix |= (uint64_t)sh.res[0] << shift;
    r_rem -= sh.res[1];
    __syncthreads();
  }
  const uint64_t kstar = prefix;
  for_each_elem<kLds>(sh, n, sc, nc, b1, [&](uint32_t ul, uint32_t p) {
    if (sel_key(ul, p) >= kstar) {
      const uint32_t slot = atomicAdd(&sh.nsel, 1u);
      if (slot < (uint32_t)kSortCap) sh.sel[slot] = (int32_t)p;
    }
  });
  __syncthreads();
}

__global__ __launch_bounds__(kThreads) void topk_finish_kernel(TopkArgs a) {
  __shared__ SelShared sh;
  const int i = blockIdx.x;
  int32_t* out = a.sel_idx ? a.sel_idx + (size_t)i * a.top_k : nullptr;
  int64_t base;
  int t;
  if (!query_desc(a.b, i, base, t)) {
    if (out)
      for (int e = threadIdx.x; e < a.top_k; e += kThreads) out[e] = -1;
    if (a.sel_count && threadIdx.x == 0) a.sel_count[i] = -1;
    return;
  }
  const int nc = cand_count(t, a.window);
  const int k = a.top_k;
  if (k == 0 || nc <= k) {
    if (out)
      for (int e = threadIdx.x; e < k; e += kThreads) out[e] = e < nc ? e : -1;
    if (a.sel_count && threadIdx.x == 0) a.sel_count[i] = min(nc, k);
    return;
  }
  const uint32_t* hq = a.hist + (size_t)i * kHistBins;
  int b1, above;
  threshold_bin(hq, k, sh.s_wave, sh.res, b1, above);
  const int r_need = k - above;
  const uint32_t n_bin = hq[b1];
  const int32_t* abv = a.above + (size_t)i * k;
  for (int e = threadIdx.x; e < above; e += kThreads) sh.sel[e] = abv[e];
  if (threadIdx.x == 0) sh.nsel = (uint32_t)above;
  const float* sc = a.scores + (size_t)i * a.score_stride;
  if (n_bin <= (uint32_t)kCandCap) {
    const uint2* cand = a.cand + (size_t)i * kCandCap;
    for (uint32_t e = threadIdx.x; e < n_bin; e += kThreads) {
      const uint2 c = cand[e];
      sh.cu[e] = c.x & kLowMask;
      sh.cp[e] = c.y;
    }
    __syncthreads();
    radix_select_append<true>(sh, n_bin, sc, nc, b1, r_need);
  } else {
    __syncthreads();
    radix_select_append<false>(sh, 0, sc, nc, b1, r_need);
  }
  // bitonic sort of the k positions, ascending (padded to a power of two)
  int P = 1;
  while (P < k) P <<= 1;
  for (int e = k + threadIdx.x; e < P; e += kThreads) sh.sel[e] = INT32_MAX;
  __syncthreads();
  for (int kk = 2; kk <= P; kk <<= 1) {
    for (int j = kk >> 1; j > 0; j >>= 1) {
      for (int idx = threadIdx.x; idx < P; idx += kThreads) {
        const int ixj = idx ^ j;
        if (ixj > idx) {
          const int32_t x = sh.sel[idx], y = sh.sel[ixj];
          const bool asc = (idx & kk) == 0;
          if ((x > y) == asc) {
            sh.sel[idx] = y;
            sh.sel[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
  }
  if (out)
    for (int e = threadIdx.x; e < k; e += kThreads) out[e] = sh.sel[e];
  if (a.sel_count && threadIdx.x == 0) a.sel_count[i] = k;
}

}  // namespace

hipError_t launch_topk_filter(const TopkArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(topk_filter_kernel, dim3(a.b.total_q * a.n_split), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_topk_finish(const TopkArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(topk_finish_kernel, dim3(a.b.total_q), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace hs2
