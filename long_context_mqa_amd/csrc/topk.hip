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
// Two kernels (the score pass already built a histogram of bits 30..19 of the scores it
// kept, and kept either every candidate's score in a row or, in the decode-shaped
// selector, per-split lists of the (score, position) pairs that can still be among the
// top k):
//   filter  (many workgroups per query): from the histogram, find the bin b1 that holds
//           the k-th largest; keys of a chunk (or of a split's lists) in a larger bin are
//           selected outright, keys in b1 are copied to a per-query candidate list (up to
//           kCandCap).
//   finish  (one workgroup per query): radix-select the remaining r keys among the b1
//           candidates in LDS (or, if b1 overflowed the list, by streaming the query's
//           scores again), then order the k positions ascending and write them.
//           Queries with at most k candidates take all of them.
#include "kernel_common.h"
#include "hs2_launch.h"

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

// True if the attention or score launch of query i was planned from host lengths that
// its device length exceeds (see last_planned): its partials or scores are incomplete.
__device__ inline bool plan_missed(const TopkArgs& a, int i) {
  return (a.miss_attn != nullptr && a.miss_attn[i] != 0) || (a.miss_score != nullptr && a.miss_score[i] != 0);
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ inline uint32_t wave_incl_scan(uint32_t x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

// ------------------------------------------------------------------------------------
// Filter: each thread takes kPerThread candidates (strided, coalesced), counts the ones
// above the threshold bin and in it, and each wave reserves its output slots with one
// atomic per list.
constexpr int kPerThread = 32;

__device__ void filter_chunk(const TopkArgs& a, int i, int nc, int split, uint32_t* s_wave, int* s_res,
                             uint32_t* s_tot) {
  const int k0 = split * a.split_len;
  if (k0 >= nc) return;
  const int k1 = min(nc, k0 + a.split_len);

  const float* sc = a.scores + (size_t)i * a.score_stride;
  uint32_t u[kPerThread];
#pragma unroll
  for (int r = 0; r < kPerThread; ++r) {
    const int p = k0 + r * kThreads + threadIdx.x;
    u[r] = p < k1 ? __float_as_uint(sc[p]) : 0u;
  }
  int b1, above;
  threshold_bin(a.hist + (size_t)i * kHistBins, a.top_k, s_wave, s_res, b1, above);

  uint32_t na = 0, nb = 0;
#pragma unroll
  for (int r = 0; r < kPerThread; ++r) {
    const int p = k0 + r * kThreads + threadIdx.x;
    const int d = (int)(u[r] >> kHistShift);
    na += (p < k1 && d > b1) ? 1u : 0u;
    nb += (p < k1 && d == b1) ? 1u : 0u;
  }
  const uint32_t ia = wave_incl_scan(na), ib = wave_incl_scan(nb);
  const int lane = threadIdx.x & 63;
  // one atomic per workgroup and list: wave totals combined in LDS
  const int wave = threadIdx.x >> 6;
  if (lane == 63) {
    s_tot[wave] = ia;
    s_tot[kThreads / 64 + wave] = ib;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t ta = 0, tb = 0;
    for (int w = 0; w < kThreads / 64; ++w) {
      ta += s_tot[w];
      tb += s_tot[kThreads / 64 + w];
    }
    s_tot[2 * (kThreads / 64)] = ta ? atomicAdd(&a.counters[(size_t)i * 4 + 0], ta) : 0u;
    s_tot[2 * (kThreads / 64) + 1] = tb ? atomicAdd(&a.counters[(size_t)i * 4 + 1], tb) : 0u;
  }
  __syncthreads();
  uint32_t oa = s_tot[2 * (kThreads / 64)] + ia - na;
  uint32_t ob = s_tot[2 * (kThreads / 64) + 1] + ib - nb;
  for (int w = 0; w < wave; ++w) {
    oa += s_tot[w];
    ob += s_tot[kThreads / 64 + w];
  }
  int32_t* abv = a.above + (size_t)i * a.top_k;
  uint2* cand = a.cand + (size_t)i * kCandCap;
#pragma unroll
  for (int r = 0; r < kPerThread; ++r) {
    const int p = k0 + r * kThreads + threadIdx.x;
    if (p >= k1) continue;
    const int d = (int)(u[r] >> kHistShift);
    if (d > b1) {
      if (oa < (uint32_t)a.top_k) abv[oa] = p;
      ++oa;
    } else if (d == b1) {
      if (ob < (uint32_t)kCandCap) cand[ob] = make_uint2(u[r], (uint32_t)p);
      ++ob;
    }
  }
}

// Filter over the candidate lists of score split `split` of query i (the lists of the
// split's waves, concatenated): entries above the threshold bin b1 go to `above`, those in
// it to `cand`. Thread t takes entries t, t + 256, ...: a first sweep counts them, one
// atomic per list reserves the workgroup's slots, a second sweep (the entries again, now
// from the L2) writes each thread's run.
__device__ void filter_lists(const TopkArgs& a, int i, int nc, int split, uint32_t* s_wave, int* s_res,
                             uint32_t* s_tot) {
  if (split * a.list_split_keys >= nc) return;  // the score pass has no list for it
  int b1, above;
  threshold_bin(a.hist + (size_t)i * kHistBins, a.top_k, s_wave, s_res, b1, above);
  const size_t l0 = ((size_t)i * a.list_splits + split) * a.list_waves;
  int off[9];  // start of each list in the concatenation (lists past list_waves are empty)
  off[0] = 0;
#pragma unroll
  for (int w = 0; w < 8; ++w) off[w + 1] = off[w] + (w < a.list_waves ? a.list_count[l0 + w] : 0);
  const int total = off[8];
  auto entry = [&](int e) {
    int w = 0, j = e;
#pragma unroll
    for (int q = 1; q < 8; ++q)
      if (e >= off[q]) {
        w = q;
        j = e - off[q];
      }
    return a.lists[(l0 + w) * a.list_cap + j];
  };
  uint32_t na = 0, nb = 0;
  for (int e = threadIdx.x; e < total; e += kThreads) {
    const int d = (int)(entry(e).x >> kHistShift);
    na += d > b1 ? 1u : 0u;
    nb += d == b1 ? 1u : 0u;
  }
  uint32_t ta, tb;
  const uint32_t pa = block_excl_scan(na, s_wave, ta);
  const uint32_t pb = block_excl_scan(nb, s_wave, tb);
  if (threadIdx.x == 0) {
    s_tot[0] = ta ? atomicAdd(&a.counters[(size_t)i * 4 + 0], ta) : 0u;
    s_tot[1] = tb ? atomicAdd(&a.counters[(size_t)i * 4 + 1], tb) : 0u;
  }
  __syncthreads();
  uint32_t oa = s_tot[0] + pa, ob = s_tot[1] + pb;
  int32_t* abv = a.above + (size_t)i * a.top_k;
  uint2* cand = a.cand + (size_t)i * kCandCap;
  for (int e = threadIdx.x; e < total; e += kThreads) {
    const uint2 c = entry(e);
    const int d = (int)(c.x >> kHistShift);
    if (d > b1) {
      if (oa < (uint32_t)a.top_k) abv[oa] = (int32_t)c.y;
      ++oa;
    } else if (d == b1) {
      if (ob < (uint32_t)kCandCap) cand[ob] = c;
      ++ob;
    }
  }
}

// ------------------------------------------------------------------------------------
// Selection inside the threshold bin. The r largest elements by (score bits, then
// smaller position) are found by a radix select over the 19 score bits below the first
// digit (passes of 11 and 8 bits); only if the last score value is shared by more
// elements than still needed are positions resolved too (four 8-bit passes over ~p).
constexpr int kSortCap = HS2_MAX_TOP_K;
constexpr int kBuckets = 1024;
constexpr uint32_t kLowMask = (1u << kHistShift) - 1u;

struct SelShared {
  uint32_t s_wave[kThreads / 64];
  uint32_t tot[2 * (kThreads / 64) + 2];
  int res[4];
  uint32_t nsel;
  int32_t sel[kSortCap];
  union {
    struct {  // selection inside the threshold bin
      uint32_t hist[2048];
      uint32_t cu[kCandCap];
      uint32_t cp[kCandCap];
    };
    struct {  // ordering of the selected positions
      int32_t sorted[kSortCap];
      uint32_t bcnt[kBuckets];
      uint32_t bfill[kBuckets];
      uint32_t bstart[kBuckets];
    };
  };
};

// Where the scores of query i are: a score row of nc entries (sc), or the candidate lists
// of the score pass (a->lists set).
struct ElemSource {
  const float* sc;
  int nc;
  const TopkArgs* a;
  int i;
};

// Visits the threshold-bin elements: from LDS (n elements) or by streaming the scores.
template <bool kLds, typename F>
__device__ inline void for_each_elem(const SelShared& sh, uint32_t n, const ElemSource& src, int b1, F&& f) {
  if (kLds) {
    for (uint32_t e = threadIdx.x; e < n; e += kThreads) f(sh.cu[e], sh.cp[e]);
  } else if (src.a->lists == nullptr) {
    for (int p = threadIdx.x; p < src.nc; p += kThreads) {
      const uint32_t u = __float_as_uint(src.sc[p]);
      if ((int)(u >> kHistShift) == b1) f(u & kLowMask, (uint32_t)p);
    }
  } else {
    // every kept list entry of the query: entries of bin b1 are at or above each split's
    // threshold (b1 is the query's k-th, at least each split's k-th)
    const TopkArgs& a = *src.a;
    const int ns = min(a.list_splits, (src.nc + a.list_split_keys - 1) / a.list_split_keys);
    for (int l = 0; l < ns * a.list_waves; ++l) {
      const size_t li = (size_t)src.i * a.list_splits * a.list_waves + l;
      const int n_l = a.list_count[li];
      const uint2* lst = a.lists + li * a.list_cap;
      for (int e = threadIdx.x; e < n_l; e += kThreads) {
        const uint2 c = lst[e];
        if ((int)(c.x >> kHistShift) == b1) f(c.x & kLowMask, c.y);
      }
    }
  }
}

// One digit pass: histogram of digit (key >> shift) & (2^width - 1) over the elements
// whose key matches `prefix` above the digit, then the digit value holding the r-th
// largest and the count of larger elements. key(ul, p) is given by `key_of`.
template <bool kLds, typename K>
__device__ inline void digit_pass(SelShared& sh, uint32_t n, const ElemSource& src, int b1,
                                  K&& key_of, uint64_t prefix, int shift, int width, int r, int& digit,
                                  int& larger) {
  const int nbins = 1 << width;
  for (int e = threadIdx.x; e < nbins; e += kThreads) sh.hist[e] = 0u;
  __syncthreads();
  const int hi = shift + width;
  for_each_elem<kLds>(sh, n, src, b1, [&](uint32_t ul, uint32_t p) {
    const uint64_t key = key_of(ul, p);
    if ((key >> hi) == (prefix >> hi)) atomicAdd(&sh.hist[(uint32_t)(key >> shift) & (uint32_t)(nbins - 1)], 1u);
  });
  __syncthreads();
  // thread tid owns bins from the top: nbins / kThreads consecutive bins, descending
  const int per = (nbins + kThreads - 1) / kThreads;
  const int top = nbins - 1 - (int)threadIdx.x * per;
  uint32_t tot = 0;
  for (int q = 0; q < per; ++q)
    if (top - q >= 0) tot += sh.hist[top - q];
  uint32_t total;
  const uint32_t excl = block_excl_scan(tot, sh.s_wave, total);
  if (threadIdx.x == 0) {
    sh.res[0] = 0;
    sh.res[1] = 0;
  }
  __syncthreads();
  if (excl < (uint32_t)r && (uint32_t)r <= excl + tot) {
    uint32_t run = excl;
    for (int q = 0; q < per; ++q) {
      if (top - q < 0) break;
      const uint32_t c = sh.hist[top - q];
      if (run < (uint32_t)r && (uint32_t)r <= run + c) {
        sh.res[0] = top - q;
        sh.res[1] = (int)run;
      }
      run += c;
    }
  }
  __syncthreads();
  digit = sh.res[0];
  larger = sh.res[1];
  __syncthreads();
}

template <bool kLds>
__device__ void select_in_bin(SelShared& sh, uint32_t n, const ElemSource& src, int b1,
                              int r_need) {
  auto score_key = [](uint32_t ul, uint32_t) { return (uint64_t)ul; };
  uint64_t pre = 0;
  int r = r_need, dg, lg;
  digit_pass<kLds>(sh, n, src, b1, score_key, pre, 8, 11, r, dg, lg);
  pre |= (uint64_t)dg << 8;
  r -= lg;
  digit_pass<kLds>(sh, n, src, b1, score_key, pre, 0, 8, r, dg, lg);
  pre |= (uint64_t)dg;
  r -= lg;
  const uint32_t ustar = (uint32_t)pre;  // score bits of the r_need-th largest
  // r elements with score bits == ustar are still needed; ties go to smaller positions
  if (threadIdx.x == 0) sh.res[2] = 0;
  __syncthreads();
  for_each_elem<kLds>(sh, n, src, b1, [&](uint32_t ul, uint32_t) {
    if (ul == ustar) atomicAdd(&sh.res[2], 1);
  });
  __syncthreads();
  const int n_eq = sh.res[2];
  uint32_t pstar_inv = 0;  // ~position threshold among the ties (0: take them all)
  if (n_eq > r) {
    auto tie_key = [ustar](uint32_t ul, uint32_t p) {
      return ul == ustar ? ((uint64_t)1 << 32) | (uint64_t)(~p) : (uint64_t)0;
    };
    uint64_t tp = (uint64_t)1 << 32;
    int rr = r;
    for (int shift = 24; shift >= 0; shift -= 8) {
      digit_pass<kLds>(sh, n, src, b1, tie_key, tp, shift, 8, rr, dg, lg);
      tp |= (uint64_t)dg << shift;
      rr -= lg;
    }
    pstar_inv = (uint32_t)tp;
  }
  __syncthreads();
  for_each_elem<kLds>(sh, n, src, b1, [&](uint32_t ul, uint32_t p) {
    const bool take = ul > ustar || (ul == ustar && (~p) >= pstar_inv);
    if (take) {
      const uint32_t slot = atomicAdd(&sh.nsel, 1u);
      if (slot < (uint32_t)kSortCap) sh.sel[slot] = (int32_t)p;
    }
  });
  __syncthreads();
}

// Final selection of query i (nc > k): run by one workgroup after every filter chunk of
// the query has been written.
__device__ void finish_query(const TopkArgs& a, SelShared& sh, int i, int nc, int32_t* out) {
  const int k = a.top_k;
  const uint32_t* hq = a.hist + (size_t)i * kHistBins;
  int b1, above;
  threshold_bin(hq, k, sh.s_wave, sh.res, b1, above);
  const int r_need = k - above;
  const uint32_t n_bin = __builtin_nontemporal_load(&hq[b1]);
  const int32_t* abv = a.above + (size_t)i * k;
  for (int e = threadIdx.x; e < above; e += kThreads) sh.sel[e] = __builtin_nontemporal_load(&abv[e]);
  if (threadIdx.x == 0) sh.nsel = (uint32_t)above;
  const ElemSource src{a.scores ? a.scores + (size_t)i * a.score_stride : nullptr, nc, &a, i};
  if (n_bin <= (uint32_t)kCandCap) {
    const uint2* cand = a.cand + (size_t)i * kCandCap;
    for (uint32_t e = threadIdx.x; e < n_bin; e += kThreads) {
      const uint32_t cx = __builtin_nontemporal_load(&cand[e].x);
      const uint32_t cy = __builtin_nontemporal_load(&cand[e].y);
      sh.cu[e] = cx & kLowMask;
      sh.cp[e] = cy;
    }
    __syncthreads();
    select_in_bin<true>(sh, n_bin, src, b1, r_need);
  } else {
    __syncthreads();
    select_in_bin<false>(sh, 0, src, b1, r_need);
  }
  // ascending order: bucket by position (kBuckets equal ranges of [0, nc)), prefix sums,
  // scatter, then the rank inside a bucket (buckets hold ~1 position on average)
  for (int e = threadIdx.x; e < kBuckets; e += kThreads) {
    sh.bcnt[e] = 0u;
    sh.bfill[e] = 0u;
  }
  __syncthreads();
  auto bucket = [nc](int32_t p) { return (int)(((int64_t)p * kBuckets) / nc); };
  for (int e = threadIdx.x; e < k; e += kThreads) atomicAdd(&sh.bcnt[bucket(sh.sel[e])], 1u);
  __syncthreads();
  {
    constexpr int per = kBuckets / kThreads;
    uint32_t c[per], tot = 0;
#pragma unroll
    for (int q = 0; q < per; ++q) {
      c[q] = sh.bcnt[threadIdx.x * per + q];
      tot += c[q];
    }
    uint32_t total;
    uint32_t run = block_excl_scan(tot, sh.s_wave, total);
#pragma unroll
    for (int q = 0; q < per; ++q) {
      sh.bstart[threadIdx.x * per + q] = run;
      run += c[q];
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < k; e += kThreads) {
    const int32_t x = sh.sel[e];
    const int bk = bucket(x);
    sh.sorted[sh.bstart[bk] + atomicAdd(&sh.bfill[bk], 1u)] = x;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < k; e += kThreads) {
    const int32_t x = sh.sorted[e];
    const int bk = bucket(x);
    const int b0 = (int)sh.bstart[bk], bn = (int)sh.bcnt[bk];
    int rank = b0;
    for (int f = b0; f < b0 + bn; ++f) rank += sh.sorted[f] < x ? 1 : 0;
    sh.sel[rank] = x;
  }
  __syncthreads();
  if (out)
    for (int e = threadIdx.x; e < k; e += kThreads) out[e] = sh.sel[e];
  if (a.sel_count && threadIdx.x == 0) a.sel_count[i] = k;
}

__global__ __launch_bounds__(kThreads) void topk_filter_kernel(TopkArgs a) {
  __shared__ uint32_t s_wave[kThreads / 64];
  __shared__ int s_res[4];
  __shared__ uint32_t s_tot[2 * (kThreads / 64) + 2];
  const int i = blockIdx.x / a.n_split;
  const int split = blockIdx.x - i * a.n_split;
  int64_t base;
  int t;
  if (!query_desc(a.b, i, base, t) || plan_missed(a, i)) return;
  const int nc = cand_count(t, a.window);
  if (a.top_k == 0 || nc <= a.top_k) return;
  filter_chunk(a, i, nc, split, s_wave, s_res, s_tot);
}

__global__ __launch_bounds__(kThreads) void topk_filter_lists_kernel(TopkArgs a) {
  __shared__ uint32_t s_wave[kThreads / 64];
  __shared__ int s_res[4];
  __shared__ uint32_t s_tot[2];
  const int i = blockIdx.x / a.list_splits;
  const int split = blockIdx.x - i * a.list_splits;
  int64_t base;
  int t;
  if (!query_desc(a.b, i, base, t) || plan_missed(a, i)) return;
  const int nc = cand_count(t, a.window);
  if (a.top_k == 0 || nc <= a.top_k) return;
  filter_lists(a, i, nc, split, s_wave, s_res, s_tot);
}

__global__ __launch_bounds__(kThreads) void topk_finish_kernel(TopkArgs a) {
  __shared__ SelShared sh;
  const int i = blockIdx.x;
  int32_t* out = a.sel_idx ? a.sel_idx + (size_t)i * a.top_k : nullptr;
  int64_t base;
  int t;
  const int k = a.top_k;
  const bool valid = query_desc(a.b, i, base, t);
  if (!valid || plan_missed(a, i)) {
    if (out)
      for (int e = threadIdx.x; e < k; e += kThreads) out[e] = -1;
    if (a.sel_count && threadIdx.x == 0) a.sel_count[i] = -1;
    if (valid) {  // a missed plan: the query's outputs are not computed either
      const size_t o0 = (size_t)i * kHeads * kDim;
      for (int e = threadIdx.x; e < kHeads * kDim; e += kThreads) {
        if (a.out_f32) static_cast<float*>(a.out)[o0 + e] = NAN;
        else static_cast<__bf16*>(a.out)[o0 + e] = (__bf16)NAN;
      }
      if (a.lse && threadIdx.x < kHeads) a.lse[(size_t)i * kHeads + threadIdx.x] = NAN;
    }
    return;
  }
  const int nc = cand_count(t, a.window);
  if (k == 0 || nc <= k) {
    if (out)
      for (int e = threadIdx.x; e < k; e += kThreads) out[e] = e < nc ? e : -1;
    if (a.sel_count && threadIdx.x == 0) a.sel_count[i] = min(nc, k);
    return;
  }
  finish_query(a, sh, i, nc, out);
}

}  // namespace

hipError_t launch_topk_filter(const TopkArgs& a, hipStream_t s) {
  if (a.lists)
    hipLaunchKernelGGL(topk_filter_lists_kernel, dim3(a.b.total_q * a.list_splits), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(topk_filter_kernel, dim3(a.b.total_q * a.n_split), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_topk_finish(const TopkArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(topk_finish_kernel, dim3(a.b.total_q), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace hs2
