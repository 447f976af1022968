// Selection score pass (pass 2) of the decode-shaped selector for gfx950: the per-key
// sum over the 64 heads of the softmax probability, from the exact log-sum-exp of pass 1.
//
// Method (page title and section): arex-research.com, "Xiaomi MiMo lead Luo Fuli
// publishes the MiMo-V3 core architecture HySparse2", section "Outer KV Bridging, inner
// KV Reuse": the full-attention layer's scores select the keys the sparse layers attend.
//
// Built with the MFMA results in VGPRs (MFMA destinations are not accumulator registers):
// the exponentials read every result element once per tile. The bf16 build (one wave per
// SIMD) takes 256 VGPRs and keeps other values in 64 accumulator registers; the FP8 build
// (two waves per SIMD) fits in 256 VGPRs.
#include "attn_common.h"
#include "hs2_launch.h"

namespace hs2 {
namespace {

using namespace attn;

// ------------------------------------------------------------------------------------
// Selection score pass: score_j = sum_h exp2(x_hj - lse2_h) for candidates j <= t-window,
// kept only where it can still be among the query's top k (see the lists below), plus a
// histogram of the first radix digit (bits 30..19) of the kept scores.
// S = Q K^T here (heads as rows): each lane sums its 32 head values of one key, and one
// exchange with lane l^32 completes the 64-head sum. K tiles stream through kScoreStages
// per-wave LDS stages (same swizzled layout and DMA as pass 1): 4 of bf16 tiles or 8 of
// FP8 tiles, the same bytes in flight.
// ------------------------------------------------------------------------------------
// LDS of a workgroup: 128 KB of K stages, the histogram and the staged scores (kSWaves x
// 32 tiles x 32 keys of fp32, 16 KB).
constexpr int kScoreStageBytes = 131072;
constexpr int kSBufTiles = 128;  // tiles of scores staged per workgroup before they are written

// Waves per workgroup: 4 for bf16 tiles (one per SIMD; the pass is bound by HBM) and 8 for
// FP8 tiles (two per SIMD), whose tiles arrive twice as fast per byte and would otherwise
// leave one wave's MFMA, conversion and exp chain exposed; its 256 registers per lane fit
// two waves per SIMD.
template <typename Kv>
struct ScoreCfg {
  static constexpr int kSWaves = score_waves(Kv::kFp8);
  static constexpr int kWaveBytes = kScoreStageBytes / kSWaves;
  static constexpr int kStages = kWaveBytes / Kv::kTileBytes;  // 4 bf16 or 4 FP8 tiles per wave
  static constexpr int kSFlush = kSBufTiles / kSWaves;          // tiles staged per wave
};

template <int kSWaves, int kSFlush>
struct ScoreSmem {
  uint8_t stage[kSWaves][kScoreStageBytes / kSWaves];
  uint32_t hist[kHistBins];
  float sbuf[kSWaves][kSFlush * kTile];
};

// The largest histogram bin b with count(bins >= b) >= k (the bin of the k-th largest
// counted element), or 0 if the histogram holds fewer than k. One wave: lane l first sums
// bins 64l .. 64l+63 (read in a rotated order, so that the 64 lanes hit 64 banks), then
// the row found is searched bin by bin. Counts still being added by other waves only lower
// the result.
__device__ inline int kth_bin(const uint32_t* hist, int k, int lane) {
  uint32_t r = 0;
  for (int j = 0; j < 64; ++j) r += hist[64 * lane + ((j + lane) & 63)];
  uint32_t suf = r;  // count of rows lane .. 63
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_down(suf, off);
    if (lane + off < 64) suf += y;
  }
  const uint64_t rows = __ballot(suf >= (uint32_t)k);
  if (rows == 0) return 0;
  const int row = 63 - __builtin_clzll(rows);
  const uint32_t above = __shfl(suf, row) - __shfl(r, row);  // count of the rows above it
  uint32_t t = hist[64 * row + lane];
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_down(t, off);
    if (lane + off < 64) t += y;
  }
  const uint64_t bins = __ballot(above + t >= (uint32_t)k);
  return 64 * row + (63 - __builtin_clzll(bins));
}

template <typename Kv>
__global__ __launch_bounds__(64 * ScoreCfg<Kv>::kSWaves) void score_bf16_kernel(ScoreArgs a, WorkList wl) {
  constexpr int kSWaves = ScoreCfg<Kv>::kSWaves;
  constexpr int kScoreStages = ScoreCfg<Kv>::kStages;
  constexpr int kSFlush = ScoreCfg<Kv>::kSFlush;
  __shared__ __align__(16) ScoreSmem<kSWaves, kSFlush> sm;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int i, split;
  work_item(wl, a.n_split, i, split);
  int64_t base;
  int t;
  const bool valid = __builtin_amdgcn_readfirstlane(query_desc(a.b, i, base, t));
  // the descriptor is the same on every lane (query i): keep the loop control scalar
  t = __builtin_amdgcn_readfirstlane(t);
  base = (int64_t)uniform_u64((uint64_t)base);
  const int nc = max(0, t - a.window + 1);
  const int k0 = split * a.split_keys;
  if (wl.n > 0 && a.plan_miss != nullptr && threadIdx.x == 0 && last_planned(wl, i))
    a.plan_miss[i] = (valid && nc > a.top_k && k0 + a.split_keys < nc) ? 1 : 0;
  if (!valid || nc <= a.top_k) return;
  if (k0 >= nc) return;
  const int k1 = min(nc, k0 + a.split_keys);
  const int ntiles = (k1 - k0 + kTile - 1) / kTile;

  for (int e = threadIdx.x; e < kHistBins; e += blockDim.x) sm.hist[e] = 0u;

  bf16x8 qop[2][8];
  {
    const __bf16* qp = static_cast<const __bf16*>(a.q) + (size_t)i * kHeads * kDim;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int s = 0; s < 8; ++s)
        qop[mb][s] = *reinterpret_cast<const bf16x8*>(qp + (32 * mb + (lane & 31)) * kDim +
                                                      (lane >> 5) * 64 + s * 8);
  }
  float l2[2][16];
  const int hrow = 4 * (lane >> 5);
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int j = 0; j < 16; ++j)
      l2[mb][j] = a.lse2[(size_t)i * kHeads + 32 * mb + 8 * (j >> 2) + hrow + (j & 3)];
  __syncthreads();  // histogram cleared; the loads above have completed

  // This wave's list of candidates: (score bits, position) of every score whose first
  // digit is at least the running threshold `thr` when its tile is flushed. thr is the
  // bin of the k-th largest score the workgroup has seen so far (kth_bin of its
  // histogram): a key below it has k keys of this split ahead of it and cannot be among
  // the query's top k.
  const size_t wl_idx = ((size_t)i * a.n_split + split) * kSWaves + wave;
  uint2* mylist = a.lists + wl_idx * a.list_cap;
  int thr = 0, cnt = 0;
  // Each wave streams its own contiguous share of the split's tiles: a workgroup then reads
  // kSWaves separate regions of K at a time instead of one region in interleaved tiles,
  // which keeps more requests in flight at the memory (64 x 131,072 decode batch: 1,029 ->
  // 1,021 us per selector call, same-box A/B in both orders).
  const int q_tiles = (ntiles + kSWaves - 1) / kSWaves;
  const int t0 = wave * q_tiles;
  const int ntw = max(0, min(q_tiles, ntiles - t0));
  // Tiles in the reverse of the attention pass's rotated order (the same per-workgroup
  // rotation, so that workgroups streaming equal splits do not read the same offsets at
  // the same time).
  const TileOrder ord = TileOrder::rotated(i * a.n_split + split, ntiles);
  auto tile_of = [&](int x) { return ord.at(ntiles - 1 - x); };
  const uint32_t wbase = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)sm.stage[wave]);
  auto issue = [&](int it, int sidx) {
    issue_tile_contig<Kv, true>(a.k, base, k0 + tile_of(t0 + it) * kTile, k1, lane,
                                wbase + sidx * Kv::kTileBytes);
  };
  for (int it = 0; it < min(ntw, kScoreStages); ++it) issue(it, it);
  for (int it = 0; it < ntw; ++it) {
    const int sidx = it % kScoreStages;
    // K(it) has landed once at most the groups issued after it are outstanding (score
    // stores issued meanwhile only make this wait longer, never shorter)
    const int later = min(ntw, it + kScoreStages) - (it + 1);
    wait_vmcnt_n(later * Kv::kDma);
    bf16x8 kc[8];
    read_k_of<Kv>(sm.stage[wave] + sidx * Kv::kTileBytes, lane, kc);
    if (it + kScoreStages < ntw) issue(it + kScoreStages, sidx);
    f32x16 acc[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      acc[mb] = f32x16{};
#pragma unroll
      for (int s = 0; s < 8; ++s) acc[mb] = mfma(qop[mb][s], kc[s], acc[mb]);
    }
    float sum = 0.0f;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int j = 0; j < 16; ++j) sum += fast_exp2(acc[mb][j] * a.c2 - l2[mb][j]);
    // lane l and l^32 hold complementary heads of the same key; add in a fixed order
    const float other = __shfl_xor(sum, 32);
    const float total = (lane < 32) ? sum + other : other + sum;
    const int p = k0 + tile_of(t0 + it) * kTile + (lane & 31);
    if (lane < 32 && p < k1) {
      sm.sbuf[wave][(it % kSFlush) * kTile + lane] = total;
      atomicAdd(&sm.hist[__float_as_uint(total) >> kHistShift], 1u);
    }
    if ((it + 1) % kSFlush == 0 || it + 1 == ntw) {
      // flush the staged tiles: the scores that pass the running threshold, compacted
      // with a ballot into the wave's list (a burst of 8-byte writes)
      wait_lgkm0();  // this wave's staged scores and histogram counts are in LDS
      thr = max(thr, kth_bin(sm.hist, a.top_k, lane));
      const int first = (it / kSFlush) * kSFlush;
      const int ne = (it + 1 - first) * kTile;
      for (int e0 = 0; e0 < ne; e0 += 64) {
        const int e = e0 + lane;
        const int p = k0 + tile_of(t0 + first + e / kTile) * kTile + (e % kTile);
        const uint32_t u = e < ne ? __float_as_uint(sm.sbuf[wave][e]) : 0u;
        const bool keep = e < ne && p < k1 && (int)(u >> kHistShift) >= thr;
        const uint64_t bal = __ballot(keep);
        if (keep) {
          const int below = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                           __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
          mylist[cnt + below] = make_uint2(u, (uint32_t)p);
        }
        cnt += __popcll(bal);
      }
    }
  }
  if (lane == 0) a.list_count[wl_idx] = cnt;
  __syncthreads();
  // the split's final threshold (every score of the split is in the histogram now; each
  // wave finds the same): only the scores at or above it are kept, and only those are
  // counted in the query's histogram
  const int thr_final = kth_bin(sm.hist, a.top_k, lane);
  if (threadIdx.x == 0) a.list_thr[(size_t)i * a.n_split + split] = thr_final;
  uint32_t* hq = a.hist + (size_t)i * kHistBins;
  for (int e = thr_final + threadIdx.x; e < kHistBins; e += blockDim.x) {
    const uint32_t c = sm.hist[e];
    if (c) atomicAdd(&hq[e], c);
  }
}

}  // namespace

hipError_t launch_score_bf16(const ScoreArgs& a, const WorkList& wl, hipStream_t s) {
  const int grid = wl.n > 0 ? wl.n : a.b.total_q * a.n_split;
  hipLaunchKernelGGL(score_bf16_kernel<KvBf16>, dim3(grid), dim3(64 * ScoreCfg<KvBf16>::kSWaves), 0, s, a, wl);
  return hipGetLastError();
}

hipError_t launch_score_fp8kv(const ScoreArgs& a, const WorkList& wl, hipStream_t s) {
  const int grid = wl.n > 0 ? wl.n : a.b.total_q * a.n_split;
  hipLaunchKernelGGL(score_bf16_kernel<KvFp8>, dim3(grid), dim3(64 * ScoreCfg<KvFp8>::kSWaves), 0, s, a, wl);
  return hipGetLastError();
}

}  // namespace hs2
