// Selection score pass (pass 2) of the decode-shaped selector for gfx950: the per-key
// sum over the 64 heads of the softmax probability, from the exact log-sum-exp of pass 1.
//
// Method (page title and section): arex-research.com, "Xiaomi MiMo lead Luo Fuli
// publishes the MiMo-V3 core architecture HySparse2", section "Outer KV Bridging, inner
// KV Reuse": the full-attention layer's scores select the keys the sparse layers attend.
//
// Built with the MFMA results in VGPRs (no accumulator registers): the loop needs about
// 180 registers, and the softmax reads every result element once per tile.
#include "attn_common.h"

namespace hs2 {
namespace {

using namespace attn;

// ------------------------------------------------------------------------------------
// Selection score pass: score_j = sum_h exp2(x_hj - lse2_h) for candidates j <= t-window,
// written per query, plus a histogram of the first radix digit (bits 30..19).
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
// leave one wave's MFMA, conversion and exp chain exposed; 186 registers per lane fit
// two waves per SIMD.
template <typename Kv>
struct ScoreCfg {
  static constexpr int kSWaves = Kv::kFp8 ? 8 : 4;
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
  if (!__builtin_amdgcn_readfirstlane(query_desc(a.b, i, base, t))) return;
  // the descriptor is the same on every lane (query i): keep the loop control scalar
  t = __builtin_amdgcn_readfirstlane(t);
  base = (int64_t)(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)base >> 32)) << 32) |
                   (uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)base));
  const int nc = max(0, t - a.window + 1);
  if (nc <= a.top_k) return;
  const int k0 = split * a.split_keys;
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

  float* srow = a.scores + (size_t)i * a.score_stride;
  const int ntw = wave < ntiles ? (ntiles - wave + kSWaves - 1) / kSWaves : 0;
  // Tiles in the reverse of the attention pass's rotated order (same rotation): the first
  // tiles read here are the last that pass read, some still in the last-level cache.
  const TileOrder ord = TileOrder::rotated(i * a.n_split + split, ntiles);
  auto tile_of = [&](int x) { return ord.at(ntiles - 1 - x); };
  const uint32_t wbase = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)sm.stage[wave]);
  auto issue = [&](int it, int sidx) {
    const int p = k0 + tile_of(wave + it * kSWaves) * kTile + (lane & 31);
    const int rel = p < k1 ? p : 0;
    issue_tile<Kv, true>(a.k, base, rel, lane, wbase + sidx * Kv::kTileBytes);
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
    const int p = k0 + tile_of(wave + it * kSWaves) * kTile + (lane & 31);
    if (lane < 32 && p < k1) {
      sm.sbuf[wave][(it % kSFlush) * kTile + lane] = total;
      atomicAdd(&sm.hist[__float_as_uint(total) >> kHistShift], 1u);
    }
    if ((it + 1) % kSFlush == 0 || it + 1 == ntw) {
      // write the staged tiles in a burst: lane e stores 4 scores of tile first + e/8
      // (16 bytes), so the writes interleave with the streaming reads as little as possible
      wait_lgkm0();
      const int first = (it / kSFlush) * kSFlush;
      const int nt = it + 1 - first;
      for (int e = lane; e < nt * 8; e += 64) {
        const int tt = first + e / 8;
        const int q0 = k0 + tile_of(wave + tt * kSWaves) * kTile + (e % 8) * 4;
        const float4 v = *reinterpret_cast<const float4*>(&sm.sbuf[wave][(tt - first) * kTile + (e % 8) * 4]);
        if (q0 + 3 < k1) {
          *reinterpret_cast<float4*>(srow + q0) = v;
        } else {
          if (q0 < k1) srow[q0] = v.x;
          if (q0 + 1 < k1) srow[q0 + 1] = v.y;
          if (q0 + 2 < k1) srow[q0 + 2] = v.z;
        }
      }
    }
  }
  __syncthreads();
  uint32_t* hq = a.hist + (size_t)i * kHistBins;
  for (int e = threadIdx.x; e < kHistBins; e += blockDim.x) {
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
