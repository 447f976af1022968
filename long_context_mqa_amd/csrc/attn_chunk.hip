// bf16 selector kernels for many queries per sequence (chunked prefill-shaped selection).
//
// Method (page title and section): arex-research.com, "Xiaomi MiMo lead Luo Fuli
// publishes the MiMo-V3 core architecture HySparse2", section "Outer KV Bridging, inner
// KV Reuse": the full-attention layer computes exact attention and its scores select
// the keys of the sparse layers. Section "Numbers computed on three 80B-A3B models":
// 64 query heads share one KV head.
//
// The decode-shaped kernels give every query its own K/V stream. When a sequence has
// many queries, the eight waves of a workgroup instead take eight consecutive queries of
// one sequence (a q-tile) and share every K/V tile: each tile is copied once into LDS
// and multiplied by eight queries, which cuts cache traffic per flop by eight and makes
// the pass matrix-bound. Two waves share each SIMD, so one wave's softmax (vector ALU)
// overlaps the other's matrix work. Each wave keeps its own online softmax state and
// reads its query's Q^T operands from LDS; the per-tile step is the one of the
// decode-shaped pass 1.
//   qtile_prep_kernel    lists the q-tiles (never straddling two sequences)
//   attn_chunk_kernel    pass 1: exact causal attention -> per-split partials
//   score_chunk_kernel   pass 2: head-summed probabilities + first-digit histograms
// This file is built with the MFMA results in VGPRs (no accumulator registers): both
// kernels stay within 256 registers, the budget of two waves per SIMD.
#include "attn_common.h"
#include "hs2_launch.h"

namespace hs2 {
namespace {

using namespace attn;

constexpr int kQT = kQTile;                           // queries per q-tile (one per wave)
constexpr int kCWaves = kQTile;                       // waves per workgroup
constexpr int kCThreads = 64 * kCWaves;
constexpr int kCStages = 2;                           // shared K+V stages of pass 1
constexpr int kSStages = 3;                           // shared K stages of the score pass
constexpr int kCopiesPerWave = kDmaPerHalf / kCWaves; // 1 of the 8 copies of a K or V tile
static_assert(kCopiesPerWave * kCWaves == kDmaPerHalf, "tile copies must split evenly");

// Raw workgroup barrier for the streaming loops. __syncthreads() carries a memory fence
// that makes the compiler wait for every vector memory operation it tracks; the loops
// only need LDS reads finished (lgkmcnt) and their LDS copies are waited for by hand.
__device__ inline void loop_barrier() {
  wait_lgkm0();
  __builtin_amdgcn_s_barrier();
}

// Block-wide exclusive scan (256 threads).
__device__ inline uint32_t excl_scan256(uint32_t v, uint32_t* s_wave, uint32_t& total) {
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
  for (int w = 0; w < 4; ++w) {
    if (w < wave) before += s_wave[w];
    total += s_wave[w];
  }
  __syncthreads();
  return before + x - v;
}

// Q-tile list: (first query, count <= kQT) per tile, in sequence order; unused entries
// get count 0. One workgroup of 256 threads. Sequences are taken 256 at a time; the
// tiles of those sequences are then written by the whole workgroup, each thread finding
// the sequence of its tile by binary search over the scanned tile offsets (a single
// sequence of 262,144 queries has 32,768 tiles).
__global__ __launch_bounds__(256) void qtile_prep_kernel(SeqsDev b, int2* tiles, int max_tiles) {
  __shared__ uint32_t s_wave[4];
  __shared__ uint32_t s_pre[256];
  __shared__ int s_q0[256], s_nq[256];
  uint32_t off = 0;
  for (int s0 = 0; s0 < b.num_seqs; s0 += 256) {
    const int s = s0 + threadIdx.x;
    int q0 = 0, nq = 0;
    if (s < b.num_seqs) {  // the tiles stay within the rows of Q: [0, total_q)
      q0 = min(max(b.q_start[s], 0), b.total_q);
      nq = max(0, min(b.q_start[s + 1], b.total_q) - q0);
    }
    const uint32_t cnt = (uint32_t)((nq + kQT - 1) / kQT);
    uint32_t total;
    const uint32_t pre = excl_scan256(cnt, s_wave, total);
    s_pre[threadIdx.x] = pre;
    s_q0[threadIdx.x] = q0;
    s_nq[threadIdx.x] = nq;
    __syncthreads();
    for (uint32_t t = threadIdx.x; t < total; t += 256) {
      // The last sequence whose first tile is at or before t owns it: a sequence with
      // no tiles shares its offset with the next one, and those at the end have offset
      // `total`, so neither is picked.
      int lo = 0, hi = 255;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_pre[mid] <= t) lo = mid; else hi = mid - 1;
      }
      const int j = (int)(t - s_pre[lo]);
      const uint32_t tix = off + t;
      if (tix < (uint32_t)max_tiles) tiles[tix] = make_int2(s_q0[lo] + j * kQT, min(kQT, s_nq[lo] - j * kQT));
    }
    off += total;
    __syncthreads();  // the next 256 sequences overwrite the shared offsets
  }
  for (uint32_t tix = off + threadIdx.x; tix < (uint32_t)max_tiles; tix += 256) tiles[tix] = make_int2(0, 0);
}

// Per-wave query of a q-tile; returns false if the wave has no valid query.
__device__ inline bool tile_query(const SeqsDev& b, int2 td, int wave, int& i, int64_t& base, int& t) {
  i = td.x + wave;
  if (wave >= td.y) return false;
  return query_desc(b, i, base, t);
}

// LDS of pass 1: 2 x 16 KB of shared K/V stages and 8 x 16 KB of Q^T operands (160 KB).
// The per-query scalars live in the stage area before and after the key loop.
struct ChunkSmem {
  union {
    uint8_t stage[kCStages][2][kTileBytes];
    struct {
      int tq[kQT];
      int64_t base[kQT];
      int redo[kQT];
    } misc;
  };
  uint8_t q[kQT][kHeads * kDim * 2];
};

// Copies this wave's share (kCopiesPerWave of the 8 wave-wide copies) of the K and V
// rows of the tile starting at key p0 into one stage. Rows past the last key are clamped.
__device__ inline void issue_shared(const __bf16* __restrict__ kp, const __bf16* __restrict__ vp, int64_t base,
                                    int p0, int plast, int wave, int lane, uint32_t lk, uint32_t lv) {
#pragma unroll
  for (int c = 0; c < kCopiesPerWave; ++c) {
    const int r = wave * kCopiesPerWave + c;
    const int row = r * 4 + (lane >> 4);
    const int p = min(p0 + row, plast);
    const int64_t g = (base + p) * kDim;
    dma16(kp + g + ((lane & 15) ^ (row & 15)) * 8, lk + r * 1024);
    dma16(vp + g + v_chunk(row, lane & 15) * 8, lv + r * 1024);
  }
}

// Streams the tiles of [k0, k1) through the shared stages; every wave issues its share
// of each tile's copies and takes part in every barrier. Waves with `compute` set run the
// tile step on the keys their query attends (kMaxOnly: only the logit maximum, into mx).
// Tile it+1 is copied while tile it is computed.
template <bool kMaxOnly>
__device__ inline void chunk_stream(WaveState& st, float (&mx)[2], ChunkSmem& sm, const uint8_t* __restrict__ qs,
                                    bool compute, int t, int k0, int k1, int ntiles, int64_t seq_base,
                                    const __bf16* __restrict__ kp, const __bf16* __restrict__ vp, float c2,
                                    int wave, int lane) {
  const uint32_t l0 = (uint32_t)(size_t)sm.stage[0][0];
  auto lk = [&](int sidx) { return __builtin_amdgcn_readfirstlane(l0 + sidx * 2 * kTileBytes); };
  auto lv = [&](int sidx) { return __builtin_amdgcn_readfirstlane(l0 + sidx * 2 * kTileBytes + kTileBytes); };
  uint32_t vb[4];
  vt_bases(lane, vb);

  if (ntiles > 0) issue_shared(kp, vp, seq_base, k0, k1 - 1, wave, lane, lk(0), lv(0));
  for (int it = 0; it < ntiles; ++it) {
    const int sidx = it & 1;
    wait_vmcnt<0>();  // this wave's copies of tile it have landed
    loop_barrier();   // every wave's copies of tile it have landed; tile it-1 is released
    if (it + 1 < ntiles)
      issue_shared(kp, vp, seq_base, k0 + (it + 1) * kTile, k1 - 1, wave, lane, lk(sidx ^ 1), lv(sidx ^ 1));
    const int p0 = k0 + it * kTile;
    if (compute && p0 <= t) {
      bf16x8 kop[8];
      read_k(sm.stage[sidx][0], lane, kop);
      const int nvalid = min(t, k1 - 1) - p0 + 1;  // keys p0 .. p0+nvalid-1 are attended
      const uint32_t vm = __builtin_amdgcn_readfirstlane(nvalid >= 32 ? 0xffffffffu : ((1u << nvalid) - 1u));
      if (kMaxOnly)
        process_tile_max<false>(mx, qs, nullptr, kop, vm, c2, lane);
      else
        process_tile<false>(st, qs, nullptr, kop, sm.stage[sidx][1], vb, vm, c2, lane);
    }
  }
}

__global__ __launch_bounds__(kCThreads) void attn_chunk_kernel(AttnArgs a, const int2* __restrict__ qtiles) {
  __shared__ __align__(16) ChunkSmem sm;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // q-tiles in reverse list order: in a prefill the tiles of the last positions hold the
  // most keys, and starting them first keeps the end of the launch from waiting on them
  const int tix = (int)(gridDim.x / a.n_split) - 1 - (int)(blockIdx.x / a.n_split);
  const int split = blockIdx.x % a.n_split;
  const int2 td = qtiles[tix];
  if (td.y <= 0) return;
  int i, t;
  int64_t base;
  const bool mine = tile_query(a.b, td, wave, i, base, t);
  if (lane == 0) {
    sm.misc.tq[wave] = mine ? t : -1;
    sm.misc.base[wave] = base;
  }
  __syncthreads();
  int t_max = -1;
  int64_t seq_base = 0;
#pragma unroll
  for (int w = 0; w < kQT; ++w) {
    if (sm.misc.tq[w] > t_max) {
      t_max = sm.misc.tq[w];
      seq_base = sm.misc.base[w];
    }
  }
  const int k0 = split * a.split_keys;
  if (t_max < 0 || k0 > t_max) return;  // the combine handles queries without partials
  const int k1 = min(t_max + 1, k0 + a.split_keys);
  const int ntiles = (k1 - k0 + kTile - 1) / kTile;

  // Q^T operands of this wave's query in LDS (read by the tile step), so that the loop
  // keeps its registers for the accumulators and no tracked global load is outstanding
  // inside it: 16-byte piece (nb, s, lane) = Q[32nb + l%32][(l/32)*64 + 8s ..]
  uint8_t* qs = sm.q[wave];
  {
    const __bf16* qp = static_cast<const __bf16*>(a.q) + (size_t)(mine ? i : 0) * kHeads * kDim;
    for (int e = lane; e < 16 * 64; e += 64) {
      const int ln = e & 63, sidx = (e >> 6) & 7, nb = e >> 9;
      *reinterpret_cast<bf16x8*>(qs + e * 16) = *reinterpret_cast<const bf16x8*>(
          qp + (32 * nb + (ln & 31)) * kDim + (ln >> 5) * 64 + sidx * 8);
    }
    __syncthreads();  // Q in place; the per-query scalars above have been read
  }

  WaveState st;
  state_init(st);
  float mx[2] = {-INFINITY, -INFINITY};
  const __bf16* kp = static_cast<const __bf16*>(a.k);
  const __bf16* vp = static_cast<const __bf16*>(a.v);
  const int tu = __builtin_amdgcn_readfirstlane(t);  // one query per wave
  chunk_stream<false>(st, mx, sm, qs, mine, tu, k0, k1, ntiles, seq_base, kp, vp, a.c2, wave, lane);

  // rare: a wave whose sums overflowed recomputes with its exact logit maximum; the
  // workgroup streams the tiles again together
  const bool bad = mine && !state_finite(st);
  __syncthreads();  // the stage area is free
  if (lane == 0) sm.misc.redo[wave] = bad ? 1 : 0;
  __syncthreads();
  int any_bad = 0;
#pragma unroll
  for (int w = 0; w < kQT; ++w) any_bad |= sm.misc.redo[w];
  if (any_bad) {
    __syncthreads();  // every wave has read the flags before the stages are reused
    chunk_stream<true>(st, mx, sm, qs, bad, tu, k0, k1, ntiles, seq_base, kp, vp, a.c2, wave, lane);
    if (bad) {
      state_init(st);
      st.m[0] = mx[0];
      st.m[1] = mx[1];
      st.have_ref = 1;
    }
    __syncthreads();
    chunk_stream<false>(st, mx, sm, qs, bad, tu, k0, k1, ntiles, seq_base, kp, vp, a.c2, wave, lane);
  }

  if (!mine) return;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    st.l[nb] += __shfl_xor(st.l[nb], 32);
    st.le[nb] += __shfl_xor(st.le[nb], 32);
  }
  const int hrow = 4 * (lane >> 5);
  if (a.direct) {
    // one split per query: its output (normalised like the split combine with a single
    // partial) and its LSE, straight from the wave's state; lane l holds head 32nb + l%32
    __bf16* out = static_cast<__bf16*>(a.out) + (size_t)i * kHeads * kDim;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const float inv = a.v_scale / st.l[nb];
      __bf16* oh = out + (32 * nb + (lane & 31)) * kDim;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int jg = 0; jg < 4; ++jg) {
          __bf16 v4[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) v4[q] = (__bf16)(st.o[nb][mb][4 * jg + q] * inv);
          *reinterpret_cast<uint2*>(oh + 32 * mb + 8 * jg + hrow) = __builtin_bit_cast(uint2, v4);
        }
      if (lane < 32) {
        const float l2 = st.m[nb] + __log2f(st.le[nb]);
        if (a.lse) a.lse[(size_t)i * kHeads + 32 * nb + lane] = l2 * kLn2;
        if (a.lse2) a.lse2[(size_t)i * kHeads + 32 * nb + lane] = l2;
      }
    }
    return;
  }
  Partial* P = a.part + (size_t)i * a.n_split + split;
  if (lane < 32) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      P->m[32 * nb + lane] = st.m[nb];
      P->l[32 * nb + lane] = st.l[nb];
      P->le[32 * nb + lane] = st.le[nb];
    }
  }
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int d = 32 * mb + 8 * (j >> 2) + hrow + (j & 3);
        P->o[d * kHeads + 32 * nb + (lane & 31)] = st.o[nb][mb][j];
      }
}

// ------------------------------------------------------------------------------------
// Score pass for q-tiles: S = Q K^T per wave on a shared K tile, the 64-head sum of
// exp2(x - lse2), written per query, and each query's first-digit histogram in LDS.
// The histogram packs two 16-bit bin counts per word (the host keeps a split below
// 2^16 keys). Scores are staged in LDS and written every kFlush tiles, so that the
// stores do not interleave with the streaming copies.
// ------------------------------------------------------------------------------------
constexpr int kFlush = 16;

struct ScoreChunkSmem {
  uint8_t stage[kSStages][kTileBytes];
  uint32_t hist[kQT][kHistBins / 2];
  float sbuf[kQT][kFlush * kTile];
  int tq[kQT];
  int64_t base[kQT];
};

__global__ __launch_bounds__(kCThreads) void score_chunk_kernel(ScoreArgs a, const int2* __restrict__ qtiles) {
  __shared__ __align__(16) ScoreChunkSmem sm;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tix = blockIdx.x / a.n_split;
  const int split = blockIdx.x - tix * a.n_split;
  const int2 td = qtiles[tix];
  if (td.y <= 0) return;
  int i, t;
  int64_t base;
  bool mine = tile_query(a.b, td, wave, i, base, t);
  const int nc = mine ? max(0, t - a.window + 1) : 0;
  mine = mine && nc > a.top_k;  // queries with at most k candidates take all of them
  if (lane == 0) {
    sm.tq[wave] = mine ? nc : 0;
    sm.base[wave] = base;
  }
  for (int e = lane; e < kHistBins / 2; e += 64) sm.hist[wave][e] = 0u;
  __syncthreads();
  int nc_max = 0;
  int64_t seq_base = 0;
#pragma unroll
  for (int w = 0; w < kQT; ++w) {
    if (sm.tq[w] > nc_max) {
      nc_max = sm.tq[w];
      seq_base = sm.base[w];
    }
  }
  const int k0 = split * a.split_keys;
  if (k0 >= nc_max) return;
  const int k1 = min(nc_max, k0 + a.split_keys);
  const int ntiles = (k1 - k0 + kTile - 1) / kTile;

  // Q operands in registers (S = Q K^T: Q is the A operand, heads as rows) and the
  // per-head log2-domain LSE in the C layout; the barrier below waits for the loads
  bf16x8 qop[2][8];
  float l2[2][16];
  const int hrow = 4 * (lane >> 5);
  {
    const __bf16* qp = static_cast<const __bf16*>(a.q) + (size_t)(mine ? i : 0) * kHeads * kDim;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int s = 0; s < 8; ++s)
        qop[mb][s] = *reinterpret_cast<const bf16x8*>(qp + (32 * mb + (lane & 31)) * kDim + (lane >> 5) * 64 + s * 8);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int j = 0; j < 16; ++j)
        l2[mb][j] = mine ? a.lse2[(size_t)i * kHeads + 32 * mb + 8 * (j >> 2) + hrow + (j & 3)] : 0.0f;
    __syncthreads();
  }

  const __bf16* kp = static_cast<const __bf16*>(a.k);
  float* srow = a.scores + (size_t)(mine ? i : 0) * a.score_stride;
  const uint32_t l0 = (uint32_t)(size_t)sm.stage[0];
  auto lk = [&](int sidx) { return __builtin_amdgcn_readfirstlane(l0 + sidx * kTileBytes); };
  auto issue_k = [&](int it2, uint32_t lds) {
#pragma unroll
    for (int c = 0; c < kCopiesPerWave; ++c) {
      const int r = wave * kCopiesPerWave + c;
      const int row = r * 4 + (lane >> 4);
      const int p = min(k0 + it2 * kTile + row, k1 - 1);
      dma16(kp + (seq_base + p) * kDim + ((lane & 15) ^ (row & 15)) * 8, lds + r * 1024);
    }
  };
  auto flush = [&](int it_end) {
    // scores of tiles [it_end - n, it_end) of this wave's query, staged in sbuf
    const int first = ((it_end - 1) / kFlush) * kFlush;
    for (int e = lane; e < (it_end - first) * kTile; e += 64) {
      const int p = k0 + first * kTile + e;
      if (p < min(k1, nc)) srow[p] = sm.sbuf[wave][e];
    }
  };

  for (int it = 0; it < min(ntiles, kSStages - 1); ++it) issue_k(it, lk(it));
  for (int it = 0; it < ntiles; ++it) {
    const int sidx = it % kSStages;
    if (it + 1 < ntiles) wait_vmcnt<kCopiesPerWave>(); else wait_vmcnt<0>();
    loop_barrier();
    if (it + kSStages - 1 < ntiles) issue_k(it + kSStages - 1, lk((it + kSStages - 1) % kSStages));
    const int p0 = k0 + it * kTile;
    if (mine && p0 < nc) {
      bf16x8 kc[8];
      read_k(sm.stage[sidx], lane, kc);
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
        for (int j = 0; j < 16; ++j) sum += fast_exp2(fmaf(acc[mb][j], a.c2, -l2[mb][j]));
      const float other = __shfl_xor(sum, 32);
      const float total = (lane < 32) ? sum + other : other + sum;
      const int p = p0 + (lane & 31);
      if (lane < 32 && p < min(k1, nc)) {
        sm.sbuf[wave][(it % kFlush) * kTile + lane] = total;
        const uint32_t bin = __float_as_uint(total) >> kHistShift;
        atomicAdd(&sm.hist[wave][bin >> 1], 1u << (16 * (bin & 1)));
      }
    }
    if (mine && ((it + 1) % kFlush == 0 || it + 1 == ntiles)) {
      wait_lgkm0();
      flush(it + 1);
    }
  }
  __syncthreads();
  if (!mine) return;
  uint32_t* hq = a.hist + (size_t)i * kHistBins;
  for (int e = lane; e < kHistBins / 2; e += 64) {
    const uint32_t c = sm.hist[wave][e];
    if (c & 0xffffu) atomicAdd(&hq[2 * e], c & 0xffffu);
    if (c >> 16) atomicAdd(&hq[2 * e + 1], c >> 16);
  }
}

}  // namespace

hipError_t launch_qtile_prep(const SeqsDev& b, int2* tiles, int max_tiles, hipStream_t s) {
  hipLaunchKernelGGL(qtile_prep_kernel, dim3(1), dim3(256), 0, s, b, tiles, max_tiles);
  return hipGetLastError();
}

hipError_t launch_attn_chunk(const AttnArgs& a, const int2* tiles, int max_tiles, hipStream_t s) {
  hipLaunchKernelGGL(attn_chunk_kernel, dim3(max_tiles * a.n_split), dim3(kCThreads), 0, s, a, tiles);
  return hipGetLastError();
}

hipError_t launch_score_chunk(const ScoreArgs& a, const int2* tiles, int max_tiles, hipStream_t s) {
  hipLaunchKernelGGL(score_chunk_kernel, dim3(max_tiles * a.n_split), dim3(kCThreads), 0, s, a, tiles);
  return hipGetLastError();
}

}  // namespace hs2
