// bf16 selector kernels for many queries per sequence (chunked prefill-shaped selection).
//
// Method (page title and section): arex-research.com, "Xiaomi MiMo lead Luo Fuli
// publishes the MiMo-V3 core architecture HySparse2", section "Outer KV Bridging, inner
// KV Reuse": the full-attention layer computes exact attention and its scores select
// the keys of the sparse layers. Section "Numbers computed on three 80B-A3B models":
// 64 query heads share one KV head.
//
// The decode-shaped kernels give every query its own K/V stream. When a sequence has
// many queries, the four waves of a workgroup instead take four consecutive queries of
// one sequence (a q-tile) and share every K/V tile: each tile is copied once into LDS
// and multiplied by four queries, which cuts cache traffic per flop by four and makes
// the pass matrix-bound. Each wave keeps its query's Q in registers and its own online
// softmax state; the per-tile step is the same as in the decode-shaped pass 1.
//   qtile_prep_kernel    lists the q-tiles (never straddling two sequences)
//   attn_chunk_kernel    pass 1: exact causal attention -> per-split partials
//   score_chunk_kernel   pass 2: head-summed probabilities + first-digit histograms
#include "attn_common.h"

namespace hs2 {
namespace {

using namespace attn;

constexpr int kQT = kWaves;       // queries per q-tile (one per wave)
constexpr int kCStages = 3;       // shared LDS stages
constexpr int kCopiesPerWave = kDmaPerHalf / kWaves;  // 2 of the 8 copies of a tile

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

// Q-tile list: (first query, count <= 4) per tile, in sequence order; unused entries
// get count 0. One workgroup.
__global__ __launch_bounds__(256) void qtile_prep_kernel(SeqsDev b, int2* tiles, int max_tiles) {
  __shared__ uint32_t s_wave[4];
  uint32_t off = 0;
  for (int s0 = 0; s0 < b.num_seqs; s0 += 256) {
    const int s = s0 + threadIdx.x;
    int q0 = 0, nq = 0;
    if (s < b.num_seqs) {
      q0 = b.q_start[s];
      nq = max(0, b.q_start[s + 1] - q0);
    }
    const uint32_t cnt = (uint32_t)((nq + kQT - 1) / kQT);
    uint32_t total;
    const uint32_t pre = excl_scan256(cnt, s_wave, total);
    for (uint32_t j = 0; j < cnt; ++j) {
      const uint32_t tix = off + pre + j;
      if (tix < (uint32_t)max_tiles) tiles[tix] = make_int2(q0 + (int)j * kQT, min(kQT, nq - (int)j * kQT));
    }
    off += total;
  }
  for (uint32_t tix = off + threadIdx.x; tix < (uint32_t)max_tiles; tix += 256) tiles[tix] = make_int2(0, 0);
}

struct ChunkSmem {
  union {
    uint8_t stage[kCStages][2][kTileBytes];  // shared K and V tiles
    uint8_t q[kQT][kHeads * kDim * 2];       // Q staging before the loop
  };
  int tq[kQT];
  int64_t base[kQT];
  int redo[kQT];
};

// Per-wave query of a q-tile; returns false if the wave has no valid query.
__device__ inline bool tile_query(const SeqsDev& b, int2 td, int wave, int& i, int64_t& base, int& t) {
  i = td.x + wave;
  if (wave >= td.y) return false;
  return query_desc(b, i, base, t);
}

// Copies this wave's share (2 of 8 wave-wide copies) of the K and V rows of the tile
// starting at key p0 into one stage. Rows past the last key are clamped.
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
template <bool kMaxOnly>
__device__ inline void chunk_stream(WaveState& st, float (&mx)[2], ChunkSmem& sm, const bf16x8 (&qop)[2][8],
                                    bool compute, int t, int k0, int k1, int ntiles, int64_t seq_base,
                                    const __bf16* __restrict__ kp, const __bf16* __restrict__ vp, float c2,
                                    int wave, int lane) {
  const uint32_t l0 = (uint32_t)(size_t)sm.stage[0][0];
  auto lk = [&](int sidx) { return __builtin_amdgcn_readfirstlane(l0 + sidx * 2 * kTileBytes); };
  auto lv = [&](int sidx) { return __builtin_amdgcn_readfirstlane(l0 + sidx * 2 * kTileBytes + kTileBytes); };
  uint32_t vb[4];
  vt_bases(lane, vb);

  for (int it = 0; it < min(ntiles, kCStages - 1); ++it)
    issue_shared(kp, vp, seq_base, k0 + it * kTile, k1 - 1, wave, lane, lk(it), lv(it));
  for (int it = 0; it < ntiles; ++it) {
    const int sidx = it % kCStages;
    if (it + 1 < ntiles) wait_vmcnt<2 * kCopiesPerWave>(); else wait_vmcnt<0>();
    loop_barrier();  // every wave's copies of tile it have landed; tile it-1 is released
    if (it + kCStages - 1 < ntiles) {
      const int nx = it + kCStages - 1;
      issue_shared(kp, vp, seq_base, k0 + nx * kTile, k1 - 1, wave, lane, lk(nx % kCStages), lv(nx % kCStages));
    }
    const int p0 = k0 + it * kTile;
    if (compute && p0 <= t) {
      bf16x8 kop[8];
      read_k(sm.stage[sidx][0], lane, kop);
      const int nvalid = min(t, k1 - 1) - p0 + 1;  // keys p0 .. p0+nvalid-1 are attended
      const uint32_t vm = __builtin_amdgcn_readfirstlane(nvalid >= 32 ? 0xffffffffu : ((1u << nvalid) - 1u));
      if (kMaxOnly)
        process_tile_max<true>(mx, nullptr, qop, kop, vm, c2, lane);
      else
        process_tile<true>(st, nullptr, qop, kop, sm.stage[sidx][1], vb, vm, c2, lane);
    }
  }
}

__global__ __launch_bounds__(256) void attn_chunk_kernel(AttnArgs a, const int2* __restrict__ qtiles) {
  __shared__ __align__(16) ChunkSmem sm;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tix = blockIdx.x / a.n_split;
  const int split = blockIdx.x - tix * a.n_split;
  const int2 td = qtiles[tix];
  if (td.y <= 0) return;
  int i, t;
  int64_t base;
  const bool mine = tile_query(a.b, td, wave, i, base, t);
  if (lane == 0) {
    sm.tq[wave] = mine ? t : -1;
    sm.base[wave] = base;
  }
  __syncthreads();
  int t_max = -1;
  int64_t seq_base = 0;
#pragma unroll
  for (int w = 0; w < kQT; ++w) {
    if (sm.tq[w] > t_max) {
      t_max = sm.tq[w];
      seq_base = sm.base[w];
    }
  }
  const int k0 = split * a.split_keys;
  if (t_max < 0 || k0 > t_max) return;  // the combine handles queries without partials
  const int k1 = min(t_max + 1, k0 + a.split_keys);
  const int ntiles = (k1 - k0 + kTile - 1) / kTile;

  // Q operands of this wave's query, staged through LDS so that no tracked global load
  // is outstanding inside the streaming loop
  bf16x8 qop[2][8];
  {
    const __bf16* qp = static_cast<const __bf16*>(a.q) + (size_t)(mine ? i : 0) * kHeads * kDim;
    uint8_t* qs = sm.q[wave];
    for (int e = lane; e < 16 * 64; e += 64) {
      const int ln = e & 63, sidx = (e >> 6) & 7, nb = e >> 9;
      *reinterpret_cast<uint4*>(qs + e * 16) = *reinterpret_cast<const uint4*>(
          qp + (32 * nb + (ln & 31)) * kDim + (ln >> 5) * 64 + sidx * 8);
    }
    __syncthreads();
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int s = 0; s < 8; ++s) qop[nb][s] = *reinterpret_cast<const bf16x8*>(qs + ((nb * 8 + s) * 64 + lane) * 16);
    __syncthreads();  // the staging area becomes the tile stages
  }

  WaveState st;
  state_init(st);
  float mx[2] = {-INFINITY, -INFINITY};
  const __bf16* kp = static_cast<const __bf16*>(a.k);
  const __bf16* vp = static_cast<const __bf16*>(a.v);
  const int tu = __builtin_amdgcn_readfirstlane(t);  // one query per wave
  chunk_stream<false>(st, mx, sm, qop, mine, tu, k0, k1, ntiles, seq_base, kp, vp, a.c2, wave, lane);

  // rare: a wave whose sums overflowed recomputes with its exact logit maximum; the
  // workgroup streams the tiles again together
  const bool bad = mine && !state_finite(st);
  if (lane == 0) sm.redo[wave] = bad ? 1 : 0;
  __syncthreads();
  if (sm.redo[0] | sm.redo[1] | sm.redo[2] | sm.redo[3]) {
    chunk_stream<true>(st, mx, sm, qop, bad, tu, k0, k1, ntiles, seq_base, kp, vp, a.c2, wave, lane);
    if (bad) {
      state_init(st);
      st.m[0] = mx[0];
      st.m[1] = mx[1];
      st.have_ref = 1;
    }
    __syncthreads();
    chunk_stream<false>(st, mx, sm, qop, bad, tu, k0, k1, ntiles, seq_base, kp, vp, a.c2, wave, lane);
  }

  if (!mine) return;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    st.l[nb] += __shfl_xor(st.l[nb], 32);
    st.le[nb] += __shfl_xor(st.le[nb], 32);
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
  const int hrow = 4 * (lane >> 5);
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
// Scores are staged in LDS and written every kFlush tiles, so that the stores do not
// interleave with the streaming copies.
// ------------------------------------------------------------------------------------
constexpr int kFlush = 16;

struct ScoreChunkSmem {
  union {
    uint8_t stage[kCStages][kTileBytes];
    uint8_t q[kQT][kHeads * kDim * 2];
  };
  uint32_t hist[kQT][kHistBins];
  float sbuf[kQT][kFlush * kTile];
  int tq[kQT];
  int64_t base[kQT];
};

__global__ __launch_bounds__(256) void score_chunk_kernel(ScoreArgs a, const int2* __restrict__ qtiles) {
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
  for (int e = lane; e < kHistBins; e += 64) sm.hist[wave][e] = 0u;
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

  bf16x8 qop[2][8];
  float l2[2][16];
  const int hrow = 4 * (lane >> 5);
  {
    const __bf16* qp = static_cast<const __bf16*>(a.q) + (size_t)(mine ? i : 0) * kHeads * kDim;
    uint8_t* qs = sm.q[wave];
    for (int e = lane; e < 16 * 64; e += 64) {
      const int ln = e & 63, sidx = (e >> 6) & 7, mb = e >> 9;
      *reinterpret_cast<uint4*>(qs + e * 16) = *reinterpret_cast<const uint4*>(
          qp + (32 * mb + (ln & 31)) * kDim + (ln >> 5) * 64 + sidx * 8);
    }
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int j = 0; j < 16; ++j)
        l2[mb][j] = mine ? a.lse2[(size_t)i * kHeads + 32 * mb + 8 * (j >> 2) + hrow + (j & 3)] : 0.0f;
    __syncthreads();
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int s = 0; s < 8; ++s) qop[mb][s] = *reinterpret_cast<const bf16x8*>(qs + ((mb * 8 + s) * 64 + lane) * 16);
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

  for (int it = 0; it < min(ntiles, kCStages - 1); ++it) issue_k(it, lk(it));
  for (int it = 0; it < ntiles; ++it) {
    const int sidx = it % kCStages;
    if (it + 1 < ntiles) wait_vmcnt<kCopiesPerWave>(); else wait_vmcnt<0>();
    loop_barrier();
    if (it + kCStages - 1 < ntiles) issue_k(it + kCStages - 1, lk((it + kCStages - 1) % kCStages));
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
        for (int j = 0; j < 16; ++j) sum += fast_exp2(acc[mb][j] * a.c2 - l2[mb][j]);
      const float other = __shfl_xor(sum, 32);
      const float total = (lane < 32) ? sum + other : other + sum;
      const int p = p0 + (lane & 31);
      if (lane < 32 && p < min(k1, nc)) {
        sm.sbuf[wave][(it % kFlush) * kTile + lane] = total;
        atomicAdd(&sm.hist[wave][__float_as_uint(total) >> kHistShift], 1u);
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
  for (int e = lane; e < kHistBins; e += 64) {
    const uint32_t c = sm.hist[wave][e];
    if (c) atomicAdd(&hq[e], c);
  }
}

}  // namespace

hipError_t launch_qtile_prep(const SeqsDev& b, int2* tiles, int max_tiles, hipStream_t s) {
  hipLaunchKernelGGL(qtile_prep_kernel, dim3(1), dim3(256), 0, s, b, tiles, max_tiles);
  return hipGetLastError();
}

hipError_t launch_attn_chunk(const AttnArgs& a, const int2* tiles, int max_tiles, hipStream_t s) {
  hipLaunchKernelGGL(attn_chunk_kernel, dim3(max_tiles * a.n_split), dim3(256), 0, s, a, tiles);
  return hipGetLastError();
}

hipError_t launch_score_chunk(const ScoreArgs& a, const int2* tiles, int max_tiles, hipStream_t s) {
  hipLaunchKernelGGL(score_chunk_kernel, dim3(max_tiles * a.n_split), dim3(256), 0, s, a, tiles);
  return hipGetLastError();
}

}  // namespace hs2
