// The decode-shaped attention kernel (one query per workgroup): the selector's exact
// causal attention (pass 1), templated on the storage format of K/V and on the number of
// waves per workgroup (4 for bf16 tiles, 8 for FP8 tiles, whose smaller tiles need two
// waves per SIMD to keep the SIMD busy).
// Included by attn_bf16.hip and attn_fp8.hip; the layout notes are in attn_bf16.hip.
#pragma once

#include "attn_common.h"

namespace hs2 {
namespace {

using namespace attn;

// Shared memory of the attention kernel: per-wave K and V stages during the key loop,
// then the cross-wave merge; Q (in MFMA operand order) stays outside the union.
constexpr int kStageArea = 131072;  // LDS of the K/V stages of a workgroup, split over its waves
constexpr int kMergeWaves = 4;      // waves of the final merge (an 8-wave group folds 4-7 into 0-3 first)

// Stages per wave: kStageArea / kW bytes hold this many (K + V) tile pairs.
template <typename Kv, int kW>
constexpr int stages_of() { return kStageArea / kW / (2 * Kv::kTileBytes); }
static_assert(stages_of<KvBf16, 4>() == 2 && stages_of<KvFp8, 4>() == 4 && stages_of<KvFp8, 8>() == 2, "stages");

template <int kW>
struct AttnSmem {
  union {
    uint8_t stage[kW][kStageArea / kW];  // stage j of a wave: K tile at 2j, V tile at 2j+1
    struct {
      float m[kMergeWaves][kHeads];
      float l[kMergeWaves][kHeads];
      float le[kMergeWaves][kHeads];
      float fm[kHeads];
      float fl[kHeads];
      float fle[kHeads];
      // per-wave O^T scaled to the common reference: [wave][d][h ^ 32 * ((d >> 2) & 1)];
      // with 8 waves, first the raw register image of wave w+4 for wave w
      float o[kMergeWaves][kDim * kHeads];
    } mg;
  };
  uint8_t q[kHeads * kDim * 2];
};

// The tiles of the workgroup's key range that one wave streams: tile x(it) = t0 + it * stride
// of the rotated order, it < n. The split is cut into kW / g contiguous chunks, each streamed
// by g waves in interleaved tiles, so that a workgroup reads 2 kW / g separate regions of K
// and V at a time. bf16 K/V (four waves): g = 2, four regions; on the 64 x 131,072 decode
// batch 7-9 us per selector call faster than g = 1 (eight regions), which was itself 6-11 us
// faster than g = 4 (two regions; same-box A/Bs, both orders). FP8 K/V (eight waves, bound by
// the per-tile conversion chain): g = 8; groups of 4 or 2 measured within noise of it.
struct WaveTiles {
  int t0, stride, n;
  template <typename Kv, int kW>
  __device__ static WaveTiles of(int wave, int ntiles) {
    constexpr int g = Kv::kFp8 ? kW : 2;  // waves per chunk
    if constexpr (g == kW) return WaveTiles{wave, kW, wave < ntiles ? (ntiles - wave + kW - 1) / kW : 0};
    const int c = wave / g, r = wave % g;
    const int qc = (ntiles + kW / g - 1) / (kW / g);  // tiles per chunk
    const int len = max(0, min(qc, ntiles - c * qc));
    return WaveTiles{c * qc + r, g, r < len ? (len - r + g - 1) / g : 0};
  }
  __device__ int at(int it) const { return t0 + it * stride; }
};

// Streams the tiles ord.at(wt.at(0)), ord.at(wt.at(1)), ... of the workgroup's key range
// through the wave's S = Kv::kStages LDS stages. DMA groups are issued in the order K0 V0 K1 V1 ..., then per
// tile K(it+S) right after the K operands of tile it are in registers and V(it+S) after
// its PV step, so S tiles stream in while one is computed. Waits count the copies issued
// later: constant in the steady state, and in the last S tiles a compile-time count per
// tile (the tail is unrolled), so the loop has no branches around its waits. The mask of
// attended keys is recomputed when a tile is processed (no per-stage state); the copies
// take their rows straight from the tile's first key (the keys are contiguous), with no
// exchange between lanes. kMaxOnly: only the logit maximum of the attended keys (into mx).
template <typename Kv, int kW, bool kMaxOnly, int kLater, bool kMore>
__device__ inline void stream_step(WaveState& st, float (&mx)[2], AttnSmem<kW>& sm, const KeyList& kl, int k0, int k1,
                                   const void* __restrict__ kp, const void* __restrict__ vp, float c2, int wave,
                                   int lane, const uint32_t (&vb)[4], uint32_t wbase, TileOrder ord, WaveTiles wt, int it) {
  constexpr int S = stages_of<Kv, kW>(), D = Kv::kDma, T = Kv::kTileBytes;
  const int sidx = it % S;
  wait_vmcnt<D * (1 + 2 * kLater)>();  // K(it) has landed
  const uint8_t* kt = sm.stage[wave] + (2 * sidx) * T;
  bf16x8 kop[8];
  read_k_of<Kv>(kt, lane, kop);
  int rel;  // unused here: the copies compute their rows from the tile's first key
  const uint32_t vm = tile_rows(kl, k0 + ord.at(wt.at(it)) * kTile, k1, lane, rel);
  const int pend = min(k1, kl.n_keys);                                  // keys past it copy row 0
  const int pn = kMore ? k0 + ord.at(wt.at(it + S)) * kTile : 0;  // first key of tile it+S
  if (kMore) issue_tile_contig<Kv, true>(kp, kl.base, pn, pend, lane, wbase + (2 * sidx) * T);
  wait_vmcnt<D * (2 * kLater + (kMore ? 1 : 0))>();  // V(it) has landed
  if (vm != 0u) {
    if (kMaxOnly)
      process_tile_max<false>(mx, sm.q, nullptr, kop, vm, c2, lane);
    else
      process_tile<false, Kv>(st, sm.q, nullptr, kop, kt + T, vb, vm, c2, lane);
  }
  if (kMore) issue_tile_contig<Kv, false>(vp, kl.base, pn, pend, lane, wbase + (2 * sidx + 1) * T);
}

template <typename Kv, int kW, bool kMaxOnly, int kLater>
__device__ inline void stream_tail(WaveState& st, float (&mx)[2], AttnSmem<kW>& sm, const KeyList& kl, int k0, int k1,
                                   const void* __restrict__ kp, const void* __restrict__ vp, float c2, int wave,
                                   int lane, const uint32_t (&vb)[4], uint32_t wbase, TileOrder ord, WaveTiles wt) {
  const int it = wt.n - 1 - kLater;
  if (it >= 0) stream_step<Kv, kW, kMaxOnly, kLater, false>(st, mx, sm, kl, k0, k1, kp, vp, c2, wave, lane, vb, wbase, ord, wt, it);
  if constexpr (kLater > 0)
    stream_tail<Kv, kW, kMaxOnly, kLater - 1>(st, mx, sm, kl, k0, k1, kp, vp, c2, wave, lane, vb, wbase, ord, wt);
}

template <typename Kv, int kW, bool kMaxOnly>
__device__ inline void stream_tiles(WaveState& st, float (&mx)[2], AttnSmem<kW>& sm, const KeyList& kl, int k0, int k1,
                                    int ntiles, const void* __restrict__ kp, const void* __restrict__ vp,
                                    float c2, int wave, int lane, TileOrder ord) {
  constexpr int S = stages_of<Kv, kW>(), T = Kv::kTileBytes;
  const WaveTiles wt = WaveTiles::of<Kv, kW>(wave, ntiles);
  const int ntw = wt.n;
  const uint32_t wbase = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)sm.stage[wave]);
  uint32_t vb[4];
  vt_bases_of<Kv>(lane, vb);
  for (int it = 0; it < min(ntw, S); ++it) {
    const int p0 = k0 + ord.at(wt.at(it)) * kTile, pend = min(k1, kl.n_keys);
    issue_tile_contig<Kv, true>(kp, kl.base, p0, pend, lane, wbase + (2 * it) * T);
    issue_tile_contig<Kv, false>(vp, kl.base, p0, pend, lane, wbase + (2 * it + 1) * T);
  }
  for (int it = 0; it + S < ntw; ++it)
    stream_step<Kv, kW, kMaxOnly, S - 1, true>(st, mx, sm, kl, k0, k1, kp, vp, c2, wave, lane, vb, wbase, ord, wt, it);
  stream_tail<Kv, kW, kMaxOnly, S - 1>(st, mx, sm, kl, k0, k1, kp, vp, c2, wave, lane, vb, wbase, ord, wt);
}

template <typename Kv, int kW>
__global__ __launch_bounds__(64 * kW) void attn_bf16_kernel(AttnArgs a, WorkList wl, uint32_t* hist,
                                                           uint32_t* counters) {
  constexpr int kThreads = 64 * kW;
  constexpr int kQPieces = kHeads * kDim * 2 / 16 / kThreads;  // 16-byte pieces of Q per thread
  __shared__ __align__(16) AttnSmem<kW> sm;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int i, split;
  work_item(wl, a.n_split, i, split);
  const int k0 = split * a.split_keys;

  // Q goes out before the descriptor is known, in MFMA operand order: 16-byte piece
  // (nb, s, lane) = Q[32nb + l%32][(l/32)*64 + 8s ..]
  bf16x8 qv[kQPieces];
  {
    const __bf16* qp = static_cast<const __bf16*>(a.q) + (size_t)i * kHeads * kDim;
#pragma unroll
    for (int u = 0; u < kQPieces; ++u) {
      const int e = (int)threadIdx.x + kThreads * u;
      const int ln = e & 63, sidx = (e >> 6) & 7, nb = e >> 9;
      qv[u] = *reinterpret_cast<const bf16x8*>(qp + (32 * nb + (ln & 31)) * kDim + (ln >> 5) * 64 + sidx * 8);
    }
  }

  int64_t base;
  int t;
  const bool valid = __builtin_amdgcn_readfirstlane(query_desc(a.b, i, base, t));
  // the descriptor is the same on every lane (query i): keep the loop control scalar
  t = __builtin_amdgcn_readfirstlane(t);
  base = (int64_t)uniform_u64((uint64_t)base);
  if (a.n_split == 1 && hist != nullptr) {
    for (int e = threadIdx.x; e < kHistBins; e += blockDim.x) hist[(size_t)i * kHistBins + e] = 0u;
    if (threadIdx.x < 4) counters[(size_t)i * 4 + threadIdx.x] = 0u;
  }
  if (wl.n > 0 && a.plan_miss != nullptr && threadIdx.x == 0 && last_planned(wl, i))
    a.plan_miss[i] = (valid && k0 + a.split_keys < t + 1) ? 1 : 0;
  if (!valid) {
    if (a.n_split == 1) {
      __bf16* out = static_cast<__bf16*>(a.out) + (size_t)i * kHeads * kDim;
      for (int e = threadIdx.x; e < kHeads * kDim; e += blockDim.x) out[e] = (__bf16)NAN;
      if (threadIdx.x < kHeads) {
        if (a.lse) a.lse[(size_t)i * kHeads + threadIdx.x] = NAN;
        if (a.lse2) a.lse2[(size_t)i * kHeads + threadIdx.x] = NAN;
      }
    }
    return;
  }

  KeyList kl;
  kl.base = base;
  kl.n_keys = t + 1;
  if (k0 >= kl.n_keys) return;  // empty split: the combine does not read it
  const int k1 = min(kl.n_keys, k0 + a.split_keys);
  const int ntiles = (k1 - k0 + kTile - 1) / kTile;
#pragma unroll
  for (int u = 0; u < kQPieces; ++u) *reinterpret_cast<bf16x8*>(sm.q + ((int)threadIdx.x + kThreads * u) * 16) = qv[u];
  __syncthreads();

  const void* kp = a.k;
  const void* vp = a.v;
  const TileOrder ord = TileOrder::rotated(i * a.n_split + split, ntiles);
  WaveState st;
  state_init(st);
  float mx[2] = {-INFINITY, -INFINITY};
  stream_tiles<Kv, kW, false>(st, mx, sm, kl, k0, k1, ntiles, kp, vp, a.c2, wave, lane, ord);
  if (!state_finite(st)) {
    // rare: a logit far above the first tile's maximum overflowed the sums; recompute
    // with the exact maximum of this wave's keys as reference (every weight <= 1)
    stream_tiles<Kv, kW, true>(st, mx, sm, kl, k0, k1, ntiles, kp, vp, a.c2, wave, lane, ord);
    state_init(st);
    st.m[0] = mx[0];
    st.m[1] = mx[1];
    st.have_ref = 1;
    stream_tiles<Kv, kW, false>(st, mx, sm, kl, k0, k1, ntiles, kp, vp, a.c2, wave, lane, ord);
  }

#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    st.l[nb] += __shfl_xor(st.l[nb], 32);
    st.le[nb] += __shfl_xor(st.le[nb], 32);
  }

  __syncthreads();  // LDS stages no longer needed
  if constexpr (kW == 8) {
    // waves 4-7 hand their state to waves 0-3 (same SIMD, same lane layout): the raw
    // register image of O^T and the per-head reference and sums
    if (wave >= kMergeWaves) {
      float* img = sm.mg.o[wave - kMergeWaves];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int j = 0; j < 16; ++j) img[((nb * 4 + mb) * 16 + j) * 64 + lane] = st.o[nb][mb][j];
      if (lane < 32) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          sm.mg.m[wave - kMergeWaves][32 * nb + lane] = st.m[nb];
          sm.mg.l[wave - kMergeWaves][32 * nb + lane] = st.l[nb];
          sm.mg.le[wave - kMergeWaves][32 * nb + lane] = st.le[nb];
        }
      }
    }
    __syncthreads();
    if (wave < kMergeWaves) {
      const float* img = sm.mg.o[wave];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int h = 32 * nb + (lane & 31);
        const float mp = sm.mg.m[wave][h];
        const float M = fmaxf(st.m[nb], mp);
        const float fa = fast_exp2(st.m[nb] - M), fb = fast_exp2(mp - M);
        st.m[nb] = M;
        st.l[nb] = st.l[nb] * fa + sm.mg.l[wave][h] * fb;
        st.le[nb] = st.le[nb] * fa + sm.mg.le[wave][h] * fb;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int j = 0; j < 16; ++j)
            st.o[nb][mb][j] = st.o[nb][mb][j] * fa + img[((nb * 4 + mb) * 16 + j) * 64 + lane] * fb;
      }
    }
    __syncthreads();
  }
  // ---- merge the four (remaining) waves (fixed order, deterministic) ----
  if (wave < kMergeWaves && lane < 32) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      sm.mg.m[wave][32 * nb + lane] = st.m[nb];
      sm.mg.l[wave][32 * nb + lane] = st.l[nb];
      sm.mg.le[wave][32 * nb + lane] = st.le[nb];
    }
  }
  __syncthreads();
  {
    float alpha[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int h = 32 * nb + (lane & 31);
      float M = sm.mg.m[0][h];
#pragma unroll
      for (int w = 1; w < kMergeWaves; ++w) M = fmaxf(M, sm.mg.m[w][h]);
      alpha[nb] = fast_exp2(st.m[nb] - M);
    }
    if (threadIdx.x < kHeads) {
      const int h = threadIdx.x;
      float M = sm.mg.m[0][h];
#pragma unroll
      for (int w = 1; w < kMergeWaves; ++w) M = fmaxf(M, sm.mg.m[w][h]);
      float L = 0.0f, LE = 0.0f;
#pragma unroll
      for (int w = 0; w < kMergeWaves; ++w) {
        const float f = fast_exp2(sm.mg.m[w][h] - M);
        L += sm.mg.l[w][h] * f;
        LE += sm.mg.le[w][h] * f;
      }
      sm.mg.fm[h] = M;
      sm.mg.fl[h] = L;
      sm.mg.fle[h] = LE;
    }
    const int hrow = 4 * (lane >> 5);
    float* ow = sm.mg.o[wave < kMergeWaves ? wave : 0];
#pragma unroll
    for (int nb = 0; nb < 2 && wave < kMergeWaves; ++nb)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int d = 32 * mb + 8 * (j >> 2) + hrow + (j & 3);
          const int h = 32 * nb + (lane & 31);
          ow[d * kHeads + (h ^ (32 * ((d >> 2) & 1)))] = st.o[nb][mb][j] * alpha[nb];
        }
  }
  __syncthreads();

  // thread (h, dq): dims 32dq .. 32dq+31 of head h, summed over the waves in order
  const int h = threadIdx.x & 63, dq = threadIdx.x >> 6;
  if (threadIdx.x >= 256) return;  // 8-wave groups: waves 4-7 are done
  if (a.n_split == 1) {
    __bf16* out = static_cast<__bf16*>(a.out) + ((size_t)i * kHeads + h) * kDim + 32 * dq;
    const float inv = a.v_scale / sm.mg.fl[h];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      bf16x8 v;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int d = 32 * dq + 8 * c + r;
        const int pos = d * kHeads + (h ^ (32 * ((d >> 2) & 1)));
        const float sum = ((sm.mg.o[0][pos] + sm.mg.o[1][pos]) + sm.mg.o[2][pos]) + sm.mg.o[3][pos];
        v[r] = (__bf16)(sum * inv);
      }
      *reinterpret_cast<bf16x8*>(out + 8 * c) = v;
    }
    if (threadIdx.x < kHeads) {
      const float l2 = sm.mg.fm[h] + __log2f(sm.mg.fle[h]);
      if (a.lse) a.lse[(size_t)i * kHeads + h] = l2 * kLn2;
      if (a.lse2) a.lse2[(size_t)i * kHeads + h] = l2;
    }
  } else {
    Partial* P = a.part + (size_t)i * a.n_split + split;
    if (threadIdx.x < kHeads) {
      P->m[h] = sm.mg.fm[h];
      P->l[h] = sm.mg.fl[h];
      P->le[h] = sm.mg.fle[h];
    }
#pragma unroll 8
    for (int r = 0; r < 32; ++r) {
      const int d = 32 * dq + r;
      const int pos = d * kHeads + (h ^ (32 * ((d >> 2) & 1)));
      P->o[d * kHeads + h] = ((sm.mg.o[0][pos] + sm.mg.o[1][pos]) + sm.mg.o[2][pos]) + sm.mg.o[3][pos];
    }
  }
}


}  // namespace
}  // namespace hs2
