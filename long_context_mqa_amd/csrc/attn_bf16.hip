// bf16 MQA attention kernels for gfx950: the selector's exact causal attention (pass 1),
// the sparse layers' gathered attention and the split combine. The selection-score pass
// is in score_bf16.hip.
//
// Method (page title and section):
//   arex-research.com, "Xiaomi MiMo lead Luo Fuli publishes the MiMo-V3 core architecture
//   HySparse2", section "Outer KV Bridging, inner KV Reuse": the full-attention layer
//   computes exact attention and its scores index the sparse layers, which reuse its KV
//   cache and indices; the 128 most recent tokens are always attended and 1,024 more
//   are picked by score. Section "Numbers computed on three 80B-A3B models": 64 query
//   heads share one KV head (MQA).
//
// Layout on the matrix cores (v_mfma_f32_32x32x16_bf16, 64-lane waves):
//   A operand [32 x 16]: lane l holds row l%32, k = 8*(l/32) + 0..7
//   B operand [16 x 32]: lane l holds col l%32, k = 8*(l/32) + 0..7
//   C/D       [32 x 32]: lane l holds col l%32, rows 8*(j/4) + 4*(l/32) + j%4, j = 0..15
// The 128-wide head dimension is contracted in 8 steps of 16. Because a contraction is
// a sum, the order of its index is free: step s, lane half h covers dims h*64 + s*8 +
// 0..7, so each lane loads one contiguous 128-byte half row of K and of Q.
//
// Pass 1 computes S^T = K Q^T (keys as rows, heads as columns), so each lane owns two
// heads and sees 16 keys of a 32-key tile. The probabilities P^T in the C layout are
// already the B operand of O^T = V^T P^T when the key index of each 16-key step is
// permuted to match; the V^T operands come from transposing LDS reads of the V tile.
// Softmax runs in the log2 domain (x = scale*log2(e)*s). The reference of each head is
// fixed at the wave's first tile with an attended key, so the accumulators are never
// rescaled inside the key loop; a wave whose sums overflowed (a logit more than ~100
// above that first maximum) recomputes its keys with its exact maximum as reference.
// P is rounded to bf16 for the MFMA and the output's denominator sums the same rounded
// values, so the output is an exactly normalised average of V rows; the LSE uses the sum
// of the unrounded values.
#include "attn_common.h"

namespace hs2 {
namespace {

using namespace attn;

// Shared memory of the attention kernel: per-wave K and V stages during the key loop,
// then the cross-wave merge; Q (in MFMA operand order) and the gathered row list stay
// outside the union.
constexpr int kSelMax = 2048;  // gathered slots per workgroup (the host caps the split)
constexpr int kSelPerThread = kSelMax / 256;

constexpr int kWaveStageBytes = 32768;  // per wave: Kv::kStages x (K + V) tiles
static_assert(KvBf16::kStages * 2 * KvBf16::kTileBytes == kWaveStageBytes, "bf16 stages");
static_assert(KvFp8::kStages * 2 * KvFp8::kTileBytes == kWaveStageBytes, "fp8 stages");

struct AttnSmem {
  union {
    uint8_t stage[kWaves][kWaveStageBytes];  // stage j of a wave: K tile at 2j, V tile at 2j+1
    struct {
      float m[kWaves][kHeads];
      float l[kWaves][kHeads];
      float le[kWaves][kHeads];
      float fm[kHeads];
      float fl[kHeads];
      float fle[kHeads];
      // per-wave O^T scaled to the common reference: [wave][d][h ^ 32 * ((d >> 2) & 1)]
      float o[kWaves][kDim * kHeads];
    } mg;
  };
  uint8_t q[kHeads * kDim * 2];
  int32_t sel[kSelMax];
};

// Streams the tiles wave, wave + 4, ... of the workgroup's key range through the wave's
// S = Kv::kStages LDS stages. DMA groups are issued in the order K0 V0 K1 V1 ..., then per
// tile K(it+S) right after the K operands of tile it are in registers and V(it+S) after
// its PV step, so S tiles stream in while one is computed. Waits count the copies issued
// later: constant in the steady state, and in the last S tiles a compile-time count per
// tile (the tail is unrolled), so the loop has no branches around its waits. The mask of
// attended keys is recomputed when a tile is processed (no per-stage state). kMaxOnly:
// only the logit maximum of the attended keys (into mx).
template <typename Kv, bool kMaxOnly, int kLater, bool kMore>
__device__ inline void stream_step(WaveState& st, float (&mx)[2], AttnSmem& sm, const KeyList& kl, int k0, int k1,
                                   const void* __restrict__ kp, const void* __restrict__ vp, float c2, int wave,
                                   int lane, const uint32_t (&vb)[4], uint32_t wbase, int it) {
  constexpr int S = Kv::kStages, D = Kv::kDma, T = Kv::kTileBytes;
  const int sidx = it % S;
  wait_vmcnt<D * (1 + 2 * kLater)>();  // K(it) has landed
  const uint8_t* kt = sm.stage[wave] + (2 * sidx) * T;
  bf16x8 kop[8];
  read_k_of<Kv>(kt, lane, kop);
  int rel;
  const uint32_t vm = tile_rows(kl, k0 + (wave + it * kWaves) * kTile, k1, lane, rel);
  if (kMore) {
    tile_rows(kl, k0 + (wave + (it + S) * kWaves) * kTile, k1, lane, rel);
    issue_tile<Kv, true>(kp, kl.base, rel, lane, wbase + (2 * sidx) * T);
  }
  wait_vmcnt<D * (2 * kLater + (kMore ? 1 : 0))>();  // V(it) has landed
  if (vm != 0u) {
    if (kMaxOnly)
      process_tile_max<false>(mx, sm.q, nullptr, kop, vm, c2, lane);
    else
      process_tile<false, Kv>(st, sm.q, nullptr, kop, kt + T, vb, vm, c2, lane);
  }
  if (kMore) issue_tile<Kv, false>(vp, kl.base, rel, lane, wbase + (2 * sidx + 1) * T);
}

template <typename Kv, bool kMaxOnly, int kLater>
__device__ inline void stream_tail(WaveState& st, float (&mx)[2], AttnSmem& sm, const KeyList& kl, int k0, int k1,
                                   const void* __restrict__ kp, const void* __restrict__ vp, float c2, int wave,
                                   int lane, const uint32_t (&vb)[4], uint32_t wbase, int ntw) {
  const int it = ntw - 1 - kLater;
  if (it >= 0) stream_step<Kv, kMaxOnly, kLater, false>(st, mx, sm, kl, k0, k1, kp, vp, c2, wave, lane, vb, wbase, it);
  if constexpr (kLater > 0)
    stream_tail<Kv, kMaxOnly, kLater - 1>(st, mx, sm, kl, k0, k1, kp, vp, c2, wave, lane, vb, wbase, ntw);
}

template <typename Kv, bool kMaxOnly>
__device__ inline void stream_tiles(WaveState& st, float (&mx)[2], AttnSmem& sm, const KeyList& kl, int k0, int k1,
                                    int ntiles, const void* __restrict__ kp, const void* __restrict__ vp,
                                    float c2, int wave, int lane) {
  constexpr int S = Kv::kStages, T = Kv::kTileBytes;
  const int ntw = wave < ntiles ? (ntiles - wave + kWaves - 1) / kWaves : 0;
  const uint32_t wbase = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)sm.stage[wave]);
  uint32_t vb[4];
  vt_bases_of<Kv>(lane, vb);
  for (int it = 0; it < min(ntw, S); ++it) {
    int rel;
    tile_rows(kl, k0 + (wave + it * kWaves) * kTile, k1, lane, rel);
    issue_tile<Kv, true>(kp, kl.base, rel, lane, wbase + (2 * it) * T);
    issue_tile<Kv, false>(vp, kl.base, rel, lane, wbase + (2 * it + 1) * T);
  }
  for (int it = 0; it + S < ntw; ++it)
    stream_step<Kv, kMaxOnly, S - 1, true>(st, mx, sm, kl, k0, k1, kp, vp, c2, wave, lane, vb, wbase, it);
  stream_tail<Kv, kMaxOnly, S - 1>(st, mx, sm, kl, k0, k1, kp, vp, c2, wave, lane, vb, wbase, ntw);
}

template <typename Kv, bool kGather>
__global__ __launch_bounds__(256) void attn_bf16_kernel(AttnArgs a, WorkList wl, uint32_t* hist,
                                                        uint32_t* counters) {
  __shared__ __align__(16) AttnSmem sm;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int i, split;
  work_item(wl, a.n_split, i, split);
  const int k0 = split * a.split_keys;

  // Loads that do not depend on the query's position go out first: the gathered slots
  // of this split (gather mode: the key count exceeds top_k, so the slot range is known)
  // and Q in MFMA operand order: 16-byte piece (nb, s, lane) = Q[32nb + l%32][(l/32)*64 + 8s ..]
  int32_t selv[kSelPerThread];
  const int s1 = kGather ? min(min(a.top_k, k0 + a.split_keys), k0 + kSelMax) : 0;
  if (kGather) {
    const int32_t* selr = a.sel + (size_t)i * a.top_k;
#pragma unroll
    for (int u = 0; u < kSelPerThread; ++u) {
      const int p = k0 + (int)threadIdx.x + 256 * u;
      selv[u] = p < s1 ? selr[p] : -1;
    }
  }
  bf16x8 qv[4];
  {
    const __bf16* qp = static_cast<const __bf16*>(a.q) + (size_t)i * kHeads * kDim;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = (int)threadIdx.x + 256 * u;
      const int ln = e & 63, sidx = (e >> 6) & 7, nb = e >> 9;
      qv[u] = *reinterpret_cast<const bf16x8*>(qp + (32 * nb + (ln & 31)) * kDim + (ln >> 5) * 64 + sidx * 8);
    }
  }

  int64_t base;
  int t;
  const bool valid = __builtin_amdgcn_readfirstlane(query_desc(a.b, i, base, t));
  // the descriptor is the same on every lane (query i): keep the loop control scalar
  t = __builtin_amdgcn_readfirstlane(t);
  base = (int64_t)(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)base >> 32)) << 32) |
                   (uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)base));
  if (a.n_split == 1 && hist != nullptr) {
    for (int e = threadIdx.x; e < kHistBins; e += blockDim.x) hist[(size_t)i * kHistBins + e] = 0u;
    if (threadIdx.x < 4) counters[(size_t)i * 4 + threadIdx.x] = 0u;
  }
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
  kl.gather = kGather;
  kl.base = base;
  kl.t = t;
  kl.top_k = a.top_k;
  kl.n_keys = logical_keys(kGather, t, a.window, a.top_k);
  kl.w_eff = min(a.window, t + 1);
  kl.cand_hi = t - a.window;
  if (k0 >= kl.n_keys) return;  // empty split: the combine does not read it
  const int k1 = min(kl.n_keys, k0 + a.split_keys);
  const int ntiles = (k1 - k0 + kTile - 1) / kTile;
  kl.sel_lds = sm.sel;
  kl.sel_k0 = k0;
  if (kGather) {
#pragma unroll
    for (int u = 0; u < kSelPerThread; ++u) {
      const int p = k0 + (int)threadIdx.x + 256 * u;
      if (p < s1) sm.sel[p - k0] = selv[u];
    }
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) *reinterpret_cast<bf16x8*>(sm.q + ((int)threadIdx.x + 256 * u) * 16) = qv[u];
  __syncthreads();

  const void* kp = a.k;
  const void* vp = a.v;
  WaveState st;
  state_init(st);
  float mx[2] = {-INFINITY, -INFINITY};
  stream_tiles<Kv, false>(st, mx, sm, kl, k0, k1, ntiles, kp, vp, a.c2, wave, lane);
  if (!state_finite(st)) {
    // rare: a logit far above the first tile's maximum overflowed the sums; recompute
    // with the exact maximum of this wave's keys as reference (every weight <= 1)
    stream_tiles<Kv, true>(st, mx, sm, kl, k0, k1, ntiles, kp, vp, a.c2, wave, lane);
    state_init(st);
    st.m[0] = mx[0];
    st.m[1] = mx[1];
    st.have_ref = 1;
    stream_tiles<Kv, false>(st, mx, sm, kl, k0, k1, ntiles, kp, vp, a.c2, wave, lane);
  }

#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    st.l[nb] += __shfl_xor(st.l[nb], 32);
    st.le[nb] += __shfl_xor(st.le[nb], 32);
  }

  // ---- merge the four waves (fixed order, deterministic) ----
  __syncthreads();  // LDS stages no longer needed
  if (lane < 32) {
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
      for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sm.mg.m[w][h]);
      alpha[nb] = fast_exp2(st.m[nb] - M);
    }
    if (threadIdx.x < kHeads) {
      const int h = threadIdx.x;
      float M = sm.mg.m[0][h];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sm.mg.m[w][h]);
      float L = 0.0f, LE = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = fast_exp2(sm.mg.m[w][h] - M);
        L += sm.mg.l[w][h] * f;
        LE += sm.mg.le[w][h] * f;
      }
      sm.mg.fm[h] = M;
      sm.mg.fl[h] = L;
      sm.mg.fle[h] = LE;
    }
    const int hrow = 4 * (lane >> 5);
    float* ow = sm.mg.o[wave];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
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

// ------------------------------------------------------------------------------------
// Split combine: merges the partials of a query in split order, writes O, LSE and the
// log2-domain LSE used by the score pass, and clears the query's selection counters.
// Grid: total_q x kCombineSlabs; a slab covers 16 dims x 64 heads of the output.
// ------------------------------------------------------------------------------------
constexpr int kCombineSlabs = kDim / 16;
constexpr int kMaxSplit = 256;

template <typename OutT>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  __shared__ float w_s[kMaxSplit][kHeads];
  __shared__ float red[4][kHeads];
  __shared__ float rede[4][kHeads];
  __shared__ float fm[kHeads], fl[kHeads];
  const int i = blockIdx.x / kCombineSlabs;
  const int slab = blockIdx.x - i * kCombineSlabs;
  const int tid = threadIdx.x;
  const int h = tid & 63, grp = tid >> 6;
  if (a.hist) {
    constexpr int per = kHistBins / kCombineSlabs;
    for (int e = tid; e < per; e += blockDim.x) a.hist[(size_t)i * kHistBins + slab * per + e] = 0u;
    if (slab == 0 && tid < 4) a.counters[(size_t)i * 4 + tid] = 0u;
  }
  int64_t base;
  int t;
  const bool valid = query_desc(a.b, i, base, t);
  OutT* out = static_cast<OutT*>(a.out) + (size_t)i * kHeads * kDim;
  const int d0 = slab * 16 + grp * 4;
  if (!valid) {
#pragma unroll
    for (int r = 0; r < 4; ++r) out[h * kDim + d0 + r] = (OutT)NAN;
    if (slab == 0 && tid < kHeads) {
      if (a.lse) a.lse[(size_t)i * kHeads + tid] = NAN;
      if (a.lse2) a.lse2[(size_t)i * kHeads + tid] = NAN;
    }
    return;
  }
  const int n_keys = logical_keys(a.gather != 0, t, a.window, a.top_k);
  const int nv = min(a.n_split, (n_keys + a.split_keys - 1) / a.split_keys);
  const Partial* P = a.part + (size_t)i * a.n_split;
  // max over splits: four groups of 64 threads take every fourth split
  float mx = -INFINITY;
  for (int s2 = grp; s2 < nv; s2 += 4) mx = fmaxf(mx, P[s2].m[h]);
  red[grp][h] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0][h], red[1][h]), fmaxf(red[2][h], red[3][h]));
  __syncthreads();
  float lsum = 0.0f, esum = 0.0f;
  for (int s2 = grp; s2 < nv; s2 += 4) {
    const float w = __builtin_amdgcn_exp2f(P[s2].m[h] - M);
    w_s[s2][h] = w;
    lsum += P[s2].l[h] * w;
    esum += P[s2].le[h] * w;
  }
  red[grp][h] = lsum;
  rede[grp][h] = esum;
  __syncthreads();
  if (tid < kHeads) {
    const float L = (red[0][h] + red[1][h]) + (red[2][h] + red[3][h]);
    const float LE = (rede[0][h] + rede[1][h]) + (rede[2][h] + rede[3][h]);
    fm[h] = M;
    fl[h] = L;
    if (slab == 0) {
      const float l2 = M + __log2f(LE);
      if (a.lse) a.lse[(size_t)i * kHeads + h] = l2 * kLn2;
      if (a.lse2) a.lse2[(size_t)i * kHeads + h] = l2;
    }
  }
  __syncthreads();
  // thread (h, grp): dims d0 .. d0+3 of head h; loads of 4 splits in flight at a time
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  int s2 = 0;
  for (; s2 + 4 <= nv; s2 += 4) {
    float v[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) v[u][r] = P[s2 + u].o[(d0 + r) * kHeads + h];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float w = w_s[s2 + u][h];
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] += v[u][r] * w;
    }
  }
  for (; s2 < nv; ++s2) {
    const float w = w_s[s2][h];
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] += P[s2].o[(d0 + r) * kHeads + h] * w;
  }
  const float inv = a.v_scale / fl[h];
#pragma unroll
  for (int r = 0; r < 4; ++r) out[h * kDim + d0 + r] = (OutT)(acc[r] * inv);
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs& a, const WorkList& wl, bool gather, int grid, uint32_t* hist,
                            uint32_t* counters, hipStream_t s) {
  if (gather)
    hipLaunchKernelGGL((attn_bf16_kernel<KvBf16, true>), dim3(grid), dim3(256), 0, s, a, wl, hist, counters);
  else
    hipLaunchKernelGGL((attn_bf16_kernel<KvBf16, false>), dim3(grid), dim3(256), 0, s, a, wl, hist, counters);
  return hipGetLastError();
}

hipError_t launch_attn_fp8kv(const AttnArgs& a, const WorkList& wl, bool gather, int grid, uint32_t* hist,
                             uint32_t* counters, hipStream_t s) {
  if (gather)
    hipLaunchKernelGGL((attn_bf16_kernel<KvFp8, true>), dim3(grid), dim3(256), 0, s, a, wl, hist, counters);
  else
    hipLaunchKernelGGL((attn_bf16_kernel<KvFp8, false>), dim3(grid), dim3(256), 0, s, a, wl, hist, counters);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, bool f32, hipStream_t s) {
  const dim3 grid(a.b.total_q * kCombineSlabs);
  if (f32)
    hipLaunchKernelGGL(combine_kernel<float>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(combine_kernel<__bf16>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}


}  // namespace hs2
