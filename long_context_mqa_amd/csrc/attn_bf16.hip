// bf16 MQA attention kernels for gfx950: the selector's exact causal attention (pass 1),
// the sparse layers' gathered attention, the split combine, and the selection-score
// pass (pass 2) that sums softmax probabilities over the 64 heads.
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
// heads and sees 16 keys of a 32-key tile: the per-head running max is an in-register
// reduction plus one exchange with lane l^32. The probabilities P^T in the C layout are
// already the B operand of O^T = V^T P^T when the key index of each 16-key step is
// permuted to match; V^T comes from a per-wave LDS copy of the V tile.
// Softmax runs in the log2 domain (x = scale*log2(e)*s) with a lazily moved reference:
// the running max only moves when a tile exceeds it by more than 8, which keeps every
// exponent <= 2^8 while avoiding a rescale of the 128 accumulators on most tiles.
// P is rounded to bf16 for the MFMA and the denominator sums the same rounded values,
// so the output is an exactly normalised average of V rows.
#include "hs2_internal.h"

namespace hs2 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kVRow = kDim + 8;     // padded LDS row (bf16 elements) of a V tile
constexpr float kNegBig = -1.0e30f; // "no key yet" reference: exp2(x - kNegBig) never used
constexpr float kLazy = 8.0f;       // reference moves only when exceeded by more than this

__device__ inline f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Logical key list of one query. Full mode: positions 0..t. Gather mode: top_k selected
// slots (entries outside the candidate range are masked) followed by the window rows.
struct KeyList {
  const int32_t* sel_row;
  int64_t base;
  int t, window, top_k, n_keys, w_eff, cand_hi;
  bool gather;

  __device__ inline void row(int p, int& rel, bool& ok) const {
    if (!gather) {
      ok = p < n_keys;
      rel = ok ? p : 0;
      return;
    }
    if (p < top_k) {
      const int s = sel_row[p];
      ok = s >= 0 && s <= cand_hi;
      rel = ok ? s : 0;
      return;
    }
    const int w = p - top_k;
    ok = w < w_eff;
    rel = ok ? (t - w_eff + 1 + w) : 0;
  }
};

struct TileRegs {
  bf16x8 k[8];   // K half-row of key l%32 (dims (l/32)*64 + s*8 ..)
  uint4 v[8];    // V piece r: key r*4 + l/16, dims (l%16)*8 .. +8
  bool ok;       // key l%32 of the tile is attended
};

__device__ inline void load_tile(const KeyList& kl, const __bf16* __restrict__ kp,
                                 const uint16_t* __restrict__ vp, int p0, int p1, int lane,
                                 TileRegs& r) {
  int rel;
  bool ok;
  const int p = p0 + (lane & 31);
  kl.row(p, rel, ok);
  ok = ok && p < p1;
  if (!ok) rel = 0;
  r.ok = ok;
  const __bf16* krow = kp + (kl.base + rel) * kDim + (lane >> 5) * 64;
#pragma unroll
  for (int s = 0; s < 8; ++s) r.k[s] = *reinterpret_cast<const bf16x8*>(krow + s * 8);
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int key = q * 4 + (lane >> 4);
    const int vrel = __shfl(rel, key);
    r.v[q] = *reinterpret_cast<const uint4*>(vp + (kl.base + vrel) * kDim + (lane & 15) * 8);
  }
}

// Online-softmax state of one wave: 64 heads x 128 dims, O^T in the C layout.
struct WaveState {
  f32x16 o[2][4];   // [head block nb][dim block mb]
  float m[2];       // reference (log2 domain) of heads 32*nb + l%32
  float l[2];       // this lane's share of the denominator
};

__device__ inline void process_tile(WaveState& st, const bf16x8 (&qop)[2][8], const TileRegs& r,
                                    uint16_t* __restrict__ vl, float c2, int lane) {
  // stage V tile in LDS (row-major, padded rows)
#pragma unroll
  for (int q = 0; q < 8; ++q)
    *reinterpret_cast<uint4*>(vl + (q * 4 + (lane >> 4)) * kVRow + (lane & 15) * 8) = r.v[q];

  // S^T = K Q^T
  f32x16 acc[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    acc[nb] = f32x16{};
#pragma unroll
    for (int s = 0; s < 8; ++s) acc[nb] = mfma(r.k[s], qop[nb][s], acc[nb]);
  }

  const uint32_t vm = (uint32_t)__ballot(r.ok);
  const int hrow = 4 * (lane >> 5);
  float x[2][16];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int j = 0; j < 16; ++j) x[nb][j] = acc[nb][j] * c2;
  if (vm != 0xffffffffu) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int key = 8 * (j >> 2) + hrow + (j & 3);
        if (!((vm >> key) & 1u)) x[nb][j] = -INFINITY;
      }
  }

  float mx[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    float v = x[nb][0];
#pragma unroll
    for (int j = 1; j < 16; ++j) v = fmaxf(v, x[nb][j]);
    mx[nb] = fmaxf(v, __shfl_xor(v, 32));
  }
  const bool need0 = mx[0] > st.m[0] + kLazy;
  const bool need1 = mx[1] > st.m[1] + kLazy;
  if (__any(need0 || need1)) {
    float alpha[2];
    alpha[0] = need0 ? fast_exp2(st.m[0] - mx[0]) : 1.0f;
    alpha[1] = need1 ? fast_exp2(st.m[1] - mx[1]) : 1.0f;
    if (need0) st.m[0] = mx[0];
    if (need1) st.m[1] = mx[1];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      st.l[nb] *= alpha[nb];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int j = 0; j < 16; ++j) st.o[nb][mb][j] *= alpha[nb];
    }
  }

  // P^T (bf16) in the B-operand layout of the 16-key steps: step ks holds registers
  // j = 8*ks .. 8*ks+7, i.e. keys 16*ks + 8*(i/4) + 4*(l/32) + i%4.
  bf16x8 pb[2][2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    float lsum = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const __bf16 pv = (__bf16)fast_exp2(x[nb][j] - st.m[nb]);
      pb[nb][j >> 3][j & 7] = pv;
      lsum += (float)pv;
    }
    st.l[nb] += lsum;
  }

  // O^T += V^T P^T; A operand: lane l holds V[key][32*mb + l%32] for the 8 keys of its slots
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 va;
#pragma unroll
      for (int ii = 0; ii < 8; ++ii) {
        const int key = 16 * ks + 8 * (ii >> 2) + hrow + (ii & 3);
        va[ii] = __builtin_bit_cast(__bf16, vl[key * kVRow + 32 * mb + (lane & 31)]);
      }
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) st.o[nb][mb] = mfma(va, pb[nb][ks], st.o[nb][mb]);
    }
  }
}

// Shared memory of the attention kernel: V tiles during the key loop, then the merge.
struct AttnSmem {
  union {
    uint16_t v[kWaves][kTile * kVRow];
    struct {
      float m[kWaves][kHeads];
      float l[kWaves][kHeads];
      float fm[kHeads];
      float fl[kHeads];
      float o[kDim][kHeads + 1];
    } mg;
  };
};

template <bool kGather>
__global__ __launch_bounds__(256) void attn_bf16_kernel(AttnArgs a, uint32_t* hist,
                                                        uint32_t* counters) {
  __shared__ AttnSmem sm;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int i = blockIdx.x / a.n_split;
  const int split = blockIdx.x - i * a.n_split;

  int64_t base;
  int t;
  const bool valid = query_desc(a.b, i, base, t);
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
  kl.sel_row = kGather ? a.sel + (size_t)i * a.top_k : nullptr;
  kl.base = base;
  kl.t = t;
  kl.window = a.window;
  kl.top_k = a.top_k;
  kl.n_keys = logical_keys(kGather, t, a.window, a.top_k);
  kl.w_eff = min(a.window, t + 1);
  kl.cand_hi = t - a.window;
  const int k0 = split * a.split_keys;
  if (k0 >= kl.n_keys) return;  // empty split: the combine does not read it
  const int k1 = min(kl.n_keys, k0 + a.split_keys);
  const int ntiles = (k1 - k0 + kTile - 1) / kTile;

  const __bf16* kp = static_cast<const __bf16*>(a.k);
  const uint16_t* vp = static_cast<const uint16_t*>(a.v);

  bf16x8 qop[2][8];
  {
    const __bf16* qp = static_cast<const __bf16*>(a.q) + (size_t)i * kHeads * kDim;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int s = 0; s < 8; ++s)
        qop[nb][s] = *reinterpret_cast<const bf16x8*>(qp + (32 * nb + (lane & 31)) * kDim +
                                                      (lane >> 5) * 64 + s * 8);
  }

  WaveState st;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    st.m[nb] = kNegBig;
    st.l[nb] = 0.0f;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) st.o[nb][mb] = f32x16{};
  }

  uint16_t* vl = sm.v[wave];
  int tau = wave;
  TileRegs cur, nxt;
  if (tau < ntiles) load_tile(kl, kp, vp, k0 + tau * kTile, k1, lane, nxt);
  for (; tau < ntiles; tau += kWaves) {
    cur = nxt;
    if (tau + kWaves < ntiles) load_tile(kl, kp, vp, k0 + (tau + kWaves) * kTile, k1, lane, nxt);
    process_tile(st, qop, cur, vl, a.c2, lane);
  }

#pragma unroll
  for (int nb = 0; nb < 2; ++nb) st.l[nb] += __shfl_xor(st.l[nb], 32);

  // ---- merge the four waves (fixed order, deterministic) ----
  __syncthreads();  // V tiles no longer needed
  if (lane < 32) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      sm.mg.m[wave][32 * nb + lane] = st.m[nb];
      sm.mg.l[wave][32 * nb + lane] = st.l[nb];
    }
  }
  __syncthreads();
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
    float L = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) L += sm.mg.l[w][h] * fast_exp2(sm.mg.m[w][h] - M);
    sm.mg.fm[h] = M;
    sm.mg.fl[h] = L;
  }
  const int hrow = 4 * (lane >> 5);
  for (int w = 0; w < kWaves; ++w) {
    if (wave == w) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int d = 32 * mb + 8 * (j >> 2) + hrow + (j & 3);
            const int h = 32 * nb + (lane & 31);
            const float val = st.o[nb][mb][j] * alpha[nb];
            sm.mg.o[d][h] = (w == 0) ? val : sm.mg.o[d][h] + val;
          }
    }
    __syncthreads();
  }

  if (a.n_split == 1) {
    __bf16* out = static_cast<__bf16*>(a.out) + (size_t)i * kHeads * kDim;
    for (int e = threadIdx.x; e < kHeads * kDim; e += blockDim.x) {
      const int h = e >> 7, d = e & 127;
      out[e] = (__bf16)(sm.mg.o[d][h] / sm.mg.fl[h]);
    }
    if (threadIdx.x < kHeads) {
      const int h = threadIdx.x;
      const float l2 = sm.mg.fm[h] + __log2f(sm.mg.fl[h]);
      if (a.lse) a.lse[(size_t)i * kHeads + h] = l2 * kLn2;
      if (a.lse2) a.lse2[(size_t)i * kHeads + h] = l2;
    }
  } else {
    Partial* P = a.part + (size_t)i * a.n_split + split;
    if (threadIdx.x < kHeads) {
      P->m[threadIdx.x] = sm.mg.fm[threadIdx.x];
      P->l[threadIdx.x] = sm.mg.fl[threadIdx.x];
    }
    for (int e = threadIdx.x; e < kHeads * kDim; e += blockDim.x) {
      const int d = e >> 6, h = e & 63;
      P->o[e] = sm.mg.o[d][h];
    }
  }
}

// ------------------------------------------------------------------------------------
// Split combine: merges the partials of a query in split order, writes O, LSE and the
// log2-domain LSE used by the score pass, and clears the query's selection counters.
// ------------------------------------------------------------------------------------
template <typename OutT>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  constexpr int kMaxSplit = 256;
  __shared__ float w_s[kMaxSplit][kHeads];
  __shared__ float fl[kHeads];
  __shared__ float ob[kDim][kHeads + 1];
  const int i = blockIdx.x;
  if (a.hist) {
    for (int e = threadIdx.x; e < kHistBins; e += blockDim.x) a.hist[(size_t)i * kHistBins + e] = 0u;
    if (threadIdx.x < 4) a.counters[(size_t)i * 4 + threadIdx.x] = 0u;
  }
  int64_t base;
  int t;
  const bool valid = query_desc(a.b, i, base, t);
  OutT* out = static_cast<OutT*>(a.out) + (size_t)i * kHeads * kDim;
  if (!valid) {
    for (int e = threadIdx.x; e < kHeads * kDim; e += blockDim.x) out[e] = (OutT)NAN;
    if (threadIdx.x < kHeads) {
      if (a.lse) a.lse[(size_t)i * kHeads + threadIdx.x] = NAN;
      if (a.lse2) a.lse2[(size_t)i * kHeads + threadIdx.x] = NAN;
    }
    return;
  }
  const int n_keys = logical_keys(a.gather != 0, t, a.window, a.top_k);
  const int nv = min(a.n_split, (n_keys + a.split_keys - 1) / a.split_keys);
  const Partial* P = a.part + (size_t)i * a.n_split;
  if (threadIdx.x < kHeads) {
    const int h = threadIdx.x;
    float M = P[0].m[h];
    for (int s = 1; s < nv; ++s) M = fmaxf(M, P[s].m[h]);
    float L = 0.0f;
    for (int s = 0; s < nv; ++s) {
      const float w = __builtin_amdgcn_exp2f(P[s].m[h] - M);
      w_s[s][h] = w;
      L += P[s].l[h] * w;
    }
    fl[h] = L;
    const float l2 = M + __log2f(L);
    if (a.lse) a.lse[(size_t)i * kHeads + h] = l2 * kLn2;
    if (a.lse2) a.lse2[(size_t)i * kHeads + h] = l2;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < kHeads * kDim; e += blockDim.x) {
    const int d = e >> 6, h = e & 63;
    float acc = 0.0f;
    for (int s = 0; s < nv; ++s) acc += P[s].o[e] * w_s[s][h];
    ob[d][h] = acc;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < kHeads * kDim; e += blockDim.x) {
    const int h = e >> 7, d = e & 127;
    out[e] = (OutT)(ob[d][h] / fl[h]);
  }
}

// ------------------------------------------------------------------------------------
// Selection score pass: score_j = sum_h exp2(x_hj - lse2_h) for candidates j <= t-window,
// written per query, plus a histogram of the first radix digit (bits 30..19).
// S = Q K^T here (heads as rows): each lane sums its 32 head values of one key, and one
// exchange with lane l^32 completes the 64-head sum.
// ------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void score_bf16_kernel(ScoreArgs a) {
  __shared__ uint32_t hist_s[kHistBins];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int i = blockIdx.x / a.n_split;
  const int split = blockIdx.x - i * a.n_split;
  int64_t base;
  int t;
  if (!query_desc(a.b, i, base, t)) return;
  const int nc = max(0, t - a.window + 1);
  if (nc <= a.top_k) return;
  const int k0 = split * a.split_keys;
  if (k0 >= nc) return;
  const int k1 = min(nc, k0 + a.split_keys);
  const int ntiles = (k1 - k0 + kTile - 1) / kTile;

  for (int e = threadIdx.x; e < kHistBins; e += blockDim.x) hist_s[e] = 0u;

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
  __syncthreads();

  const __bf16* kp = static_cast<const __bf16*>(a.k);
  float* srow = a.scores + (size_t)i * a.score_stride;
  bf16x8 kc[8], kn[8];
  auto load = [&](int tau, bf16x8 (&kr)[8]) {
    const int p = k0 + tau * kTile + (lane & 31);
    const int rel = p < k1 ? p : 0;
    const __bf16* krow = kp + (base + rel) * kDim + (lane >> 5) * 64;
#pragma unroll
    for (int s = 0; s < 8; ++s) kr[s] = *reinterpret_cast<const bf16x8*>(krow + s * 8);
  };
  int tau = wave;
  if (tau < ntiles) load(tau, kn);
  for (; tau < ntiles; tau += kWaves) {
#pragma unroll
    for (int s = 0; s < 8; ++s) kc[s] = kn[s];
    if (tau + kWaves < ntiles) load(tau + kWaves, kn);
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
    const int p = k0 + tau * kTile + (lane & 31);
    if (lane < 32 && p < k1) {
      srow[p] = total;
      atomicAdd(&hist_s[__float_as_uint(total) >> kHistShift], 1u);
    }
  }
  __syncthreads();
  uint32_t* hq = a.hist + (size_t)i * kHistBins;
  for (int e = threadIdx.x; e < kHistBins; e += blockDim.x) {
    const uint32_t c = hist_s[e];
    if (c) atomicAdd(&hq[e], c);
  }
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs& a, bool gather, int grid, uint32_t* hist,
                            uint32_t* counters, hipStream_t s) {
  if (gather)
    hipLaunchKernelGGL(attn_bf16_kernel<true>, dim3(grid), dim3(256), 0, s, a, hist, counters);
  else
    hipLaunchKernelGGL(attn_bf16_kernel<false>, dim3(grid), dim3(256), 0, s, a, hist, counters);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, bool f32, hipStream_t s) {
  if (f32)
    hipLaunchKernelGGL(combine_kernel<float>, dim3(a.b.total_q), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(combine_kernel<__bf16>, dim3(a.b.total_q), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_score_bf16(const ScoreArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(score_bf16_kernel, dim3(a.b.total_q * a.n_split), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace hs2
