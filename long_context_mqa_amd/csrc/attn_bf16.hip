// bf16 MQA attention for gfx950: the selector's exact causal attention (pass 1, the
// decode-shaped kernel of attn_decode.h with four waves per workgroup) and the split
// combine (also used by the sparse layers of sparse_attn.hip). The selection-score pass is
// in score_bf16.hip, the FP8 K/V instantiation in attn_fp8.hip.
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
#include "attn_decode.h"
#include "hs2_launch.h"

namespace hs2 {
namespace {

using namespace attn;

// ------------------------------------------------------------------------------------
// Split combine: merges the partials of a query in split order, writes O, LSE and the
// log2-domain LSE used by the score pass, and clears the query's selection counters.
// Grid: total_q x kCombineSlabs; a slab covers 16 dims x 64 heads of the output. Thread
// (h, g) merges head h's partials for 4 dims on its own (online, with a running
// reference, in split order), so that the loads of several splits are in flight at once
// and no barrier separates them; every thread of a head computes the same denominators.
// ------------------------------------------------------------------------------------
constexpr int kCombineSlabs = kDim / 16;

struct MergeAcc {
  float m = -INFINITY, l = 0.0f, le = 0.0f;
  float o[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  __device__ inline void add(float ms, float ls, float les, const float (&os)[4]) {
    const float mn = fmaxf(m, ms);
    const float fa = __builtin_amdgcn_exp2f(m - mn), fb = __builtin_amdgcn_exp2f(ms - mn);
    l = l * fa + ls * fb;
    le = le * fa + les * fb;
#pragma unroll
    for (int r = 0; r < 4; ++r) o[r] = o[r] * fa + os[r] * fb;
    m = mn;
  }
};

template <typename OutT>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int i = blockIdx.x / kCombineSlabs;
  const int slab = blockIdx.x - i * kCombineSlabs;
  const int tid = threadIdx.x;
  const int h = tid & 63, grp = tid >> 6;
  if (a.hist) {
    constexpr int per = kHistBins / kCombineSlabs;
    for (int e = tid; e < per; e += blockDim.x) a.hist[(size_t)i * kHistBins + slab * per + e] = 0u;
    if (slab == 0 && tid < 4) a.counters[(size_t)i * 4 + tid] = 0u;
  }
  // The partials are loaded kMergeBatch at a time, every load of a batch in flight at once,
  // and merged in split order; the first batch goes out with the query's descriptor loads
  // (partials past the query's valid splits are in the workspace and simply not used).
  constexpr int kMergeBatch = 16;
  const Partial* P = a.part + (size_t)i * a.n_split;
  const int d0 = slab * 16 + grp * 4;
  float m[kMergeBatch], l[kMergeBatch], le[kMergeBatch], v[kMergeBatch][4];
  auto load_batch = [&](int s0, int n) {
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      if (u < n) {
        m[u] = P[s0 + u].m[h];
        l[u] = P[s0 + u].l[h];
        le[u] = P[s0 + u].le[h];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[u][r] = P[s0 + u].o[(d0 + r) * kHeads + h];
      }
    }
  };
  load_batch(0, min(kMergeBatch, a.n_split));
  int64_t base;
  int t;
  const bool valid = query_desc(a.b, i, base, t) && !(a.plan_miss != nullptr && a.plan_miss[i] != 0);
  OutT* out = static_cast<OutT*>(a.out) + (size_t)i * kHeads * kDim;
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
  MergeAcc acc;
  for (int s0 = 0; s0 < nv; s0 += kMergeBatch) {
    const int n = min(kMergeBatch, nv - s0);
    if (s0 > 0) load_batch(s0, n);
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u)
      if (u < n) acc.add(m[u], l[u], le[u], v[u]);
  }
  if (slab == 0 && grp == 0) {
    const float l2 = acc.m + __log2f(acc.le);
    if (a.lse) a.lse[(size_t)i * kHeads + h] = l2 * kLn2;
    if (a.lse2) a.lse2[(size_t)i * kHeads + h] = l2;
  }
  const float inv = a.v_scale / acc.l;
#pragma unroll
  for (int r = 0; r < 4; ++r) out[h * kDim + d0 + r] = (OutT)(acc.o[r] * inv);
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs& a, const WorkList& wl, int grid, uint32_t* hist, uint32_t* counters,
                            hipStream_t s) {
  hipLaunchKernelGGL((attn_bf16_kernel<KvBf16, 4>), dim3(grid), dim3(256), 0, s, a, wl, hist, counters);
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

