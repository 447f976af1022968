// bf16 MQA attention for gfx950: the selector's exact causal attention (pass 1) and the
// sparse layers' gathered attention (the decode-shaped kernel of attn_decode.h with four
// waves per workgroup), and the split combine. The selection-score pass is in
// score_bf16.hip, the FP8 K/V instantiation in attn_fp8.hip.
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

namespace hs2 {
namespace {

using namespace attn;

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
    hipLaunchKernelGGL((attn_bf16_kernel<KvBf16, true, 4>), dim3(grid), dim3(256), 0, s, a, wl, hist, counters);
  else
    hipLaunchKernelGGL((attn_bf16_kernel<KvBf16, false, 4>), dim3(grid), dim3(256), 0, s, a, wl, hist, counters);
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

