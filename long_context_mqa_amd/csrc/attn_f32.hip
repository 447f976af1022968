// float32 storage path of the attention kernels (plain fp32 vector arithmetic).
//
// Same operations, split structure, partial format and log2-domain conventions as the
// bf16 MFMA kernels, so the split combine and the top-k kernels are shared:
//   attn_f32_kernel   exact causal attention (pass 1) or gathered sparse attention
//   score_f32_kernel  head-summed softmax probability of every candidate key (pass 2)
// Method (page title and section): arex-research.com, "Xiaomi MiMo lead Luo Fuli
// publishes the MiMo-V3 core architecture HySparse2", section "Outer KV Bridging, inner
// KV Reuse".
//
// Thread layout: 256 threads = 64 heads x 4 slices of 32 dims. A logit is the sum of the
// four slice dot products (two xor-shuffles within the four lanes of a head).
#include "kernel_common.h"
#include "hs2_launch.h"

namespace hs2 {
namespace {

constexpr int kT = 32;            // keys per LDS tile
constexpr int kRow = kDim + 4;    // padded LDS row (floats)
constexpr float kNegBig = -1.0e30f;

__device__ inline float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <bool kGather>
__global__ __launch_bounds__(256) void attn_f32_kernel(AttnArgs a, uint32_t* hist,
                                                       uint32_t* counters) {
  __shared__ float ks[kT][kRow];
  __shared__ float vs[kT][kRow];
  __shared__ int rows[kT];
  __shared__ int oks[kT];
  const int tid = threadIdx.x;
  const int h = tid >> 2, sl = tid & 3;
  const int i = blockIdx.x / a.n_split;
  const int split = blockIdx.x - i * a.n_split;
  int64_t base;
  int t;
  const bool valid = query_desc(a.b, i, base, t);
  if (a.n_split == 1 && hist != nullptr) {
    for (int e = tid; e < kHistBins; e += blockDim.x) hist[(size_t)i * kHistBins + e] = 0u;
    if (tid < 4) counters[(size_t)i * 4 + tid] = 0u;
  }
  float* outp = static_cast<float*>(a.out) + (size_t)i * kHeads * kDim;
  if (!valid) {
    if (a.n_split == 1) {
      for (int e = tid; e < kHeads * kDim; e += blockDim.x) outp[e] = NAN;
      if (tid < kHeads) {
        if (a.lse) a.lse[(size_t)i * kHeads + tid] = NAN;
        if (a.lse2) a.lse2[(size_t)i * kHeads + tid] = NAN;
      }
    }
    return;
  }
  const int n_keys = logical_keys(kGather, t, a.window, a.top_k);
  const int k0 = split * a.split_keys;
  if (k0 >= n_keys) return;
  const int k1 = min(n_keys, k0 + a.split_keys);
  const int w_eff = min(a.window, t + 1);
  const int cand_hi = t - a.window;
  const int32_t* selr = kGather ? a.sel + (size_t)i * a.top_k : nullptr;

  const float* q = static_cast<const float*>(a.q) + ((size_t)i * kHeads + h) * kDim + 32 * sl;
  float qv[32];
#pragma unroll
  for (int r = 0; r < 32; ++r) qv[r] = q[r];
  float o[32];
#pragma unroll
  for (int r = 0; r < 32; ++r) o[r] = 0.0f;
  float m = kNegBig, l = 0.0f;
  const float* kp = static_cast<const float*>(a.k);
  const float* vp = static_cast<const float*>(a.v);

  for (int p0 = k0; p0 < k1; p0 += kT) {
    if (tid < kT) {
      const int p = p0 + tid;
      int rel = 0;
      bool ok = p < k1;
      if (ok) {
        if (!kGather) {
          rel = p;
        } else if (p < a.top_k) {
          const int s = selr[p];
          ok = s >= 0 && s <= cand_hi;
          rel = ok ? s : 0;
        } else {
          const int w = p - a.top_k;
          ok = w < w_eff;
          rel = ok ? t - w_eff + 1 + w : 0;
        }
      }
      rows[tid] = rel;
      oks[tid] = ok;
    }
    __syncthreads();
    for (int e = tid; e < kT * kDim; e += blockDim.x) {
      const int key = e >> 7, d = e & 127;
      const size_t r = (size_t)(base + rows[key]) * kDim + d;
      ks[key][d] = kp[r];
      vs[key][d] = vp[r];
    }
    __syncthreads();
    for (int key = 0; key < kT; ++key) {
      if (!oks[key]) continue;
      float part = 0.0f;
#pragma unroll
      for (int r = 0; r < 32; ++r) part = fmaf(qv[r], ks[key][32 * sl + r], part);
      part += __shfl_xor(part, 1);
      part += __shfl_xor(part, 2);
      const float x = part * a.c2;
      const float mn = fmaxf(m, x);
      const float alpha = fexp2(m - mn);
      const float p = fexp2(x - mn);
      l = l * alpha + p;
#pragma unroll
      for (int r = 0; r < 32; ++r) o[r] = fmaf(o[r], alpha, p * vs[key][32 * sl + r]);
      m = mn;
    }
    __syncthreads();
  }

  if (a.n_split == 1) {
#pragma unroll
    for (int r = 0; r < 32; ++r) outp[h * kDim + 32 * sl + r] = o[r] / l;
    if (sl == 0) {
      const float l2 = m + __log2f(l);
      if (a.lse) a.lse[(size_t)i * kHeads + h] = l2 * kLn2;
      if (a.lse2) a.lse2[(size_t)i * kHeads + h] = l2;
    }
  } else {
    Partial* P = a.part + (size_t)i * a.n_split + split;
    if (sl == 0) {
      P->m[h] = m;
      P->l[h] = l;
      P->le[h] = l;
    }
#pragma unroll
    for (int r = 0; r < 32; ++r) P->o[(32 * sl + r) * kHeads + h] = o[r];
  }
}

__global__ __launch_bounds__(256) void score_f32_kernel(ScoreArgs a) {
  __shared__ float ks[kT][kRow];
  __shared__ float pb[kT][kHeads + 1];
  __shared__ uint32_t hist_s[kHistBins];
  const int tid = threadIdx.x;
  const int h = tid >> 2, sl = tid & 3;
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
  for (int e = tid; e < kHistBins; e += blockDim.x) hist_s[e] = 0u;

  const float* q = static_cast<const float*>(a.q) + ((size_t)i * kHeads + h) * kDim + 32 * sl;
  float qv[32];
#pragma unroll
  for (int r = 0; r < 32; ++r) qv[r] = q[r];
  const float l2 = a.lse2[(size_t)i * kHeads + h];
  const float* kp = static_cast<const float*>(a.k);
  float* srow = a.scores + (size_t)i * a.score_stride;

  for (int p0 = k0; p0 < k1; p0 += kT) {
    __syncthreads();
    for (int e = tid; e < kT * kDim; e += blockDim.x) {
      const int key = e >> 7, d = e & 127;
      const int p = min(p0 + key, k1 - 1);
      ks[key][d] = kp[(size_t)(base + p) * kDim + d];
    }
    __syncthreads();
    for (int key = 0; key < kT; ++key) {
      float part = 0.0f;
#pragma unroll
      for (int r = 0; r < 32; ++r) part = fmaf(qv[r], ks[key][32 * sl + r], part);
      part += __shfl_xor(part, 1);
      part += __shfl_xor(part, 2);
      if (sl == 0) pb[key][h] = fexp2(part * a.c2 - l2);
    }
    __syncthreads();
    if (tid < kT && p0 + tid < k1) {
      float s = 0.0f;
      for (int hh = 0; hh < kHeads; ++hh) s += pb[tid][hh];
      srow[p0 + tid] = s;
      atomicAdd(&hist_s[__float_as_uint(s) >> kHistShift], 1u);
    }
  }
  __syncthreads();
  uint32_t* hq = a.hist + (size_t)i * kHistBins;
  for (int e = tid; e < kHistBins; e += blockDim.x) {
    const uint32_t c = hist_s[e];
    if (c) atomicAdd(&hq[e], c);
  }
}

}  // namespace

hipError_t launch_attn_f32(const AttnArgs& a, bool gather, int grid, uint32_t* hist,
                           uint32_t* counters, hipStream_t s) {
  if (gather)
    hipLaunchKernelGGL(attn_f32_kernel<true>, dim3(grid), dim3(256), 0, s, a, hist, counters);
  else
    hipLaunchKernelGGL(attn_f32_kernel<false>, dim3(grid), dim3(256), 0, s, a, hist, counters);
  return hipGetLastError();
}

hipError_t launch_score_f32(const ScoreArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(score_f32_kernel, dim3(a.b.total_q * a.n_split), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace hs2
