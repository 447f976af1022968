// Decode-time KV Bridging for gfx950: each new token's hidden state through every
// bridged layer's K and V projections, written into that layer's caches at the token's
// row, ahead of the selector of the same decode step.
//
// Method (page title and section): arex-research.com, "Xiaomi MiMo lead Luo Fuli
// publishes the MiMo-V3 core architecture HySparse2", section "Outer KV Bridging, inner
// KV Reuse": each cross-decoder full-attention layer builds its own KV cache from the
// input hidden states of the matching self-decoder full-attention layer through its own
// K/V projection; in decode every new token adds one row to each of those caches.
//
// A decode batch brings a few dozen rows against 2L weight matrices of 2,048 x 128, so
// the weights are the bytes to move and the work is split over the contraction: a
// partial workgroup takes one matrix, 128 of the contraction and 32 new rows, and a
// finishing pass sums the partials in a fixed order and writes bf16 rows into the caches.
// A weight matrix [d_model][128] is laid out like a V cache, so its 32-row tiles go
// through the V-tile copy and the transposing operand reads of the attention kernels:
// out^T = W^T H^T with W^T as the A operand and H^T as the B operand in the same
// permuted contraction order as the P^T operand of O^T += V^T P^T.
#include "attn_common.h"
#include "hs2_launch.h"

namespace hs2 {
namespace {

using namespace attn;

constexpr int kSliceTiles = kAppendSlice / kTile;  // 32-row weight tiles per partial workgroup

// Grid (slice, matrix, 32-row block); wave w computes output columns 32w .. 32w+31.
__global__ __launch_bounds__(256) void append_partial_kernel(AppendArgs a) {
  __shared__ __align__(16) uint8_t wt[kSliceTiles][kTileBytes];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int s = blockIdx.x, m = blockIdx.y, rb = blockIdx.z;
  const int k0 = s * kAppendSlice;
  // wave w copies weight rows k0 + 32w .. k0 + 32w + 31 (tile w) into LDS, V layout
  issue_rows<false>(reinterpret_cast<const __bf16*>(a.w[m]), (int64_t)(k0 + kTile * wave), lane & 31, lane,
                    __builtin_amdgcn_readfirstlane((uint32_t)(size_t)wt[wave]));
  // B operand (H^T): lane l holds new row 32rb + l%32 at contraction positions
  // 16ks + 8(e/4) + 4(l/32) + e%4 of tile t (two 8-byte pieces per 16-step)
  const int r = kTile * rb + (lane & 31);
  const __bf16* hr = reinterpret_cast<const __bf16*>(a.h) + (size_t)min(r, a.n_new - 1) * a.d_model + k0 +
                     4 * (lane >> 5);
  bf16x8 hb[kSliceTiles][2];
#pragma unroll
  for (int t = 0; t < kSliceTiles; ++t)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint2 lo = *reinterpret_cast<const uint2*>(hr + kTile * t + 16 * ks);
      const uint2 hi = *reinterpret_cast<const uint2*>(hr + kTile * t + 16 * ks + 8);
      hb[t][ks] = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
    }
  wait_vmcnt<0>();
  __syncthreads();  // every wave's tile has landed

  uint32_t vb[4];
  vt_bases(lane, vb);
  f32x16 acc = f32x16{};
#pragma unroll
  for (int t = 0; t < kSliceTiles; ++t)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) acc = mfma(read_vt(wt[t], vb[wave], ks), hb[t][ks], acc);

  // C layout: lane l holds new row 32rb + l%32, output columns 32w + 8(j/4) + 4(l/32) + j%4
  if (r < a.n_new) {
    const int cols = a.n_mats * kDim;
    float* dst = a.part + ((size_t)s * a.n_new + r) * cols + m * kDim + kTile * wave + 4 * (lane >> 5);
#pragma unroll
    for (int jg = 0; jg < 4; ++jg)
      *reinterpret_cast<float4*>(dst + 8 * jg) =
          make_float4(acc[4 * jg], acc[4 * jg + 1], acc[4 * jg + 2], acc[4 * jg + 3]);
  }
}

// Thread (new row, 8 consecutive output columns): the partials summed in slice order,
// rounded to bf16 (or, FP8 caches: scaled by the matrix's reciprocal scale, clamped to
// +-448 and converted to E4M3 codes, round to nearest even) and written to the cache row
// of that token; rows outside [0, cache_rows) are skipped.
template <bool kFp8>
__global__ __launch_bounds__(256) void append_finish_kernel(AppendArgs a, BridgeOut o) {
  const int cols = a.n_mats * kDim;
  const int per_row = cols / 8;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= a.n_new * per_row) return;
  const int r = idx / per_row, c = (idx - r * per_row) * 8;
  float acc[8] = {};
  for (int s = 0; s < a.n_slices; ++s) {
    const float4* p = reinterpret_cast<const float4*>(a.part + ((size_t)s * a.n_new + r) * cols + c);
    const float4 x = p[0], y = p[1];
    acc[0] += x.x; acc[1] += x.y; acc[2] += x.z; acc[3] += x.w;
    acc[4] += y.x; acc[5] += y.y; acc[6] += y.z; acc[7] += y.w;
  }
  const int64_t row = a.rows[r];
  if (row < 0 || row >= a.cache_rows) return;
  if constexpr (kFp8) {
    const float is = o.inv_scale[c / kDim];
    float v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = fminf(fmaxf(acc[q] * is, -448.0f), 448.0f);
    int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], w0, true);
    int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(v[4], v[5], 0, false);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(v[6], v[7], w1, true);
    *reinterpret_cast<int2*>(reinterpret_cast<uint8_t*>(a.outs[c / kDim]) + row * kDim + (c % kDim)) =
        make_int2(w0, w1);
  } else {
    bf16x8 v;
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = (__bf16)acc[q];
    *reinterpret_cast<bf16x8*>(a.outs[c / kDim] + row * kDim + (c % kDim)) = v;
  }
}

}  // namespace

hipError_t launch_bridge_append(const AppendArgs& a, const BridgeOut& o, hipStream_t s) {
  const dim3 grid(a.n_slices, a.n_mats, (a.n_new + kTile - 1) / kTile);
  hipLaunchKernelGGL(append_partial_kernel, grid, dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int threads = a.n_new * (a.n_mats * kDim / 8);
  if (o.fp8)
    hipLaunchKernelGGL(append_finish_kernel<true>, dim3((threads + 255) / 256), dim3(256), 0, s, a, o);
  else
    hipLaunchKernelGGL(append_finish_kernel<false>, dim3((threads + 255) / 256), dim3(256), 0, s, a, o);
  return hipGetLastError();
}

}  // namespace hs2
