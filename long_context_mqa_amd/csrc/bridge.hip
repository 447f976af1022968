// KV Bridging fan-out GEMM for gfx950: K_l = H W_K^l, V_l = H W_V^l for all bridged
// layers l, from one pass over the hidden states H.
//
// Method (page title and section): arex-research.com, "Xiaomi MiMo lead Luo Fuli
// publishes the MiMo-V3 core architecture HySparse2", section "Outer KV Bridging, inner
// KV Reuse": each cross-decoder full-attention layer builds its own KV cache from the
// input hidden states of the matching self-decoder full-attention layer, through its
// own K/V projection, and one source may feed several layers. Section "Numbers computed
// on three 80B-A3B models": hidden size 2,048.
//
// The 2L projection matrices are treated as one [d_model x 128*2L] right-hand side. The
// weights are first transposed into the workspace (k contiguous), so that both MFMA
// operands read 16 contiguous bytes per lane. Each workgroup computes a 256-row x
// 256-column tile of C^T = W^T H^T (two output matrices) with four waves of 128 x 128;
// tiles of the same rows run back to back on one XCD, so H is read from HBM once and
// re-served from that XCD's L2 for the other column tiles.
#include "hs2_internal.h"

namespace hs2 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 256;   // H rows per workgroup
constexpr int kBN = 256;   // output columns per workgroup (two matrices of 128)
constexpr int kBK = 64;    // contraction step
constexpr int kXcds = 8;

struct WPtrs {
  const uint16_t* w[16];
};

// wt[m][n][k] = w_m[k][n]  (64 x 64 tiles through LDS)
__global__ __launch_bounds__(256) void transpose_w_kernel(WPtrs wp, uint16_t* wt, int d_model) {
  __shared__ uint16_t tile[64][66];
  const int m = blockIdx.z;
  const int k0 = blockIdx.x * 64, n0 = blockIdx.y * 64;
  const uint16_t* w = wp.w[m];
  for (int e = threadIdx.x; e < 64 * 64; e += 256) {
    const int kk = e >> 6, nn = e & 63;
    tile[kk][nn] = w[(size_t)(k0 + kk) * kDim + n0 + nn];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 64 * 64; e += 256) {
    const int nn = e >> 6, kk = e & 63;
    wt[((size_t)m * kDim + n0 + nn) * d_model + k0 + kk] = tile[kk][nn];
  }
}

__device__ inline int swz(int row, int chunk) { return row * kBK + ((chunk ^ (row & 7)) << 3); }

__global__ __launch_bounds__(256) void bridge_gemm_kernel(BridgeArgs a) {
  __shared__ __align__(16) uint16_t As[kBN * kBK];  // Wt tile [n][k]
  __shared__ __align__(16) uint16_t Bs[kBM * kBK];  // H tile  [row][k]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n_nt = a.n_mats / 2;
  const int64_t n_rt = (a.n_rows + kBM - 1) / kBM;
  // XCD-aware order: workgroup b runs on XCD b % 8; consecutive slots of one XCD take
  // the column tiles of one row tile.
  const int xcd = blockIdx.x % kXcds;
  const int slot = blockIdx.x / kXcds;
  const int64_t rt = (int64_t)(slot / n_nt) * kXcds + xcd;
  const int nt = slot % n_nt;
  if (rt >= n_rt) return;
  const int64_t r0 = rt * kBM;

  const uint16_t* wt = a.wt + (size_t)nt * kBN * a.d_model;
  const int wr = wave & 1;   // 128-row half
  const int wn = wave >> 1;  // 128-column half (one output matrix)

  f32x16 acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = f32x16{};

  uint4 ra[8], rb[8];
  auto gload = [&](int k0) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int e = threadIdx.x + 256 * r;
      const int row = e >> 3, c = e & 7;
      ra[r] = *reinterpret_cast<const uint4*>(wt + (size_t)row * a.d_model + k0 + 8 * c);
      int64_t hr = r0 + row;
      if (hr >= a.n_rows) hr = a.n_rows - 1;
      rb[r] = *reinterpret_cast<const uint4*>(a.h + hr * a.d_model + k0 + 8 * c);
    }
  };
  const int KT = a.d_model / kBK;
  gload(0);
  for (int kt = 0; kt < KT; ++kt) {
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int e = threadIdx.x + 256 * r;
      const int row = e >> 3, c = e & 7;
      *reinterpret_cast<uint4*>(&As[swz(row, c)]) = ra[r];
      *reinterpret_cast<uint4*>(&Bs[swz(row, c)]) = rb[r];
    }
    __syncthreads();
    if (kt + 1 < KT) gload((kt + 1) * kBK);
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int c = 2 * ks + (lane >> 5);
      bf16x8 av[4], bv[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int nrow = wn * 128 + 32 * x + (lane & 31);
        av[x] = *reinterpret_cast<const bf16x8*>(&As[swz(nrow, c)]);
        const int hrow = wr * 128 + 32 * x + (lane & 31);
        bv[x] = *reinterpret_cast<const bf16x8*>(&Bs[swz(hrow, c)]);
      }
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y)
          acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[x], bv[y], acc[x][y], 0, 0, 0);
    }
  }

  // C^T[n][row]: lane holds rows 32*y + l%32, columns 32*x + 8*(j/4) + 4*(l/32) + j%4
  uint16_t* out = a.outs[2 * nt + wn];
#pragma unroll
  for (int y = 0; y < 4; ++y) {
    const int64_t grow = r0 + wr * 128 + 32 * y + (lane & 31);
    if (grow >= a.n_rows) continue;
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const int n0 = 32 * x + 8 * jg + 4 * (lane >> 5);
        __bf16 v4[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v4[q] = (__bf16)acc[x][y][4 * jg + q];
        *reinterpret_cast<uint2*>(out + grow * kDim + n0) = __builtin_bit_cast(uint2, v4);
      }
  }
}

}  // namespace

hipError_t launch_bridge_transpose(const BridgeArgs& a, const uint16_t* const* w, int32_t n_mats, uint16_t* wt,
                                   hipStream_t s) {
  WPtrs wp{};
  for (int m = 0; m < n_mats; ++m) wp.w[m] = w[m];
  hipLaunchKernelGGL(transpose_w_kernel, dim3(a.d_model / 64, kDim / 64, n_mats), dim3(256), 0, s, wp,
                     wt, a.d_model);
  return hipGetLastError();
}

hipError_t launch_bridge_gemm(const BridgeArgs& a, hipStream_t s) {
  const int64_t n_rt = (a.n_rows + kBM - 1) / kBM;
  const int64_t per_xcd = (n_rt + kXcds - 1) / kXcds;
  const int64_t grid = per_xcd * kXcds * (a.n_mats / 2);
  hipLaunchKernelGGL(bridge_gemm_kernel, dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace hs2
