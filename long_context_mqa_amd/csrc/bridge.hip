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
// 256-column tile of C^T = W^T H^T (two output matrices) with four waves of 128 x 128
// (accumulators in the AGPRs); operand tiles stream through three LDS stages by
// direct-to-LDS loads. Tiles of the same rows run back to back on one XCD, so H is read
// from HBM once and re-served from that XCD's L2 for the other column tiles.
#include "hs2_internal.h"

namespace hs2 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 256;   // H rows per workgroup
constexpr int kBN = 256;   // output columns per workgroup (two matrices of 128)
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

constexpr int kStagesG = 3;      // LDS stages of the contraction loop
constexpr int kKStep = 32;       // contraction step (two MFMA k-steps of 16)
constexpr int kTileB = 256 * kKStep * 2;  // 16 KB: one 256 x 32 bf16 operand tile

// Operand tiles in LDS: 256 rows of 64 bytes (32 bf16 of the contraction); the 16-byte
// chunk c of row r sits at chunk position c ^ ((r >> 2) & 3), so that the eight lanes an
// LDS read serves together (eight consecutive rows, same chunk) hit distinct banks.
__device__ inline uint32_t op_off(int row, int chunk) {
  return (uint32_t)(row * 64 + ((chunk ^ ((row >> 2) & 3)) << 4));
}

struct GemmSmem {
  uint8_t a[kStagesG][kTileB];  // transposed weights: [n][k]
  uint8_t b[kStagesG][kTileB];  // hidden states:      [row][k]
};

__global__ __launch_bounds__(256) void bridge_gemm_kernel(BridgeArgs a) {
  __shared__ __align__(16) GemmSmem sm;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n_nt = a.n_mats / 2;
  const int64_t n_rt = (a.n_rows + kBM - 1) / kBM;
  // XCD-aware order: workgroup b runs on XCD b % 8; consecutive slots of one XCD take
  // the column tiles of one row tile, so the H rows are re-read from that XCD's L2.
  const int xcd = blockIdx.x % kXcds;
  const int slot = blockIdx.x / kXcds;
  const int64_t rt = (int64_t)(slot / n_nt) * kXcds + xcd;
  const int nt = slot % n_nt;
  if (rt >= n_rt) return;
  const int64_t r0 = rt * kBM;
  const uint16_t* wt = a.wt + (size_t)nt * kBN * a.d_model;
  const int wr = wave & 1;   // 128-row half
  const int wn = wave >> 1;  // 128-column half (one output matrix)

  const uint32_t la0 = (uint32_t)(size_t)sm.a[0];
  const uint32_t lb0 = (uint32_t)(size_t)sm.b[0];
  // this wave's copy rows: copies r = 4*wave .. 4*wave+3 cover rows 16r .. 16r+15
  const uint16_t* ga[4];
  const uint16_t* gb[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = 4 * wave + q;
    const int row = 16 * r + (lane >> 2);
    const int chunk = (lane & 3) ^ ((row >> 2) & 3);
    ga[q] = wt + (size_t)row * a.d_model + chunk * 8;
    int64_t hr = r0 + row;
    if (hr >= a.n_rows) hr = a.n_rows - 1;
    gb[q] = a.h + hr * a.d_model + chunk * 8;
  }
  auto issue = [&](int kt, int st) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = 4 * wave + q;
      dma16(ga[q] + kt * kKStep, __builtin_amdgcn_readfirstlane(la0 + st * kTileB + r * 1024));
      dma16(gb[q] + kt * kKStep, __builtin_amdgcn_readfirstlane(lb0 + st * kTileB + r * 1024));
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = f32x16{};

  const int KT = a.d_model / kKStep;
  issue(0, 0);
  if (KT > 1) issue(1, 1);
  for (int kt = 0; kt < KT; ++kt) {
    const int st = kt % kStagesG;
    // this wave's 8 copies of stage kt have landed once only those of stage kt+1 remain
    if (kt + 1 < KT)
      asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // the whole stage has landed; stage kt-1 is no longer read
    if (kt + 2 < KT) issue(kt + 2, (kt + 2) % kStagesG);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int c = 2 * ks + (lane >> 5);
      bf16x8 av[4], bv[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        av[x] = *reinterpret_cast<const bf16x8*>(sm.a[st] + op_off(wn * 128 + 32 * x + (lane & 31), c));
        bv[x] = *reinterpret_cast<const bf16x8*>(sm.b[st] + op_off(wr * 128 + 32 * x + (lane & 31), c));
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
