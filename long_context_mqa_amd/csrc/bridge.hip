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
// operands read 16 contiguous bytes per lane. Each workgroup computes a tile of 256 rows
// x 384 columns (three output matrices; 256 when 2L is not a multiple of 3) of
// C^T = W^T H^T with eight waves, two per SIMD, of 128 rows x 96 columns (64 x 128 for the
// 256-column tile). The wider tile re-reads each H row 2L/3 times instead of L times; the
// 128 x 96 wave tile reads 7 operand fragments from LDS per 12 MFMAs (8 for 64 x 192, which
// measured 1.5-2% slower), and its 192 fp32 accumulators per lane still allow two
// waves per SIMD (251 registers in all). Operand tiles stream through two LDS stages 64 deep in the contraction
// (80 KB each) by direct-to-LDS loads: one barrier per 64 of depth (half as many as with
// 32-deep stages, which measured 15% slower on random data even with a third stage).
// Tiles of the same rows run back to back on one XCD, so H is read from HBM once and
// re-served from that XCD's L2 for the other column tiles.
//
// The results leave through LDS: a store straight from the MFMA layout writes 32 rows x 16
// bytes per instruction, and those stores cost about 10% of the kernel; written as bf16 rows
// into the (then idle) stage area and read back, each store instruction covers four whole
// 256-byte rows (5% faster overall). For an FP8 KV cache ([arex] "Numbers computed on three
// 80B-A3B models" accounts the cache in FP8) the same epilogue writes OCP E4M3 codes instead:
// each value times its output matrix's reciprocal scale, clamped to +-448, converted with
// round to nearest even; a store then covers eight 128-byte rows (no slower than bf16). Measured and not kept: four waves (one per SIMD) on
// 256 x 256 tiles with AGPR accumulators and double-buffered operand registers (2% slower);
// a persistent grid carrying the copy stream across tiles (8% slower); touching the lines of
// stage k+3 ahead of their copies (4% slower: the copies were not waiting on HBM).
#include "kernel_common.h"
#include "hs2_launch.h"

namespace hs2 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 256;   // H rows per workgroup
constexpr int kXcds = 8;
constexpr int kGWaves = 8;

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

constexpr int kStagesG = 2;      // LDS stages of the contraction loop
constexpr int kKStep = 64;       // contraction depth per stage (four MFMA k-steps of 16)
constexpr int kRowB = kKStep * 2;           // bytes of one operand row in a stage
constexpr int kRowsPerCopy = 1024 / kRowB;  // rows filled by one wave-wide 16-byte copy
constexpr int kLanesPerRow = 64 / kRowsPerCopy;

// Operand tiles in LDS: rows of 128 bytes (64 bf16 of the contraction); the 16-byte chunk
// c of row r sits at chunk position c ^ ((r >> 1) & 7), so that the 16 lanes an LDS read
// serves together (16 consecutive rows, same chunk) hit 16 distinct bank groups.
__device__ inline int op_swz(int row) { return (row >> 1) & 7; }
__device__ inline uint32_t op_off(int row, int chunk) {
  return (uint32_t)(row * kRowB + ((chunk ^ op_swz(row)) << 4));
}

template <int N>
__device__ inline void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// kCols output columns per workgroup (256 or 384). Wave w: rows kWR*(w%kRW) .. of the
// tile, columns kWC*(w/kRW) .., as kXB x kYB blocks of 32 x 32.
template <int kCols, bool kFp8Out>
__global__ __launch_bounds__(64 * kGWaves) void bridge_gemm_kernel(BridgeArgs a, BridgeOut o) {
  constexpr int kTA = kCols * kKStep * 2;        // W^T tile bytes per stage
  constexpr int kTB = kBM * kKStep * 2;          // H tile bytes per stage
  constexpr int kCopA = kCols / kRowsPerCopy / kGWaves;  // 1 KB copies per wave per stage
  constexpr int kCopB = kBM / kRowsPerCopy / kGWaves;
  static_assert(kCopA * kRowsPerCopy * kGWaves == kCols && kCopB * kRowsPerCopy * kGWaves == kBM,
                "copies must split evenly");
  __shared__ __align__(16) uint8_t lds_all[kStagesG * (kTA + kTB)];
  uint8_t(*lds_a)[kTA] = reinterpret_cast<uint8_t(*)[kTA]>(lds_all);
  uint8_t(*lds_b)[kTB] = reinterpret_cast<uint8_t(*)[kTB]>(lds_all + kStagesG * kTA);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_nt = a.n_mats * kDim / kCols;
  const int64_t n_rt = (a.n_rows + kBM - 1) / kBM;
  // XCD-aware order: workgroup b runs on XCD b % 8; consecutive slots of one XCD take
  // the column tiles of one row tile, so the H rows are re-read from that XCD's L2.
  const int xcd = blockIdx.x % kXcds;
  const int slot = blockIdx.x / kXcds;
  const int64_t rt = (int64_t)(slot / n_nt) * kXcds + xcd;
  const int nt = slot % n_nt;
  if (rt >= n_rt) return;
  const int64_t r0 = rt * kBM;
  const uint16_t* wt = a.wt + (size_t)nt * kCols * a.d_model;
  // kCols == 384: 2 x 4 waves of 128 rows x 96 columns; kCols == 256: 4 x 2 of 64 x 128
  constexpr int kRW = kCols == 384 ? 2 : 4;          // wave rows
  constexpr int kWR = kBM / kRW;                     // rows per wave
  constexpr int kWC = kCols / (kGWaves / kRW);       // columns per wave
  const int wr = wave % kRW;
  const int wc = wave / kRW;
  const uint32_t la0 = (uint32_t)(size_t)lds_a[0];
  const uint32_t lb0 = (uint32_t)(size_t)lds_b[0];
  // this wave's copies: A copies kCopA*wave + q, B copies kCopB*wave + q, kRowsPerCopy
  // rows each; lane l fills chunk position l % kLanesPerRow of its row
  const uint16_t* ga[kCopA];
  const uint16_t* gb[kCopB];
#pragma unroll
  for (int q = 0; q < kCopA; ++q) {
    const int row = kRowsPerCopy * (kCopA * wave + q) + lane / kLanesPerRow;
    ga[q] = wt + (size_t)row * a.d_model + ((lane % kLanesPerRow) ^ op_swz(row)) * 8;
  }
#pragma unroll
  for (int q = 0; q < kCopB; ++q) {
    const int row = kRowsPerCopy * (kCopB * wave + q) + lane / kLanesPerRow;
    int64_t hr = r0 + row;
    if (hr >= a.n_rows) hr = a.n_rows - 1;
    gb[q] = a.h + hr * a.d_model + ((lane % kLanesPerRow) ^ op_swz(row)) * 8;
  }
  auto issue = [&](int kt, int st) {
#pragma unroll
    for (int q = 0; q < kCopA; ++q)
      dma16(ga[q] + kt * kKStep, la0 + st * kTA + (kCopA * wave + q) * 1024);
#pragma unroll
    for (int q = 0; q < kCopB; ++q)
      dma16(gb[q] + kt * kKStep, lb0 + st * kTB + (kCopB * wave + q) * 1024);
  };

  constexpr int kXB = kWC / 32, kYB = kWR / 32;
  f32x16 acc[kXB][kYB];
#pragma unroll
  for (int x = 0; x < kXB; ++x)
#pragma unroll
    for (int y = 0; y < kYB; ++y) acc[x][y] = f32x16{};

  const int KT = a.d_model / kKStep;  // >= 1 (d_model is a multiple of 64)
  static_assert(kStagesG == 2, "the loop below keeps one stage in flight");
  issue(0, 0);
  for (int kt = 0; kt < KT; ++kt) {
    const int st = kt % kStagesG;
    wait_vm<0>();  // this wave's copies of stage kt have landed (the only ones in flight)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();  // the whole stage has landed; stage kt-1 is no longer read
    if (kt + 1 < KT) issue(kt + 1, (kt + 1) % kStagesG);
#pragma unroll
    for (int ks = 0; ks < kKStep / 16; ++ks) {
      const int c = 2 * ks + (lane >> 5);
      bf16x8 av[kXB], bv[kYB];
#pragma unroll
      for (int x = 0; x < kXB; ++x)
        av[x] = *reinterpret_cast<const bf16x8*>(lds_a[st] + op_off(wc * kWC + 32 * x + (lane & 31), c));
#pragma unroll
      for (int y = 0; y < kYB; ++y)
        bv[y] = *reinterpret_cast<const bf16x8*>(lds_b[st] + op_off(wr * kWR + 32 * y + (lane & 31), c));
#pragma unroll
      for (int x = 0; x < kXB; ++x)
#pragma unroll
        for (int y = 0; y < kYB; ++y)
          acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[x], bv[y], acc[x][y], 0, 0, 0);
    }
  }

  // Results through LDS, 128 rows at a time: the waves holding those rows write them as bf16
  // rows of kCols columns, then every store instruction writes four whole 256-byte rows of one
  // output matrix. C^T[n][row]: lane l holds rows 32 y + l % 32, columns 32 x + 8 jg + 4 (l / 32)
  // + 0..3 of block (x, y). FP8 output: the four values are scaled by their matrix's
  // reciprocal scale, clamped to the largest E4M3 magnitude (448) and converted (round to
  // nearest even) into one 32-bit word of codes; rows are then 128 bytes per matrix and each
  // store instruction writes eight of them.
  constexpr int kEB = kFp8Out ? 1 : 2;                 // bytes per output element
  constexpr int kPitch = kCols * kEB + 16;
  static_assert(128 * kPitch <= kStagesG * (kTA + kTB), "a half tile fits in the stage area");
  uint8_t* epi = lds_all;  // the stage area, free once every wave is past the last stage
  const int last = (int)(a.n_rows - r0 < kBM ? a.n_rows - r0 : kBM) - 1;
  constexpr int kRowsPerStore = 1024 / (kDim * kEB);   // whole output rows per store instruction
  constexpr int kLanesPerRowOut = 64 / kRowsPerStore;
  constexpr int kSegsPerMat = 128 / kRowsPerStore;
  constexpr int kSegs = kSegsPerMat * (kCols / kDim);  // 1 KB stores per half tile
  static_assert(kSegs % kGWaves == 0, "stores must split evenly");
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    __syncthreads();  // stage reads (or the previous half's stores) are done
    if ((wr * kWR) / 128 == half) {
#pragma unroll
      for (int y = 0; y < kYB; ++y)
#pragma unroll
        for (int x = 0; x < kXB; ++x)
#pragma unroll
          for (int jg = 0; jg < 4; ++jg) {
            const int row = wr * kWR - 128 * half + 32 * y + (lane & 31);
            const int col = wc * kWC + 32 * x + 8 * jg + 4 * (lane >> 5);
            if constexpr (kFp8Out) {
              const float is = o.inv_scale[nt * (kCols / kDim) + col / kDim];  // this column's output matrix
              float v[4];
#pragma unroll
              for (int q = 0; q < 4; ++q) v[q] = fminf(fmaxf(acc[x][y][4 * jg + q] * is, -448.0f), 448.0f);
              int w = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
              w = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], w, true);
              *reinterpret_cast<int*>(epi + row * kPitch + col) = w;
            } else {
              __bf16 v4[4];
#pragma unroll
              for (int q = 0; q < 4; ++q) v4[q] = (__bf16)acc[x][y][4 * jg + q];
              *reinterpret_cast<uint2*>(epi + row * kPitch + col * 2) = __builtin_bit_cast(uint2, v4);
            }
          }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kSegs / kGWaves; ++i) {
      const int idx = wave * (kSegs / kGWaves) + i;
      const int m = idx / kSegsPerMat;                                  // output matrix of the tile
      const int row = (idx % kSegsPerMat) * kRowsPerStore + lane / kLanesPerRowOut;  // row within the half
      const int chunk = lane % kLanesPerRowOut;                          // 16-byte chunk of the row
      const uint4 v = *reinterpret_cast<const uint4*>(epi + row * kPitch + m * kDim * kEB + chunk * 16);
      const int trow = 128 * half + row;
      if (trow <= last)
        *reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(a.outs[nt * (kCols / kDim) + m]) +
                                  ((r0 + trow) * kDim + chunk * (16 / kEB)) * kEB) = v;
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

hipError_t launch_bridge_gemm(const BridgeArgs& a, const BridgeOut& o, hipStream_t s) {
  const int64_t n_rt = (a.n_rows + kBM - 1) / kBM;
  const int64_t per_xcd = (n_rt + kXcds - 1) / kXcds;
  const bool wide = a.n_mats % 3 == 0;
  const int64_t grid = per_xcd * kXcds * (a.n_mats * kDim / (wide ? 384 : 256));
  const dim3 g((unsigned)grid), b(64 * kGWaves);
  if (wide && o.fp8)
    hipLaunchKernelGGL((bridge_gemm_kernel<384, true>), g, b, 0, s, a, o);
  else if (wide)
    hipLaunchKernelGGL((bridge_gemm_kernel<384, false>), g, b, 0, s, a, o);
  else if (o.fp8)
    hipLaunchKernelGGL((bridge_gemm_kernel<256, true>), g, b, 0, s, a, o);
  else
    hipLaunchKernelGGL((bridge_gemm_kernel<256, false>), g, b, 0, s, a, o);
  return hipGetLastError();
}

}  // namespace hs2
