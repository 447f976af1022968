// Device helpers shared by the bf16 attention kernels (decode-shaped and chunked):
// LDS tile layout and copies, the key list of a query, and the per-tile online softmax
// step on the matrix cores. See attn_bf16.hip for the layout of the MFMA operands.
#pragma once

#include "hs2_internal.h"

namespace hs2 {
namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kNegBig = -1.0e30f; // "no key yet" reference
constexpr float kLazy = 8.0f;       // reference moves only when exceeded by more than this
constexpr int kTileBytes = kTile * kDim * 2;  // 8 KB: one K or V tile
constexpr int kStages = 2;                    // per-wave LDS stages (K + V each)
constexpr int kDmaPerHalf = kTileBytes / 1024;     // 8 wave-wide 16-byte loads per K or V tile

__device__ inline f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }


template <int N>
__device__ inline void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

__device__ inline void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory"); }

// Tile layouts in LDS (32 rows of 256 bytes, filled by row-coalesced DMA):
//  K: the 16-byte chunk c of row r is stored at chunk position c ^ (r & 15), so that the
//     MFMA-operand reads (32 rows, same chunk) are free of bank conflicts;
//  V: plain row-major, so that all V^T operand reads of a lane share one base address
//     and differ by immediate offsets.
__device__ inline uint32_t tile_off(int row, int chunk) {
  return (uint32_t)(row * 256 + ((chunk ^ (row & 15)) << 4));
}

// Logical key list of one query. Full mode: positions 0..t. Gather mode: top_k selected
// slots (entries outside the candidate range are masked) followed by the window rows.
struct KeyList {
  const int32_t* sel_lds;  // gather mode: selected rows of slots [sel_k0, ...) in LDS
  int sel_k0;
  int64_t base;
  int t, top_k, n_keys, w_eff, cand_hi;
  bool gather;

  __device__ inline void row(int p, int& rel, bool& ok) const {
    if (!gather) {
      ok = p < n_keys;
      rel = ok ? p : 0;
      return;
    }
    if (p < top_k) {
      const int s = sel_lds[p - sel_k0];
      ok = s >= 0 && s <= cand_hi;
      rel = ok ? s : 0;
      return;
    }
    const int w = p - top_k;
    ok = w < w_eff;
    rel = ok ? (t - w_eff + 1 + w) : 0;
  }
};

// Row of key (p0 + l%32) of a tile for lane l, and the mask of attended keys of the tile.
__device__ inline uint32_t tile_rows(const KeyList& kl, int p0, int p1, int lane, int& rel) {
  bool ok;
  const int p = p0 + (lane & 31);
  kl.row(p, rel, ok);
  ok = ok && p < p1;
  if (!ok) rel = 0;
  return (uint32_t)__ballot(ok);
}

// Enqueues the 32 rows of a K tile (swizzled) or a V tile (row-major) into LDS. `rel` is
// the row of key l%32 held by lane l; earlier LDS reads of the stage must have completed.
template <bool kSwizzle>
__device__ inline void issue_rows(const __bf16* __restrict__ src, int64_t base, int rel, int lane, uint32_t lds) {
  wait_lgkm0();
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int row = r * 4 + (lane >> 4);
    const int chunk = kSwizzle ? ((lane & 15) ^ (row & 15)) : (lane & 15);
    dma16(src + (base + __shfl(rel, row)) * kDim + chunk * 8, lds + r * 1024);
  }
}

// Online-softmax state of one wave: 64 heads x 128 dims, O^T in the C layout.
struct WaveState {
  f32x16 o[2][4];   // [head block nb][dim block mb]
  float m[2];       // reference (log2 domain) of heads 32*nb + l%32
  float l[2];       // this lane's share of the denominator of the bf16-rounded P
  float le[2];      // ... and of the unrounded P (for the LSE)
};

// One 32-key tile: S^T = K Q^T, online softmax, O^T += V^T P^T. Q^T operands and the V
// tile are read from LDS; the K operands were read already (its stage is reused).
template <bool kQReg>
__device__ inline void process_tile(WaveState& st, const uint8_t* __restrict__ qs, const bf16x8 (*qreg)[8],
                                    const bf16x8 (&kop)[8], const uint8_t* __restrict__ vt, uint32_t vm, float c2,
                                    int lane) {
  f32x16 acc[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    acc[nb] = f32x16{};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bf16x8 q = kQReg ? qreg[nb][s] : *reinterpret_cast<const bf16x8*>(qs + ((nb * 8 + s) * 64 + lane) * 16);
      acc[nb] = mfma(kop[s], q, acc[nb]);
    }
  }

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
      st.le[nb] *= alpha[nb];
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
    float lsum = 0.0f, esum = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float pf = fast_exp2(x[nb][j] - st.m[nb]);
      const __bf16 pv = (__bf16)pf;
      pb[nb][j >> 3][j & 7] = pv;
      lsum += (float)pv;
      esum += pf;
    }
    st.l[nb] += lsum;
    st.le[nb] += esum;
  }

  // O^T += V^T P^T. A operand: lane l holds V[key][32*mb + l%32] for the 8 keys
  // 16*ks + 8*(i/4) + 4*(l/32) + i%4 of its slots (row-major V tile: immediate offsets).
  const uint16_t* vb = reinterpret_cast<const uint16_t*>(vt) + hrow * kDim + (lane & 31);
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 va;
#pragma unroll
      for (int ii = 0; ii < 8; ++ii)
        va[ii] = __builtin_bit_cast(__bf16, vb[(16 * ks + 8 * (ii >> 2) + (ii & 3)) * kDim + 32 * mb]);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) st.o[nb][mb] = mfma(va, pb[nb][ks], st.o[nb][mb]);
    }
}

// K A-operands of the 8 contraction steps from a swizzled K tile.
__device__ inline void read_k(const uint8_t* __restrict__ kt, int lane, bf16x8 (&kop)[8]) {
  const int row = lane & 31;
#pragma unroll
  for (int s = 0; s < 8; ++s)
    kop[s] = *reinterpret_cast<const bf16x8*>(kt + tile_off(row, (lane >> 5) * 8 + s));
}

// s_waitcnt vmcnt(n) for a run-time n in {0, 8, 16, 24}
__device__ inline void wait_vmcnt_dyn(int n) {
  if (n >= 24) wait_vmcnt<24>();
  else if (n >= 16) wait_vmcnt<16>();
  else if (n >= 8) wait_vmcnt<8>();
  else wait_vmcnt<0>();
}

}  // namespace attn
}  // namespace hs2
