// Device helpers shared by the bf16 attention kernels (decode-shaped and chunked):
// LDS tile layout and copies, the key list of a query, and the per-tile online softmax
// step on the matrix cores. See attn_bf16.hip for the layout of the MFMA operands.
#pragma once

#include "kernel_common.h"

namespace hs2 {
namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kNegBig = -1.0e30f; // "no key yet" reference
constexpr int kTileBytes = kTile * kDim * 2;  // 8 KB: one bf16 K or V tile
constexpr int kStages = 2;                    // per-wave LDS stages (K + V each)
constexpr int kDmaPerHalf = kTileBytes / 1024;     // 8 wave-wide 16-byte loads per K or V tile

// Storage formats of the K and V rows. The MFMA operands are bf16 in both: an OCP FP8
// E4M3 value converts to bf16 exactly (3 mantissa bits, exponents 2^-9 .. 2^8), and the
// per-tensor scales are applied in fp32 outside the products (the K scale in the logit
// scale, the V scale in the output normalisation).
struct KvBf16 {
  static constexpr bool kFp8 = false;
  static constexpr int kRowBytes = kDim * 2;              // 256
  static constexpr int kTileBytes = kTile * kRowBytes;    // 8 KB
  static constexpr int kDma = kTileBytes / 1024;          // wave-wide 16-byte copies per tile
  static constexpr int kStages = 2;                       // pass-1 stages per wave (K + V)
};
struct KvFp8 {
  static constexpr bool kFp8 = true;
  static constexpr int kRowBytes = kDim;                  // 128
  static constexpr int kTileBytes = kTile * kRowBytes;    // 4 KB
  static constexpr int kDma = kTileBytes / 1024;
  static constexpr int kStages = 4;                       // same bytes in flight as bf16
};

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
//  V: chunk c of row r at position c ^ (4 * (r & 3)), so that the transposing reads of
//     the V^T operands (8 rows x 64 bytes per instruction) cover all 64 banks twice.
__device__ inline uint32_t tile_off(int row, int chunk) {
  return (uint32_t)(row * 256 + ((chunk ^ (row & 15)) << 4));
}
__device__ inline int v_chunk(int row, int pos) { return pos ^ ((row & 3) << 2); }

// FP8 tiles (32 rows of 128 bytes = 8 chunks of 16):
//  K: chunk c of row r at position c ^ ((r >> 1) & 7): the operand reads (16 rows, same
//     chunk, per 256 bytes of LDS) cover all 16 bank groups;
//  V: chunk c of row r at position c ^ ((r & 2) | ((r >> 1) & 4)): the transposing reads
//     take 8 rows x 2 adjacent chunks (rows {0,1,2,3,8,9,10,11} + 4h of a 16-key step),
//     which this maps onto 16 distinct bank groups.
__device__ inline int k8_swz(int row) { return (row >> 1) & 7; }
__device__ inline int v8_swz(int row) { return (row & 2) | ((row >> 1) & 4); }

// Key list of one query in the selector's attention pass: positions 0 .. n_keys-1 (the
// causal range 0..t) of the sequence whose first row is `base`.
struct KeyList {
  int64_t base;
  int n_keys;

  __device__ inline void row(int p, int& rel, bool& ok) const {
    ok = p < n_keys;
    rel = ok ? p : 0;
  }
};

// Order in which a workgroup visits the tiles of its key range: tile x of the stream is
// tile (x + rot) mod n. Workgroups streaming equal-sized splits in the same order would
// read the same offsets of their splits at the same moment; a per-workgroup rotation
// (97 x the work index, modulo the tiles) staggers them. On the 64 x 131,072 decode
// batch the selector's attention pass ran 3% faster with it (same-box A/B).
struct TileOrder {
  int rot, n;
  __device__ static TileOrder rotated(int work, int ntiles) {
    return TileOrder{(int)(((uint32_t)work * 97u) % (uint32_t)ntiles), ntiles};
  }
  __device__ int at(int x) const { return x + rot < n ? x + rot : x + rot - n; }  // 0 <= x < n
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

// Enqueues the 32 rows of a K tile or a V tile (each in its swizzle) into LDS. `rel` is
// the row of key l%32 held by lane l; earlier LDS reads of the stage must have completed.
// Copy r writes rows 4r .. 4r+3: lane l fills chunk position l%16 of row 4r + l/16.
template <bool kIsK>
__device__ inline void issue_rows(const __bf16* __restrict__ src, int64_t base, int rel, int lane, uint32_t lds) {
  wait_lgkm0();
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int row = r * 4 + (lane >> 4);
    const int chunk = kIsK ? ((lane & 15) ^ (row & 15)) : v_chunk(row, lane & 15);
    dma16(src + (base + __shfl(rel, row)) * kDim + chunk * 8, lds + r * 1024);
  }
}

// The same for either storage format (src: the K or V tensor): copy r writes the
// 1024/kRowBytes rows that follow row r*1024/kRowBytes, each lane one 16-byte position.
template <typename Kv, bool kIsK>
__device__ inline void issue_tile(const void* __restrict__ src, int64_t base, int rel, int lane, uint32_t lds) {
  if constexpr (!Kv::kFp8) {
    issue_rows<kIsK>(static_cast<const __bf16*>(src), base, rel, lane, lds);
  } else {
    wait_lgkm0();
    const uint8_t* s8 = static_cast<const uint8_t*>(src);
#pragma unroll
    for (int r = 0; r < Kv::kDma; ++r) {
      const int row = r * 8 + (lane >> 3);
      const int pos = lane & 7;
      const int chunk = pos ^ (kIsK ? k8_swz(row) : v8_swz(row));
      dma16(s8 + (base + __shfl(rel, row)) * Kv::kRowBytes + chunk * 16, lds + r * 1024);
    }
  }
}

// The same copies for a contiguous tile: keys p0 .. p0+31 of the sequence whose first row
// is `base`; a key at or past `pend` (not attended) copies row `base` instead, as
// tile_rows' row 0 does. Each lane computes its rows' addresses itself. The decode passes
// read each of these rows once, so the copies are marked non-temporal.
template <typename Kv, bool kIsK>
__device__ inline void issue_tile_contig(const void* __restrict__ src, int64_t base, int p0, int pend, int lane,
                                         uint32_t lds) {
  wait_lgkm0();
  if constexpr (!Kv::kFp8) {
    const __bf16* s = static_cast<const __bf16*>(src);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int row = r * 4 + (lane >> 4);
      const int p = p0 + row;
      const int rel = p < pend ? p : 0;
      const int chunk = kIsK ? ((lane & 15) ^ (row & 15)) : v_chunk(row, lane & 15);
      dma16_nt(s + (base + rel) * kDim + chunk * 8, lds + r * 1024);
    }
  } else {
    const uint8_t* s8 = static_cast<const uint8_t*>(src);
#pragma unroll
    for (int r = 0; r < Kv::kDma; ++r) {
      const int row = r * 8 + (lane >> 3);
      const int p = p0 + row;
      const int rel = p < pend ? p : 0;
      const int chunk = (lane & 7) ^ (kIsK ? k8_swz(row) : v8_swz(row));
      dma16_nt(s8 + (base + rel) * Kv::kRowBytes + chunk * 16, lds + r * 1024);
    }
  }
}

// Online-softmax state of one wave: 64 heads x 128 dims, O^T in the C layout.
// The softmax reference m of a head is fixed at the first tile that holds an attended
// key (that tile's maximum); later tiles are not rescaled. exp2(x - m) may then exceed 1,
// which floating point represents exactly up to 2^127; a wave whose state overflowed is
// recomputed with the exact maximum as reference (see state_finite).
struct WaveState {
  f32x16 o[2][4];   // [head block nb][dim block mb]
  float m[2];       // reference (log2 domain) of heads 32*nb + l%32
  float l[2];       // this lane's share of the denominator of the bf16-rounded P
  float le[2];      // ... and of the unrounded P (for the LSE)
  int have_ref;     // wave-uniform: m holds a reference
};

__device__ inline void state_init(WaveState& st) {
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    st.m[nb] = kNegBig;
    st.l[nb] = 0.0f;
    st.le[nb] = 0.0f;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) st.o[nb][mb] = f32x16{};
  }
  st.have_ref = 0;
}

// True on every lane if no accumulator or denominator of the wave is inf or NaN.
__device__ inline bool state_finite(const WaveState& st) {
  float z = 0.0f;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    z = fmaf(st.l[nb], 0.0f, z);
    z = fmaf(st.le[nb], 0.0f, z);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int j = 0; j < 16; ++j) z = fmaf(st.o[nb][mb][j], 0.0f, z);
  }
  return __all(z == 0.0f);  // inf * 0 and NaN * 0 are NaN
}

// Per-lane base addresses of the transposing V^T reads. Instruction (mb, ks, half) on
// lane l returns V[16ks + 8half + 4(l/32) + i][32mb + l%32], i = 0..3: the A-operand
// entries of MFMA k = 8(l/32) + 4half + i under the key order of the P^T operand.
// Source lane l addresses row 16ks + 8half + 4(l/32) + (l/4)%4 at dims
// 32mb + 16((l/16)%2) + 4(l%4) .. +3 (8 bytes).
__device__ inline void vt_bases(int lane, uint32_t (&vb)[4]) {
  const int r4 = lane & 3, c = (lane >> 2) & 3, gp = (lane >> 4) & 1, h = lane >> 5;
  const uint32_t lb = (uint32_t)((4 * h + c) * 256 + 32 * gp + 8 * r4);
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) vb[mb] = lb + 64u * (uint32_t)(mb ^ c);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// FP8 V^T operands (ds_read_b64_tr_b8). In each 16-lane group g, output lane j receives
// as its byte c the byte j%8 of the 8 bytes addressed by lane 2c + j/8 of the group
// (lane mapping established with an in-bounds probe on the GPU). Lane 2c + h of group g
// addresses row key(c) = 16ks + 8(c/4) + 4(g/2) + c%4 at dims 32mb + 16(g%2) + 8h, so
// output lane l holds V[key(c)][32mb + l%32] for c = 0..7: the A operand of
// O^T += V^T P^T in the key order of the P^T operand (see process_tile).
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

__device__ inline void vt8_bases(int lane, uint32_t (&vb)[4]) {
  const int g = lane >> 4, c = (lane & 15) >> 1, h = lane & 1;
  const int row = 8 * (c >> 2) + 4 * (g >> 1) + (c & 3);
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
    vb[mb] = (uint32_t)(row * 128 + (((2 * mb + (g & 1)) ^ v8_swz(row)) << 4) + 8 * h);
}

template <typename Kv>
__device__ inline void vt_bases_of(int lane, uint32_t (&vb)[4]) {
  if constexpr (Kv::kFp8) vt8_bases(lane, vb);
  else vt_bases(lane, vb);
}

// Eight OCP E4M3 codes (bytes of w0, then w1) to bf16, exactly (scale 1).
__device__ inline bf16x8 fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w0, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w0, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w1, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w1, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ inline bf16x8 read_vt8(const uint8_t* vt, uint32_t vbase, int ks) {
  const __attribute__((address_space(3))) char* p =
      (const __attribute__((address_space(3))) char*)(vt) + vbase + ks * 16 * 128;
  const i32x2 w = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)p);
  return fp8x8_to_bf16((uint32_t)w[0], (uint32_t)w[1]);
}

__device__ inline bf16x8 read_vt(const uint8_t* vt, uint32_t vbase, int ks) {
  const __attribute__((address_space(3))) char* p =
      (const __attribute__((address_space(3))) char*)(vt) + vbase + ks * 16 * 256;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 8 * 256));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// S^T = K Q^T of one tile: acc[nb] holds keys (C rows) x heads 32nb.. (C columns).
template <bool kQReg>
__device__ inline void tile_logits(f32x16 (&acc)[2], const uint8_t* __restrict__ qs, const bf16x8 (*qreg)[8],
                                   const bf16x8 (&kop)[8], int lane) {
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    acc[nb] = f32x16{};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bf16x8 q = kQReg ? qreg[nb][s] : *reinterpret_cast<const bf16x8*>(qs + ((nb * 8 + s) * 64 + lane) * 16);
      acc[nb] = mfma(kop[s], q, acc[nb]);
    }
  }
}

// Maximum over the attended keys of the tile (mask vm, bit = key) of the raw logits of
// heads 32nb + l%32, times c2 (> 0); -inf if no key is attended.
__device__ inline void tile_max(const f32x16 (&acc)[2], uint32_t vm, float c2, int lane, float (&mx)[2]) {
  const int hrow = 4 * (lane >> 5);
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    float v = -INFINITY;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int key = 8 * (j >> 2) + hrow + (j & 3);
      v = ((vm >> key) & 1u) ? fmaxf(v, acc[nb][j]) : v;
    }
    v = fmaxf(v, __shfl_xor(v, 32));
    mx[nb] = v * c2;
  }
}

// One 32-key tile with at least one attended key: S^T = K Q^T, P = exp2(c2 S - m) with
// the fixed reference, O^T += V^T P^T. Q^T operands come from LDS or registers, K
// operands were read already, V^T is read from the tile's stage in LDS.
template <bool kQReg, typename Kv = KvBf16>
__device__ inline void process_tile(WaveState& st, const uint8_t* __restrict__ qs, const bf16x8 (*qreg)[8],
                                    const bf16x8 (&kop)[8], const uint8_t* __restrict__ vt, const uint32_t (&vb)[4],
                                    uint32_t vm, float c2, int lane) {
  f32x16 acc[2];
  tile_logits<kQReg>(acc, qs, qreg, kop, lane);
  if (__builtin_amdgcn_readfirstlane(st.have_ref) == 0) {  // wave-uniform, first attended tile only
    tile_max(acc, vm, c2, lane, st.m);
    st.have_ref = 1;
  }

  float p[2][16];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const float nm = -st.m[nb];
#pragma unroll
    for (int j = 0; j < 16; ++j) p[nb][j] = fast_exp2(fmaf(acc[nb][j], c2, nm));
  }
  if (__builtin_amdgcn_readfirstlane(vm) != 0xffffffffu) {  // wave-uniform: edge tiles only
    const int hrow = 4 * (lane >> 5);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int key = 8 * (j >> 2) + hrow + (j & 3);
        if (!((vm >> key) & 1u)) p[nb][j] = 0.0f;
      }
  }

  // P^T (bf16) in the B-operand layout of the 16-key steps: step ks holds registers
  // j = 8*ks .. 8*ks+7, i.e. keys 16*ks + 8*(i/4) + 4*(l/32) + i%4.
  bf16x8 pb[2][2];
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    float esum = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      pb[nb][j >> 3][j & 7] = (__bf16)p[nb][j];
      esum += p[nb][j];
    }
    float lsum = st.l[nb];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        lsum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[nb][ks][2 * u], pb[nb][ks][2 * u + 1]}, ones, lsum, false);
    st.l[nb] = lsum;
    st.le[nb] += esum;
  }

  // O^T += V^T P^T
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 va;
      if constexpr (Kv::kFp8) va = read_vt8(vt, vb[mb], ks);
      else va = read_vt(vt, vb[mb], ks);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) st.o[nb][mb] = mfma(va, pb[nb][ks], st.o[nb][mb]);
    }
}

// Logit maximum only (the recomputation of an overflowed wave): mx = max(mx, tile max).
template <bool kQReg>
__device__ inline void process_tile_max(float (&mx)[2], const uint8_t* __restrict__ qs, const bf16x8 (*qreg)[8],
                                        const bf16x8 (&kop)[8], uint32_t vm, float c2, int lane) {
  f32x16 acc[2];
  tile_logits<kQReg>(acc, qs, qreg, kop, lane);
  float t[2];
  tile_max(acc, vm, c2, lane, t);
  mx[0] = fmaxf(mx[0], t[0]);
  mx[1] = fmaxf(mx[1], t[1]);
}

// K A-operands of the 8 contraction steps from a swizzled K tile.
__device__ inline void read_k(const uint8_t* __restrict__ kt, int lane, bf16x8 (&kop)[8]) {
  const int row = lane & 31;
#pragma unroll
  for (int s = 0; s < 8; ++s)
    kop[s] = *reinterpret_cast<const bf16x8*>(kt + tile_off(row, (lane >> 5) * 8 + s));
}

// K A-operands from an FP8 K tile: lane l reads the 64 bytes of dims (l/32)*64 .. +63 of
// row l%32 (4 chunks; each holds the 8-dim slices of two contraction steps) and
// converts them to bf16.
__device__ inline void read_k8(const uint8_t* __restrict__ kt, int lane, bf16x8 (&kop)[8]) {
  const int row = lane & 31;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int chunk = 4 * (lane >> 5) + u;
    const uint4 w = *reinterpret_cast<const uint4*>(kt + row * 128 + ((chunk ^ k8_swz(row)) << 4));
    kop[2 * u] = fp8x8_to_bf16(w.x, w.y);
    kop[2 * u + 1] = fp8x8_to_bf16(w.z, w.w);
  }
}

template <typename Kv>
__device__ inline void read_k_of(const uint8_t* __restrict__ kt, int lane, bf16x8 (&kop)[8]) {
  if constexpr (Kv::kFp8) read_k8(kt, lane, kop);
  else read_k(kt, lane, kop);
}

// s_waitcnt vmcnt(n) for a run-time, wave-uniform n, a multiple of 4 below 64
__device__ inline void wait_vmcnt_n(int n) {
  switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 4: wait_vmcnt<4>(); break;
    case 8: wait_vmcnt<8>(); break;
    case 12: wait_vmcnt<12>(); break;
    case 16: wait_vmcnt<16>(); break;
    case 20: wait_vmcnt<20>(); break;
    case 24: wait_vmcnt<24>(); break;
    case 28: wait_vmcnt<28>(); break;
    case 32: wait_vmcnt<32>(); break;
    case 36: wait_vmcnt<36>(); break;
    case 40: wait_vmcnt<40>(); break;
    case 44: wait_vmcnt<44>(); break;
    case 48: wait_vmcnt<48>(); break;
    case 52: wait_vmcnt<52>(); break;
    case 56: wait_vmcnt<56>(); break;
    case 60: wait_vmcnt<60>(); break;
    default: wait_vmcnt<0>(); break;
  }
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
