// Sparse attention layers of the hybrid block on gfx950: each query attends to its forced
// window plus the selector's rows only, on the selector's KV cache (bf16 or FP8 E4M3).
//
// Method (page title and section): arex-research.com, "Xiaomi MiMo lead Luo Fuli
// publishes the MiMo-V3 core architecture HySparse2", section "Outer KV Bridging, inner
// KV Reuse": the sparse layers reuse the full-attention layer's KV cache and its index
// set, attending the 128 most recent tokens plus the 1,024 selected ones; section
// "Numbers computed on three 80B-A3B models": one KV head serves all 64 query heads,
// so every gathered row is used by all of them.
//
// The layer is bound by gathering scattered 256-byte rows (128-byte with FP8), not by
// arithmetic: 1,152 K and V rows per query. A workgroup takes a slice of one query's
// logical keys (selected slots first, then the window rows) and requests the K and V rows
// of all of its tiles up front, each 32-key tile into its own LDS slot, so the whole
// slice is in flight at once. Since every tile's rows are scattered, tiles land at about
// the same time, near the end of the transfer: the arithmetic after that is spread over
// all four SIMDs. Wave w owns the 32 query heads of head block w%2 and the tiles of parity
// w/2; the two waves of a parity copy the K and the V rows of their tiles respectively
// and compute every one of them for their own heads. The two parities are merged through
// LDS at the end; the key split over workgroups is merged by the split combine of
// attn_bf16.hip. The tile step is the one of the full-attention kernels (attn_common.h:
// S^T = K Q^T, a softmax reference fixed at the first attended tile, O^T += V^T P^T)
// restricted to one 32-head block, with the wave's Q operands in registers.
#include "attn_common.h"
#include "hs2_launch.h"

namespace hs2 {
namespace {

using namespace attn;

constexpr int kSpWaves = 4;                 // waves per workgroup: 2 head blocks x 2 tile parities

// Tile slots of a workgroup: the wide form (144 KB of LDS, one workgroup per CU) for
// batches whose slices fill the GPU about once; the narrow form (64 KB, two per CU, so
// one's gather overlaps the other's arithmetic) for batches of many queries, where each
// workgroup takes a whole query in batches of kNarrow tiles.
template <typename Kv>
struct SparseCfg {
  static constexpr int kSlots = kSparseStageBytes / (2 * Kv::kTileBytes);  // 9 bf16 tiles, 18 FP8 tiles
  static constexpr int kNarrow = kSparseNarrowBytes / (2 * Kv::kTileBytes);  // 4 bf16 tiles, 8 FP8 tiles
};
static_assert(SparseCfg<KvBf16>::kSlots == sparse_slots(false) && SparseCfg<KvFp8>::kSlots == sparse_slots(true),
              "slots");

// Online-softmax state of one wave's 32 heads: O^T [128 dims][32 heads] in the C layout
// (dim block mb), the reference m (log2 domain) of head l%32, this lane's shares of the
// denominators of the bf16-rounded (l) and unrounded (le) probabilities.
struct HeadsState {
  f32x16 o[4];
  float m, l, le;
  int have_ref;
};

__device__ inline void heads_init(HeadsState& st) {
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) st.o[mb] = f32x16{};
  st.m = kNegBig;
  st.l = 0.0f;
  st.le = 0.0f;
  st.have_ref = 0;
}

__device__ inline bool heads_finite(const HeadsState& st) {
  float z = fmaf(st.l, 0.0f, 0.0f);
  z = fmaf(st.le, 0.0f, z);
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int j = 0; j < 16; ++j) z = fmaf(st.o[mb][j], 0.0f, z);
  return __all(z == 0.0f);
}

// S^T = K Q^T of one tile for the wave's 32 heads: acc[j] = logit of key 8(j/4) + 4(l/32)
// + j%4 for head l%32 (raw dot products).
__device__ inline f32x16 heads_logits(const bf16x8 (&kop)[8], const bf16x8 (&q)[8]) {
  f32x16 acc = f32x16{};
#pragma unroll
  for (int s = 0; s < 8; ++s) acc = mfma(kop[s], q[s], acc);
  return acc;
}

// Maximum of c2 * logit over the attended keys (mask vm) of the tile, per head; -inf if none.
__device__ inline float heads_max(const f32x16& acc, uint32_t vm, float c2, int lane) {
  const int hrow = 4 * (lane >> 5);
  float v = -INFINITY;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int key = 8 * (j >> 2) + hrow + (j & 3);
    v = ((vm >> key) & 1u) ? fmaxf(v, acc[j]) : v;
  }
  return fmaxf(v, __shfl_xor(v, 32)) * c2;
}

// One tile with at least one attended key: P = exp2(c2 S - m) with the fixed reference,
// O^T += V^T P^T; l sums the bf16-rounded P (the output's denominator), le the unrounded.
template <typename Kv>
__device__ inline void heads_tile(HeadsState& st, const bf16x8 (&q)[8], const uint8_t* __restrict__ kt,
                                  const uint8_t* __restrict__ vt, const uint32_t (&vb)[4], uint32_t vm, float c2,
                                  int lane) {
  bf16x8 kop[8];
  read_k_of<Kv>(kt, lane, kop);
  const f32x16 acc = heads_logits(kop, q);
  if (__builtin_amdgcn_readfirstlane(st.have_ref) == 0) {
    st.m = heads_max(acc, vm, c2, lane);
    st.have_ref = 1;
  }
  float p[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) p[j] = fast_exp2(fmaf(acc[j], c2, -st.m));
  if (__builtin_amdgcn_readfirstlane(vm) != 0xffffffffu) {
    const int hrow = 4 * (lane >> 5);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int key = 8 * (j >> 2) + hrow + (j & 3);
      if (!((vm >> key) & 1u)) p[j] = 0.0f;
    }
  }
  // P^T in the B-operand layout of the 16-key steps (step ks: registers 8ks .. 8ks+7)
  bf16x8 pb[2];
  float esum = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    pb[j >> 3][j & 7] = (__bf16)p[j];
    esum += p[j];
  }
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  float lsum = st.l;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int u = 0; u < 4; ++u)
      lsum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[ks][2 * u], pb[ks][2 * u + 1]}, ones, lsum, false);
  st.l = lsum;
  st.le += esum;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 va;
      if constexpr (Kv::kFp8) va = read_vt8(vt, vb[mb], ks);
      else va = read_vt(vt, vb[mb], ks);
      st.o[mb] = mfma(va, pb[ks], st.o[mb]);
    }
}

// s_waitcnt vmcnt(n) for a wave-uniform n (capped at 63, the counter's range: waiting
// for fewer outstanding copies than needed is only more conservative).
__device__ inline void wait_vm_upto(int n) {
  if (n >= 63) wait_vmcnt<63>();
  else if (n >= 56) wait_vmcnt<56>();
  else if (n >= 48) wait_vmcnt<48>();
  else if (n >= 40) wait_vmcnt<40>();
  else if (n >= 32) wait_vmcnt<32>();
  else if (n >= 24) wait_vmcnt<24>();
  else if (n >= 16) wait_vmcnt<16>();
  else if (n >= 8) wait_vmcnt<8>();
  else wait_vmcnt<0>();
}

__device__ inline void slot_barrier() {
  wait_lgkm0();
  __builtin_amdgcn_s_barrier();
}

// The logical keys [k0, k1) of query i in tiles of 32: tile j holds keys k0 + 32j + l%32.
// Key p < top_k is selected slot p (attended if 0 <= sel[p] <= t - window); key p >= top_k
// is window row t - w_eff + 1 + (p - top_k). Returns the row of lane l's key (0 if not
// attended) and the mask of attended keys.
struct SparseKeys {
  const int32_t* sel;  // this query's top_k slots
  int64_t base;
  int t, top_k, w_eff, cand_hi, k0, k1;
  __device__ inline uint32_t tile(int j, int32_t slot, int lane, int& rel) const {
    const int p = k0 + 32 * j + (lane & 31);
    bool ok;
    if (p < top_k) {
      ok = slot >= 0 && slot <= cand_hi;
      rel = ok ? slot : 0;
    } else {
      const int w = p - top_k;
      ok = w < w_eff;
      rel = ok ? t - w_eff + 1 + w : 0;
    }
    ok = ok && p < k1;
    if (!ok) rel = 0;
    return (uint32_t)__ballot(ok);
  }
  __device__ inline int32_t slot_of(int j, int lane) const {
    const int p = k0 + 32 * j + (lane & 31);
    return (p < top_k && p < k1) ? sel[p] : -1;
  }
};

// Gathers and computes the tiles [0, ntiles) of the slice in batches of kSlots. Tile j of
// a batch goes to slot j; the waves of parity j%2 compute it, the one of head block 0
// copying its K rows and the one of head block 1 its V rows. Each round of two tiles ends
// with a barrier of the workgroup, after each wave has waited for its own copies. The
// first batch's slot values come in `slot0` (this wave's tiles j = 2u + par).
template <typename Kv, int T, bool kMaxOnly>
__device__ inline void sparse_pass(HeadsState& st, float& mx, uint8_t (*stage)[2][Kv::kTileBytes],
                                   const SparseKeys& sk, const int32_t (&slot0)[(T + 1) / 2], int ntiles,
                                   const bf16x8 (&q)[8], const void* __restrict__ kp, const void* __restrict__ vp,
                                   float c2, int hb, int par, int lane) {
  constexpr int U = (T + 1) / 2;  // tiles of one parity in a batch
  uint32_t vb[4];
  vt_bases_of<Kv>(lane, vb);
  for (int b0 = 0; b0 < ntiles; b0 += T) {
    const int nb = min(T, ntiles - b0);
    const int mine = (nb - par + 1) / 2;  // tiles of this parity in the batch
    int32_t slot[U];
    if (b0 == 0) {
#pragma unroll
      for (int u = 0; u < U; ++u) slot[u] = slot0[u];
    } else {
      slot_barrier();  // every wave is done with the previous batch's slots
#pragma unroll
      for (int u = 0; u < U; ++u) slot[u] = sk.slot_of(b0 + 2 * u + par, lane);
    }
    // every compiler-tracked load has completed before the copies are issued (their waits
    // are placed by hand and count only the copies)
#pragma unroll
    for (int u = 0; u < U; ++u) asm volatile("" : : "v"(slot[u]));
    uint32_t vm[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      vm[u] = 0u;
      if (u < mine) {
        const int j = 2 * u + par;
        int rel;
        vm[u] = sk.tile(b0 + j, slot[u], lane, rel);
        const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)stage[j][hb]);
        if (hb == 0) issue_tile<Kv, true>(kp, sk.base, rel, lane, lds);
        else issue_tile<Kv, false>(vp, sk.base, rel, lane, lds);
      }
    }
    const int rounds = (nb + 1) / 2;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (u < rounds) {
        if (u < mine) wait_vm_upto(Kv::kDma * (mine - 1 - u));  // this wave's copies of its tile u landed
        slot_barrier();                                           // ... and its partner's
        if (u < mine && vm[u] != 0u) {
          const int j = 2 * u + par;
          if (kMaxOnly) {
            bf16x8 kop[8];
            read_k_of<Kv>(stage[j][0], lane, kop);
            mx = fmaxf(mx, heads_max(heads_logits(kop, q), vm[u], c2, lane));
          } else {
            heads_tile<Kv>(st, q, stage[j][0], stage[j][1], vb, vm[u], c2, lane);
          }
        }
      }
    }
  }
}

template <typename Kv, int T>
__global__ __launch_bounds__(64 * kSpWaves) void sparse_attn_kernel(AttnArgs a) {
  constexpr int U = (T + 1) / 2;
  // K/V slots during the key loop; afterwards the state of the parity-1 waves for the merge
  struct MergeArea {
    float o[2][64 * 64];  // [head block][register image: element e of lane l at e * 64 + l]
    float m[2][32], l[2][32], le[2][32];
  };
  constexpr int kSlotBytes = T * 2 * Kv::kTileBytes;
  constexpr int kBytes = kSlotBytes > (int)sizeof(MergeArea) ? kSlotBytes : (int)sizeof(MergeArea);
  __shared__ __align__(16) uint8_t lds[kBytes];
  uint8_t(*stage)[2][Kv::kTileBytes] = reinterpret_cast<uint8_t(*)[2][Kv::kTileBytes]>(lds);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hb = wave & 1, par = wave >> 1;
  const int i = blockIdx.x / a.n_split;
  const int split = blockIdx.x - i * a.n_split;
  const int k0 = split * a.split_keys;

  // One round of loads before anything depends on them: the query's descriptor, this
  // slice's first batch of slot values and the wave's Q operands (heads 32w .. 32w+31:
  // piece s of lane l = Q[32w + l%32][(l/32)*64 + 8s .. +7]).
  SparseKeys sk;
  sk.sel = a.top_k > 0 ? a.sel + (size_t)i * a.top_k : nullptr;
  sk.top_k = a.top_k;
  sk.k0 = k0;
  sk.k1 = k0 + a.split_keys;  // narrowed below once t is known
  int32_t slot0[U];
#pragma unroll
  for (int u = 0; u < U; ++u) slot0[u] = sk.slot_of(2 * u + par, lane);
  bf16x8 q[8];
  {
    const __bf16* qp = static_cast<const __bf16*>(a.q) + ((size_t)i * kHeads + 32 * hb + (lane & 31)) * kDim +
                       (lane >> 5) * 64;
#pragma unroll
    for (int s = 0; s < 8; ++s) q[s] = *reinterpret_cast<const bf16x8*>(qp + 8 * s);
  }
  int64_t base;
  int t;
  const bool valid = __builtin_amdgcn_readfirstlane(query_desc(a.b, i, base, t));
  t = __builtin_amdgcn_readfirstlane(t);
  base = (int64_t)uniform_u64((uint64_t)base);
  // the copies below are waited for by hand: every compiler-tracked load (Q included) must
  // have completed before the first one is issued
#pragma unroll
  for (int s = 0; s < 8; ++s) asm volatile("" : : "v"(q[s]));
  if (!valid) {
    if (a.n_split == 1 && par == 0) {
      __bf16* out = static_cast<__bf16*>(a.out) + ((size_t)i * kHeads + 32 * hb + (lane & 31)) * kDim;
      for (int d = (lane >> 5) * 64; d < (lane >> 5) * 64 + 64; ++d) out[d] = (__bf16)NAN;
      if (lane < 32 && a.lse) a.lse[(size_t)i * kHeads + 32 * hb + lane] = NAN;
    }
    return;
  }
  sk.base = base;
  sk.t = t;
  sk.w_eff = min(a.window, t + 1);
  sk.cand_hi = t - a.window;
  const int n_keys = a.top_k + sk.w_eff;
  if (k0 >= n_keys) return;  // an empty slice: the combine does not read it
  sk.k1 = min(n_keys, k0 + a.split_keys);
  const int ntiles = (sk.k1 - k0 + kTile - 1) / kTile;

  HeadsState st;
  heads_init(st);
  float mx = -INFINITY;
  sparse_pass<Kv, T, false>(st, mx, stage, sk, slot0, ntiles, q, a.k, a.v, a.c2, hb, par, lane);
  // rare: a logit far above the first tile's maximum overflowed a wave's sums. Every wave
  // then gathers the slice again (each copies its share of the tiles and joins every
  // barrier): once for the exact maximum of each head over its tiles, once more with it
  // as the reference.
  __shared__ int s_bad[kSpWaves];
  const bool finite = heads_finite(st);  // a vote of the whole wave: every lane takes part
  if (lane == 0) s_bad[wave] = finite ? 0 : 1;
  __syncthreads();  // also: every wave is done with the slots
  if (s_bad[0] | s_bad[1] | s_bad[2] | s_bad[3]) {
    sparse_pass<Kv, T, true>(st, mx, stage, sk, slot0, ntiles, q, a.k, a.v, a.c2, hb, par, lane);
    heads_init(st);
    st.m = mx;
    st.have_ref = 1;
    slot_barrier();
    sparse_pass<Kv, T, false>(st, mx, stage, sk, slot0, ntiles, q, a.k, a.v, a.c2, hb, par, lane);
    __syncthreads();  // the slots are free for the merge area
  }
  st.l += __shfl_xor(st.l, 32);
  st.le += __shfl_xor(st.le, 32);

  // merge the two parities of each head block (fixed order: parity 0, then 1); a wave that
  // attended no key (a slice of a single tile) has the "no key yet" reference and weight 0
  MergeArea& mg = *reinterpret_cast<MergeArea*>(lds);
  if (par == 1) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int j = 0; j < 16; ++j) mg.o[hb][(16 * mb + j) * 64 + lane] = st.o[mb][j];
    if (lane < 32) {
      mg.m[hb][lane] = st.m;
      mg.l[hb][lane] = st.l;
      mg.le[hb][lane] = st.le;
    }
  }
  __syncthreads();
  if (par == 1) return;
  {
    const float m1 = mg.m[hb][lane & 31];
    const float M = fmaxf(st.m, m1);
    const float f0 = fast_exp2(st.m - M), f1 = fast_exp2(m1 - M);
    st.l = st.l * f0 + mg.l[hb][lane & 31] * f1;
    st.le = st.le * f0 + mg.le[hb][lane & 31] * f1;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int j = 0; j < 16; ++j) st.o[mb][j] = st.o[mb][j] * f0 + mg.o[hb][(16 * mb + j) * 64 + lane] * f1;
    st.m = M;
  }

  const int h = 32 * hb + (lane & 31);
  const int hrow = 4 * (lane >> 5);
  if (a.n_split == 1) {
    __bf16* out = static_cast<__bf16*>(a.out) + ((size_t)i * kHeads + h) * kDim;
    const float inv = a.v_scale / st.l;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        __bf16 v4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v4[r] = (__bf16)(st.o[mb][4 * jg + r] * inv);
        *reinterpret_cast<uint2*>(out + 32 * mb + 8 * jg + hrow) = __builtin_bit_cast(uint2, v4);
      }
    if (lane < 32 && a.lse) a.lse[(size_t)i * kHeads + h] = (st.m + __log2f(st.le)) * kLn2;
    return;
  }
  Partial* P = a.part + (size_t)i * a.n_split + split;
  if (lane < 32) {
    P->m[h] = st.m;
    P->l[h] = st.l;
    P->le[h] = st.le;
  }
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int j = 0; j < 16; ++j) P->o[(32 * mb + 8 * (j >> 2) + hrow + (j & 3)) * kHeads + h] = st.o[mb][j];
}

}  // namespace

hipError_t launch_sparse_attn(const AttnArgs& a, bool fp8, bool narrow, int grid, hipStream_t s) {
  const dim3 g(grid), blk(64 * kSpWaves);
  if (fp8) {
    if (narrow) hipLaunchKernelGGL((sparse_attn_kernel<KvFp8, SparseCfg<KvFp8>::kNarrow>), g, blk, 0, s, a);
    else hipLaunchKernelGGL((sparse_attn_kernel<KvFp8, SparseCfg<KvFp8>::kSlots>), g, blk, 0, s, a);
  } else {
    if (narrow) hipLaunchKernelGGL((sparse_attn_kernel<KvBf16, SparseCfg<KvBf16>::kNarrow>), g, blk, 0, s, a);
    else hipLaunchKernelGGL((sparse_attn_kernel<KvBf16, SparseCfg<KvBf16>::kSlots>), g, blk, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace hs2
