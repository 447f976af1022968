// First-generation HySparse layout on gfx950 (the comparison variant): GQA attention with
// 4 KV heads of 16 query heads, 64-token block selection per KV head, and sparse layers
// whose selected-block branch and sliding-window branch are fused through gates.
//
// Method (page title and section):
//   arex-research.com, "Xiaomi MiMo lead Luo Fuli publishes the MiMo-V3 core architecture
//   HySparse2", section "Outer KV Bridging, inner KV Reuse": the predecessor picks its
//   1,024 global tokens as 64-token blocks, and its sparse layers add a separate
//   128-token SWA branch fused through a gate; the full layer hands its KV cache and
//   top-k block indices to the sparse layers. Section "Numbers computed on three 80B-A3B
//   models": the predecessor uses GQA, 64 query heads on 4 KV heads. Section "Lost
//   points, the 290B check and open questions": the SWA branch has its own projections
//   and local KV cache.
//
// Work decomposition. One workgroup of four waves takes one query and one part of its
// keys; wave g serves KV head g and its 16 query heads, so the four waves stream
// disjoint 256-byte slices of the same 1 KB cache rows and no cross-wave merge is needed.
// Tiles of 32 keys go through two per-wave LDS stages by direct-to-LDS copies, as in the
// MQA kernels, and use the same MFMA operand layouts (v_mfma_f32_32x32x16_bf16 with keys
// as rows and heads as columns): the 16 heads fill half of the 32 columns and the other
// half carries zero queries. The wasted half of the matrix work costs nothing here: at
// 32 x 512 bytes of K and V per tile the kernel is bound by HBM with several times the
// matrix throughput to spare.
//
// Softmax is online in the log2 domain with a running maximum per head (the accumulators
// are rescaled when it grows). The selector also writes, per 64-key block and head, the
// log2-sum of the block's weights: block score = sum over the group's heads of
// 2^(block LSE - head LSE), computed after the split combine, so no second pass over K
// is needed for block-level selection.
#include "attn_common.h"
#include "v1_internal.h"
#include "hs2_launch.h"

namespace hs2 {
namespace {

using namespace attn;

constexpr int kV1Stages = 2;
constexpr int kV1WaveBytes = kV1Stages * 2 * kTileBytes;  // 32 KB per wave
constexpr int kV1D = kTileBytes / 1024;                   // wave-wide copies per K or V tile
constexpr int kRowElems = kV1Groups * kDim;               // elements of one cache row (4 heads)
constexpr uint32_t kWaitVm0 = 0x0F70;
constexpr int kMaxV1Split = 256;                         // bound of the selector's parts per query                     // s_waitcnt vmcnt(0), others unbounded

enum { kModeFull = 0, kModeSparse = 1, kModeSwa = 2 };

// Query i: sequence s, first cache row of the sequence and position t; false when the
// descriptor is inconsistent.
__device__ inline bool v1_query(const SeqsDev& b, int i, int& s, int64_t& base, int& t) {
  int lo = (int)(((int64_t)i * b.num_seqs) / max(1, b.total_q));
  if (lo >= b.num_seqs) lo = b.num_seqs - 1;
  if (!(b.q_start[lo] <= i && i < b.q_start[lo + 1])) {
    lo = 0;
    int hi = b.num_seqs - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (b.q_start[mid] <= i) lo = mid; else hi = mid - 1;
    }
  }
  s = lo;
  base = b.kv_start[lo];
  const int n = b.kv_len[lo];
  t = b.q_pos[i];
  const bool ok = b.q_start[lo] <= i && i < b.q_start[lo + 1] && t >= 0 && t < n && base >= 0 &&
                  base + (int64_t)n <= b.total_rows;
  if (!ok) { base = 0; t = 0; }
  return ok;
}

__device__ inline int64_t uniform64(int64_t x) {
  return (int64_t)uniform_u64((uint64_t)x);
}

// Where the keys of one wave's tile list live. Tile `it` holds 32 keys; key kk of it is
//   full:   position p0 + 32 it + kk                        (rows base + p)
//   sparse: position 64 b + 32 (it % 2) + kk, b = block of slot it / 2   (rows base + p)
//   SWA:    position p0 + 32 it + kk, kept in ring slot p mod ring      (rows base + slot)
// and is attended when its position is <= t (and, sparse, the slot holds a block >= 0).
struct TileSrc {
  const __bf16* k;   // K tensor, offset to the wave's KV head
  const __bf16* v;
  int64_t base;
  int t, tb, p0, r0, ring;  // tb = t / 64, the last block with a position <= t
  int bl;            // sparse: lane j holds the block of slot j of the part
};

template <int kMode>
__device__ inline int64_t key_row(const TileSrc& ts, int it, int kk, bool& ok) {
  if constexpr (kMode == kModeFull) {
    const int p = ts.p0 + 32 * it + kk;
    ok = p <= ts.t;
    return ts.base + (ok ? p : 0);
  } else if constexpr (kMode == kModeSparse) {
    const int b = __shfl(ts.bl, it >> 1);
    const bool inb = b >= 0 && b <= ts.tb;  // entries outside the candidate blocks are ignored
    const int p = kV1Block * (inb ? b : 0) + 32 * (it & 1) + kk;
    ok = inb && p <= ts.t;
    return ts.base + (ok ? p : 0);
  } else {
    const int d = 32 * it + kk;  // valid keys: d <= t - p0 < window <= ring
    ok = ts.p0 + d <= ts.t;
    int r = ts.r0 + d;
    r = r >= ts.ring ? r - ts.ring : r;
    return ts.base + (ok ? r : 0);
  }
}

// Mask of the attended keys of tile it (bit kk).
template <int kMode>
__device__ inline uint32_t tile_mask(const TileSrc& ts, int it, int lane) {
  bool ok;
  key_row<kMode>(ts, it, lane & 31, ok);
  return (uint32_t)__ballot(ok);
}

// Enqueues the 32 rows of the K or V tile `it` into LDS in the swizzles of the MQA tiles
// (copy r writes rows 4r .. 4r+3; lane l fills chunk position l%16 of row 4r + l/16).
// Earlier LDS reads of the stage must have completed. The selector pass reads each row
// once (non-temporal copies); the sparse layers gather rows that later layers read again.
template <int kMode, bool kIsK>
__device__ inline void issue_v1(const TileSrc& ts, int it, int lane, uint32_t lds) {
  wait_lgkm0();
  const __bf16* src = kIsK ? ts.k : ts.v;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int kk = r * 4 + (lane >> 4);
    bool ok;
    const int64_t row = key_row<kMode>(ts, it, kk, ok);
    const int chunk = kIsK ? ((lane & 15) ^ (kk & 15)) : v_chunk(kk, lane & 15);
    if constexpr (kMode == kModeFull)
      dma16_nt(src + row * kRowElems + chunk * 8, lds + r * 1024);
    else
      dma16(src + row * kRowElems + chunk * 8, lds + r * 1024);
  }
}

// Online-softmax state of one wave: 16 heads (columns 0..15 of the C layout; columns
// 16..31 carry zero queries and are never written out) x 128 dims.
struct V1Wave {
  f32x16 o[4];  // O^T, dim block mb
  float m;      // running maximum (log2 domain) of head l%32
  float l;      // this lane's share of the denominator of the bf16-rounded P
  float le;     // ... of the unrounded P
  float bs;     // ... of the unrounded P of the current 64-key block
};

// One tile with at least one attended key.
__device__ inline void v1_tile(V1Wave& st, const bf16x8 (&qop)[8], const bf16x8 (&kop)[8],
                               const uint8_t* __restrict__ vt, const uint32_t (&vb)[4], uint32_t vm, float c2,
                               int lane) {
  f32x16 acc = {};
#pragma unroll
  for (int s = 0; s < 8; ++s) acc = mfma(kop[s], qop[s], acc);
  const int hrow = 4 * (lane >> 5);
  float tmax = -INFINITY;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int key = 8 * (j >> 2) + hrow + (j & 3);
    tmax = ((vm >> key) & 1u) ? fmaxf(tmax, acc[j]) : tmax;
  }
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
  const float mnew = fmaxf(st.m, tmax * c2);
  const float alpha = fast_exp2(st.m - mnew);  // 0 on the first tile (m = -inf)
  st.m = mnew;
  st.l *= alpha;
  st.le *= alpha;
  st.bs *= alpha;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int j = 0; j < 16; ++j) st.o[mb][j] *= alpha;

  float p[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) p[j] = fast_exp2(fmaf(acc[j], c2, -mnew));
  if (__builtin_amdgcn_readfirstlane(vm) != 0xffffffffu) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int key = 8 * (j >> 2) + hrow + (j & 3);
      if (!((vm >> key) & 1u)) p[j] = 0.0f;
    }
  }
  // P^T (bf16) as the B operand of the two 16-key steps (the key order of the V^T reads)
  bf16x8 pb[2];
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  float esum = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    pb[j >> 3][j & 7] = (__bf16)p[j];
    esum += p[j];
  }
  float lsum = st.l;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int u = 0; u < 4; ++u)
      lsum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[ks][2 * u], pb[ks][2 * u + 1]}, ones, lsum, false);
  st.l = lsum;
  st.le += esum;
  st.bs += esum;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) st.o[mb] = mfma(read_vt(vt, vb[mb], ks), pb[ks], st.o[mb]);
}

// Selector only: after the last tile of a 64-key block, the block's log2-sum of weights
// per head, m + log2(sum over the block of 2^(x - m)), into the block LSE table.
__device__ inline void block_flush(V1Wave& st, float* __restrict__ dst, int lane) {
  const float tot = st.bs + __shfl_xor(st.bs, 32);
  if (lane < kV1GroupHeads) dst[lane] = st.m + __log2f(tot);
  st.bs = 0.0f;
}

// One tile of the stream with kLater tiles in flight behind it and, when kMore, tile
// it+2 to enqueue into the stage this one frees. Copies are issued K0 V0 K1 V1 ...; the
// waits count the copies issued after the awaited one (stores in between only make the
// waits stricter: loads complete in order).
template <int kMode, int kLater, bool kMore>
__device__ inline void v1_step(V1Wave& st, const TileSrc& ts, const bf16x8 (&qop)[8], float c2, int lane,
                               const uint32_t (&vb)[4], const uint8_t* wst, uint32_t wbase, int it, int ntw,
                               float* blse) {
  const int sidx = it & 1;
  wait_vmcnt<kV1D * (1 + 2 * kLater)>();  // K(it) has landed
  const uint8_t* kt = wst + (2 * sidx) * kTileBytes;
  bf16x8 kop[8];
  read_k(kt, lane, kop);
  const uint32_t vm = tile_mask<kMode>(ts, it, lane);
  if (kMore) issue_v1<kMode, true>(ts, it + 2, lane, wbase + (2 * sidx) * kTileBytes);
  wait_vmcnt<kV1D * (2 * kLater + (kMore ? 1 : 0))>();  // V(it) has landed
  if (vm != 0u) v1_tile(st, qop, kop, kt + kTileBytes, vb, vm, c2, lane);
  if constexpr (kMode == kModeFull) {
    if ((it & 1) || it == ntw - 1) block_flush(st, blse + (it >> 1) * kV1GroupHeads, lane);
  }
  if (kMore) issue_v1<kMode, false>(ts, it + 2, lane, wbase + (2 * sidx + 1) * kTileBytes);
}

template <int kMode>
__device__ inline void v1_stream(V1Wave& st, const TileSrc& ts, int ntw, const bf16x8 (&qop)[8], float c2,
                                 int lane, uint8_t* wst, float* blse) {
  const uint32_t wbase = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)wst);
  uint32_t vb[4];
  vt_bases(lane, vb);
  for (int it = 0; it < min(ntw, kV1Stages); ++it) {
    issue_v1<kMode, true>(ts, it, lane, wbase + (2 * it) * kTileBytes);
    issue_v1<kMode, false>(ts, it, lane, wbase + (2 * it + 1) * kTileBytes);
  }
  int it = 0;
  for (; it + kV1Stages < ntw; ++it) v1_step<kMode, 1, true>(st, ts, qop, c2, lane, vb, wst, wbase, it, ntw, blse);
  if (ntw >= 2) v1_step<kMode, 1, false>(st, ts, qop, c2, lane, vb, wst, wbase, ntw - 2, ntw, blse);
  if (ntw >= 1) v1_step<kMode, 0, false>(st, ts, qop, c2, lane, vb, wst, wbase, ntw - 1, ntw, blse);
}

template <bool kSparse>
__global__ __launch_bounds__(256) void v1_attn_kernel(V1AttnArgs a) {
  __shared__ __align__(16) uint8_t stage[kV1Groups][kV1WaveBytes];
  const int lane = threadIdx.x & 63;
  const int g = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = blockIdx.x / a.n_split;
  const int split = blockIdx.x - i * a.n_split;
  int s, t;
  int64_t base;
  // a position beyond the blocks the parts cover (a kv_len above max_kv_len) is invalid
  const bool valid = __builtin_amdgcn_readfirstlane(v1_query(a.b, i, s, base, t) &&
                                                    (kSparse || t < a.blse_stride * kV1Block));
  if (!valid) return;  // the combine writes this query's NaN outputs
  t = __builtin_amdgcn_readfirstlane(t);
  s = __builtin_amdgcn_readfirstlane(s);
  base = uniform64(base);

  TileSrc ts;
  ts.t = t;
  ts.tb = t / kV1Block;
  ts.base = base;
  ts.k = a.k + g * kDim;
  ts.v = a.v + g * kDim;
  ts.p0 = 0;
  ts.r0 = 0;
  ts.ring = 1;
  ts.bl = -1;
  int ntw;
  int mode;
  if (!kSparse) {
    mode = kModeFull;
    ts.p0 = split * a.split_units * kV1Block;
    if (ts.p0 > t) return;  // beyond the query's keys: the combine does not read this part
    ntw = (min(t + 1, ts.p0 + a.split_units * kV1Block) - ts.p0 + 31) / 32;
  } else if (split < a.n_split - 1) {
    mode = kModeSparse;
    const int s0 = split * a.split_units;
    const int nslot = min(a.split_units, a.top_blocks - s0);
    ts.bl = lane < nslot ? a.blk[((size_t)i * kV1Groups + g) * a.top_blocks + s0 + lane] : -1;
    ntw = 2 * nslot;
  } else {
    mode = kModeSwa;
    ts.p0 = max(0, t - a.window + 1);
    ts.ring = a.swa_slots;
    ts.r0 = ts.p0 % a.swa_slots;
    ts.base = (int64_t)s * a.swa_slots;
    ts.k = a.k_swa + g * kDim;
    ts.v = a.v_swa + g * kDim;
    ntw = (t - ts.p0 + 1 + 31) / 32;
  }

  // Q^T operand of the wave's 16 heads: piece s of lane l = Q[i][16g + l%32][64(l/32) + 8s ..]
  // for l%32 < 16, zero for the padding columns
  bf16x8 qop[8];
  {
    const int h = lane & 31;
    const __bf16* qp = a.q + ((size_t)i * kHeads + kV1GroupHeads * g + min(h, kV1GroupHeads - 1)) * kDim +
                       64 * (lane >> 5);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const bf16x8 x = *reinterpret_cast<const bf16x8*>(qp + 8 * u);
      qop[u] = h < kV1GroupHeads ? x : bf16x8{};
    }
  }
  // the Q and block-list loads complete here, so that no wait for them lands in the loop
  __builtin_amdgcn_s_waitcnt(kWaitVm0);

  float* blse = kSparse ? nullptr
                        : a.blse + (((size_t)i * kV1Groups + g) * a.blse_stride + (size_t)split * a.split_units) *
                                       kV1GroupHeads;
  V1Wave st;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) st.o[mb] = f32x16{};
  st.m = -INFINITY;
  st.l = 0.0f;
  st.le = 0.0f;
  st.bs = 0.0f;
  uint8_t* wst = stage[g];
  if constexpr (!kSparse)
    v1_stream<kModeFull>(st, ts, ntw, qop, a.c2, lane, wst, blse);
  else if (mode == kModeSparse)
    v1_stream<kModeSparse>(st, ts, ntw, qop, a.c2, lane, wst, nullptr);
  else
    v1_stream<kModeSwa>(st, ts, ntw, qop, a.c2, lane, wst, nullptr);

  // partial of (i, g, split): lanes with l%32 < 16 hold head l%32; the two lane halves
  // hold the dims 4(l/32) + 8q .. of each 32-dim block
  const float lt = st.l + __shfl_xor(st.l, 32);
  const float let = st.le + __shfl_xor(st.le, 32);
  V1Partial* P = a.part + ((size_t)i * kV1Groups + g) * a.n_split + split;
  const int h = lane & 31;
  if (h < kV1GroupHeads) {
    if (lane < 32) {
      P->m[h] = st.m;
      P->l[h] = lt;
      P->le[h] = let;
    }
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int d = 32 * mb + 8 * q + 4 * (lane >> 5);
        *reinterpret_cast<float4*>(&P->o[h][d]) =
            float4{st.o[mb][4 * q], st.o[mb][4 * q + 1], st.o[mb][4 * q + 2], st.o[mb][4 * q + 3]};
      }
  }
}

// ------------------------------------------------------------------------------------
// Selector combine and block selection. Workgroup (i, g): merges the parts of query i
// for the 16 heads of KV head g (output and LSE), then scores every candidate block,
// score[b] = sum over the heads of 2^(block LSE - head LSE), and keeps the top_blocks
// best (ties to the smaller index), written ascending and padded with -1.
// ------------------------------------------------------------------------------------

__device__ inline int wave_sum(int x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d);
  return x;
}

// Sum over the workgroup (256 threads); `slot` holds 4 ints no other thread reads or
// writes between this call's barrier and the next call's barrier on the same slot.
__device__ inline int block_sum(int x, int* slot) {
  x = wave_sum(x);
  if ((threadIdx.x & 63) == 0) slot[threadIdx.x >> 6] = x;
  __syncthreads();
  return (slot[0] + slot[1]) + (slot[2] + slot[3]);
}

// Exclusive prefix sum over the workgroup in thread order.
__device__ inline int block_exscan(int x, int* slot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int v = x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(v, d);
    if (lane >= d) v += y;
  }
  if (lane == 63) slot[wave] = v;
  __syncthreads();
  int off = 0;
  for (int w = 0; w < wave; ++w) off += slot[w];
  return off + v - x;
}

__global__ __launch_bounds__(256) void v1_select_kernel(V1SelectArgs a) {
  extern __shared__ float sc[];  // [blse_stride] block scores
  __shared__ float lse2_s[kV1GroupHeads];
  __shared__ int red[2][4];
  __shared__ int red2[4], scan1[4], scan2[4];
  const int i = blockIdx.x / kV1Groups;
  const int g = blockIdx.x - i * kV1Groups;
  const int tid = threadIdx.x;
  const int h = tid & 15, dg = tid >> 4;
  int s, t;
  int64_t base;
  const bool valid = v1_query(a.b, i, s, base, t) && t < a.blse_stride * kV1Block;
  __bf16* out = a.out + ((size_t)i * kHeads + kV1GroupHeads * g + h) * kDim + 8 * dg;
  int32_t* bi = a.blk_idx + ((size_t)i * kV1Groups + g) * a.top_blocks;
  if (!valid) {
    bf16x8 nanv;
#pragma unroll
    for (int r = 0; r < 8; ++r) nanv[r] = (__bf16)NAN;
    *reinterpret_cast<bf16x8*>(out) = nanv;
    if (dg == 0 && a.lse) a.lse[(size_t)i * kHeads + kV1GroupHeads * g + h] = NAN;
    for (int e = tid; e < a.top_blocks; e += 256) bi[e] = -1;
    if (tid == 0 && a.blk_count) a.blk_count[(size_t)i * kV1Groups + g] = -1;
    return;
  }
  const int nblk = t / kV1Block + 1;
  const int nv = (nblk + a.split_units - 1) / a.split_units;
  const V1Partial* P = a.part + ((size_t)i * kV1Groups + g) * a.n_split;
  float M = -INFINITY;
  for (int p = 0; p < nv; ++p) M = fmaxf(M, P[p].m[h]);
  float L = 0.0f, LE = 0.0f;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int p = 0; p < nv; ++p) {
    const float w = fast_exp2(P[p].m[h] - M);
    L += P[p].l[h] * w;
    LE += P[p].le[h] * w;
    const float4 x0 = *reinterpret_cast<const float4*>(&P[p].o[h][8 * dg]);
    const float4 x1 = *reinterpret_cast<const float4*>(&P[p].o[h][8 * dg + 4]);
    acc[0] += x0.x * w; acc[1] += x0.y * w; acc[2] += x0.z * w; acc[3] += x0.w * w;
    acc[4] += x1.x * w; acc[5] += x1.y * w; acc[6] += x1.z * w; acc[7] += x1.w * w;
  }
  {
    const float inv = 1.0f / L;
    bf16x8 ov;
#pragma unroll
    for (int r = 0; r < 8; ++r) ov[r] = (__bf16)(acc[r] * inv);
    *reinterpret_cast<bf16x8*>(out) = ov;
  }
  if (dg == 0) {
    const float l2 = M + __log2f(LE);
    lse2_s[h] = l2;
    if (a.lse) a.lse[(size_t)i * kHeads + kV1GroupHeads * g + h] = l2 * kLn2;
  }
  __syncthreads();

  const int K = a.top_blocks;
  int32_t* cnt = a.blk_count ? a.blk_count + (size_t)i * kV1Groups + g : nullptr;
  if (nblk <= K) {  // every block is kept
    for (int e = tid; e < K; e += 256) bi[e] = e < nblk ? e : -1;
    if (tid == 0 && cnt) *cnt = nblk;
    return;
  }
  const float* B = a.blse + ((size_t)i * kV1Groups + g) * a.blse_stride * kV1GroupHeads;
  for (int b = tid; b < nblk; b += 256) {
    const float4* x = reinterpret_cast<const float4*>(B + (size_t)b * kV1GroupHeads);
    float v = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 y = x[q];
      v += fast_exp2(y.x - lse2_s[4 * q]);
      v += fast_exp2(y.y - lse2_s[4 * q + 1]);
      v += fast_exp2(y.z - lse2_s[4 * q + 2]);
      v += fast_exp2(y.w - lse2_s[4 * q + 3]);
    }
    sc[b] = v >= 0.0f ? v : 0.0f;  // a NaN score (from NaN inputs) ranks as zero
  }
  __syncthreads();

  // the K-th largest score: the largest bit pattern T with #{score >= T} >= K (scores are
  // non-negative, so their bit patterns order as the values)
  const int per = (nblk + 255) / 256;
  const int lo = min(nblk, tid * per), hi = min(nblk, lo + per);
  uint32_t T = 0;
  for (int bit = 30; bit >= 0; --bit) {
    const uint32_t cand = T | (1u << bit);
    int c = 0;
    for (int b = lo; b < hi; ++b) c += __float_as_uint(sc[b]) >= cand ? 1 : 0;
    if (block_sum(c, red[bit & 1]) >= K) T = cand;
  }
  int ngt = 0, neq = 0;
  for (int b = lo; b < hi; ++b) {
    const uint32_t u = __float_as_uint(sc[b]);
    ngt += u > T ? 1 : 0;
    neq += u == T ? 1 : 0;
  }
  const int need = K - block_sum(ngt, red2);  // >= 1 blocks equal to T, smallest indices first
  const int eq0 = block_exscan(neq, scan1);
  int eqr = eq0;
  int nsel = 0;
  for (int b = lo; b < hi; ++b) {
    const uint32_t u = __float_as_uint(sc[b]);
    const bool take = u > T || (u == T && eqr < need);
    eqr += u == T ? 1 : 0;
    nsel += take ? 1 : 0;
  }
  int pos = block_exscan(nsel, scan2);
  eqr = eq0;
  for (int b = lo; b < hi; ++b) {
    const uint32_t u = __float_as_uint(sc[b]);
    const bool take = u > T || (u == T && eqr < need);
    eqr += u == T ? 1 : 0;
    if (take && pos < K) bi[pos++] = b;
  }
  if (tid == 0 && cnt) *cnt = K;
}

// ------------------------------------------------------------------------------------
// Sparse-layer combine: per (query, KV head), the block-slot parts merge into the
// selected-block branch, the last part is the window branch, and
//   out_h = gate_sparse[h] * O_sparse,h + gate_swa[h] * O_swa,h
// A branch without attended keys contributes zero.
// ------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void v1_gate_kernel(V1GateArgs a) {
  const int i = blockIdx.x / kV1Groups;
  const int g = blockIdx.x - i * kV1Groups;
  const int tid = threadIdx.x;
  const int h = tid & 15, dg = tid >> 4;
  int s, t;
  int64_t base;
  const bool valid = v1_query(a.b, i, s, base, t);
  const int hq = kV1GroupHeads * g + h;
  __bf16* out = a.out + ((size_t)i * kHeads + hq) * kDim + 8 * dg;
  if (!valid) {
    bf16x8 nanv;
#pragma unroll
    for (int r = 0; r < 8; ++r) nanv[r] = (__bf16)NAN;
    *reinterpret_cast<bf16x8*>(out) = nanv;
    return;
  }
  const V1Partial* P = a.part + ((size_t)i * kV1Groups + g) * a.n_split;
  const int nsp = a.n_split - 1;
  float M = -INFINITY;
  for (int p = 0; p < nsp; ++p) M = fmaxf(M, P[p].m[h]);
  float L = 0.0f;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (M != -INFINITY) {
    for (int p = 0; p < nsp; ++p) {
      const float w = fast_exp2(P[p].m[h] - M);  // 0 for a part without keys
      L += P[p].l[h] * w;
      const float4 x0 = *reinterpret_cast<const float4*>(&P[p].o[h][8 * dg]);
      const float4 x1 = *reinterpret_cast<const float4*>(&P[p].o[h][8 * dg + 4]);
      acc[0] += x0.x * w; acc[1] += x0.y * w; acc[2] += x0.z * w; acc[3] += x0.w * w;
      acc[4] += x1.x * w; acc[5] += x1.y * w; acc[6] += x1.z * w; acc[7] += x1.w * w;
    }
  }
  const float gs = a.gate_sparse[(size_t)i * kHeads + hq];
  const float gw = a.gate_swa[(size_t)i * kHeads + hq];
  const float fs = L > 0.0f ? gs / L : 0.0f;
  const V1Partial& W = P[nsp];
  const float fw = gw / W.l[h];
  const float4 y0 = *reinterpret_cast<const float4*>(&W.o[h][8 * dg]);
  const float4 y1 = *reinterpret_cast<const float4*>(&W.o[h][8 * dg + 4]);
  const float yv[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
  bf16x8 ov;
#pragma unroll
  for (int r = 0; r < 8; ++r) ov[r] = (__bf16)(acc[r] * fs + yv[r] * fw);
  *reinterpret_cast<bf16x8*>(out) = ov;
}

}  // namespace

hipError_t launch_v1_attn(const V1AttnArgs& a, bool sparse, int grid, hipStream_t s) {
  if (sparse)
    hipLaunchKernelGGL(v1_attn_kernel<true>, dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(v1_attn_kernel<false>, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_v1_select(const V1SelectArgs& a, hipStream_t s) {
  const size_t lds = (size_t)a.blse_stride * sizeof(float);
  static bool attr_set = false;  // the attribute is per function; setting it twice is harmless
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute((const void*)v1_select_kernel,
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (kV1MaxBlocks + kMaxV1Split) * (int)sizeof(float));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(v1_select_kernel, dim3(a.b.total_q * kV1Groups), dim3(256), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_v1_gate(const V1GateArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(v1_gate_kernel, dim3(a.b.total_q * kV1Groups), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace hs2
