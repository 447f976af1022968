// Internal declarations shared by the HIP kernels and the host entry points of libhs2.
// Target: gfx950 (MI355X) only: 64-lane wavefronts, bf16 MFMA 32x32x16.
#pragma once

#include <hip/hip_runtime.h>

#include "hs2.h"
#include <stddef.h>
#include <stdint.h>

namespace hs2 {

constexpr int kHeads = 64;     // query heads sharing the single KV head (MQA 64:1)
constexpr int kDim = 128;      // head_dim
constexpr int kTile = 32;      // keys per MFMA tile (one 32x32 output block)
constexpr int kWaves = 4;      // waves per attention workgroup
constexpr int kHistBits = 12;  // first radix digit: bits 30..19 of a non-negative fp32 score
constexpr int kHistBins = 1 << kHistBits;
constexpr int kHistShift = 31 - kHistBits;
constexpr int kCandCap = 4096; // threshold-bin candidates kept per query for the in-LDS select
constexpr int kQTile = 8;      // queries per q-tile of the chunked selector (one wave each)
constexpr int kScoreSplitMax = 32768;  // keys per chunked score workgroup (16-bit LDS bin counts)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Device view of the ragged batch descriptor.
struct SeqsDev {
  const int64_t* kv_start;
  const int32_t* kv_len;
  const int32_t* q_start;
  const int32_t* q_pos;
  int32_t num_seqs;
  int32_t total_q;
  int64_t total_rows;
  int32_t max_kv_len;  // the host's bound of every kv_len, which sizes splits and score rows
};

// Partial result of one workgroup's key range for one query: running max m (log2
// domain), the softmax denominator summed from the probabilities as rounded for the
// P.V product (l, normalises the output) and from the unrounded probabilities (le, gives
// the LSE), and the unnormalised output transposed to [dim][head].
struct Partial {
  float m[kHeads];
  float l[kHeads];
  float le[kHeads];
  float o[kDim * kHeads];
};

// Arguments of the attention kernels (full causal range, or gathered window + selection).
struct AttnArgs {
  SeqsDev b;
  const void* q;          // [total_q][64][128]
  const void* k;          // [rows][128]
  const void* v;          // [rows][128]
  const int32_t* sel;     // gather mode: [total_q][top_k]
  int32_t window;
  int32_t top_k;
  float c2;               // softmax scale * log2(e)
  int32_t n_split;        // workgroups per query
  int32_t split_keys;     // logical keys per workgroup (multiple of kTile)
  Partial* part;          // [total_q][n_split] when n_split > 1
  void* out;              // [total_q][64][128] when n_split == 1
  float* lse;             // [total_q][64] natural log, nullable (n_split == 1)
  float* lse2;            // [total_q][64] log2 domain, nullable (n_split == 1)
  float v_scale;          // output factor (the V scale of FP8 storage; 1 otherwise)
  int32_t direct;         // q-tile kernel with n_split == 1: write out/lse itself (no partials)
};

// (query, split) pairs of a launch in launch order: workgroup b takes item b, so that the
// active pairs fill the XCDs (b % 8) evenly and no workgroup is launched without work.
// n == 0: the grid is total_q x n_split in query-major order.
constexpr int kMaxWorkItems = 512;
struct WorkList {
  int32_t n;
  uint32_t item[kMaxWorkItems];  // query << 9 | split (split < 512)
};

__device__ inline void work_item(const WorkList& wl, int n_split, int& i, int& split) {
  if (wl.n > 0) {
    const uint32_t it = wl.item[blockIdx.x];
    i = (int)(it >> 9);
    split = (int)(it & 511u);
  } else {
    i = blockIdx.x / n_split;
    split = blockIdx.x - i * n_split;
  }
}

struct CombineArgs {
  SeqsDev b;
  const Partial* part;
  int32_t n_split;
  int32_t split_keys;
  int32_t gather;         // logical key count: t+1 (full) or window+top_k (gather)
  int32_t window;
  int32_t top_k;
  void* out;
  float* lse;             // nullable
  float* lse2;            // nullable
  uint32_t* hist;         // nullable: [total_q][kHistBins] zeroed here for the score pass
  uint32_t* counters;     // nullable: [total_q][4] zeroed here
  float v_scale;          // output factor (the V scale of FP8 storage; 1 otherwise)
};

struct ScoreArgs {
  SeqsDev b;
  const void* q;
  const void* k;
  const float* lse2;      // [total_q][64]
  float c2;
  int32_t window;
  int32_t top_k;
  int32_t n_split;
  int32_t split_keys;
  int64_t score_stride;   // floats per query in `scores`
  float* scores;          // [total_q][score_stride]
  uint32_t* hist;         // [total_q][kHistBins]
};

struct TopkArgs {
  SeqsDev b;
  int32_t window;
  int32_t top_k;
  int32_t n_split;        // filter workgroups per query
  int32_t split_len;      // candidates per filter workgroup
  int64_t score_stride;
  const float* scores;
  const uint32_t* hist;
  uint32_t* counters;     // [total_q][4]: 0 = above count, 1 = threshold-bin count
  int32_t* above;         // [total_q][top_k]
  uint2* cand;            // [total_q][kCandCap]: (score bits, position)
  int32_t* sel_idx;       // [total_q][top_k]
  int32_t* sel_count;     // nullable
};

struct BridgeArgs {
  const uint16_t* h;      // [n_rows][d_model]
  const uint16_t* wt;     // [n_mats][128][d_model]  (transposed weights, workspace)
  uint16_t* outs[16];     // n_mats output matrices [n_rows][128]
  int64_t n_rows;
  int32_t d_model;
  int32_t n_mats;
};

// Decode-time KV Bridging: the new tokens' hidden states through every bridged layer's
// projections, written into the caches at the tokens' rows.
constexpr int kAppendSlice = 128;  // contraction depth of one partial workgroup
struct AppendArgs {
  const uint16_t* h;       // [n_new][d_model] bf16
  const int64_t* rows;     // device [n_new]: cache row of each new token
  const uint16_t* w[16];   // n_mats weights [d_model][128] bf16 (K of layer l at 2l, V at 2l+1)
  uint16_t* outs[16];      // n_mats caches [cache_rows][128] bf16
  float* part;             // [n_slices][n_new][n_mats * 128] fp32 partial sums
  int64_t cache_rows;
  int32_t n_new;
  int32_t d_model;
  int32_t n_mats;
  int32_t n_slices;        // d_model / kAppendSlice
};

// Resolves query i: sequence row base and position t. Returns false when the
// descriptor is inconsistent (the query is then not computed), which includes a position
// at or beyond max_kv_len: the key splits and score rows are sized from that bound. The sequence is first
// guessed proportionally (exact for batches with equal query counts per sequence), and
// found by binary search over q_start otherwise.
__device__ inline bool query_desc(const SeqsDev& b, int i, int64_t& base, int& t) {
  int lo = (int)(((int64_t)i * b.num_seqs) / max(1, b.total_q));
  if (lo >= b.num_seqs) lo = b.num_seqs - 1;
  if (!(b.q_start[lo] <= i && i < b.q_start[lo + 1])) {
    lo = 0;
    int hi = b.num_seqs - 1;
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (b.q_start[mid] <= i) lo = mid; else hi = mid - 1;
    }
  }
  base = b.kv_start[lo];
  const int n = b.kv_len[lo];
  t = b.q_pos[i];
  const bool ok = b.q_start[lo] <= i && i < b.q_start[lo + 1] && t >= 0 && t < n && t < b.max_kv_len &&
                  base >= 0 && base + (int64_t)n <= b.total_rows;
  if (!ok) { base = 0; t = 0; }
  return ok;
}

// One wave-wide 16-byte-per-lane copy from global memory straight into LDS: lane l's
// 16 bytes land at LDS byte address `lds` + 16*l (`lds` must be wave-uniform). Issued as
// asm so that the wait for it can be placed by hand with s_waitcnt vmcnt (the compiler
// otherwise waits for every pending LDS copy before any LDS read). The asm has no
// register results; M0, which holds the LDS address, is saved and restored around it.
__device__ inline void dma16(const void* g, uint32_t lds) {
  lds = __builtin_amdgcn_readfirstlane(lds);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0\n"
      : "=&s"(saved)
      : "v"(g), "s"(lds)
      : "memory");
}

// Number of logical keys of a query: t+1 (full causal) or top_k + min(window, t+1)
// (gather: selected slots first, then the window rows oldest first).
__device__ inline int logical_keys(bool gather, int t, int window, int top_k) {
  return gather ? top_k + min(window, t + 1) : t + 1;
}

// ---------------------------------------------------------------------------------
// Host-side launchers (defined next to their kernels).
// ---------------------------------------------------------------------------------
hipError_t launch_attn_bf16(const AttnArgs& a, const WorkList& wl, bool gather, int grid, uint32_t* hist,
                            uint32_t* counters, hipStream_t s);
hipError_t launch_attn_fp8kv(const AttnArgs& a, const WorkList& wl, bool gather, int grid, uint32_t* hist,
                             uint32_t* counters, hipStream_t s);
hipError_t launch_attn_f32(const AttnArgs& a, bool gather, int grid, uint32_t* hist,
                           uint32_t* counters, hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, bool f32, hipStream_t s);
hipError_t launch_qtile_prep(const SeqsDev& b, int2* tiles, int max_tiles, hipStream_t s);
hipError_t launch_attn_chunk(const AttnArgs& a, const int2* tiles, int max_tiles, hipStream_t s);
hipError_t launch_score_chunk(const ScoreArgs& a, const int2* tiles, int max_tiles, hipStream_t s);
hipError_t launch_score_bf16(const ScoreArgs& a, const WorkList& wl, hipStream_t s);
hipError_t launch_score_fp8kv(const ScoreArgs& a, const WorkList& wl, hipStream_t s);
hipError_t launch_score_f32(const ScoreArgs& a, hipStream_t s);
hipError_t launch_topk_filter(const TopkArgs& a, hipStream_t s);
hipError_t launch_topk_finish(const TopkArgs& a, hipStream_t s);
hipError_t launch_bridge_transpose(const BridgeArgs& a, const uint16_t* const* w, int32_t n_mats,
                                   uint16_t* wt, hipStream_t s);
hipError_t launch_bridge_gemm(const BridgeArgs& a, hipStream_t s);
hipError_t launch_bridge_append(const AppendArgs& a, hipStream_t s);

}  // namespace hs2
