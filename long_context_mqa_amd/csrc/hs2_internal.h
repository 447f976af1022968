// Internal declarations shared by the HIP kernels and the host entry points of libhs2:
// constants and kernel argument structs. The launchers and host helpers are declared in
// hs2_launch.h, the device helpers in kernel_common.h.
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
constexpr int kSparseStageBytes = 147456;  // LDS of a sparse-layer workgroup's K/V tile slots
constexpr int kSparseNarrowBytes = 65536;  // ... in the narrow form (batches of many queries)
// K/V tiles (32 rows each) a sparse-layer workgroup holds in LDS at once
constexpr int sparse_slots(bool fp8) { return kSparseStageBytes / (2 * kTile * kDim * (fp8 ? 1 : 2)); }
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
  int32_t* plan_miss;     // work-list launches: [total_q], 1 if query i's keys run past its
                          // planned splits (written by the last planned split), else 0
};

// (query, split) pairs of a launch in launch order: workgroup b takes item b, so that the
// active pairs fill the XCDs (b % 8) evenly and no workgroup is launched without work.
// n == 0: the grid is total_q x n_split in query-major order.
constexpr int kMaxWorkItems = 512;
struct WorkList {
  int32_t n;
  uint32_t item[kMaxWorkItems];  // query << 9 | split (split < 512)
};

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
  const int32_t* plan_miss;  // nullable: the attention launch's plan-miss flags
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
  float* scores;          // q-tile and fp32 kernels: [total_q][score_stride]
  uint32_t* hist;         // [total_q][kHistBins]
  int32_t* plan_miss;     // work-list launches: [total_q] plan-miss flags of the score pass
  // decode-shaped bf16 and FP8 kernels: candidate lists instead of score rows
  uint2* lists;           // [total_q][n_split][waves][list_cap]: (score bits, position)
  int32_t* list_count;    // [total_q][n_split][waves]: entries of each list
  int32_t* list_thr;      // [total_q][n_split]: the split's final threshold (first digit)
  int32_t list_cap;
};

struct TopkArgs {
  SeqsDev b;
  int32_t window;
  int32_t top_k;
  int32_t n_split;        // filter workgroups per query
  int32_t split_len;      // candidates per filter workgroup
  int64_t score_stride;
  const float* scores;    // score rows (null when the score pass wrote candidate lists)
  const uint2* lists;     // candidate lists of the score pass (see ScoreArgs), or null
  const int32_t* list_count;
  const int32_t* list_thr;
  int32_t list_cap;
  int32_t list_waves;     // lists per score split
  int32_t list_splits;    // score splits per query
  int32_t list_split_keys;  // candidates per score split
  const uint32_t* hist;
  uint32_t* counters;     // [total_q][4]: 0 = above count, 1 = threshold-bin count
  int32_t* above;         // [total_q][top_k]
  uint2* cand;            // [total_q][kCandCap]: (score bits, position)
  int32_t* sel_idx;       // [total_q][top_k]
  int32_t* sel_count;     // nullable
  const int32_t* miss_attn;   // nullable: plan-miss flags of the attention launch
  const int32_t* miss_score;  // nullable: plan-miss flags of the score launch
  void* out;              // with the flags: outputs of a missed query are set to NaN
  float* lse;             // nullable
  int32_t out_f32;        // out holds fp32 (else bf16)
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

}  // namespace hs2
