// Internal declarations of the first-generation HySparse layout (the comparison variant):
// GQA with 4 KV heads of 16 query heads each, selection of 64-token blocks per KV head,
// and sparse layers that fuse a selected-block branch with a sliding-window branch on
// their own K/V through per-head gates.
#pragma once

#include "hs2_internal.h"

namespace hs2 {

constexpr int kV1Groups = 4;        // KV heads
constexpr int kV1GroupHeads = 16;   // query heads per KV head
constexpr int kV1Block = 64;        // positions per selection block
constexpr int kV1MaxTopBlocks = 64; // bound of the blocks kept per query and KV head
constexpr int kV1MaxBlocks = 32768; // bound of the blocks of one sequence (2^21 positions)

// Partial result of one (query, KV head, part): running maximum m (log2 domain), the
// denominators of the bf16-rounded (l) and unrounded (le) probabilities, and the
// unnormalised output of the 16 heads.
struct V1Partial {
  float m[kV1GroupHeads];
  float l[kV1GroupHeads];
  float le[kV1GroupHeads];
  float pad[kV1GroupHeads];
  float o[kV1GroupHeads][kDim];
};

struct V1AttnArgs {
  SeqsDev b;
  const __bf16* q;        // [total_q][64][128]
  const __bf16* k;        // [total_rows][4][128]
  const __bf16* v;        // [total_rows][4][128]
  const __bf16* k_swa;    // sparse: [num_seqs][swa_slots][4][128]
  const __bf16* v_swa;
  int32_t swa_slots;
  int32_t window;
  const int32_t* blk;     // sparse: [total_q][4][top_blocks]
  int32_t top_blocks;
  float c2;               // softmax scale * log2(e)
  int32_t n_split;        // parts per query (sparse: block-slot parts, then the window part)
  int32_t split_units;    // blocks (selector) or block slots (sparse) per part
  V1Partial* part;        // [total_q][4][n_split]
  float* blse;            // selector: [total_q][4][blse_stride][16], log2-domain block LSEs
  int32_t blse_stride;
};

struct V1SelectArgs {
  SeqsDev b;
  const V1Partial* part;
  int32_t n_split;
  int32_t split_units;
  const float* blse;
  int32_t blse_stride;
  __bf16* out;            // [total_q][64][128]
  float* lse;             // [total_q][64] natural log, nullable
  int32_t* blk_idx;       // [total_q][4][top_blocks]
  int32_t* blk_count;     // [total_q][4], nullable
  int32_t top_blocks;
};

struct V1GateArgs {
  SeqsDev b;
  const V1Partial* part;
  int32_t n_split;        // block-slot parts + 1 (the window part, last)
  const float* gate_sparse;  // [total_q][64]
  const float* gate_swa;     // [total_q][64]
  __bf16* out;               // [total_q][64][128]
};

}  // namespace hs2
