// Host-side declarations of libhs2: the kernel launchers (defined next to their kernels)
// and the helpers the entry points share.
#pragma once

#include "hs2_internal.h"
#include "v1_internal.h"

namespace hs2 {

// Waves per workgroup of the decode-shaped score pass (4 for bf16 tiles, 8 for FP8 tiles).
// Each wave keeps its own candidate list, so the kernel's launch shape and the planner's
// list area are both sized from this one value.
constexpr int score_waves(bool fp8) { return fp8 ? 8 : 4; }

// Sets the calling thread's hs2_last_error() text and returns st (for entry points
// defined outside hs2_api.cpp).
hs2_status set_error(hs2_status st, const char* msg);

// Every argument check of hs2_sparse_attn except the workspace's (sets hs2_last_error).
hs2_status sparse_check(const hs2_seqs* batch, const void* q, const void* k, const void* v, const int32_t* sel_idx,
                        int32_t n_heads, int32_t head_dim, int32_t window, int32_t top_k, float scale,
                        const void* out, const float* lse, hs2_dtype dt);

// ---------------------------------------------------------------------------------
// Host-side launchers (defined next to their kernels).
// ---------------------------------------------------------------------------------
hipError_t launch_attn_bf16(const AttnArgs& a, const WorkList& wl, int grid, uint32_t* hist, uint32_t* counters,
                            hipStream_t s);
hipError_t launch_attn_fp8kv(const AttnArgs& a, const WorkList& wl, int grid, uint32_t* hist, uint32_t* counters,
                             hipStream_t s);
hipError_t launch_attn_f32(const AttnArgs& a, bool gather, int grid, uint32_t* hist,
                           uint32_t* counters, hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, bool f32, hipStream_t s);
hipError_t launch_sparse_attn(const AttnArgs& a, bool fp8, bool narrow, int grid, hipStream_t s);
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
// Output form of the bridging GEMM: bf16 rows, or (fp8 set) OCP E4M3 codes of
// min(max(value * inv_scale[m], -448), 448) for output matrix m, rows of 128 bytes.
struct BridgeOut {
  int32_t fp8;
  float inv_scale[16];
};
hipError_t launch_bridge_gemm(const BridgeArgs& a, const BridgeOut& o, hipStream_t s);
hipError_t launch_bridge_append(const AppendArgs& a, const BridgeOut& o, hipStream_t s);

hipError_t launch_v1_attn(const V1AttnArgs& a, bool sparse, int grid, hipStream_t s);
hipError_t launch_v1_select(const V1SelectArgs& a, hipStream_t s);
hipError_t launch_v1_gate(const V1GateArgs& a, hipStream_t s);

}  // namespace hs2
