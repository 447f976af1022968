// FP8 (OCP E4M3) K/V instantiation of the decode-shaped attention kernel (attn_decode.h):
// eight waves per workgroup, two per SIMD, each streaming its own 4 KB tiles through two
// LDS stages. FP8 tiles carry half the bytes of bf16 tiles for the same matrix and vector
// work, so one wave per SIMD leaves its per-tile chain (LDS reads, conversion, MFMA,
// exp2, MFMA) exposed; with two, one wave's vector work runs under the other's MFMAs.
// Built with the MFMA results in VGPRs: the kernel fits the 256 registers of two waves
// per SIMD only without accumulator registers.
//
// Method (page title and section): arex-research.com, "Xiaomi MiMo lead Luo Fuli
// publishes the MiMo-V3 core architecture HySparse2", section "Numbers computed on three
// 80B-A3B models": the KV cache is accounted in FP8.
#include "attn_decode.h"
#include "hs2_launch.h"

namespace hs2 {

// The selector's pass 1 over an FP8 cache (the sparse layers' FP8 attention is in
// sparse_attn.hip).
hipError_t launch_attn_fp8kv(const AttnArgs& a, const WorkList& wl, int grid, uint32_t* hist, uint32_t* counters,
                             hipStream_t s) {
  hipLaunchKernelGGL((attn_bf16_kernel<KvFp8, 8>), dim3(grid), dim3(512), 0, s, a, wl, hist, counters);
  return hipGetLastError();
}

}  // namespace hs2
