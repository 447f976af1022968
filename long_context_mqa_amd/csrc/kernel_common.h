// Device helpers shared by the kernels of libhs2: work items, the descriptor of a query,
// the direct-to-LDS copy and the logical key count of a query.
#pragma once

#include "hs2_internal.h"

namespace hs2 {

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

// A work list is planned from the host's copy of the sequence lengths: query i gets the
// splits 0 .. n_i-1 (at least one), listed in split order. The workgroup of the last of
// them tells whether the query's keys on the device end within its range; if not (the
// host copy was smaller than the device lengths), the splits beyond were never launched
// and the query is reported as inconsistent by the kernels that read its partials.
__device__ inline bool last_planned(const WorkList& wl, int i) {
  const int b = (int)blockIdx.x;
  return b + 1 >= wl.n || (int)(wl.item[b + 1] >> 9) != i;
}

// Resolves query i: sequence row base and position t. Returns false when the
// descriptor is inconsistent (the query is then not computed), which includes a position
// at or beyond max_kv_len: the key splits and score rows are sized from that bound. The
// sequence is first guessed proportionally (exact for batches with equal query counts per
// sequence) and every value of that guess is loaded at once, so that the common case
// costs one round of loads; a wrong guess is corrected by binary search over q_start.
__device__ inline bool query_desc(const SeqsDev& b, int i, int64_t& base, int& t) {
  // the query index must name a row of Q, and q_start must run from 0 to total_q (a
  // q_start beyond total_q would otherwise map a kernel's query onto rows past the
  // caller's Q, out, LSE and selection buffers)
  if (i < 0 || i >= b.total_q) {
    base = 0;
    t = 0;
    return false;
  }
  int lo = (int)(((int64_t)i * b.num_seqs) / max(1, b.total_q));
  if (lo >= b.num_seqs) lo = b.num_seqs - 1;
  const int qs0 = b.q_start[0], qsn = b.q_start[b.num_seqs];
  int ql = b.q_start[lo], qh = b.q_start[lo + 1];
  base = b.kv_start[lo];
  int n = b.kv_len[lo];
  t = b.q_pos[i];
  if (!(ql <= i && i < qh)) {
    lo = 0;
    int hi = b.num_seqs - 1;
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (b.q_start[mid] <= i) lo = mid; else hi = mid - 1;
    }
    ql = b.q_start[lo];
    qh = b.q_start[lo + 1];
    base = b.kv_start[lo];
    n = b.kv_len[lo];
  }
  const bool ok = qs0 == 0 && qsn == b.total_q && ql <= i && i < qh && t >= 0 && t < n && t < b.max_kv_len &&
                  base >= 0 && base + (int64_t)n <= b.total_rows;
  if (!ok) { base = 0; t = 0; }
  return ok;
}

// A wave-uniform 64-bit value moved to scalar registers, half by half. readfirstlane
// returns a signed int, so each half goes back through uint32_t before it is widened: a low
// half with bit 31 set would otherwise sign-extend over the high half.
__device__ inline uint64_t uniform_u64(uint64_t x) {
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(x >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)x);
  return ((uint64_t)hi << 32) | (uint64_t)lo;
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

// The same copy marked non-temporal, for data read once (the decode passes' K/V stream):
// the caches keep these lines only briefly, leaving room for what is read again. On the
// 64 x 131,072 decode batch it took a selector call from 1,126 to 1,029 us.
__device__ inline void dma16_nt(const void* g, uint32_t lds) {
  lds = __builtin_amdgcn_readfirstlane(lds);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off nt\n\t"
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

}  // namespace hs2
