// Host entry points of libhs2: argument checks, workspace planning and kernel launches.
// Every check runs before anything is enqueued; the library allocates nothing.
#include <algorithm>
#include <cmath>
#include <limits>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "hs2.h"
#include "hs2_launch.h"


namespace {

using namespace hs2;

thread_local std::string g_err;

hs2_status fail(hs2_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

hs2_status ok() {
  g_err.clear();
  return HS2_OK;
}

}  // namespace

namespace hs2 {
hs2_status set_error(hs2_status st, const char* msg) {
  g_err = msg;
  return st;
}
}  // namespace hs2

namespace {

constexpr size_t kAlign = 256;
constexpr int kTargetGroups = 256;  // workgroups per launch: one per CU
constexpr int kMaxSplit = 256;      // bound of the split combine
constexpr int kSparseSplitMax = 2048;
constexpr int kChunkMinQueries = 8;   // queries per sequence from which K/V tiles are shared  // keys per sparse workgroup (LDS row list)
constexpr int kFilterLen = 8192;    // candidates per top-k filter workgroup (256 threads x 32)

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
bool aligned(const void* p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

struct Split {
  int n_split;
  int split_keys;
};

// Splits the logical key range [0, max_keys) of each query over workgroups so that the
// launch fills the GPU once (kTargetGroups workgroups of work, one per CU at the LDS
// size of the attention and score kernels). `work` estimates the keys of the whole
// launch; splits are multiples of one 32-key tile. Workgroups beyond a query's own
// range exit at once.
Split plan_split(int64_t work, int64_t max_keys) {
  Split s;
  if (max_keys <= 0) return Split{1, kTile};
  int64_t keys = std::max<int64_t>(ceil_div(std::max<int64_t>(work, 1), kTargetGroups), ceil_div(max_keys, kMaxSplit));
  keys = ceil_div(keys, kTile) * kTile;
  s.split_keys = (int)std::min<int64_t>(keys, ceil_div(max_keys, kTile) * kTile);
  s.n_split = (int)ceil_div(max_keys, s.split_keys);
  return s;
}

// Split of ragged single-query sequences from their host lengths: the smallest split
// (a multiple of one tile) whose active workgroups, sum over sequences of
// ceil(keys_s / split), fit one round of kTargetGroups; or two rounds, if their total is
// at least 10% shorter (each round adds its own prologue, merge and partial writes).
// keys_s = n_s - sub (clamped at 0).
bool plan_split_lengths(const hs2_seqs* b, int64_t sub, int64_t max_keys, Split& out, WorkList* wl) {
  if (!b->kv_len_host || b->max_q_per_seq > 1 || max_keys <= 0) return false;
  // every query gets at least one workgroup: the one that reports a length beyond the plan
  auto splits_of = [&](int s, int64_t sk) {
    const int64_t k = std::max<int64_t>(0, (int64_t)b->kv_len_host[s] - sub);
    return std::max<int64_t>(1, ceil_div(k, sk));
  };
  auto active = [&](int64_t sk) {
    int64_t n = 0;
    for (int s = 0; s < b->num_seqs; ++s) n += splits_of(s, sk);
    return n;
  };
  const int64_t hi_tiles = ceil_div(max_keys, kTile);
  const int64_t lo_tiles = std::max<int64_t>(1, ceil_div(hi_tiles, kMaxSplit));  // the combine's bound
  auto smallest = [&](int64_t cap) {  // smallest split (in tiles) with at most cap active groups
    int64_t lo = lo_tiles, hi = hi_tiles;
    if (active(hi * kTile) > cap) return (int64_t)-1;
    while (lo < hi) {
      const int64_t mid = (lo + hi) / 2;
      if (active(mid * kTile) <= cap) hi = mid; else lo = mid + 1;
    }
    return lo;
  };
  int64_t best = smallest(kTargetGroups);
  const int64_t two = smallest(2 * kTargetGroups);
  if (best < 0 || (two > 0 && 20 * two < 9 * best)) best = two;
  if (best < 0) return false;
  out.split_keys = (int)(best * kTile);
  out.n_split = (int)ceil_div(max_keys, out.split_keys);
  // the active (query, split) pairs, when query s is the one query of sequence s
  if (wl) {
    wl->n = 0;
    if (b->total_q == b->num_seqs && active(out.split_keys) <= kMaxWorkItems && out.n_split <= 512) {
      for (int q = 0; q < b->num_seqs; ++q) {
        const int64_t ns = splits_of(q, out.split_keys);
        for (int64_t sp = 0; sp < ns; ++sp) wl->item[wl->n++] = ((uint32_t)q << 9) | (uint32_t)sp;
      }
    }
  }
  return true;
}

// Keys processed by one launch: every query over up to max_keys, bounded for ragged
// single-query sequences by the rows of the batch.
int64_t launch_work(const hs2_seqs* b, int64_t max_keys) {
  const int64_t tq = std::max(0, b->total_q);
  const int64_t by_rows = b->total_kv_rows * std::max(1, b->max_q_per_seq);
  return std::min(tq * max_keys, std::max<int64_t>(by_rows, max_keys));
}

struct SelectPlan {
  bool chunk = false;     // many queries per sequence: q-tile kernels sharing K/V tiles
  WorkList attn_wl{}, score_wl{};  // bf16 decode path with host lengths: the active pairs
  int max_tiles = 0;      // q-tiles launched (upper bound of the tiles of the batch)
  size_t off_tiles = 0;
  Split attn, score;
  int f_split = 1, f_len = kFilterLen;
  int64_t score_stride = 0;
  bool score_lists = false;  // decode-shaped bf16/FP8 score pass: candidate lists, not score rows
  int list_waves = 0, list_cap = 0;
  size_t off_part = 0, off_lse2 = 0, off_scores = 0, off_hist = 0, off_counters = 0,
         off_above = 0, off_cand = 0, off_miss = 0, off_lists = 0, off_lcount = 0, off_lthr = 0, total = 0;
  bool lists() const { return attn_wl.n > 0 || score_wl.n > 0; }
};

// selection == false: exact causal attention only (hs2_causal_attn): no LSE copy, score
// histograms or selection counters, and a query with one split gets its output directly.
SelectPlan plan_select(const hs2_seqs* b, int window, int top_k, hs2_dtype dt, bool selection = true) {
  SelectPlan p;
  const int64_t tq = std::max(0, b->total_q);
  const int64_t max_cand = std::max<int64_t>(0, (int64_t)b->max_kv_len - window + 1);
  p.chunk = dt == HS2_BF16 && b->max_q_per_seq >= kChunkMinQueries;
  if (p.chunk) {
    // q-tiles of kQTile queries of one sequence; splits fill one round of workgroups.
    // A score split stays below 2^16 keys (the kernel's 16-bit LDS bin counts).
    p.max_tiles = (int)(tq / kQTile + b->num_seqs + 1);
    const int64_t want = std::max<int64_t>(1, kTargetGroups / std::max(1, p.max_tiles));
    auto split_of = [&](int64_t keys, int64_t cap) {
      Split sp;
      if (keys <= 0) return Split{1, kTile};
      sp.split_keys = (int)std::min<int64_t>(
          ceil_div(ceil_div(keys, std::min<int64_t>(want, kMaxSplit)), kTile) * kTile, cap);
      sp.n_split = (int)ceil_div(keys, sp.split_keys);
      return sp;
    };
    p.attn = split_of(b->max_kv_len, std::numeric_limits<int>::max());
    p.score = split_of(max_cand, kScoreSplitMax);
  } else {
    const bool lists = dt != HS2_F32;  // the bf16 and FP8 decode-shaped kernels take work lists
    if (!plan_split_lengths(b, 0, b->max_kv_len, p.attn, lists ? &p.attn_wl : nullptr))
      p.attn = plan_split(launch_work(b, b->max_kv_len), b->max_kv_len);
    if (!plan_split_lengths(b, window - 1, max_cand, p.score, lists ? &p.score_wl : nullptr))
      p.score = plan_split(launch_work(b, max_cand), max_cand);
  }
  p.f_split = (int)std::max<int64_t>(1, ceil_div(max_cand, kFilterLen));
  p.score_stride = (max_cand + 63) / 64 * 64;
  size_t off = 0;
  p.off_part = off;
  if (p.attn.n_split > 1 || (p.chunk && selection)) off += align_up((size_t)tq * p.attn.n_split * sizeof(Partial));
  if (selection) {
    p.off_lse2 = off;
    off += align_up((size_t)tq * kHeads * sizeof(float));
    p.off_hist = off;
    off += align_up((size_t)tq * kHistBins * sizeof(uint32_t));
    p.off_counters = off;
    off += align_up((size_t)tq * 4 * sizeof(uint32_t));
  }
  if (p.chunk) {
    p.off_tiles = off;
    off += align_up((size_t)p.max_tiles * sizeof(int2));
  }
  if (p.lists()) {  // plan-miss flags of the work-list launches: attention, then score pass
    p.off_miss = off;
    off += align_up((size_t)2 * tq * sizeof(int32_t));
  }
  if (top_k > 0) {
    p.score_lists = !p.chunk && dt != HS2_F32;
    if (p.score_lists) {
      // per (query, score split, wave): up to all of the wave's candidates as 8-byte pairs
      p.list_waves = score_waves(dt == HS2_FP8_E4M3);  // one list per wave of the score pass
      p.list_cap = (int)(ceil_div(ceil_div(p.score.split_keys, kTile), p.list_waves) * kTile);
      const size_t nl = (size_t)tq * p.score.n_split * p.list_waves;
      p.off_lists = off;
      off += align_up(nl * p.list_cap * sizeof(uint2));
      p.off_lcount = off;
      off += align_up(nl * sizeof(int32_t));
      p.off_lthr = off;
      off += align_up((size_t)tq * p.score.n_split * sizeof(int32_t));
    } else {
      p.off_scores = off;
      off += align_up((size_t)tq * p.score_stride * sizeof(float));
    }
    p.off_above = off;
    off += align_up((size_t)tq * top_k * sizeof(int32_t));
    p.off_cand = off;
    off += align_up((size_t)tq * kCandCap * sizeof(uint2));
  }
  p.total = off;
  return p;
}

struct SparsePlan {
  Split attn;
  bool narrow = false;  // bf16 / FP8: the narrow-slot kernel, one workgroup per query
  size_t total = 0;
};

// bf16 and FP8 K/V: slices of whole tiles, at most sparse_slots() of them in LDS at once,
// sized so that the launch holds about one workgroup per CU; a batch of at least two
// queries per CU instead takes the narrow-slot kernel with one workgroup per query (two
// workgroups share a CU; no split combine). fp32 K/V: key splits of the fp32 gather kernel
// (at most kSparseSplitMax keys, the bound of its LDS row list).
SparsePlan plan_sparse(const hs2_seqs* b, int window, int top_k, hs2_dtype dt) {
  SparsePlan p;
  const int64_t tq = std::max(0, b->total_q);
  const int64_t max_keys = (int64_t)top_k + std::min<int64_t>(window, b->max_kv_len);
  if (dt == HS2_F32) {
    p.attn = plan_split(tq * max_keys, max_keys);
    if (p.attn.split_keys > kSparseSplitMax) {  // gathered slots of a workgroup are staged in LDS
      p.attn.split_keys = kSparseSplitMax;
      p.attn.n_split = (int)ceil_div(max_keys, kSparseSplitMax);
    }
  } else if (tq >= 2 * kTargetGroups) {
    p.narrow = true;
    p.attn.split_keys = (int)(std::max<int64_t>(1, ceil_div(max_keys, kTile)) * kTile);
    p.attn.n_split = 1;
  } else {
    const int64_t tiles = std::max<int64_t>(1, ceil_div(max_keys, kTile));
    int64_t per = std::min<int64_t>(ceil_div(std::max<int64_t>(1, tq) * tiles, kTargetGroups),
                                    sparse_slots(dt == HS2_FP8_E4M3));
    per = std::max<int64_t>({per, 1, ceil_div(tiles, kMaxSplit)});  // a very wide window: several batches
    p.attn.split_keys = (int)(per * kTile);
    p.attn.n_split = (int)ceil_div(tiles, per);
  }
  p.total = p.attn.n_split > 1 ? align_up((size_t)tq * p.attn.n_split * sizeof(Partial)) : 0;
  return p;
}

hs2_status check_batch(const hs2_seqs* b) {
  if (!b) return fail(HS2_ERR_INVALID_ARG, "batch descriptor is NULL");
  if (b->num_seqs < 1) return fail(HS2_ERR_INVALID_ARG, "num_seqs must be >= 1 (got %d)", b->num_seqs);
  if (b->total_q < 0) return fail(HS2_ERR_INVALID_ARG, "total_q must be >= 0 (got %d)", b->total_q);
  if (b->max_kv_len < 1) return fail(HS2_ERR_INVALID_ARG, "max_kv_len must be >= 1 (got %d)", b->max_kv_len);
  if (b->total_kv_rows < 0) return fail(HS2_ERR_INVALID_ARG, "total_kv_rows must be >= 0");
  if (b->max_q_per_seq < 0) return fail(HS2_ERR_INVALID_ARG, "max_q_per_seq must be >= 0");
  if (!b->kv_start || !b->kv_len || !b->q_start || (b->total_q > 0 && !b->q_pos))
    return fail(HS2_ERR_INVALID_ARG, "batch descriptor has a NULL device array");
  if (!aligned(b->kv_start, 8) || !aligned(b->kv_len, 4) || !aligned(b->q_start, 4) ||
      (b->q_pos && !aligned(b->q_pos, 4)))
    return fail(HS2_ERR_INVALID_ARG, "batch descriptor arrays are misaligned");
  if (b->kv_len_host) {  // the split planner sizes work items from these
    for (int s = 0; s < b->num_seqs; ++s)
      if (b->kv_len_host[s] < 0 || b->kv_len_host[s] > b->max_kv_len)
        return fail(HS2_ERR_INVALID_ARG, "kv_len_host[%d] = %d is outside [0, max_kv_len = %d]", s,
                    b->kv_len_host[s], b->max_kv_len);
  }
  return HS2_OK;
}

hs2_status check_attn_common(const hs2_seqs* b, const void* q, const void* k, const void* v,
                             int32_t n_heads, int32_t head_dim, int32_t window, int32_t top_k,
                             float scale, const void* out, const float* lse, hs2_dtype dt) {
  hs2_status st = check_batch(b);
  if (st != HS2_OK) return st;
  if (dt != HS2_BF16 && dt != HS2_F32 && dt != HS2_FP8_E4M3)
    return fail(HS2_ERR_UNSUPPORTED, "dtype %d is not supported", (int)dt);
  if (n_heads != kHeads || head_dim != kDim)
    return fail(HS2_ERR_UNSUPPORTED, "only n_heads=64, head_dim=128 are supported (got %d, %d)", n_heads,
                head_dim);
  if (window < 1 || window > (1 << 18)) return fail(HS2_ERR_INVALID_ARG, "window must be in [1, 2^18] (got %d)", window);
  if (top_k < 0 || top_k > HS2_MAX_TOP_K)
    return fail(HS2_ERR_INVALID_ARG, "top_k must be in [0, %d] (got %d)", HS2_MAX_TOP_K, top_k);
  if (!(scale > 0.0f) || !std::isfinite(scale)) return fail(HS2_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (b->total_q > 0 && (!q || !out)) return fail(HS2_ERR_INVALID_ARG, "q and out must not be NULL");
  if (b->total_kv_rows > 0 && (!k || !v)) return fail(HS2_ERR_INVALID_ARG, "k and v must not be NULL");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
    return fail(HS2_ERR_INVALID_ARG, "q, k, v and out must be 16-byte aligned");
  if (lse && !aligned(lse, 4)) return fail(HS2_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  if (out && (out == q || out == k || out == v)) return fail(HS2_ERR_INVALID_ARG, "out aliases an input");
  return HS2_OK;
}

SeqsDev to_dev(const hs2_seqs* b) {
  SeqsDev d;
  d.kv_start = b->kv_start;
  d.kv_len = b->kv_len;
  d.q_start = b->q_start;
  d.q_pos = b->q_pos;
  d.num_seqs = b->num_seqs;
  d.total_q = b->total_q;
  d.total_rows = b->total_kv_rows;
  d.max_kv_len = b->max_kv_len;
  return d;
}

// Kernel timing hook state (see hs2_set_kernel_events): per calling thread.
constexpr int kMaxEventPairs = 16;
thread_local hipEvent_t g_events[2 * kMaxEventPairs];
thread_local int g_event_pairs = 0;

// Brackets the kernel of pipeline slot j of one entry-point call with the attached events.
struct LaunchMarks {
  hipStream_t s;
  explicit LaunchMarks(hipStream_t st) : s(st) {}
  hipError_t before(int j) const {
    return j < g_event_pairs ? hipEventRecord(g_events[2 * j], s) : hipSuccess;
  }
  hipError_t after(int j) const {
    return j < g_event_pairs ? hipEventRecord(g_events[2 * j + 1], s) : hipSuccess;
  }
};

hs2_status hip_fail(hipError_t e, const char* what) {
  return fail(HS2_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

}  // namespace

extern "C" {

int32_t hs2_version(void) { return HS2_VERSION; }

hs2_status hs2_set_kernel_events(void* const* events, int32_t n_pairs) {
  if (n_pairs < 0 || n_pairs > kMaxEventPairs)
    return fail(HS2_ERR_INVALID_ARG, "n_pairs must be in [0, %d] (got %d)", kMaxEventPairs, n_pairs);
  if (!events || n_pairs == 0) {
    g_event_pairs = 0;
    return ok();
  }
  for (int i = 0; i < 2 * n_pairs; ++i)
    if (!events[i]) return fail(HS2_ERR_INVALID_ARG, "event %d is NULL", i);
  for (int i = 0; i < 2 * n_pairs; ++i) g_events[i] = static_cast<hipEvent_t>(events[i]);
  g_event_pairs = n_pairs;
  return ok();
}

const char* hs2_last_error(void) { return g_err.c_str(); }

size_t hs2_full_attn_select_workspace_size(const hs2_seqs* batch, int32_t n_heads, int32_t head_dim,
                                           int32_t window, int32_t top_k, hs2_dtype dt) {
  (void)n_heads;
  (void)head_dim;
  if (!batch || batch->total_q < 0 || batch->max_kv_len < 1 || window < 1 || top_k < 0) return 0;
  return plan_select(batch, window, top_k, dt).total;
}

}  // extern "C"

namespace {

// FP8 K/V: the per-tensor scales must be finite and positive.
hs2_status check_kv_scales(float k_scale, float v_scale) {
  if (!(k_scale > 0.0f) || !std::isfinite(k_scale) || !(v_scale > 0.0f) || !std::isfinite(v_scale))
    return fail(HS2_ERR_INVALID_ARG, "k_scale and v_scale must be finite and > 0");
  return HS2_OK;
}

// Softmax constant of the kernels: scale * log2(e), times the K scale of FP8 storage
// (logit = scale * <q, k_scale * code> = (scale * k_scale) * <q, code>).
float logit_c2(float scale, hs2_dtype dt, float k_scale) {
  if (dt != HS2_FP8_E4M3) return scale * kLog2e;
  return (float)((double)scale * (double)k_scale * 1.4426950408889634);
}

hs2_status select_impl(const hs2_seqs* batch, const void* q, const void* k, const void* v, float k_scale,
                       float v_scale, int32_t n_heads, int32_t head_dim, int32_t window, int32_t top_k,
                       float scale, void* out, float* lse, int32_t* sel_idx, int32_t* sel_count, void* workspace,
                       size_t workspace_bytes, hs2_dtype dt, void* stream) {
  hs2_status st = check_attn_common(batch, q, k, v, n_heads, head_dim, window, top_k, scale, out, lse, dt);
  if (st != HS2_OK) return st;
  if (top_k > 0 && batch->total_q > 0 && !sel_idx)
    return fail(HS2_ERR_INVALID_ARG, "sel_idx must not be NULL when top_k > 0");
  if ((sel_idx && !aligned(sel_idx, 4)) || (sel_count && !aligned(sel_count, 4)))
    return fail(HS2_ERR_INVALID_ARG, "sel_idx and sel_count must be 4-byte aligned");
  const SelectPlan p = plan_select(batch, window, top_k, dt);
  if (workspace_bytes < p.total || (p.total > 0 && !workspace))
    return fail(HS2_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the required %zu", workspace_bytes,
                p.total);
  if (workspace && !aligned(workspace, kAlign)) return fail(HS2_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (batch->total_q == 0) return ok();

  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool f32 = dt == HS2_F32;
  const bool fp8 = dt == HS2_FP8_E4M3;
  const int tq = batch->total_q;
  float* lse2 = at<float>(workspace, p.off_lse2);
  uint32_t* hist = at<uint32_t>(workspace, p.off_hist);
  uint32_t* counters = at<uint32_t>(workspace, p.off_counters);

  AttnArgs a{};
  a.b = to_dev(batch);
  a.q = q;
  a.k = k;
  a.v = v;
  a.sel = nullptr;
  a.window = window;
  a.top_k = top_k;
  a.c2 = logit_c2(scale, dt, k_scale);
  a.n_split = p.attn.n_split;
  a.split_keys = p.attn.split_keys;
  a.part = p.attn.n_split > 1 ? at<Partial>(workspace, p.off_part) : nullptr;
  a.out = out;
  a.lse = lse;
  a.lse2 = lse2;
  a.v_scale = fp8 ? v_scale : 1.0f;
  int32_t* miss = p.lists() ? at<int32_t>(workspace, p.off_miss) : nullptr;
  a.plan_miss = p.attn_wl.n > 0 ? miss : nullptr;
  const int grid = tq * p.attn.n_split;
  int2* tiles = p.chunk ? at<int2>(workspace, p.off_tiles) : nullptr;
  LaunchMarks mk(s);
  hipError_t e = hipSuccess;
  if (p.chunk) {
    a.part = at<Partial>(workspace, p.off_part);
    e = launch_qtile_prep(a.b, tiles, p.max_tiles, s);
    if (e != hipSuccess) return hip_fail(e, "q-tile list launch");
  }
  e = mk.before(0);
  if (e == hipSuccess) {
    if (p.chunk)
      e = launch_attn_chunk(a, tiles, p.max_tiles, s);
    else if (f32)
      e = launch_attn_f32(a, false, grid, hist, counters, s);
    else if (fp8)
      e = launch_attn_fp8kv(a, p.attn_wl, p.attn_wl.n > 0 ? p.attn_wl.n : grid, hist, counters, s);
    else
      e = launch_attn_bf16(a, p.attn_wl, p.attn_wl.n > 0 ? p.attn_wl.n : grid, hist, counters, s);
  }
  if (e == hipSuccess) e = mk.after(0);
  if (e != hipSuccess) return hip_fail(e, "full attention launch");
  if (p.attn.n_split > 1 || p.chunk) {
    CombineArgs c{};
    c.b = a.b;
    c.part = a.part;
    c.n_split = p.attn.n_split;
    c.split_keys = p.attn.split_keys;
    c.gather = 0;
    c.window = window;
    c.top_k = top_k;
    c.out = out;
    c.lse = lse;
    c.lse2 = lse2;
    c.hist = hist;
    c.counters = counters;
    c.v_scale = a.v_scale;
    c.plan_miss = a.plan_miss;
    e = mk.before(1);
    if (e == hipSuccess) e = launch_combine(c, f32, s);
    if (e == hipSuccess) e = mk.after(1);
    if (e != hipSuccess) return hip_fail(e, "split combine launch");
  }
  TopkArgs tk{};
  tk.b = a.b;
  tk.window = window;
  tk.top_k = top_k;
  tk.n_split = p.f_split;
  tk.split_len = p.f_len;
  tk.score_stride = p.score_stride;
  tk.scores = top_k > 0 && !p.score_lists ? at<float>(workspace, p.off_scores) : nullptr;
  if (top_k > 0 && p.score_lists) {
    tk.lists = at<uint2>(workspace, p.off_lists);
    tk.list_count = at<int32_t>(workspace, p.off_lcount);
    tk.list_thr = at<int32_t>(workspace, p.off_lthr);
    tk.list_cap = p.list_cap;
    tk.list_waves = p.list_waves;
    tk.list_splits = p.score.n_split;
    tk.list_split_keys = p.score.split_keys;
  }
  tk.hist = hist;
  tk.counters = counters;
  tk.above = top_k > 0 ? at<int32_t>(workspace, p.off_above) : nullptr;
  tk.cand = top_k > 0 ? at<uint2>(workspace, p.off_cand) : nullptr;
  tk.sel_idx = sel_idx;
  tk.sel_count = sel_count;
  tk.miss_attn = a.plan_miss;
  tk.miss_score = top_k > 0 && p.score_wl.n > 0 ? miss + tq : nullptr;
  tk.out = out;
  tk.lse = lse;
  tk.out_f32 = f32 ? 1 : 0;
  if (top_k > 0) {
    ScoreArgs sc{};
    sc.b = a.b;
    sc.q = q;
    sc.k = k;
    sc.lse2 = lse2;
    sc.c2 = a.c2;
    sc.window = window;
    sc.top_k = top_k;
    sc.n_split = p.score.n_split;
    sc.split_keys = p.score.split_keys;
    sc.score_stride = p.score_stride;
    sc.scores = tk.scores ? const_cast<float*>(tk.scores) : nullptr;
    sc.lists = const_cast<uint2*>(tk.lists);
    sc.list_count = const_cast<int32_t*>(tk.list_count);
    sc.list_thr = const_cast<int32_t*>(tk.list_thr);
    sc.list_cap = tk.list_cap;
    sc.hist = hist;
    sc.plan_miss = tk.miss_score ? miss + tq : nullptr;
    e = mk.before(2);
    if (e == hipSuccess) {
      if (p.chunk)
        e = launch_score_chunk(sc, tiles, p.max_tiles, s);
      else if (f32)
        e = launch_score_f32(sc, s);
      else if (fp8)
        e = launch_score_fp8kv(sc, p.score_wl, s);
      else
        e = launch_score_bf16(sc, p.score_wl, s);
    }
    if (e == hipSuccess) e = mk.after(2);
    if (e != hipSuccess) return hip_fail(e, "score launch");
    e = mk.before(3);
    if (e == hipSuccess) e = launch_topk_filter(tk, s);
    if (e == hipSuccess) e = mk.after(3);
    if (e != hipSuccess) return hip_fail(e, "top-k filter launch");
  }
  e = mk.before(4);
  if (e == hipSuccess) e = launch_topk_finish(tk, s);
  if (e == hipSuccess) e = mk.after(4);
  if (e != hipSuccess) return hip_fail(e, "top-k finish launch");
  return ok();
}

}  // namespace

namespace hs2 {
// Every argument check of a sparse-layer call except the workspace's.
hs2_status sparse_check(const hs2_seqs* batch, const void* q, const void* k, const void* v, const int32_t* sel_idx,
                        int32_t n_heads, int32_t head_dim, int32_t window, int32_t top_k, float scale,
                        const void* out, const float* lse, hs2_dtype dt) {
  hs2_status st = check_attn_common(batch, q, k, v, n_heads, head_dim, window, top_k, scale, out, lse, dt);
  if (st != HS2_OK) return st;
  if (top_k > 0 && batch->total_q > 0 && !sel_idx)
    return fail(HS2_ERR_INVALID_ARG, "sel_idx must not be NULL when top_k > 0");
  if (sel_idx && !aligned(sel_idx, 4)) return fail(HS2_ERR_INVALID_ARG, "sel_idx must be 4-byte aligned");
  return HS2_OK;
}
}  // namespace hs2

namespace {

hs2_status sparse_impl(const hs2_seqs* batch, const void* q, const void* k, const void* v, float k_scale,
                       float v_scale, const int32_t* sel_idx, int32_t n_heads, int32_t head_dim, int32_t window,
                       int32_t top_k, float scale, void* out, float* lse, void* workspace, size_t workspace_bytes,
                       hs2_dtype dt, void* stream) {
  hs2_status st = sparse_check(batch, q, k, v, sel_idx, n_heads, head_dim, window, top_k, scale, out, lse, dt);
  if (st != HS2_OK) return st;
  const SparsePlan p = plan_sparse(batch, window, top_k, dt);
  if (workspace_bytes < p.total || (p.total > 0 && !workspace))
    return fail(HS2_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the required %zu", workspace_bytes,
                p.total);
  if (workspace && !aligned(workspace, kAlign)) return fail(HS2_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (batch->total_q == 0) return ok();

  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool f32 = dt == HS2_F32;
  const bool fp8 = dt == HS2_FP8_E4M3;
  AttnArgs a{};
  a.b = to_dev(batch);
  a.q = q;
  a.k = k;
  a.v = v;
  a.sel = sel_idx;
  a.window = window;
  a.top_k = top_k;
  a.c2 = logit_c2(scale, dt, k_scale);
  a.n_split = p.attn.n_split;
  a.split_keys = p.attn.split_keys;
  a.part = p.attn.n_split > 1 ? static_cast<Partial*>(workspace) : nullptr;
  a.out = out;
  a.lse = lse;
  a.lse2 = nullptr;
  a.v_scale = fp8 ? v_scale : 1.0f;
  const int grid = batch->total_q * p.attn.n_split;
  LaunchMarks mk(s);
  hipError_t e = mk.before(0);
  if (e == hipSuccess)
    e = f32 ? launch_attn_f32(a, true, grid, nullptr, nullptr, s) : launch_sparse_attn(a, fp8, p.narrow, grid, s);
  if (e == hipSuccess) e = mk.after(0);
  if (e != hipSuccess) return hip_fail(e, "sparse attention launch");
  if (p.attn.n_split > 1) {
    CombineArgs c{};
    c.b = a.b;
    c.part = a.part;
    c.n_split = p.attn.n_split;
    c.split_keys = p.attn.split_keys;
    c.gather = 1;
    c.window = window;
    c.top_k = top_k;
    c.out = out;
    c.lse = lse;
    c.lse2 = nullptr;
    c.hist = nullptr;
    c.counters = nullptr;
    c.v_scale = a.v_scale;
    e = mk.before(1);
    if (e == hipSuccess) e = launch_combine(c, f32, s);
    if (e == hipSuccess) e = mk.after(1);
    if (e != hipSuccess) return hip_fail(e, "split combine launch");
  }
  return ok();
}

// Exact causal attention of every query, no selection (the self-decoder's full-attention
// layer in prefill): pass 1 alone, plus the split combine when a query's keys are split.
hs2_status causal_impl(const hs2_seqs* batch, const void* q, const void* k, const void* v, int32_t n_heads,
                       int32_t head_dim, float scale, void* out, float* lse, void* workspace, size_t workspace_bytes,
                       hs2_dtype dt, void* stream) {
  if (dt == HS2_FP8_E4M3) return fail(HS2_ERR_UNSUPPORTED, "causal attention takes bf16 or fp32 K/V");
  hs2_status st = check_attn_common(batch, q, k, v, n_heads, head_dim, 1, 0, scale, out, lse, dt);
  if (st != HS2_OK) return st;
  const SelectPlan p = plan_select(batch, 1, 0, dt, false);
  if (workspace_bytes < p.total || (p.total > 0 && !workspace))
    return fail(HS2_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the required %zu", workspace_bytes,
                p.total);
  if (workspace && !aligned(workspace, kAlign)) return fail(HS2_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (batch->total_q == 0) return ok();

  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool f32 = dt == HS2_F32;
  AttnArgs a{};
  a.b = to_dev(batch);
  a.q = q;
  a.k = k;
  a.v = v;
  a.sel = nullptr;
  a.window = 1;
  a.top_k = 0;
  a.c2 = scale * kLog2e;
  a.n_split = p.attn.n_split;
  a.split_keys = p.attn.split_keys;
  a.part = p.attn.n_split > 1 ? at<Partial>(workspace, p.off_part) : nullptr;
  a.out = out;
  a.lse = lse;
  a.lse2 = nullptr;
  a.v_scale = 1.0f;
  a.direct = p.chunk && p.attn.n_split == 1;
  a.plan_miss = p.attn_wl.n > 0 ? at<int32_t>(workspace, p.off_miss) : nullptr;
  const int grid = batch->total_q * p.attn.n_split;
  LaunchMarks mk(s);
  hipError_t e = hipSuccess;
  int2* tiles = p.chunk ? at<int2>(workspace, p.off_tiles) : nullptr;
  if (p.chunk) {
    e = launch_qtile_prep(a.b, tiles, p.max_tiles, s);
    if (e != hipSuccess) return hip_fail(e, "q-tile list launch");
  }
  e = mk.before(0);
  if (e == hipSuccess) {
    if (p.chunk)
      e = launch_attn_chunk(a, tiles, p.max_tiles, s);
    else if (f32)
      e = launch_attn_f32(a, false, grid, nullptr, nullptr, s);
    else
      e = launch_attn_bf16(a, p.attn_wl, p.attn_wl.n > 0 ? p.attn_wl.n : grid, nullptr, nullptr, s);
  }
  if (e == hipSuccess) e = mk.after(0);
  if (e != hipSuccess) return hip_fail(e, "causal attention launch");
  if (p.attn.n_split > 1) {
    CombineArgs c{};
    c.b = a.b;
    c.part = a.part;
    c.n_split = p.attn.n_split;
    c.split_keys = p.attn.split_keys;
    c.gather = 0;
    c.window = 1;
    c.top_k = 0;
    c.out = out;
    c.lse = lse;
    c.lse2 = nullptr;
    c.hist = nullptr;
    c.counters = nullptr;
    c.v_scale = 1.0f;
    c.plan_miss = a.plan_miss;
    e = mk.before(1);
    if (e == hipSuccess) e = launch_combine(c, f32, s);
    if (e == hipSuccess) e = mk.after(1);
    if (e != hipSuccess) return hip_fail(e, "split combine launch");
  }
  return ok();
}

// Both append entry points: bf16 cache rows, or (k_scale and v_scale given) FP8 E4M3 codes.
hs2_status append_impl(const void* hidden, int32_t n_new, const int64_t* rows, int64_t cache_rows, int32_t d_model,
                       int32_t n_layers, const void* const* w_k, const void* const* w_v, void* const* k_cache,
                       void* const* v_cache, const float* k_scale, const float* v_scale, int32_t head_dim,
                       void* workspace, size_t workspace_bytes, void* stream) {
  if (head_dim != kDim) return fail(HS2_ERR_UNSUPPORTED, "bridging supports head_dim=128 only (got %d)", head_dim);
  if (d_model < kAppendSlice || d_model > 65536 || d_model % kAppendSlice != 0)
    return fail(HS2_ERR_UNSUPPORTED, "d_model must be a multiple of %d in [%d, 65536] (got %d)", kAppendSlice,
                kAppendSlice, d_model);
  if (n_layers < 1 || n_layers > 8) return fail(HS2_ERR_UNSUPPORTED, "n_layers must be in [1, 8] (got %d)", n_layers);
  if (n_new < 0 || n_new > 65536) return fail(HS2_ERR_INVALID_ARG, "n_new must be in [0, 65536] (got %d)", n_new);
  if (cache_rows < 0) return fail(HS2_ERR_INVALID_ARG, "cache_rows must be >= 0");
  if (!w_k || !w_v || !k_cache || !v_cache) return fail(HS2_ERR_INVALID_ARG, "pointer arrays must not be NULL");
  if (n_new > 0 && (!hidden || !rows)) return fail(HS2_ERR_INVALID_ARG, "hidden and rows must not be NULL");
  if (!aligned(hidden, 16) || !aligned(rows, 8)) return fail(HS2_ERR_INVALID_ARG, "hidden must be 16-byte and rows 8-byte aligned");
  AppendArgs a{};
  BridgeOut o{};
  o.fp8 = k_scale != nullptr ? 1 : 0;
  for (int l = 0; l < n_layers; ++l) {
    if (!w_k[l] || !w_v[l] || !k_cache[l] || !v_cache[l])
      return fail(HS2_ERR_INVALID_ARG, "a weight or cache pointer of layer %d is NULL", l);
    if (!aligned(w_k[l], 16) || !aligned(w_v[l], 16) || !aligned(k_cache[l], 16) || !aligned(v_cache[l], 16))
      return fail(HS2_ERR_INVALID_ARG, "weights and caches must be 16-byte aligned (layer %d)", l);
    if (o.fp8) {
      const float ks = k_scale[l], vs = v_scale[l];
      if (!(std::isfinite(ks) && ks > 0.0f && std::isfinite(vs) && vs > 0.0f))
        return fail(HS2_ERR_INVALID_ARG, "k_scale and v_scale must be finite and > 0 (layer %d)", l);
      const float ik = 1.0f / ks, iv = 1.0f / vs;
      if (!std::isfinite(ik) || !std::isfinite(iv))
        return fail(HS2_ERR_INVALID_ARG, "the reciprocal of a scale overflows (layer %d)", l);
      o.inv_scale[2 * l] = ik;
      o.inv_scale[2 * l + 1] = iv;
    }
    a.w[2 * l] = static_cast<const uint16_t*>(w_k[l]);
    a.w[2 * l + 1] = static_cast<const uint16_t*>(w_v[l]);
    a.outs[2 * l] = static_cast<uint16_t*>(k_cache[l]);
    a.outs[2 * l + 1] = static_cast<uint16_t*>(v_cache[l]);
  }
  const size_t need = hs2_bridge_kv_append_workspace_size(n_new, d_model, n_layers, head_dim);
  if (workspace_bytes < need || (need > 0 && !workspace))
    return fail(HS2_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the required %zu", workspace_bytes, need);
  if (workspace && !aligned(workspace, kAlign)) return fail(HS2_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (n_new == 0) return ok();
  a.h = static_cast<const uint16_t*>(hidden);
  a.rows = rows;
  a.part = static_cast<float*>(workspace);
  a.cache_rows = cache_rows;
  a.n_new = n_new;
  a.d_model = d_model;
  a.n_mats = 2 * n_layers;
  a.n_slices = d_model / kAppendSlice;
  hipStream_t s = static_cast<hipStream_t>(stream);
  LaunchMarks mk(s);
  hipError_t e = mk.before(0);
  if (e == hipSuccess) e = launch_bridge_append(a, o, s);
  if (e == hipSuccess) e = mk.after(0);
  if (e != hipSuccess) return hip_fail(e, "bridging append launch");
  return ok();
}

}  // namespace

extern "C" {

size_t hs2_causal_attn_workspace_size(const hs2_seqs* batch, int32_t n_heads, int32_t head_dim, hs2_dtype dt) {
  (void)n_heads;
  (void)head_dim;
  if (!batch || batch->total_q < 0 || batch->max_kv_len < 1) return 0;
  return plan_select(batch, 1, 0, dt, false).total;
}

hs2_status hs2_causal_attn(const hs2_seqs* batch, const void* q, const void* k, const void* v, int32_t n_heads,
                           int32_t head_dim, float scale, void* out, float* lse, void* workspace,
                           size_t workspace_bytes, hs2_dtype dt, void* stream) {
  return causal_impl(batch, q, k, v, n_heads, head_dim, scale, out, lse, workspace, workspace_bytes, dt, stream);
}

hs2_status hs2_full_attn_select(const hs2_seqs* batch, const void* q, const void* k, const void* v,
                                int32_t n_heads, int32_t head_dim, int32_t window, int32_t top_k,
                                float scale, void* out, float* lse, int32_t* sel_idx,
                                int32_t* sel_count, void* workspace, size_t workspace_bytes,
                                hs2_dtype dt, void* stream) {
  if (dt == HS2_FP8_E4M3)
    return fail(HS2_ERR_UNSUPPORTED, "FP8 K/V needs its scales: use hs2_full_attn_select_fp8kv");
  return select_impl(batch, q, k, v, 1.0f, 1.0f, n_heads, head_dim, window, top_k, scale, out, lse, sel_idx,
                     sel_count, workspace, workspace_bytes, dt, stream);
}

hs2_status hs2_full_attn_select_fp8kv(const hs2_seqs* batch, const void* q, const void* k, const void* v,
                                      float k_scale, float v_scale, int32_t n_heads, int32_t head_dim,
                                      int32_t window, int32_t top_k, float scale, void* out, float* lse,
                                      int32_t* sel_idx, int32_t* sel_count, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  hs2_status st = check_kv_scales(k_scale, v_scale);
  if (st != HS2_OK) return st;
  return select_impl(batch, q, k, v, k_scale, v_scale, n_heads, head_dim, window, top_k, scale, out, lse, sel_idx,
                     sel_count, workspace, workspace_bytes, HS2_FP8_E4M3, stream);
}

hs2_status hs2_sparse_attn(const hs2_seqs* batch, const void* q, const void* k, const void* v,
                           const int32_t* sel_idx, int32_t n_heads, int32_t head_dim, int32_t window,
                           int32_t top_k, float scale, void* out, float* lse, void* workspace,
                           size_t workspace_bytes, hs2_dtype dt, void* stream) {
  if (dt == HS2_FP8_E4M3) return fail(HS2_ERR_UNSUPPORTED, "FP8 K/V needs its scales: use hs2_sparse_attn_fp8kv");
  return sparse_impl(batch, q, k, v, 1.0f, 1.0f, sel_idx, n_heads, head_dim, window, top_k, scale, out, lse,
                     workspace, workspace_bytes, dt, stream);
}

hs2_status hs2_sparse_attn_fp8kv(const hs2_seqs* batch, const void* q, const void* k, const void* v,
                                 float k_scale, float v_scale, const int32_t* sel_idx, int32_t n_heads,
                                 int32_t head_dim, int32_t window, int32_t top_k, float scale, void* out,
                                 float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  hs2_status st = check_kv_scales(k_scale, v_scale);
  if (st != HS2_OK) return st;
  return sparse_impl(batch, q, k, v, k_scale, v_scale, sel_idx, n_heads, head_dim, window, top_k, scale, out, lse,
                     workspace, workspace_bytes, HS2_FP8_E4M3, stream);
}


size_t hs2_sparse_attn_workspace_size(const hs2_seqs* batch, int32_t n_heads, int32_t head_dim, int32_t window,
                                      int32_t top_k, hs2_dtype dt) {
  (void)n_heads;
  (void)head_dim;
  if (!batch || batch->total_q < 0 || batch->max_kv_len < 1 || window < 1 || top_k < 0) return 0;
  return plan_sparse(batch, window, top_k, dt).total;
}

size_t hs2_bridge_kv_append_workspace_size(int32_t n_new, int32_t d_model, int32_t n_layers, int32_t head_dim) {
  if (n_new <= 0 || d_model <= 0 || n_layers <= 0 || head_dim <= 0) return 0;
  return align_up((size_t)(d_model / kAppendSlice) * n_new * 2 * n_layers * head_dim * sizeof(float));
}

hs2_status hs2_bridge_kv_append(const void* hidden, int32_t n_new, const int64_t* rows, int64_t cache_rows,
                                int32_t d_model, int32_t n_layers, const void* const* w_k, const void* const* w_v,
                                void* const* k_cache, void* const* v_cache, int32_t head_dim, void* workspace,
                                size_t workspace_bytes, hs2_dtype dt, void* stream) {
  if (dt != HS2_BF16) return fail(HS2_ERR_UNSUPPORTED, "bridging supports bf16 only");
  return append_impl(hidden, n_new, rows, cache_rows, d_model, n_layers, w_k, w_v, k_cache, v_cache, nullptr,
                     nullptr, head_dim, workspace, workspace_bytes, stream);
}

hs2_status hs2_bridge_kv_append_fp8kv(const void* hidden, int32_t n_new, const int64_t* rows, int64_t cache_rows,
                                      int32_t d_model, int32_t n_layers, const void* const* w_k,
                                      const void* const* w_v, void* const* k_cache, void* const* v_cache,
                                      const float* k_scale, const float* v_scale, int32_t head_dim, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  if (!k_scale || !v_scale) return fail(HS2_ERR_INVALID_ARG, "k_scale and v_scale must not be NULL");
  return append_impl(hidden, n_new, rows, cache_rows, d_model, n_layers, w_k, w_v, k_cache, v_cache, k_scale,
                     v_scale, head_dim, workspace, workspace_bytes, stream);
}

size_t hs2_bridge_kv_workspace_size(int32_t d_model, int32_t n_layers, int32_t head_dim) {
  if (d_model <= 0 || n_layers <= 0 || head_dim <= 0) return 0;
  return align_up((size_t)2 * n_layers * head_dim * d_model * sizeof(uint16_t));
}

}  // extern "C"

namespace {

// Both bridging entry points: bf16 outputs, or (k_scale and v_scale given) FP8 E4M3 codes.
hs2_status bridge_impl(const void* hidden, int64_t n_rows, int32_t d_model, int32_t n_layers,
                       const void* const* w_k, const void* const* w_v, void* const* k_out, void* const* v_out,
                       const float* k_scale, const float* v_scale, int32_t head_dim, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (head_dim != kDim) return fail(HS2_ERR_UNSUPPORTED, "bridging supports head_dim=128 only (got %d)", head_dim);
  if (d_model < 64 || d_model > 65536 || d_model % 64 != 0)
    return fail(HS2_ERR_UNSUPPORTED, "d_model must be a multiple of 64 in [64, 65536] (got %d)", d_model);
  if (n_layers < 1 || n_layers > 8) return fail(HS2_ERR_UNSUPPORTED, "n_layers must be in [1, 8] (got %d)", n_layers);
  if (n_rows < 0) return fail(HS2_ERR_INVALID_ARG, "n_rows must be >= 0");
  if (!w_k || !w_v || !k_out || !v_out) return fail(HS2_ERR_INVALID_ARG, "pointer arrays must not be NULL");
  if (n_rows > 0 && !hidden) return fail(HS2_ERR_INVALID_ARG, "hidden must not be NULL");
  if (!aligned(hidden, 16)) return fail(HS2_ERR_INVALID_ARG, "hidden must be 16-byte aligned");
  const bool fp8 = k_scale != nullptr;
  const uint16_t* w[16];
  BridgeArgs a{};
  BridgeOut o{};
  o.fp8 = fp8 ? 1 : 0;
  for (int l = 0; l < n_layers; ++l) {
    if (!w_k[l] || !w_v[l] || !k_out[l] || !v_out[l])
      return fail(HS2_ERR_INVALID_ARG, "a weight or output pointer of layer %d is NULL", l);
    if (!aligned(w_k[l], 16) || !aligned(w_v[l], 16) || !aligned(k_out[l], 16) || !aligned(v_out[l], 16))
      return fail(HS2_ERR_INVALID_ARG, "weights and outputs must be 16-byte aligned (layer %d)", l);
    if (k_out[l] == hidden || v_out[l] == hidden) return fail(HS2_ERR_INVALID_ARG, "an output aliases hidden");
    if (fp8) {
      const float ks = k_scale[l], vs = v_scale[l];
      if (!(std::isfinite(ks) && ks > 0.0f && std::isfinite(vs) && vs > 0.0f))
        return fail(HS2_ERR_INVALID_ARG, "k_scale and v_scale must be finite and > 0 (layer %d)", l);
      const float ik = 1.0f / ks, iv = 1.0f / vs;
      if (!std::isfinite(ik) || !std::isfinite(iv))
        return fail(HS2_ERR_INVALID_ARG, "the reciprocal of a scale overflows (layer %d)", l);
      o.inv_scale[2 * l] = ik;
      o.inv_scale[2 * l + 1] = iv;
    }
    w[2 * l] = static_cast<const uint16_t*>(w_k[l]);
    w[2 * l + 1] = static_cast<const uint16_t*>(w_v[l]);
    a.outs[2 * l] = static_cast<uint16_t*>(k_out[l]);
    a.outs[2 * l + 1] = static_cast<uint16_t*>(v_out[l]);
  }
  const size_t need = hs2_bridge_kv_workspace_size(d_model, n_layers, head_dim);
  if (workspace_bytes < need || !workspace)
    return fail(HS2_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the required %zu", workspace_bytes, need);
  if (!aligned(workspace, kAlign)) return fail(HS2_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  a.h = static_cast<const uint16_t*>(hidden);
  a.wt = static_cast<const uint16_t*>(workspace);
  a.n_rows = n_rows;
  a.d_model = d_model;
  a.n_mats = 2 * n_layers;
  hipStream_t s = static_cast<hipStream_t>(stream);
  LaunchMarks mk(s);
  hipError_t e = mk.before(0);
  if (e == hipSuccess) e = launch_bridge_transpose(a, w, 2 * n_layers, static_cast<uint16_t*>(workspace), s);
  if (e == hipSuccess) e = mk.after(0);
  if (e != hipSuccess) return hip_fail(e, "bridging weight transpose launch");
  if (n_rows == 0) return ok();
  e = mk.before(1);
  if (e == hipSuccess) e = launch_bridge_gemm(a, o, s);
  if (e == hipSuccess) e = mk.after(1);
  if (e != hipSuccess) return hip_fail(e, "bridging launch");
  return ok();
}

}  // namespace

extern "C" {

hs2_status hs2_bridge_kv(const void* hidden, int64_t n_rows, int32_t d_model, int32_t n_layers,
                         const void* const* w_k, const void* const* w_v, void* const* k_out,
                         void* const* v_out, int32_t head_dim, void* workspace, size_t workspace_bytes,
                         hs2_dtype dt, void* stream) {
  if (dt != HS2_BF16) return fail(HS2_ERR_UNSUPPORTED, "bridging supports bf16 only");
  return bridge_impl(hidden, n_rows, d_model, n_layers, w_k, w_v, k_out, v_out, nullptr, nullptr, head_dim,
                     workspace, workspace_bytes, stream);
}

hs2_status hs2_bridge_kv_fp8kv(const void* hidden, int64_t n_rows, int32_t d_model, int32_t n_layers,
                               const void* const* w_k, const void* const* w_v, void* const* k_out,
                               void* const* v_out, const float* k_scale, const float* v_scale, int32_t head_dim,
                               void* workspace, size_t workspace_bytes, void* stream) {
  if (!k_scale || !v_scale) return fail(HS2_ERR_INVALID_ARG, "k_scale and v_scale must not be NULL");
  return bridge_impl(hidden, n_rows, d_model, n_layers, w_k, w_v, k_out, v_out, k_scale, v_scale, head_dim,
                     workspace, workspace_bytes, stream);
}

}  // extern "C"

// ------------------------------------------------------------------------------------
// First-generation HySparse layout (GQA 64:4, 64-token block selection, gated window
// branch): the comparison variant.
// ------------------------------------------------------------------------------------
namespace {

struct V1SelPlan {
  int n_split = 1, units = 1, stride = 1;
  size_t off_blse = 0, total = 0;
};

// Parts of 'units' blocks per query so that the launch holds about four workgroups per
// CU (one resident at a time: 128 KB of LDS each), at most kMaxSplit parts per query.
V1SelPlan plan_v1_select(const hs2_seqs* b) {
  V1SelPlan p;
  const int64_t tq = std::max(0, b->total_q);
  const int64_t nblk = ceil_div(std::max(1, b->max_kv_len), kV1Block);
  int64_t u = std::max<int64_t>(2, ceil_div(std::max<int64_t>(1, tq * nblk), 4 * kTargetGroups));
  u = std::max<int64_t>(u, ceil_div(nblk, kMaxSplit));
  p.n_split = (int)ceil_div(nblk, u);
  p.units = (int)ceil_div(nblk, p.n_split);  // rebalanced: n_split * units < nblk + n_split
  p.stride = p.n_split * p.units;  // blocks the parts cover (>= the blocks of max_kv_len)
  p.off_blse = align_up((size_t)tq * kV1Groups * p.n_split * sizeof(V1Partial));
  p.total = p.off_blse + align_up((size_t)tq * kV1Groups * p.stride * kV1GroupHeads * sizeof(float));
  return p;
}

constexpr int kV1SparseUnits = 2;  // block slots per sparse part (4 tiles, as the window part)

struct V1SpPlan {
  int n_split = 2;
  size_t total = 0;
};

V1SpPlan plan_v1_sparse(const hs2_seqs* b, int top_blocks) {
  V1SpPlan p;
  const int64_t tq = std::max(0, b->total_q);
  p.n_split = (int)ceil_div(std::max(1, top_blocks), kV1SparseUnits) + 1;
  p.total = align_up((size_t)tq * kV1Groups * p.n_split * sizeof(V1Partial));
  return p;
}

hs2_status check_v1_common(const hs2_seqs* b, const void* q, const void* k, const void* v, int32_t n_heads,
                           int32_t n_kv_heads, int32_t head_dim, int32_t top_blocks, float scale, const void* out,
                           hs2_dtype dt) {
  hs2_status st = check_batch(b);
  if (st != HS2_OK) return st;
  if (dt != HS2_BF16) return fail(HS2_ERR_UNSUPPORTED, "the v1 layout supports bf16 only (dtype %d)", (int)dt);
  if (n_heads != kHeads || n_kv_heads != kV1Groups || head_dim != kDim)
    return fail(HS2_ERR_UNSUPPORTED, "only n_heads=64, n_kv_heads=4, head_dim=128 are supported (got %d, %d, %d)",
                n_heads, n_kv_heads, head_dim);
  if (b->max_kv_len > kV1MaxBlocks * kV1Block)
    return fail(HS2_ERR_UNSUPPORTED, "max_kv_len must be <= %d for the v1 layout (got %d)", kV1MaxBlocks * kV1Block,
                b->max_kv_len);
  if (top_blocks < 1 || top_blocks > kV1MaxTopBlocks)
    return fail(HS2_ERR_INVALID_ARG, "top_blocks must be in [1, %d] (got %d)", kV1MaxTopBlocks, top_blocks);
  if (!(scale > 0.0f) || !std::isfinite(scale)) return fail(HS2_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (b->total_q > 0 && (!q || !out)) return fail(HS2_ERR_INVALID_ARG, "q and out must not be NULL");
  if (b->total_kv_rows > 0 && (!k || !v)) return fail(HS2_ERR_INVALID_ARG, "k and v must not be NULL");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
    return fail(HS2_ERR_INVALID_ARG, "q, k, v and out must be 16-byte aligned");
  if (out && (out == q || out == k || out == v)) return fail(HS2_ERR_INVALID_ARG, "out aliases an input");
  return HS2_OK;
}

}  // namespace

extern "C" {

size_t hs2_v1_full_attn_select_workspace_size(const hs2_seqs* batch, int32_t n_heads, int32_t n_kv_heads,
                                              int32_t head_dim, int32_t top_blocks, hs2_dtype dt) {
  (void)n_heads;
  (void)n_kv_heads;
  (void)head_dim;
  (void)top_blocks;
  (void)dt;
  if (!batch || batch->total_q < 0 || batch->max_kv_len < 1) return 0;
  return plan_v1_select(batch).total;
}

hs2_status hs2_v1_full_attn_select(const hs2_seqs* batch, const void* q, const void* k, const void* v,
                                   int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, int32_t top_blocks,
                                   float scale, void* out, float* lse, int32_t* blk_idx, int32_t* blk_count,
                                   void* workspace, size_t workspace_bytes, hs2_dtype dt, void* stream) {
  hs2_status st = check_v1_common(batch, q, k, v, n_heads, n_kv_heads, head_dim, top_blocks, scale, out, dt);
  if (st != HS2_OK) return st;
  if (batch->total_q > 0 && !blk_idx) return fail(HS2_ERR_INVALID_ARG, "blk_idx must not be NULL");
  if ((blk_idx && !aligned(blk_idx, 4)) || (blk_count && !aligned(blk_count, 4)) || (lse && !aligned(lse, 4)))
    return fail(HS2_ERR_INVALID_ARG, "blk_idx, blk_count and lse must be 4-byte aligned");
  const V1SelPlan p = plan_v1_select(batch);
  if (workspace_bytes < p.total || (p.total > 0 && !workspace))
    return fail(HS2_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the required %zu", workspace_bytes,
                p.total);
  if (workspace && !aligned(workspace, kAlign)) return fail(HS2_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (batch->total_q == 0) return ok();

  hipStream_t s = static_cast<hipStream_t>(stream);
  V1AttnArgs a{};
  a.b = to_dev(batch);
  a.q = static_cast<const __bf16*>(q);
  a.k = static_cast<const __bf16*>(k);
  a.v = static_cast<const __bf16*>(v);
  a.c2 = scale * kLog2e;
  a.n_split = p.n_split;
  a.split_units = p.units;
  a.part = static_cast<V1Partial*>(workspace);
  a.blse = at<float>(workspace, p.off_blse);
  a.blse_stride = p.stride;
  LaunchMarks mk(s);
  hipError_t e = mk.before(0);
  if (e == hipSuccess) e = launch_v1_attn(a, false, batch->total_q * p.n_split, s);
  if (e == hipSuccess) e = mk.after(0);
  if (e != hipSuccess) return hip_fail(e, "v1 attention launch");
  V1SelectArgs c{};
  c.b = a.b;
  c.part = a.part;
  c.n_split = p.n_split;
  c.split_units = p.units;
  c.blse = a.blse;
  c.blse_stride = p.stride;
  c.out = static_cast<__bf16*>(out);
  c.lse = lse;
  c.blk_idx = blk_idx;
  c.blk_count = blk_count;
  c.top_blocks = top_blocks;
  e = mk.before(1);
  if (e == hipSuccess) e = launch_v1_select(c, s);
  if (e == hipSuccess) e = mk.after(1);
  if (e != hipSuccess) return hip_fail(e, "v1 combine and block selection launch");
  return ok();
}

size_t hs2_v1_sparse_attn_workspace_size(const hs2_seqs* batch, int32_t n_heads, int32_t n_kv_heads,
                                         int32_t head_dim, int32_t top_blocks, hs2_dtype dt) {
  (void)n_heads;
  (void)n_kv_heads;
  (void)head_dim;
  (void)dt;
  if (!batch || batch->total_q < 0 || top_blocks < 1) return 0;
  return plan_v1_sparse(batch, top_blocks).total;
}

hs2_status hs2_v1_sparse_attn(const hs2_seqs* batch, const void* q, const void* k, const void* v,
                              const int32_t* blk_idx, int32_t top_blocks, const void* k_swa, const void* v_swa,
                              int32_t swa_slots, int32_t window, const float* gate_sparse, const float* gate_swa,
                              int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, float scale, void* out,
                              void* workspace, size_t workspace_bytes, hs2_dtype dt, void* stream) {
  hs2_status st = check_v1_common(batch, q, k, v, n_heads, n_kv_heads, head_dim, top_blocks, scale, out, dt);
  if (st != HS2_OK) return st;
  if (window < 1 || swa_slots < window || swa_slots > (1 << 20))
    return fail(HS2_ERR_INVALID_ARG, "need 1 <= window <= swa_slots <= 2^20 (got window %d, swa_slots %d)", window,
                swa_slots);
  if (batch->total_q > 0 && (!blk_idx || !k_swa || !v_swa || !gate_sparse || !gate_swa))
    return fail(HS2_ERR_INVALID_ARG, "blk_idx, k_swa, v_swa, gate_sparse and gate_swa must not be NULL");
  if (!aligned(k_swa, 16) || !aligned(v_swa, 16) || !aligned(blk_idx, 4) || !aligned(gate_sparse, 4) ||
      !aligned(gate_swa, 4))
    return fail(HS2_ERR_INVALID_ARG, "k_swa and v_swa must be 16-byte aligned, blk_idx and the gates 4-byte");
  if (out && (out == k_swa || out == v_swa)) return fail(HS2_ERR_INVALID_ARG, "out aliases an input");
  const V1SpPlan p = plan_v1_sparse(batch, top_blocks);
  if (workspace_bytes < p.total || (p.total > 0 && !workspace))
    return fail(HS2_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the required %zu", workspace_bytes,
                p.total);
  if (workspace && !aligned(workspace, kAlign)) return fail(HS2_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (batch->total_q == 0) return ok();

  hipStream_t s = static_cast<hipStream_t>(stream);
  V1AttnArgs a{};
  a.b = to_dev(batch);
  a.q = static_cast<const __bf16*>(q);
  a.k = static_cast<const __bf16*>(k);
  a.v = static_cast<const __bf16*>(v);
  a.k_swa = static_cast<const __bf16*>(k_swa);
  a.v_swa = static_cast<const __bf16*>(v_swa);
  a.swa_slots = swa_slots;
  a.window = window;
  a.blk = blk_idx;
  a.top_blocks = top_blocks;
  a.c2 = scale * kLog2e;
  a.n_split = p.n_split;
  a.split_units = kV1SparseUnits;
  a.part = static_cast<V1Partial*>(workspace);
  LaunchMarks mk(s);
  hipError_t e = mk.before(0);
  if (e == hipSuccess) e = launch_v1_attn(a, true, batch->total_q * p.n_split, s);
  if (e == hipSuccess) e = mk.after(0);
  if (e != hipSuccess) return hip_fail(e, "v1 sparse attention launch");
  V1GateArgs c{};
  c.b = a.b;
  c.part = a.part;
  c.n_split = p.n_split;
  c.gate_sparse = gate_sparse;
  c.gate_swa = gate_swa;
  c.out = static_cast<__bf16*>(out);
  e = mk.before(1);
  if (e == hipSuccess) e = launch_v1_gate(c, s);
  if (e == hipSuccess) e = mk.after(1);
  if (e != hipSuccess) return hip_fail(e, "v1 gated combine launch");
  return ok();
}

}  // extern "C"
