// Host-only driver of libhs2's entry points, built with AddressSanitizer and
// UndefinedBehaviorSanitizer together with csrc/hs2_api.cpp (the argument checks, the
// split planner and the workspace layout) and run without a GPU.
//
// The kernel launchers are replaced by stubs that launch nothing. Each stub checks what
// the planner hands it: every pointer it derived from the workspace, with the extent the
// kernel addresses through it, lies inside the workspace the size query reported; work
// lists hold distinct (query, split) items in query order with split 0 first and every
// query present; grids are positive. The driver calls every entry point with fuzzed
// descriptors (a workspace of exactly the reported size must be accepted, one byte less
// rejected) and every rejection path. Exit status 0 means every check held.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "hs2.h"
#include "hs2_launch.h"

namespace {

int g_fail = 0;
const char* g_where = "";
uintptr_t g_ws_lo = 0, g_ws_hi = 0;  // workspace of the call in progress
int g_launches = 0;

#define CHECK(c)                                                                        \
  do {                                                                                  \
    if (!(c)) {                                                                         \
      std::fprintf(stderr, "check failed (%s): %s, line %d\n", g_where, #c, __LINE__); \
      if (++g_fail > 20) std::exit(1);                                                  \
    }                                                                                   \
  } while (0)

// p .. p+bytes must lie inside the workspace (null pointers are not addressed).
void in_ws(const void* p, size_t bytes) {
  if (!p || bytes == 0) return;
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  CHECK(a >= g_ws_lo && a + bytes <= g_ws_hi);
}

void check_list(const hs2::WorkList& wl, int total_q, int n_split) {
  if (wl.n == 0) return;
  CHECK(wl.n <= hs2::kMaxWorkItems);
  int prev_q = -1, prev_s = -1;
  std::vector<char> seen(total_q, 0);
  for (int j = 0; j < wl.n; ++j) {
    const int q = (int)(wl.item[j] >> 9), s = (int)(wl.item[j] & 511u);
    CHECK(q >= 0 && q < total_q && s >= 0 && s < n_split);
    if (q == prev_q) CHECK(s == prev_s + 1);
    else CHECK(q > prev_q && s == 0);
    if (q >= 0 && q < total_q) seen[q] = 1;
    prev_q = q;
    prev_s = s;
  }
  for (int q = 0; q < total_q; ++q) CHECK(seen[q]);
}

size_t part_bytes(const hs2::SeqsDev& b, int n_split) { return (size_t)b.total_q * n_split * sizeof(hs2::Partial); }

}  // namespace

// ---- stubs of the HIP runtime calls the entry points make ----
extern "C" hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
extern "C" const char* hipGetErrorString(hipError_t) { return "stub"; }

// ---- stub launchers ----
namespace hs2 {

static void attn_common(const AttnArgs& a, const WorkList& wl, bool gather, int grid, uint32_t* hist,
                        uint32_t* counters) {
  ++g_launches;
  CHECK(grid > 0 && a.n_split >= 1 && a.split_keys >= kTile && a.split_keys % kTile == 0);
  CHECK((int64_t)a.n_split * a.split_keys >= (gather ? 0 : 1));
  check_list(wl, a.b.total_q, a.n_split);
  if (wl.n > 0) CHECK(grid == wl.n);
  else CHECK(grid == a.b.total_q * a.n_split);
  if (!gather) CHECK((int64_t)a.n_split * a.split_keys >= a.b.max_kv_len || wl.n > 0);
  if (a.n_split > 1) in_ws(a.part, part_bytes(a.b, a.n_split));
  in_ws(a.lse2, (size_t)a.b.total_q * kHeads * 4);
  in_ws(hist, (size_t)a.b.total_q * kHistBins * 4);
  in_ws(counters, (size_t)a.b.total_q * 16);
  in_ws(a.plan_miss, (size_t)a.b.total_q * 4);
  if (wl.n > 0 && !gather) CHECK(a.plan_miss != nullptr);
}
hipError_t launch_attn_bf16(const AttnArgs& a, const WorkList& wl, int grid, uint32_t* hist, uint32_t* counters,
                            hipStream_t) {
  attn_common(a, wl, false, grid, hist, counters);
  return hipSuccess;
}
hipError_t launch_attn_fp8kv(const AttnArgs& a, const WorkList& wl, int grid, uint32_t* hist, uint32_t* counters,
                             hipStream_t) {
  attn_common(a, wl, false, grid, hist, counters);
  return hipSuccess;
}
hipError_t launch_attn_f32(const AttnArgs& a, bool gather, int grid, uint32_t* hist, uint32_t* counters,
                           hipStream_t) {
  attn_common(a, WorkList{}, gather, grid, hist, counters);
  return hipSuccess;
}
hipError_t launch_sparse_attn(const AttnArgs& a, bool, bool, int grid, hipStream_t) {
  ++g_launches;
  CHECK(grid == a.b.total_q * a.n_split && a.split_keys % kTile == 0 && a.split_keys >= kTile);
  CHECK(a.n_split <= 256 || a.split_keys > sparse_slots(false) * kTile);
  if (a.n_split > 1) in_ws(a.part, part_bytes(a.b, a.n_split));
  else CHECK(a.part == nullptr);
  return hipSuccess;
}
hipError_t launch_combine(const CombineArgs& a, bool, hipStream_t) {
  ++g_launches;
  CHECK(a.n_split >= 1);
  in_ws(a.part, part_bytes(a.b, a.n_split));
  in_ws(a.lse2, (size_t)a.b.total_q * kHeads * 4);
  in_ws(a.hist, (size_t)a.b.total_q * kHistBins * 4);
  in_ws(a.counters, (size_t)a.b.total_q * 16);
  in_ws(a.plan_miss, (size_t)a.b.total_q * 4);
  return hipSuccess;
}
static int g_max_tiles = 0;
hipError_t launch_qtile_prep(const SeqsDev& b, int2* tiles, int max_tiles, hipStream_t) {
  ++g_launches;
  CHECK(max_tiles >= b.total_q / kQTile + b.num_seqs);
  in_ws(tiles, (size_t)max_tiles * sizeof(int2));
  g_max_tiles = max_tiles;
  return hipSuccess;
}
hipError_t launch_attn_chunk(const AttnArgs& a, const int2* tiles, int max_tiles, hipStream_t) {
  ++g_launches;
  CHECK(max_tiles == g_max_tiles && a.n_split >= 1);
  in_ws(tiles, (size_t)max_tiles * sizeof(int2));
  if (!a.direct) in_ws(a.part, part_bytes(a.b, a.n_split));
  CHECK(!a.direct || a.n_split == 1);
  in_ws(a.lse2, (size_t)a.b.total_q * kHeads * 4);
  return hipSuccess;
}
static void score_common(const ScoreArgs& a, const WorkList& wl) {
  ++g_launches;
  check_list(wl, a.b.total_q, a.n_split);
  CHECK(a.score_stride >= (int64_t)a.b.max_kv_len - a.window + 1);
  in_ws(a.scores, (size_t)a.b.total_q * a.score_stride * 4);
  in_ws(a.hist, (size_t)a.b.total_q * kHistBins * 4);
  in_ws(a.lse2, (size_t)a.b.total_q * kHeads * 4);
  in_ws(a.plan_miss, (size_t)a.b.total_q * 4);
  CHECK((int64_t)a.n_split * a.split_keys >= (int64_t)a.b.max_kv_len - a.window + 1 || wl.n > 0);
  CHECK((a.scores == nullptr) != (a.lists == nullptr));
  if (a.lists) {  // the regions of all of a split's lists are checked by the top-k stubs
    CHECK(a.list_cap >= 32 && a.list_cap % 32 == 0);
    CHECK((int64_t)a.list_cap * 8 >= a.split_keys);
    in_ws(a.list_thr, (size_t)a.b.total_q * a.n_split * sizeof(int32_t));
  }
}
hipError_t launch_score_chunk(const ScoreArgs& a, const int2* tiles, int max_tiles, hipStream_t) {
  score_common(a, WorkList{});
  CHECK(a.split_keys <= kScoreSplitMax);
  in_ws(tiles, (size_t)max_tiles * sizeof(int2));
  return hipSuccess;
}
hipError_t launch_score_bf16(const ScoreArgs& a, const WorkList& wl, hipStream_t) {
  score_common(a, wl);
  return hipSuccess;
}
hipError_t launch_score_fp8kv(const ScoreArgs& a, const WorkList& wl, hipStream_t) {
  score_common(a, wl);
  return hipSuccess;
}
hipError_t launch_score_f32(const ScoreArgs& a, hipStream_t) {
  score_common(a, WorkList{});
  return hipSuccess;
}
static void topk_common(const TopkArgs& a) {
  ++g_launches;
  CHECK(a.n_split >= 1 && (int64_t)a.n_split * a.split_len >= (int64_t)a.b.max_kv_len - a.window + 1);
  if (a.top_k > 0) {
    in_ws(a.scores, (size_t)a.b.total_q * a.score_stride * 4);
    in_ws(a.above, (size_t)a.b.total_q * a.top_k * 4);
    in_ws(a.cand, (size_t)a.b.total_q * kCandCap * sizeof(uint2));
  }
  in_ws(a.hist, (size_t)a.b.total_q * kHistBins * 4);
  in_ws(a.counters, (size_t)a.b.total_q * 16);
  in_ws(a.miss_attn, (size_t)a.b.total_q * 4);
  in_ws(a.miss_score, (size_t)a.b.total_q * 4);
  if (a.lists) {
    CHECK(a.scores == nullptr && (a.list_waves == 4 || a.list_waves == 8));
    CHECK((int64_t)a.list_splits * a.list_split_keys >= (int64_t)a.b.max_kv_len - a.window + 1);
    CHECK((int64_t)a.list_cap * a.list_waves >= a.list_split_keys);
    const size_t nl = (size_t)a.b.total_q * a.list_splits * a.list_waves;
    in_ws(a.lists, nl * a.list_cap * sizeof(uint2));
    in_ws(a.list_count, nl * sizeof(int32_t));
    in_ws(a.list_thr, (size_t)a.b.total_q * a.list_splits * sizeof(int32_t));
  }
}
hipError_t launch_topk_filter(const TopkArgs& a, hipStream_t) {
  topk_common(a);
  return hipSuccess;
}
hipError_t launch_topk_finish(const TopkArgs& a, hipStream_t) {
  topk_common(a);
  return hipSuccess;
}
hipError_t launch_bridge_transpose(const BridgeArgs& a, const uint16_t* const* w, int32_t n_mats, uint16_t* wt,
                                   hipStream_t) {
  ++g_launches;
  CHECK(n_mats == a.n_mats && w != nullptr);
  in_ws(wt, (size_t)n_mats * kDim * a.d_model * 2);
  return hipSuccess;
}
hipError_t launch_bridge_gemm(const BridgeArgs& a, const BridgeOut&, hipStream_t) {
  ++g_launches;
  CHECK(a.n_rows > 0);
  in_ws(a.wt, (size_t)a.n_mats * kDim * a.d_model * 2);
  return hipSuccess;
}
hipError_t launch_bridge_append(const AppendArgs& a, const BridgeOut&, hipStream_t) {
  ++g_launches;
  CHECK(a.n_slices * kAppendSlice == a.d_model);
  in_ws(a.part, (size_t)a.n_slices * a.n_new * a.n_mats * kDim * 4);
  return hipSuccess;
}
hipError_t launch_v1_attn(const V1AttnArgs& a, bool sparse, int grid, hipStream_t) {
  ++g_launches;
  CHECK(grid == a.b.total_q * a.n_split);
  in_ws(a.part, (size_t)a.b.total_q * kV1Groups * a.n_split * sizeof(V1Partial));
  if (!sparse) in_ws(a.blse, (size_t)a.b.total_q * kV1Groups * a.blse_stride * kV1GroupHeads * 4);
  return hipSuccess;
}
hipError_t launch_v1_select(const V1SelectArgs& a, hipStream_t) {
  ++g_launches;
  in_ws(a.part, (size_t)a.b.total_q * kV1Groups * a.n_split * sizeof(V1Partial));
  in_ws(a.blse, (size_t)a.b.total_q * kV1Groups * a.blse_stride * kV1GroupHeads * 4);
  return hipSuccess;
}
hipError_t launch_v1_gate(const V1GateArgs& a, hipStream_t) {
  ++g_launches;
  in_ws(a.part, (size_t)a.b.total_q * kV1Groups * a.n_split * sizeof(V1Partial));
  return hipSuccess;
}

}  // namespace hs2

namespace {

// Device pointers of the calls below are never dereferenced on the host: fake, aligned.
void* fake(uintptr_t k) { return reinterpret_cast<void*>((uintptr_t)0x100000000ull * k); }

struct Desc {
  std::vector<int32_t> lens;
  std::vector<int32_t> qper;  // queries per sequence
  bool host_lens = false;
  hs2_seqs b{};
  void make() {
    b.num_seqs = (int32_t)lens.size();
    b.kv_start = (const int64_t*)fake(1);
    b.kv_len = (const int32_t*)fake(2);
    b.q_start = (const int32_t*)fake(3);
    b.q_pos = (const int32_t*)fake(4);
    int64_t rows = 0;
    int tq = 0, mx = 1, mq = 0;
    for (size_t s = 0; s < lens.size(); ++s) {
      rows += lens[s];
      tq += qper[s];
      mx = std::max(mx, lens[s]);
      mq = std::max(mq, qper[s]);
    }
    b.total_q = tq;
    b.max_kv_len = mx;
    b.total_kv_rows = rows;
    b.max_q_per_seq = mq;
    b.kv_len_host = host_lens ? lens.data() : nullptr;
  }
};

// Calls fn(ws, bytes) with a workspace of exactly `need` bytes (accepted) and with one
// byte less (rejected with HS2_ERR_WORKSPACE when need > 0). The workspace is device
// memory the host never touches, so a fake 256-byte aligned address stands for it.
template <typename F>
void with_workspace(size_t need, F&& fn) {
  char* ws = static_cast<char*>(fake(4096));
  g_ws_lo = reinterpret_cast<uintptr_t>(ws);
  g_ws_hi = g_ws_lo + need;
  const int st = fn(need > 0 ? ws : nullptr, need);
  CHECK(st == HS2_OK);
  if (st != HS2_OK) std::fprintf(stderr, "  status %d: %s\n", st, hs2_last_error());
  if (need > 0) CHECK(fn(ws, need - 1) == HS2_ERR_WORKSPACE);
}

void run_attention_calls(Desc& d, std::mt19937& rng) {
  d.make();
  const hs2_seqs* b = &d.b;
  const int window = std::uniform_int_distribution<int>(1, 300)(rng) == 1 ? (1 << 18)
                                                                       : std::uniform_int_distribution<int>(1, 256)(rng);
  const int top_k = std::uniform_int_distribution<int>(0, 8)(rng) == 0 ? 0 : std::uniform_int_distribution<int>(1, HS2_MAX_TOP_K)(rng);
  const float sc = 0.088f;
  for (hs2_dtype dt : {HS2_BF16, HS2_F32, HS2_FP8_E4M3}) {
    g_where = "select";
    const size_t need = hs2_full_attn_select_workspace_size(b, 64, 128, window, top_k, dt);
    with_workspace(need, [&](void* ws, size_t n) {
      if (dt == HS2_FP8_E4M3)
        return (int)hs2_full_attn_select_fp8kv(b, fake(5), fake(6), fake(7), 0.05f, 0.03f, 64, 128, window, top_k, sc,
                                               fake(8), (float*)fake(9), (int32_t*)fake(10), (int32_t*)fake(11), ws, n,
                                               nullptr);
      return (int)hs2_full_attn_select(b, fake(5), fake(6), fake(7), 64, 128, window, top_k, sc, fake(8),
                                       (float*)fake(9), (int32_t*)fake(10), (int32_t*)fake(11), ws, n, dt, nullptr);
    });
    g_where = "sparse";
    const size_t need2 = hs2_sparse_attn_workspace_size(b, 64, 128, window, top_k, dt);
    if (need2 > 0) with_workspace(need2, [&](void* ws, size_t n) {
      if (dt == HS2_FP8_E4M3)
        return (int)hs2_sparse_attn_fp8kv(b, fake(5), fake(6), fake(7), 0.05f, 0.03f, (const int32_t*)fake(10), 64, 128,
                                          window, top_k, sc, fake(8), nullptr, ws, n, nullptr);
      return (int)hs2_sparse_attn(b, fake(5), fake(6), fake(7), (const int32_t*)fake(10), 64, 128, window, top_k, sc,
                                  fake(8), nullptr, ws, n, dt, nullptr);
    });
    if (dt != HS2_FP8_E4M3) {
      g_where = "causal";
      const size_t need3 = hs2_causal_attn_workspace_size(b, 64, 128, dt);
      if (need3 > 0) with_workspace(need3, [&](void* ws, size_t n) {
        return (int)hs2_causal_attn(b, fake(5), fake(6), fake(7), 64, 128, sc, fake(8), (float*)fake(9), ws, n, dt,
                                    nullptr);
      });
    }
  }
  if (d.b.max_kv_len <= hs2::kV1MaxBlocks * hs2::kV1Block) {
    const int tb = std::uniform_int_distribution<int>(1, hs2::kV1MaxTopBlocks)(rng);
    g_where = "v1 select";
    with_workspace(hs2_v1_full_attn_select_workspace_size(b, 64, 4, 128, tb, HS2_BF16), [&](void* ws, size_t n) {
      return (int)hs2_v1_full_attn_select(b, fake(5), fake(6), fake(7), 64, 4, 128, tb, sc, fake(8), (float*)fake(9),
                                          (int32_t*)fake(10), (int32_t*)fake(11), ws, n, HS2_BF16, nullptr);
    });
    g_where = "v1 sparse";
    with_workspace(hs2_v1_sparse_attn_workspace_size(b, 64, 4, 128, tb, HS2_BF16), [&](void* ws, size_t n) {
      return (int)hs2_v1_sparse_attn(b, fake(5), fake(6), fake(7), (const int32_t*)fake(10), tb, fake(12), fake(13),
                                     std::max(window, 128), 128, (const float*)fake(14), (const float*)fake(15), 64, 4,
                                     128, sc, fake(8), ws, n, HS2_BF16, nullptr);
    });
  }
}

void rejections() {
  g_where = "rejections";
  Desc d;
  d.lens = {5000, 3000};
  d.qper = {1, 1};
  d.host_lens = true;
  d.make();
  void* ws = fake(4096);
  const size_t n = (size_t)1 << 34;
  auto sel = [&](const hs2_seqs* b, int h, int dim, int w, int k, float sc, void* q, void* out, int32_t* si) {
    return hs2_full_attn_select(b, q, fake(6), fake(7), h, dim, w, k, sc, out, nullptr, si, nullptr, ws, n, HS2_BF16,
                                nullptr);
  };
  CHECK(sel(nullptr, 64, 128, 128, 1024, 0.1f, fake(5), fake(8), (int32_t*)fake(10)) == HS2_ERR_INVALID_ARG);
  CHECK(sel(&d.b, 32, 128, 128, 1024, 0.1f, fake(5), fake(8), (int32_t*)fake(10)) == HS2_ERR_UNSUPPORTED);
  CHECK(sel(&d.b, 64, 64, 128, 1024, 0.1f, fake(5), fake(8), (int32_t*)fake(10)) == HS2_ERR_UNSUPPORTED);
  CHECK(sel(&d.b, 64, 128, 0, 1024, 0.1f, fake(5), fake(8), (int32_t*)fake(10)) == HS2_ERR_INVALID_ARG);
  CHECK(sel(&d.b, 64, 128, (1 << 18) + 1, 1024, 0.1f, fake(5), fake(8), (int32_t*)fake(10)) == HS2_ERR_INVALID_ARG);
  CHECK(sel(&d.b, 64, 128, 128, HS2_MAX_TOP_K + 1, 0.1f, fake(5), fake(8), (int32_t*)fake(10)) == HS2_ERR_INVALID_ARG);
  CHECK(sel(&d.b, 64, 128, 128, 1024, 0.0f, fake(5), fake(8), (int32_t*)fake(10)) == HS2_ERR_INVALID_ARG);
  CHECK(sel(&d.b, 64, 128, 128, 1024, 1.0f / 0.0f, fake(5), fake(8), (int32_t*)fake(10)) == HS2_ERR_INVALID_ARG);
  CHECK(sel(&d.b, 64, 128, 128, 1024, 0.1f, nullptr, fake(8), (int32_t*)fake(10)) == HS2_ERR_INVALID_ARG);
  CHECK(sel(&d.b, 64, 128, 128, 1024, 0.1f, fake(5), fake(5), (int32_t*)fake(10)) == HS2_ERR_INVALID_ARG);  // alias
  CHECK(sel(&d.b, 64, 128, 128, 1024, 0.1f, fake(5), fake(8), nullptr) == HS2_ERR_INVALID_ARG);
  CHECK(sel(&d.b, 64, 128, 128, 1024, 0.1f, (char*)fake(5) + 8, fake(8), (int32_t*)fake(10)) == HS2_ERR_INVALID_ARG);
  std::vector<int32_t> bad_host = {5000, 9000};  // above max_kv_len
  hs2_seqs b2 = d.b;
  b2.kv_len_host = bad_host.data();
  CHECK(sel(&b2, 64, 128, 128, 1024, 0.1f, fake(5), fake(8), (int32_t*)fake(10)) == HS2_ERR_INVALID_ARG);
  bad_host[1] = -1;
  CHECK(sel(&b2, 64, 128, 128, 1024, 0.1f, fake(5), fake(8), (int32_t*)fake(10)) == HS2_ERR_INVALID_ARG);
  b2 = d.b;
  b2.num_seqs = 0;
  CHECK(sel(&b2, 64, 128, 128, 1024, 0.1f, fake(5), fake(8), (int32_t*)fake(10)) == HS2_ERR_INVALID_ARG);
  b2 = d.b;
  b2.kv_len = nullptr;
  CHECK(sel(&b2, 64, 128, 128, 1024, 0.1f, fake(5), fake(8), (int32_t*)fake(10)) == HS2_ERR_INVALID_ARG);
  b2 = d.b;
  b2.max_kv_len = 0;
  CHECK(sel(&b2, 64, 128, 128, 1024, 0.1f, fake(5), fake(8), (int32_t*)fake(10)) == HS2_ERR_INVALID_ARG);
  CHECK(hs2_full_attn_select(&d.b, fake(5), fake(6), fake(7), 64, 128, 128, 1024, 0.1f, fake(8), nullptr,
                             (int32_t*)fake(10), nullptr, ws, 16, HS2_BF16, nullptr) == HS2_ERR_WORKSPACE);
  CHECK(hs2_full_attn_select(&d.b, fake(5), fake(6), fake(7), 64, 128, 128, 1024, 0.1f, fake(8), nullptr,
                             (int32_t*)fake(10), nullptr, (char*)ws + 64, n - 64, HS2_BF16, nullptr) == HS2_ERR_WORKSPACE);
  CHECK(hs2_full_attn_select(&d.b, fake(5), fake(6), fake(7), 64, 128, 128, 1024, 0.1f, fake(8), nullptr,
                             (int32_t*)fake(10), nullptr, ws, n, HS2_FP8_E4M3, nullptr) == HS2_ERR_UNSUPPORTED);
  CHECK(hs2_full_attn_select_fp8kv(&d.b, fake(5), fake(6), fake(7), 0.0f, 0.03f, 64, 128, 128, 1024, 0.1f, fake(8),
                                   nullptr, (int32_t*)fake(10), nullptr, ws, n, nullptr) == HS2_ERR_INVALID_ARG);
  CHECK(hs2_sparse_attn(&d.b, fake(5), fake(6), fake(7), nullptr, 64, 128, 128, 1024, 0.1f, fake(8), nullptr, ws, n,
                        HS2_BF16, nullptr) == HS2_ERR_INVALID_ARG);
  CHECK(hs2_causal_attn(&d.b, fake(5), fake(6), fake(7), 64, 128, 0.1f, fake(8), nullptr, ws, n, HS2_FP8_E4M3,
                        nullptr) == HS2_ERR_UNSUPPORTED);
  // bridging
  void* wk[8] = {fake(20), fake(21), fake(22), fake(23), fake(24), fake(25), fake(26), fake(27)};
  void* ko[8] = {fake(30), fake(31), fake(32), fake(33), fake(34), fake(35), fake(36), fake(37)};
  CHECK(hs2_bridge_kv(fake(40), 1000, 2048, 3, wk, wk, ko, ko, 64, ws, n, HS2_BF16, nullptr) == HS2_ERR_UNSUPPORTED);
  CHECK(hs2_bridge_kv(fake(40), 1000, 2000, 3, wk, wk, ko, ko, 128, ws, n, HS2_BF16, nullptr) == HS2_ERR_UNSUPPORTED);
  CHECK(hs2_bridge_kv(fake(40), 1000, 2048, 9, wk, wk, ko, ko, 128, ws, n, HS2_BF16, nullptr) == HS2_ERR_UNSUPPORTED);
  CHECK(hs2_bridge_kv(fake(40), -1, 2048, 3, wk, wk, ko, ko, 128, ws, n, HS2_BF16, nullptr) == HS2_ERR_INVALID_ARG);
  CHECK(hs2_bridge_kv(fake(40), 1000, 2048, 3, nullptr, wk, ko, ko, 128, ws, n, HS2_BF16, nullptr) == HS2_ERR_INVALID_ARG);
  CHECK(hs2_bridge_kv(fake(40), 1000, 2048, 3, wk, wk, ko, ko, 128, ws, 8, HS2_BF16, nullptr) == HS2_ERR_WORKSPACE);
  CHECK(hs2_bridge_kv(fake(40), 1000, 2048, 3, wk, wk, ko, ko, 128, ws, n, HS2_F32, nullptr) == HS2_ERR_UNSUPPORTED);
  void* ko_alias[3] = {fake(40), fake(31), fake(32)};
  CHECK(hs2_bridge_kv(fake(40), 1000, 2048, 3, wk, wk, ko_alias, ko, 128, ws, n, HS2_BF16, nullptr) == HS2_ERR_INVALID_ARG);
  CHECK(hs2_bridge_kv_append(fake(40), 65537, (const int64_t*)fake(41), 100, 2048, 3, wk, wk, ko, ko, 128, ws, n,
                             HS2_BF16, nullptr) == HS2_ERR_INVALID_ARG);
  CHECK(hs2_bridge_kv_append(fake(40), 4, (const int64_t*)fake(41), 100, 2000, 3, wk, wk, ko, ko, 128, ws, n, HS2_BF16,
                             nullptr) == HS2_ERR_UNSUPPORTED);
  CHECK(hs2_set_kernel_events(nullptr, 17) == HS2_ERR_INVALID_ARG);
  CHECK(hs2_set_kernel_events(nullptr, 0) == HS2_OK);
}

void bridging_calls(std::mt19937& rng) {
  for (int it = 0; it < 40; ++it) {
    const int d_model = 64 * std::uniform_int_distribution<int>(1, 64)(rng);
    const int L = std::uniform_int_distribution<int>(1, 8)(rng);
    const int64_t rows = std::uniform_int_distribution<int64_t>(0, 3000000)(rng);
    void* wk[8];
    void* ko[8];
    for (int l = 0; l < 8; ++l) {
      wk[l] = fake(50 + l);
      ko[l] = fake(60 + l);
    }
    g_where = "bridge";
    with_workspace(hs2_bridge_kv_workspace_size(d_model, L, 128), [&](void* ws, size_t n) {
      return (int)hs2_bridge_kv(fake(40), rows, d_model, L, wk, wk, ko, ko, 128, ws, n, HS2_BF16, nullptr);
    });
    if (d_model % hs2::kAppendSlice == 0) {
      const int n_new = std::uniform_int_distribution<int>(1, 65536)(rng);
      g_where = "bridge append";
      with_workspace(hs2_bridge_kv_append_workspace_size(n_new, d_model, L, 128), [&](void* ws, size_t n) {
        return (int)hs2_bridge_kv_append(fake(40), n_new, (const int64_t*)fake(41), rows, d_model, L, wk, wk, ko, ko,
                                         128, ws, n, HS2_BF16, nullptr);
      });
    }
  }
}

}  // namespace

int main() {
  std::mt19937 rng(20261203u);
  rejections();
  bridging_calls(rng);
  // fixed shapes of the benchmark workloads
  {
    Desc d;
    d.lens.assign(64, 131072);
    d.qper.assign(64, 1);
    d.host_lens = true;
    run_attention_calls(d, rng);
    d.host_lens = false;
    run_attention_calls(d, rng);
    Desc c;
    c.lens = {262144};
    c.qper = {4096};
    run_attention_calls(c, rng);
  }
  // fuzzed descriptors: decode batches (one query per sequence, with and without host
  // lengths) and batches with several queries per sequence
  for (int it = 0; it < 300; ++it) {
    Desc d;
    const int S = std::uniform_int_distribution<int>(1, it % 3 == 0 ? 600 : 40)(rng);
    const bool decode = it % 2 == 0;
    const int len_hi = std::uniform_int_distribution<int>(0, 4)(rng) == 0 ? 3000000 : 300000;
    for (int s = 0; s < S; ++s) {
      d.lens.push_back(std::uniform_int_distribution<int>(0, 20)(rng) == 0 ? 0
                                                                           : std::uniform_int_distribution<int>(1, len_hi)(rng));
      d.qper.push_back(decode ? 1 : std::uniform_int_distribution<int>(0, 40)(rng));
    }
    d.host_lens = std::uniform_int_distribution<int>(0, 1)(rng) == 1;
    run_attention_calls(d, rng);
  }
  std::printf("launches checked: %d, failures: %d\n", g_launches, g_fail);
  return g_fail == 0 ? 0 : 1;
}
