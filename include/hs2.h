/*
 * hs2.h -- C ABI of the HySparse2 attention hot path on AMD Instinct MI355X (gfx950).
 *
 * The HySparse2 operations, with one KV head shared by 64 query heads (MQA), and at the
 * end the first-generation layout (GQA 64:4, block selection, gated window branch) as a
 * comparison variant (hs2_v1_*):
 *   hs2_bridge_kv         KV Bridging: one read of the self-decoder hidden states is
 *                         projected through separate K/V weights for several layers.
 *   hs2_full_attn_select  the cross-decoder full-attention (selector) layer: exact
 *                         causal attention, plus, for each query, the top_k keys outside
 *                         the forced window ranked by their softmax probability summed
 *                         over the query heads.
 *   hs2_sparse_attn       a sparse layer of the same hybrid block: attention over the
 *                         forced window plus the selector's rows only, on the selector's
 *                         KV cache.
 *
 * Sources (page title and section; the pages are news and commentary on the HySparse2
 * paper):
 *   [arex]     arex-research.com, "Xiaomi MiMo lead Luo Fuli publishes the MiMo-V3 core
 *              architecture HySparse2", sections "Outer KV Bridging, inner KV Reuse" and
 *              "Numbers computed on three 80B-A3B models".
 *   [toolnavs] toolnavs.com (German) article on the core architecture of Xiaomi MiMo-V3,
 *              section "Was HySparse2 tut".
 *   [zgeo]     zgeo.com.cn, "Xiaomi HySparse2 architecture deep dive", section
 *              "Core technical principles".
 *
 * Conventions shared by every call
 *   - All tensors are row-major, contiguous and 16-byte aligned device memory unless a
 *     parameter says "host".
 *   - Q:   [total_q][n_heads][head_dim]          (query rows of one layer)
 *   - K,V: [total_kv_rows][head_dim]             (one KV head; sequences packed)
 *   - Positions are sequence-local: row kv_start[s] + j holds position j of sequence s.
 *   - The window of query position t is the `window` most recent positions including t:
 *     rows max(0, t-window+1) .. t. Candidates for selection are rows 0 .. t-window.
 *   - Selected indices are sequence-local candidate positions, ascending, padded with -1.
 *   - LSE outputs are natural-log log-sum-exp of the scaled logits, fp32.
 *   - The caller owns every buffer and the stream. The library allocates nothing, keeps
 *     no state between calls (apart from the per-thread attachment of the measurement
 *     hook hs2_set_kernel_events) and never synchronises the stream. Inputs are read-only;
 *     outputs and the workspace must not alias any input or each other.
 *   - `stream` is a hipStream_t (NULL = the null stream). Work is enqueued and the call
 *     returns; device faults surface at the caller's next synchronisation.
 *   - Argument checks run on the host before anything is enqueued. A failing check
 *     returns a negative hs2_status, enqueues nothing and sets hs2_last_error().
 *     A failing launch returns HS2_ERR_HIP.
 *   - Device-side descriptor values are not read by the host. A query whose descriptor
 *     is inconsistent (q_pos outside [0, kv_len) or not below max_kv_len, rows outside
 *     [0, total_kv_rows)) is not computed: its outputs are NaN and its sel_count is -1.
 *     No memory outside the given buffers is touched. A kv_len_host value outside
 *     [0, max_kv_len] returns HS2_ERR_INVALID_ARG.
 *   - Supported shapes: n_heads == 64, head_dim == 128 (the MQA layout of the pages,
 *     [arex] "Numbers computed on three 80B-A3B models"); anything else returns
 *     HS2_ERR_UNSUPPORTED. 1 <= window <= 1<<18, 0 <= top_k <= HS2_MAX_TOP_K.
 *   - Sequence lengths up to 2^31-1 rows; total rows up to 2^62.
 */
#ifndef HS2_H_
#define HS2_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HS2_VERSION 10000 /* 1.0.0 */
#define HS2_MAX_TOP_K 4096

typedef enum hs2_status {
  HS2_OK = 0,
  HS2_ERR_INVALID_ARG = -1, /* a null pointer, a negative size, inconsistent sizes     */
  HS2_ERR_UNSUPPORTED = -2, /* a valid but unsupported shape or dtype                  */
  HS2_ERR_WORKSPACE = -3,   /* workspace missing or smaller than the size query says   */
  HS2_ERR_HIP = -4          /* the HIP runtime reported an error while enqueueing      */
} hs2_status;

typedef enum hs2_dtype {
  HS2_BF16 = 0,    /* bfloat16 storage, fp32 arithmetic (bf16 MFMA with fp32 accumulation) */
  HS2_F32 = 1,     /* float32 storage and arithmetic                                      */
  HS2_FP8_E4M3 = 2 /* K and V stored as OCP FP8 E4M3 codes with one scale per tensor; Q and
                      out bfloat16. Taken by the *_fp8kv entry points and the workspace
                      size queries (the other entry points return HS2_ERR_UNSUPPORTED)  */
} hs2_dtype;

/* A ragged batch of sequences and their queries. */
typedef struct hs2_seqs {
  int32_t num_seqs;        /* host: number of sequences, >= 1                               */
  const int64_t* kv_start; /* device [num_seqs]: first row of sequence s in K and V         */
  const int32_t* kv_len;   /* device [num_seqs]: n_s, cached rows of s (current token incl.)*/
  const int32_t* q_start;  /* device [num_seqs+1]: queries of s are rows q_start[s] ..
                              q_start[s+1]-1 of Q; q_start[0] == 0, non-decreasing,
                              q_start[num_seqs] == total_q (otherwise every query is
                              inconsistent; a q_start that decreases somewhere leaves the
                              results of the queries it covers undefined, never touching
                              memory outside the given buffers)                          */
  const int32_t* q_pos;    /* device [total_q]: position t of each query, 0 <= t < n_s      */
  int32_t total_q;         /* host: q_start[num_seqs]                                      */
  int32_t max_kv_len;      /* host: an upper bound of every kv_len                         */
  int64_t total_kv_rows;   /* host: rows of K and V                                        */
  int32_t max_q_per_seq;   /* host: an upper bound of the queries of any one sequence      */
  const int32_t* kv_len_host; /* host, nullable: a copy of kv_len. Used only to size the
                              split of each query's keys over workgroups when every
                              sequence has at most one query (ragged decode); without it
                              the split assumes equal lengths, which may leave a second,
                              mostly idle round of workgroups. It must not be below the
                              device kv_len (also for every replay of a captured call):
                              a query whose keys run past the workgroups planned from it
                              is reported as inconsistent (NaN outputs, sel_count -1) */
} hs2_seqs;

/* Library version: HS2_VERSION of the built library. */
int32_t hs2_version(void);

/* Text of the last failed check on the calling thread; "" if none. Valid until the
 * next call on the same thread. */
const char* hs2_last_error(void);

/* ------------------------------------------------------------------------------------
 * KV Bridging ([arex] "Outer KV Bridging, inner KV Reuse"; [toolnavs] "Was HySparse2
 * tut"): every cross-decoder full-attention layer l builds its own K and V from the
 * input hidden states H of the matching self-decoder full-attention layer, through its
 * own projections, and one source may feed several layers:
 *     K_l = H W_K^l,   V_l = H W_V^l,   l = 0 .. n_layers-1
 * Plain linear maps: no bias, normalisation or rotary embedding is applied.
 *
 *   hidden   device [n_rows][d_model], bf16
 *   w_k,w_v  HOST arrays of n_layers DEVICE pointers, each [d_model][head_dim] bf16
 *   k_out,   HOST arrays of n_layers DEVICE pointers, each [n_rows][head_dim] bf16,
 *   v_out    written with round-to-nearest-even from fp32 accumulation
 *   Limits: dt == HS2_BF16; head_dim == 128; d_model a multiple of 64, <= 65536;
 *           1 <= n_layers <= 8; n_rows >= 0 (0 enqueues nothing).
 * ------------------------------------------------------------------------------------ */
size_t hs2_bridge_kv_workspace_size(int32_t d_model, int32_t n_layers, int32_t head_dim);

hs2_status hs2_bridge_kv(const void* hidden, int64_t n_rows, int32_t d_model, int32_t n_layers,
                         const void* const* w_k, const void* const* w_v, void* const* k_out,
                         void* const* v_out, int32_t head_dim, void* workspace,
                         size_t workspace_bytes, hs2_dtype dt, void* stream);

/* ------------------------------------------------------------------------------------
 * KV Bridging into FP8 caches: the same projections, written as the OCP FP8 E4M3 caches
 * that the *_fp8kv entry points read ([arex] "Numbers computed on three 80B-A3B models"
 * accounts the KV cache in FP8). With one scale per output tensor, element (r, c) of
 * layer l's K cache is the E4M3 code nearest to (H W_K^l)[r][c] / k_scale[l] (ties to
 * the even mantissa; magnitudes above 448 saturate to 448), and likewise for V.
 *
 *   hidden, w_k, w_v, workspace: as for hs2_bridge_kv (bf16, same workspace size)
 *   k_out,   HOST arrays of n_layers DEVICE pointers, each [n_rows][head_dim] bytes of
 *   v_out    E4M3 codes, 16-byte aligned
 *   k_scale, HOST arrays of n_layers scales, each finite and > 0 (the value a code
 *   v_scale  stands for is scale * its E4M3 value); the products are computed in fp32
 *            as (H W)[r][c] * (1 / scale), then converted
 *   Limits: as for hs2_bridge_kv. HS2_ERR_INVALID_ARG for a NULL array or a bad scale.
 * ------------------------------------------------------------------------------------ */
hs2_status hs2_bridge_kv_fp8kv(const void* hidden, int64_t n_rows, int32_t d_model, int32_t n_layers,
                               const void* const* w_k, const void* const* w_v, void* const* k_out,
                               void* const* v_out, const float* k_scale, const float* v_scale,
                               int32_t head_dim, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------
 * Full-attention selector layer ([arex] "Outer KV Bridging, inner KV Reuse": the few
 * full-attention layers act as the indexer, with their exact attention scores;
 * [toolnavs] "Was HySparse2 tut"). For each query i at position t of sequence s:
 *     s_hj  = scale * <q_h, k_j>,  j = 0..t           (all 64 heads share k_j, v_j)
 *     out_h = sum_j softmax_j(s_h) v_j,  lse_h = log sum_j exp(s_hj)
 *     score_j = sum_h exp(s_hj - lse_h)  for candidates j = 0..t-window
 *     sel   = the top_k candidates by score (all of them if fewer), ties to the smaller
 *             position, written ascending and padded with -1.
 *
 *   q        device [total_q][64][128], dtype dt
 *   k, v     device [total_kv_rows][128], dtype dt
 *   scale    softmax scale, finite and > 0 (1/sqrt(128) for the pages' layout)
 *   out      device [total_q][64][128], dtype dt
 *   lse      device [total_q][64] fp32, or NULL
 *   sel_idx  device [total_q][top_k] int32 (may be NULL when top_k == 0)
 *   sel_count device [total_q] int32 = min(top_k, candidates), or NULL
 *   workspace device scratch of at least hs2_full_attn_select_workspace_size(...) bytes,
 *            256-byte aligned; its contents on entry do not matter. The size depends on
 *            the descriptor's host fields (kv_len_host included): query it with the
 *            descriptor that the call will use.
 * ------------------------------------------------------------------------------------ */
size_t hs2_full_attn_select_workspace_size(const hs2_seqs* batch, int32_t n_heads,
                                           int32_t head_dim, int32_t window, int32_t top_k,
                                           hs2_dtype dt);

hs2_status hs2_full_attn_select(const hs2_seqs* batch, const void* q, const void* k,
                                const void* v, int32_t n_heads, int32_t head_dim,
                                int32_t window, int32_t top_k, float scale, void* out,
                                float* lse, int32_t* sel_idx, int32_t* sel_count,
                                void* workspace, size_t workspace_bytes, hs2_dtype dt,
                                void* stream);

/* ------------------------------------------------------------------------------------
 * Sparse attention layer with KV Reuse ([arex] "Outer KV Bridging, inner KV Reuse";
 * [zgeo] "Core technical principles"): a sparse layer reuses the selector's KV cache
 * and index set; each query attends to its window plus the selected rows only:
 *     A_t   = {max(0,t-window+1) .. t}  U  {sel_idx[i][r] : 0 <= sel_idx[i][r] <= t-window}
 *     out_h = sum_{j in A_t} softmax_j(scale * <q_h, k_j>) v_j
 * Entries of sel_idx outside [0, t-window] (the -1 padding) are ignored. Entries must
 * be distinct; a repeated entry is counted twice.
 *
 *   q        device [total_q][64][128] of this layer, dtype dt
 *   k, v     the selector's cache, device [total_kv_rows][128]
 *   sel_idx  device [total_q][top_k] int32 (the selector's output); NULL iff top_k == 0
 *   out      device [total_q][64][128], dtype dt;  lse device [total_q][64] fp32 or NULL
 *   workspace as for the selector, sized by hs2_sparse_attn_workspace_size(...)
 * ------------------------------------------------------------------------------------ */
size_t hs2_sparse_attn_workspace_size(const hs2_seqs* batch, int32_t n_heads, int32_t head_dim,
                                      int32_t window, int32_t top_k, hs2_dtype dt);

hs2_status hs2_sparse_attn(const hs2_seqs* batch, const void* q, const void* k, const void* v,
                           const int32_t* sel_idx, int32_t n_heads, int32_t head_dim,
                           int32_t window, int32_t top_k, float scale, void* out, float* lse,
                           void* workspace, size_t workspace_bytes, hs2_dtype dt, void* stream);

/* ------------------------------------------------------------------------------------
 * hs2_sparse_attn for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. The same operation and
 * arguments as hs2_sparse_attn (dt HS2_BF16 or HS2_F32), without a workspace: the split
 * partials live in a device array of HS2_NOALLOC_SCRATCH_BYTES that the library holds on
 * every GPU it runs on until the process ends (no memory is allocated by the call). A
 * batch whose hs2_sparse_attn_workspace_size exceeds HS2_NOALLOC_SCRATCH_BYTES returns
 * HS2_ERR_WORKSPACE. The stream must belong to the current device (HS2_ERR_INVALID_ARG
 * otherwise). Calls on one GPU share its array: calls that overlap there (other streams or
 * threads) race and must be serialised by the caller.
 * ------------------------------------------------------------------------------------ */
#define HS2_NOALLOC_SCRATCH_BYTES (16u << 20) /* 16 MiB per GPU: e.g. 64 queries x 7 splits */

hs2_status hs2_sparse_attn_noalloc(const hs2_seqs* batch, const void* q, const void* k, const void* v,
                                   const int32_t* sel_idx, int32_t n_heads, int32_t head_dim,
                                   int32_t window, int32_t top_k, float scale, void* out, float* lse,
                                   hs2_dtype dt, void* stream);

/* ------------------------------------------------------------------------------------
 * Decode-time KV Bridging ([arex] "Outer KV Bridging, inner KV Reuse"): in decode each
 * new token's hidden state h_i (the input of the matching self-decoder full-attention
 * layer) goes through every bridged layer's own projections, and the results become
 * that token's row of each layer's cache, before the selector of the step reads it:
 *     K_l[rows[i]] = h_i W_K^l,   V_l[rows[i]] = h_i W_V^l,   i < n_new, l < n_layers
 *
 *   hidden     device [n_new][d_model] bf16
 *   rows       device [n_new] int64: cache row of each new token; rows outside
 *              [0, cache_rows) are not written; repeated rows are written in no set order
 *   cache_rows host: rows of every cache (the bound of rows)
 *   w_k, w_v   HOST arrays of n_layers DEVICE pointers, each [d_model][head_dim] bf16
 *   k_cache,   HOST arrays of n_layers DEVICE pointers, each [cache_rows][head_dim] bf16;
 *   v_cache    only the given rows are written (fp32 accumulation, round to nearest even)
 *   workspace  device scratch of hs2_bridge_kv_append_workspace_size(...) bytes, 256-byte
 *              aligned; contents on entry do not matter
 *   Limits: dt == HS2_BF16; head_dim == 128; d_model a multiple of 128, <= 65536;
 *           1 <= n_layers <= 8; 0 <= n_new <= 65536 (0 enqueues nothing).
 * ------------------------------------------------------------------------------------ */
size_t hs2_bridge_kv_append_workspace_size(int32_t n_new, int32_t d_model, int32_t n_layers,
                                           int32_t head_dim);

hs2_status hs2_bridge_kv_append(const void* hidden, int32_t n_new, const int64_t* rows,
                                int64_t cache_rows, int32_t d_model, int32_t n_layers,
                                const void* const* w_k, const void* const* w_v,
                                void* const* k_cache, void* const* v_cache, int32_t head_dim,
                                void* workspace, size_t workspace_bytes, hs2_dtype dt,
                                void* stream);

/* The same append into FP8 E4M3 caches (the caches of hs2_bridge_kv_fp8kv and the *_fp8kv
 * entry points): element c of the new row of layer l's K cache is the E4M3 code nearest
 * to (h_i W_K^l)[c] / k_scale[l] (ties to the even mantissa, saturating at 448), computed
 * as the fp32 sum times 1 / k_scale[l]; likewise for V.
 *   k_cache, v_cache  HOST arrays of n_layers DEVICE pointers, each [cache_rows][head_dim]
 *                     bytes of E4M3 codes, 16-byte aligned
 *   k_scale, v_scale  HOST arrays of n_layers scales, each finite and > 0
 *   Everything else as for hs2_bridge_kv_append (same workspace size).
 */
hs2_status hs2_bridge_kv_append_fp8kv(const void* hidden, int32_t n_new, const int64_t* rows,
                                      int64_t cache_rows, int32_t d_model, int32_t n_layers,
                                      const void* const* w_k, const void* const* w_v,
                                      void* const* k_cache, void* const* v_cache,
                                      const float* k_scale, const float* v_scale, int32_t head_dim,
                                      void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------
 * Exact causal attention of every query, without selection: the self-decoder's
 * full-attention layer in prefill ([arex] "Outer KV Bridging, inner KV Reuse": prefill
 * runs the self-decoder and the cross-decoder's KV projections; [toolnavs] "Prefill
 * endet nach der Hälfte"), whose hidden states then feed hs2_bridge_kv:
 *     out_h = sum_{j<=t} softmax_j(scale * <q_h, k_j>) v_j,   lse_h = log sum_{j<=t} exp(...)
 * The batch is usually one sequence with every position as a query (q_pos = 0..n-1),
 * but any descriptor accepted by hs2_full_attn_select is.
 *
 *   q        device [total_q][64][128], dtype dt (HS2_BF16 or HS2_F32)
 *   k, v     device [total_kv_rows][128], dtype dt
 *   scale    softmax scale, finite and > 0
 *   out      device [total_q][64][128], dtype dt;  lse device [total_q][64] fp32 or NULL
 *   workspace device scratch of hs2_causal_attn_workspace_size(...) bytes (0 when every
 *            query's keys fit one workgroup), 256-byte aligned; contents on entry do
 *            not matter
 * ------------------------------------------------------------------------------------ */
size_t hs2_causal_attn_workspace_size(const hs2_seqs* batch, int32_t n_heads, int32_t head_dim,
                                      hs2_dtype dt);

hs2_status hs2_causal_attn(const hs2_seqs* batch, const void* q, const void* k, const void* v,
                           int32_t n_heads, int32_t head_dim, float scale, void* out, float* lse,
                           void* workspace, size_t workspace_bytes, hs2_dtype dt, void* stream);

/* ------------------------------------------------------------------------------------
 * FP8 KV cache ([arex] "Numbers computed on three 80B-A3B models": the pages' KV-cache
 * accounting at 1M tokens stores K and V in FP8). The same two operations as
 * hs2_full_attn_select and hs2_sparse_attn, on a cache whose rows are OCP FP8 E4M3
 * codes (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; subnormals; 0x7F and
 * 0xFF are NaN; no infinities; largest finite 448). Row j of the cache stands for
 *     k_j = k_scale * decode(k[j][:]),   v_j = v_scale * decode(v[j][:])
 * and every result is that of the bf16 operation on those values: the codes convert to
 * bf16 exactly, K's scale multiplies the logit scale and V's the output, in fp32.
 *
 *   k, v      device [total_kv_rows][128] uint8 (E4M3 codes), 16-byte aligned
 *   k_scale,  per-tensor scales, finite and > 0
 *   v_scale
 *   q, out    bf16 as in the bf16 operations; other arguments as there. Workspace sizes
 *             come from the size queries with dt = HS2_FP8_E4M3. The selector always
 *             uses its one-query-per-workgroup kernels (no q-tile path for FP8).
 * ------------------------------------------------------------------------------------ */
hs2_status hs2_full_attn_select_fp8kv(const hs2_seqs* batch, const void* q, const void* k,
                                      const void* v, float k_scale, float v_scale,
                                      int32_t n_heads, int32_t head_dim, int32_t window,
                                      int32_t top_k, float scale, void* out, float* lse,
                                      int32_t* sel_idx, int32_t* sel_count, void* workspace,
                                      size_t workspace_bytes, void* stream);

hs2_status hs2_sparse_attn_fp8kv(const hs2_seqs* batch, const void* q, const void* k,
                                 const void* v, float k_scale, float v_scale,
                                 const int32_t* sel_idx, int32_t n_heads, int32_t head_dim,
                                 int32_t window, int32_t top_k, float scale, void* out,
                                 float* lse, void* workspace, size_t workspace_bytes,
                                 void* stream);

/* ------------------------------------------------------------------------------------
 * First-generation HySparse layout, the comparison variant ([arex] "Outer KV Bridging,
 * inner KV Reuse": the predecessor selects its 1,024 global tokens as 64-token blocks and
 * adds a separate 128-token sliding-window (SWA) branch fused through a gate; [arex]
 * "Numbers computed on three 80B-A3B models": GQA, 64 query heads on 4 KV heads; [arex]
 * "Lost points, the 290B check and open questions": the SWA branch has its own
 * projections and local KV cache; [toolnavs] "Was HySparse2 tut": block-level selection).
 *
 * Layout: K and V rows hold the 4 KV heads, [total_kv_rows][4][128] bf16; query head h
 * reads KV head h / 16. A block is the 64 positions 64b .. 64b+63 of a sequence.
 *
 * Selector (exact causal attention plus block selection), query i at position t:
 *     out_h = sum_{j<=t} softmax_j(scale * <q_h, k_{j,h/16}>) v_{j,h/16},  lse_h as above
 *     score_{g,b} = sum over the 16 heads h of KV head g of the softmax probabilities of
 *                   the positions j <= t of block b,   b = 0 .. t/64
 *     blk_idx[i][g] = the top_blocks best blocks of KV head g (all of them if t/64 + 1 <=
 *                   top_blocks), ties to the smaller index, ascending, padded with -1;
 *     blk_count[i][g] = min(top_blocks, t/64 + 1)
 *
 *   q        device [total_q][64][128] bf16;  k, v device [total_kv_rows][4][128] bf16
 *   out      device [total_q][64][128] bf16;  lse device [total_q][64] fp32 or NULL
 *   blk_idx  device [total_q][4][top_blocks] int32; blk_count device [total_q][4] or NULL
 *   workspace device scratch of hs2_v1_full_attn_select_workspace_size(...) bytes, 256-byte
 *            aligned, contents on entry irrelevant
 *   Limits: dt == HS2_BF16, n_heads == 64, n_kv_heads == 4, head_dim == 128,
 *           1 <= top_blocks <= 64, max_kv_len <= 2^21. A query whose position lies beyond
 *           max_kv_len is treated as an inconsistent descriptor (NaN outputs, counts -1).
 * ------------------------------------------------------------------------------------ */
size_t hs2_v1_full_attn_select_workspace_size(const hs2_seqs* batch, int32_t n_heads,
                                              int32_t n_kv_heads, int32_t head_dim,
                                              int32_t top_blocks, hs2_dtype dt);

hs2_status hs2_v1_full_attn_select(const hs2_seqs* batch, const void* q, const void* k,
                                   const void* v, int32_t n_heads, int32_t n_kv_heads,
                                   int32_t head_dim, int32_t top_blocks, float scale, void* out,
                                   float* lse, int32_t* blk_idx, int32_t* blk_count,
                                   void* workspace, size_t workspace_bytes, hs2_dtype dt,
                                   void* stream);

/* Sparse layer of the v1 layout, query i at position t, head h of KV head g = h / 16:
 *     o_sparse_h = softmax attention over the positions j <= t of the blocks
 *                  blk_idx[i][g][*] (entries < 0 or > t/64 are ignored; entries must be
 *                  distinct) on the shared cache k, v
 *     o_swa_h    = softmax attention over positions max(0, t-window+1) .. t of this
 *                  layer's own cache k_swa, v_swa
 *     out_h      = gate_sparse[i][h] * o_sparse_h + gate_swa[i][h] * o_swa_h
 * A branch without attended positions contributes zero.
 *
 *   k, v          the selector's cache, device [total_kv_rows][4][128] bf16
 *   blk_idx       device [total_q][4][top_blocks] int32 (the selector's output)
 *   k_swa, v_swa  device [num_seqs][swa_slots][4][128] bf16: a ring per sequence, position p
 *                 of sequence s in row s * swa_slots + p % swa_slots. Every position a query
 *                 reads must be present: swa_slots >= window plus the spread of the
 *                 positions of one sequence's queries.
 *   gate_sparse,  device [total_q][64] fp32: the gate values of the two branches (how they
 *   gate_swa      are computed is the caller's)
 *   out           device [total_q][64][128] bf16
 *   workspace     device scratch of hs2_v1_sparse_attn_workspace_size(...) bytes
 *   Limits: as for the selector; 1 <= window <= swa_slots <= 2^20.
 * ------------------------------------------------------------------------------------ */
size_t hs2_v1_sparse_attn_workspace_size(const hs2_seqs* batch, int32_t n_heads,
                                         int32_t n_kv_heads, int32_t head_dim,
                                         int32_t top_blocks, hs2_dtype dt);

hs2_status hs2_v1_sparse_attn(const hs2_seqs* batch, const void* q, const void* k,
                              const void* v, const int32_t* blk_idx, int32_t top_blocks,
                              const void* k_swa, const void* v_swa, int32_t swa_slots,
                              int32_t window, const float* gate_sparse, const float* gate_swa,
                              int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, float scale,
                              void* out, void* workspace, size_t workspace_bytes, hs2_dtype dt,
                              void* stream);

/* ------------------------------------------------------------------------------------
 * Kernel timing hook, for benchmarks and profilers that need per-kernel durations on the
 * library's own stream (not an operation of the method, and the one exception to "no
 * state between calls": an attachment lasts until it is detached, on the thread that
 * made it, and changes no result). While attached, every hs2_*
 * compute call records events[2*j] right before and events[2*j+1] right after its
 * kernel of pipeline slot j (j < n_pairs), on that call's stream. Slots:
 *   hs2_full_attn_select: 0 attention, 1 split combine, 2 score pass, 3 top-k filter,
 *                         4 top-k finish
 *   hs2_sparse_attn:      0 attention, 1 split combine
 *   hs2_bridge_kv:        0 weight transpose, 1 fan-out GEMM
 *   hs2_v1_full_attn_select: 0 attention, 1 combine and block selection
 *   hs2_v1_sparse_attn:      0 attention (both branches), 1 gated combine
 * A slot whose kernel a call does not need (e.g. no split combine when one workgroup
 * covers a query) is not recorded. The events are hipEvent_t handles created and owned
 * by the caller and must stay valid while attached. events == NULL or n_pairs == 0
 * detaches. The attachment is per calling thread: calls made on other threads record
 * nothing. 0 <= n_pairs <= 16.
 * ------------------------------------------------------------------------------------ */
hs2_status hs2_set_kernel_events(void* const* events, int32_t n_pairs);

#ifdef __cplusplus
} /* extern "C" */
#endif

#endif /* HS2_H_ */
