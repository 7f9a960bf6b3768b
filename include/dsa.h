/*
 * dsa.h -- C ABI of the MI355X (gfx950) DeepSeek-style sparse attention layer:
 * lightning indexer -> per-row top-k -> page translation -> sparse MLA.
 *
 * The method (Kimi K3.1 Pro day-0 page, "Sparse attention in K3.1 Pro"):
 * every sparse-attention layer keeps a small indexer beside MLA; 32 light
 * heads score every earlier token of the query against a per-token FP8 index
 * key (132 bytes with its scale), the 2,048 best tokens are kept, and MLA then
 * runs exactly, but only over those tokens.  The indexer score reads as the
 * DeepSeek-V3.2 form the page defers to,
 *     score(t, s) = sum_h w_h(t) * ReLU(q_h(t) . k_s),
 * accumulated in FP32 with a weighted reduction across heads (same page, AMD
 * section "native MXFP4 indexer").
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE memory owned and allocated by the caller.
 *     The library never allocates, frees or synchronises; scratch memory is a
 *     caller-provided workspace sized by dsa_workspace_size().
 *   - Work is enqueued asynchronously on `stream` (0 = the null stream).
 *   - Arguments are validated on the host before anything is launched; on any
 *     error nothing is launched and a status is returned.  There is no silent
 *     fallback to another path.  dsa_last_error() describes the last failure
 *     of the calling thread.
 *   - Device-resident metadata (visible counts, block-table entries, row ids)
 *     cannot be checked on the host.  Kernels bound every access by them;
 *     visible counts are clamped to max_vis.  A block-table entry outside
 *     [0, num_pages) names no page (an absent page) and nothing is read from
 *     it: the indexer writes -inf as the score of its tokens, the top-k ranks
 *     -inf below every finite score (equal -inf scores by lower index, like
 *     any tie) and translation turns its tokens into row -1, which attention
 *     skips, as it skips any row id < 0 or past the pool's last row.  A row
 *     whose tok_req names no request (outside [0, num_requests)) translates
 *     to no rows (-1) and the MSA variant reads no block for it.  The debug
 *     build notes every such clamp or skip (dsa_check_debug_flag).
 *   - Calls are re-entrant and may run concurrently on different streams with
 *     different buffers.  The only state the library holds is the per-GPU
 *     scratch of sparse_mla_decode_noalloc (whose calls must not overlap on
 *     one GPU) and, in the debug build, its status words.
 *
 * Paged caches (same page, "One KV cache, three states": the engine turns the
 * block table into kernel page addresses before each step).  A pool is a
 * sequence of physical pages `page_bytes` apart; a page holds P = 2^p tokens.
 * Index-key pages are scanned whole, so they are structure-of-arrays, each
 * region starting on a 16-byte boundary:
 *     key   FP8    [P x 128 E4M3][P x fp32 scale]                     132 B/token
 *     key   MXFP4  [P x 64 B E2M1 pairs, low nibble first][P x 4 E8M0]  68 B/token
 *     key   NVFP4  [P x 64 B E2M1 pairs, low nibble first]
 *                  [P x 8 E4M3 block scales, one per 16 dims]            72 B/token
 * (NVFP4 index keys: MiniMax-M3.1-Flash day-0 page, "Quick start" and AMD
 * "NVFP4 indexer DCP"; a value is E2M1 x its block scale, no second-level
 * scale.)
 * Latent rows are gathered one by one, so a latent page is P rows, each row
 * padded to whole 128-byte lines and holding all of its bytes (a gathered row
 * then fetches only its own lines; page_bytes a multiple of 128 keeps rows
 * line-aligned):
 *     lat   BF16   row 1152 B: [576 bf16]                              1152 B/token
 *     lat   FP8    row  640 B: [576 E4M3][fp32 scale][60 B unused]      580 B/token
 *     lat   NVFP4  row  384 B: [256 B E2M1 pairs (dims 0..511)]
 *                              [32 E4M3 scales, one per 16 dims]
 *                              [64 E4M3 rope dims 512..575, unscaled]
 *                              [32 B unused]                           352 B/token
 * (B/token counts the data bytes.)  page_bytes may exceed P x (bytes per row
 * or token): several layers' pages can share one block row.  Logical token s
 * of request r lives in physical page block_table[r * bt_stride + (s >> p)],
 * slot s & (P-1); with block_table == NULL the cache is non-paged and request
 * r owns physical page r.  A physical row id is page * P + slot.  Keys and
 * latents of one token share page ids.
 *
 * Latent rows are 576-d: 512 "nope" dims followed by 64 "rope" dims; the value
 * vector is the first 512 dims.  FP8 E4M3 is OCP E4M3FN (bias 7, max 448).
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_ABI_VERSION 2
#define DSA_INDEX_HEADS 32
#define DSA_INDEX_DIM 128
#define DSA_LATENT_DIM 576
#define DSA_VALUE_DIM 512
#define DSA_MAX_TOPK 2048
#define DSA_MAX_HEADS 128

typedef enum dsa_status {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad size or shape      */
  DSA_ERR_UNSUPPORTED = 2, /* format or combination this build does not run   */
  DSA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required      */
  DSA_ERR_HIP = 4          /* the HIP runtime reported a launch error         */
} dsa_status;

/* Cache and query formats. */
enum { DSA_KEY_FP8 = 1, DSA_KEY_MXFP4 = 2, DSA_KEY_NVFP4 = 3 };
enum { DSA_LAT_BF16 = 1, DSA_LAT_FP8 = 2, DSA_LAT_NVFP4 = 3 };
enum { DSA_Q_BF16 = 1, DSA_Q_FP8 = 2, DSA_Q_MXFP4 = 3 };

/* Operation ids for dsa_workspace_size(). */
enum { DSA_OP_INDEXER = 1, DSA_OP_TOPK = 2, DSA_OP_MLA_DECODE = 3, DSA_OP_MLA_PREFILL = 4,
       DSA_OP_TOPK_SHARDED = 5, DSA_OP_MSA_DECODE = 6, DSA_OP_INDEXER_PREFIX = 7 };

/* One paged pool (index keys or latents) of one layer. */
typedef struct dsa_cache {
  const void* base;       /* device, 16-byte aligned: physical page 0         */
  int64_t page_bytes;     /* stride between physical pages, multiple of 16    */
  int32_t page_size_log2; /* p: P = 2^p tokens per page, 4 <= p <= 24         */
  int32_t num_pages;      /* physical pages in the pool (bounds page ids)     */
  int32_t fmt;            /* DSA_KEY_* for key pools, DSA_LAT_* for latents   */
} dsa_cache;

/* Query rows of one step, grouped by request.  Rows of request r are
 * [req_row_start[r], req_row_start[r+1]); row t sees logical keys
 * 0 .. tok_vis[t]-1 (speculative rows of one request see one more key each;
 * prefill rows see their prefix plus themselves). */
typedef struct dsa_batch {
  int32_t num_requests;          /* R >= 1                                     */
  int32_t num_rows;              /* T >= 1 query rows                          */
  const int32_t* req_row_start;  /* device int32 [R+1], non-decreasing, 0..T   */
  const int32_t* tok_req;        /* device int32 [T]: request of each row      */
  const int32_t* tok_vis;        /* device int32 [T]: visible keys, 1..max_vis */
  const int32_t* block_table;    /* device int32 [R, bt_stride] or NULL        */
  int32_t bt_stride;             /* entries per block-table row                */
  int32_t max_vis;               /* host bound on tok_vis (sizes the grid)     */
  int32_t max_rows_per_req;      /* host bound on rows of one request          */
} dsa_batch;

/* dsa_indexer_scores -- stage 1, the lightning indexer.
 * For every row t and visible key s < tok_vis[t]:
 *     scores[t*ld + s] = sum_{h<32} w[t,h] * max(0, q[t,h,:] . k_s)
 * with k_s the dequantised key (FP8: codes x per-token scale; MXFP4: E2M1 x
 * 2^(E8M0-127) per 32 dims; NVFP4: E2M1 x its E4M3 block scale per 16 dims)
 * and q BF16, FP8 codes x q_scale[t,h], or MXFP4 (E2M1 x 2^(E8M0-127) per 32
 * dims).  Products are exact and accumulate in fp32; keys on absent pages
 * score -inf.  Positions >= tok_vis[t] are not written.  Rows of one request
 * share each key load (speculative verify rows reuse keys, same page, AMD
 * "native MXFP4 indexer").  BF16 q (any key format) runs on BF16 MFMA over
 * keys dequantised exactly in registers; FP8 q (FP8 keys) on FP8 MFMA, the
 * compute-bound prefill shape; MXFP4 q (MXFP4 keys) on the FP4 MFMA with the
 * E8M0 scales applied by the instruction (the AMD section's native FP4 matrix
 * instructions).  A request with more rows than max_rows_per_req still has
 * every row scored.  Errors: DSA_ERR_INVALID_ARG for a bad batch or cache,
 * null or unaligned pointers, ld below max_vis or not a multiple of 4;
 * DSA_ERR_UNSUPPORTED for an unknown format or a q / key pairing other than
 * the three above. */
typedef struct dsa_indexer_args {
  dsa_batch batch;
  dsa_cache keys;                /* fmt DSA_KEY_FP8, _MXFP4 or _NVFP4          */
  const void* q;                 /* device: bf16 [T,32,128], E4M3 [T,32,128],
                                    or E2M1 pairs [T,32,64], 16-byte aligned   */
  int32_t q_fmt;                 /* DSA_Q_BF16, DSA_Q_FP8 or DSA_Q_MXFP4       */
  const void* q_scale;           /* device: fp32 [T,32] (FP8 q), E8M0 uint8
                                    [T,32,4] (MXFP4 q), else NULL              */
  const float* w;                /* device fp32 [T,32] head weights            */
  float* scores;                 /* device fp32 [T, ld]                        */
  int64_t ld;                    /* row stride of scores, >= max_vis, %4 == 0  */
} dsa_indexer_args;
dsa_status dsa_indexer_scores(const dsa_indexer_args* args, hipStream_t stream);

/* dsa_indexer_scores_prefix -- the indexer for batches whose requests share
 * a cached prefix (high-concurrency decode over one long shared context; the
 * MiniMax M3.1 page's AMD section dequantises a shared-prefix page once for
 * up to 64 requests).  Requests form groups of consecutive requests whose
 * rows are consecutive: group g owns rows [group_row_start[g],
 * group_row_start[g+1]); every request of a group maps its first
 * prefix_len / P logical pages to the same physical pages, those of request
 * group_first_req[g].  The shared pages are streamed once for all rows of the
 * group (one multi-row pass), the rest of every request once for its own
 * rows.  The scores are those of dsa_indexer_scores(&base) on the same
 * inputs, up to the order of fp32 additions (the shared pass may run on the
 * multi-row kernel where the plain call runs the single-row one).
 * prefix_len is a multiple of the page size, 0 <= prefix_len <= max_vis;
 * BF16 q only; groups of at most 64 requests' rows are the intended case.
 * Errors as dsa_indexer_scores, plus DSA_ERR_INVALID_ARG for a bad group
 * description and DSA_ERR_WORKSPACE below dsa_workspace_size(
 * DSA_OP_INDEXER_PREFIX, args). */
typedef struct dsa_indexer_prefix_args {
  dsa_indexer_args base;         /* the plain call's arguments (block table required) */
  int32_t num_groups;            /* G >= 1                                       */
  const int32_t* group_row_start;/* device int32 [G+1], from 0 to num_rows       */
  const int32_t* group_first_req;/* device int32 [G]: a request of each group    */
  int32_t prefix_len;            /* shared tokens per group                      */
  int32_t max_rows_per_group;    /* host bound on rows of one group              */
  void* workspace;               /* device, 256-byte aligned                     */
  size_t workspace_bytes;
} dsa_indexer_prefix_args;
dsa_status dsa_indexer_scores_prefix(const dsa_indexer_prefix_args* args, hipStream_t stream);

/* dsa_topk -- stage 2, per-row top-k with a deterministic tie-break.
 * Keeps K_t = min(k, tok_vis[t]) positions of row t: the highest scores, and
 * among equal scores the lower index (a unique set).  idx[t, 0..K_t) holds
 * them in ascending index order, idx[t, K_t..k) = -1.  If rows != NULL the
 * same entries are also translated to physical latent rows (page * P + slot,
 * P = 2^page_size_log2) through batch.block_table, so attention can read them
 * directly (same page, "Low-latency fused DSA decode path": the fused indexer
 * emits physical KV rows).  count[t] = K_t if count != NULL.  Scores are
 * finite or -inf (the indexer's score of a token on an absent page); -inf
 * ranks below every finite score and -0.0 equal to +0.0.  The result of a row
 * does not depend on the other rows of the batch.  Errors: DSA_ERR_INVALID_ARG
 * for k outside [1, 2048], an empty batch, a null or unaligned scores or idx,
 * ld below max_vis or not a multiple of 4, and (rows != NULL) page_size_log2
 * outside [4, 24], num_pages < 1 or num_pages x P above 2^31 - 1, a null
 * tok_req or a block table too short for max_vis; DSA_ERR_WORKSPACE when the
 * workspace is missing, unaligned or smaller than dsa_workspace_size(
 * DSA_OP_TOPK, args). */
typedef struct dsa_topk_args {
  dsa_batch batch;
  const float* scores;           /* device fp32 [T, ld]                        */
  int64_t ld;
  int32_t k;                     /* 1 .. 2048                                  */
  int32_t* idx;                  /* device int32 [T, k]                        */
  int32_t* rows;                 /* device int32 [T, k] or NULL                */
  int32_t page_size_log2;        /* page size of the latent pool (rows != NULL)*/
  int32_t num_pages;             /* pages of the latent pool (rows != NULL)    */
  int32_t* count;                /* device int32 [T] or NULL                   */
  void* workspace;               /* device, 256-byte aligned                   */
  size_t workspace_bytes;
} dsa_topk_args;
dsa_status dsa_topk(const dsa_topk_args* args, hipStream_t stream);

/* dsa_translate_pages -- logical selected indices -> physical rows (Kimi K3.1
 * Pro day-0 page, "One KV cache, three states": the block table becomes kernel
 * page addresses before each step).
 * rows[t*k+j] = page * P + (i & (P-1)) with page = block_table[r*bt_stride +
 * (i >> p)], r = tok_req[t], i = idx[t*k+j]; -1, an index outside the
 * request's block-table row, or a page outside [0, num_pages) gives -1.
 * Non-paged (block_table NULL): page = r.  Errors: DSA_ERR_INVALID_ARG for a
 * null pointer, k outside [1, 2048], num_rows < 1, page_size_log2 outside
 * [4, 24], num_pages < 1 or num_pages x P above 2^31 - 1. */
dsa_status dsa_translate_pages(const int32_t* idx, int32_t k, const dsa_batch* batch,
                               int32_t page_size_log2, int32_t num_pages, int32_t* rows, hipStream_t stream);

/* dsa_topk_sharded -- the exact top-k merge of decode context parallelism,
 * its W shards emulated on this device (Kimi K3.1 Pro day-0 page, "Long
 * context: decode context parallel" and "Exact top-k merge").  Shard r of W
 * holds every W-th token of a row: global token s = j*W + r sits at local
 * position j, and the shard's scores of row t are
 *     scores[(r*num_rows + t)*ld + j],  j < n_r(t) = ceil((tok_vis[t] - r)/W)
 * (the layout each shard's indexer writes).  Steps, all on `stream`:
 *   1. every shard keeps its local top-min(k, n_r) of each row and sends the
 *      `cand` best of them as (fp32 score, global index) candidates;
 *   2. per row, the K_t = min(k, tok_vis[t]) best candidates of the union are
 *      selected; a shard all of whose candidates were selected while it sent
 *      fewer than min(k, n_r) is flagged, since it may hold more of the top-k;
 *   3. flagged shards send their full local top-k and flagged rows are
 *      selected again (one round always suffices).
 * The result is the unsharded top-k of the row -- the same as dsa_topk on the
 * row in global order: idx[t, 0..K_t) the ascending global indices, -1
 * padded to k; count[t] = K_t (if count != NULL); resend[t*W + r] = 1 for the
 * flagged shards, else 0 (if resend != NULL).  Scores must be finite.
 * Errors: DSA_ERR_INVALID_ARG for num_rows < 1, W outside [1, 16], k outside
 * [1, 2048], cand outside [0, k], max_vis < 1, ld < ceil(max_vis / W) or not
 * a multiple of 4, a null or unaligned pointer; DSA_ERR_WORKSPACE when the
 * workspace is missing, unaligned or smaller than dsa_workspace_size(
 * DSA_OP_TOPK_SHARDED, args). */
typedef struct dsa_topk_sharded_args {
  int32_t num_rows;              /* T >= 1                                     */
  int32_t num_shards;            /* W, 1 .. 16                                 */
  const float* scores;           /* device fp32 [W, T, ld], 16-byte aligned    */
  int64_t ld;                    /* >= ceil(max_vis / W), multiple of 4        */
  const int32_t* tok_vis;        /* device int32 [T]: global visible count     */
  int32_t max_vis;               /* host bound on tok_vis (values are clamped) */
  int32_t k;                     /* 1 .. 2048                                  */
  int32_t cand;                  /* candidates a shard sends, 0 = ceil(1.5k/W) */
  int32_t* idx;                  /* device int32 [T, k]                        */
  int32_t* count;                /* device int32 [T] or NULL                   */
  int32_t* resend;               /* device int32 [T, W] or NULL                */
  void* workspace;               /* device, 256-byte aligned                   */
  size_t workspace_bytes;
} dsa_topk_sharded_args;
dsa_status dsa_topk_sharded(const dsa_topk_sharded_args* args, hipStream_t stream);

/* sparse_mla_decode / sparse_mla_prefill -- stage 3, exact MLA over the
 * selected rows.  For row t and head h < num_heads, over the valid entries s
 * of rows[t, 0..k) (entries < 0 or outside the pool are skipped):
 *     l_s = sm_scale * q[t,h,:] . c_s        (c_s the dequantised 576-d latent)
 *     out[t,h,:] = sum_s softmax(l)_s * c_s[0:512],  lse[t,h] = log sum_s e^{l_s}
 * A row with no valid entry gives out = 0 and lse = -inf.  Heads are padded in
 * the kernel to a multiple of 16 (the MFMA tile; MI355X Kimi K3 page, section
 * 4 "MLA": padding 12 -> 16 heads leaves the real heads unchanged); padded
 * heads are never written.  Decode splits each row's list into num_splits
 * pieces (0 = automatic) whose partial results merge by log-sum-exp (Kimi
 * K3.1 Pro day-0 page, "Long context: decode context parallel"); prefill runs
 * one workgroup per query row over all heads (same page, AMD "Prefill").
 * q is BF16; products accumulate in fp32; softmax weights enter the value
 * product as BF16. */
typedef struct dsa_mla_args {
  int32_t num_rows;              /* T                                           */
  int32_t num_heads;             /* H, 1 .. 128                                 */
  const void* q;                 /* device bf16 [T, H, 576]                     */
  dsa_cache latents;             /* fmt DSA_LAT_*                               */
  const int32_t* rows;           /* device int32 [T, k] physical rows           */
  int32_t k;                     /* 1 .. 2048                                   */
  float sm_scale;                /* softmax scale (finite, > 0)                 */
  int32_t num_splits;            /* 0 = automatic, else 1 .. k/16; at most 64
                                    are used (decode)                           */
  float* out;                    /* device fp32 [T, H, 512]                     */
  float* lse;                    /* device fp32 [T, H] or NULL                  */
  void* workspace;               /* device, 256-byte aligned                    */
  size_t workspace_bytes;
} dsa_mla_args;
dsa_status sparse_mla_decode(const dsa_mla_args* args, hipStream_t stream);
dsa_status sparse_mla_prefill(const dsa_mla_args* args, hipStream_t stream);

/* sparse_mla_decode_noalloc -- sparse_mla_decode for callers that cannot
 * allocate (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same arguments, kernels and results as
 * sparse_mla_decode, except that args->workspace / workspace_bytes are
 * ignored: the split partials live in a device array inside the library, 32
 * MiB per GPU (DSA_MLA_SCRATCH_BYTES), held until the process ends.  The call
 * allocates nothing; its first call on a device resolves that device's copy
 * of the array (a symbol-address query, no allocation).  With num_splits = 0
 * the automatic split count is lowered until the partials, T x splits x H x
 * 2052 bytes, fit; an explicit num_splits whose partials do not fit returns
 * DSA_ERR_WORKSPACE.  Every call on one GPU shares that GPU's array: calls
 * that overlap on one GPU (different streams, or different threads) race and
 * must be serialised by the caller.  Errors as sparse_mla_decode, plus
 * DSA_ERR_HIP when the scratch address cannot be resolved. */
#define DSA_MLA_SCRATCH_BYTES (32u << 20)
dsa_status sparse_mla_decode_noalloc(const dsa_mla_args* args, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Front end of a step (Kimi K3.1 Pro day-0 page, "Low-latency decoding: the
 * fused DSA decode path": the indexer front end quantises the index query to
 * FP8 or MXFP4 with the head weights folded into the quantisation and writes
 * the new token's index key; the MLA query step writes the new token's latent
 * into the KV cache).  Quantisation rules, shared by both calls:
 *   FP8 row   s = amax / 448 (1 for an all-zero row); code = E4M3(x / s)
 *   MXFP4     per 32 values E8M0 = (fp32 exponent field of amax) - 2,
 *             clamped to 0..254; code = E2M1(x / 2^(E8M0 - 127))
 *   NVFP4     per 16 values s = E4M3(amax / 6); code = E2M1(x / value(s)),
 *             0 when s decodes to 0; rope dims 512..575 E4M3(x), unscaled
 * E4M3 / E2M1 codes are the nearest value (ties to the even code, saturating
 * at 448 / 6; zero stored as +0); each division is an IEEE fp32 division
 * (subnormals kept).  Inputs are BF16. */

/* dsa_quantize_q -- index-query quantisation per (row, head).
 * FP8: q_out uint8 [T, 32, 128] E4M3, q_scale fp32 [T, 32]; with w_folded
 * != NULL also w_folded[t, h] = w[t, h] * q_scale[t, h] (fp32), the head
 * weight folded into the scale (w' ReLU(code . k) = w ReLU((s code) . k) as
 * s > 0).  The FP8-q indexer takes q_out with either q_scale and w, or a
 * unit scale and w_folded.  MXFP4: q_out uint8 [T, 32, 64] E2M1 pairs (low
 * nibble first), q_scale uint8 [T, 32, 4] E8M0; w and w_folded are unused.
 * T = 0 launches nothing. */
typedef struct dsa_quant_q_args {
  int32_t num_rows;              /* T >= 0                                      */
  const void* q;                 /* device bf16 [T, 32, 128], 16-byte aligned   */
  const float* w;                /* device fp32 [T, 32] or NULL                 */
  int32_t fmt;                   /* DSA_Q_FP8 or DSA_Q_MXFP4                    */
  void* q_out;                   /* device, 16-byte aligned (see above)         */
  void* q_scale;                 /* device, fp32 [T, 32] or uint8 [T, 32, 4]    */
  float* w_folded;               /* device fp32 [T, 32] or NULL (FP8; needs w)  */
} dsa_quant_q_args;
dsa_status dsa_quantize_q(const dsa_quant_q_args* args, hipStream_t stream);

/* dsa_cache_insert -- write n new tokens into the paged pools.
 * Token i (request tok_req[i], logical position tok_pos[i]) goes to page
 * block_table[r * bt_stride + (pos >> p)] (block_table NULL: page r), slot
 * pos & (P-1), of the key pool (key_vals bf16 [n, 128] quantised to the
 * pool's format) and of the latent pool (lat_vals bf16 [n, 576]); either may
 * be NULL.  Only the token's own bytes are written (its codes and scale
 * words; a latent row's unused tail is left as it is).  A token with a
 * request outside [0, num_requests), a negative position, a position past its
 * block-table row or a page outside [0, num_pages) is skipped.  Tokens that
 * map to the same slot race.  The pools are written through keys.base and
 * latents.base (device memory the caller owns; the other calls only read it). */
typedef struct dsa_insert_args {
  int32_t num_tokens;            /* n >= 0                                      */
  int32_t num_requests;
  const int32_t* tok_req;        /* device int32 [n]                            */
  const int32_t* tok_pos;        /* device int32 [n]                            */
  const int32_t* block_table;    /* device int32 [R, bt_stride] or NULL         */
  int32_t bt_stride;
  const void* key_vals;          /* device bf16 [n, 128] or NULL, 4-byte aligned */
  dsa_cache keys;                /* fmt DSA_KEY_FP8, _MXFP4 or _NVFP4           */
  const void* lat_vals;          /* device bf16 [n, 576] or NULL, 16-byte aligned */
  dsa_cache latents;             /* fmt DSA_LAT_*; same page size as keys       */
} dsa_insert_args;
dsa_status dsa_cache_insert(const dsa_insert_args* args, hipStream_t stream);

/* dsa_msa_decode -- the MSA block-sparse variant (MiniMax M3.1 page, "MSA
 * primer"), one decode step over a paged cache of 128-token blocks.
 * For row t (request r = tok_req[t], visible tokens 0 .. tok_vis[t]-1) and
 * group g < Hkv:
 *   score(g, s)  = q_idx[t,g,:] . k_s        (k_s: the token's 128 E4M3 index
 *                                              values, unscaled; exact products,
 *                                              fp32 accumulation)
 *   block b      = max of score over its visible tokens
 *   sel[t,g,:]   = the most recent block plus the top_blocks-1 best other
 *                  blocks (ties to the lower id), ascending, -1 padded; every
 *                  block when there are at most top_blocks
 *   out[t,h,:]   = softmax_s(sm_scale * q[t,h,:] . K_g(s)) weighted sum of
 *                  V_g(s) over the visible tokens of the selected blocks, for
 *                  every head h of group g = h / (Hq/Hkv); lse[t,h] in nats.
 * K_g(s) / V_g(s) = k_scale / v_scale x the E4M3 values of head g.
 * Layouts (device, 16-byte aligned): index_keys [num_blocks][128][128] bytes;
 * kv [num_blocks][128][2][Hkv][128] bytes (per token: K of every head, then
 * V); batch.block_table [R, bt_stride] maps logical block b of request r to a
 * pool block (entries < 0 or >= num_blocks: absent, their tokens score -inf
 * and are never attended); q_idx bf16 [T, Hkv, 128]; q bf16 [T, Hq, 128].
 * Errors: DSA_ERR_INVALID_ARG for Hkv outside [1, 8], Hq not a multiple of
 * Hkv or Hq/Hkv > 16, top_blocks outside [1, 16], a bad batch, null or
 * unaligned pointers; DSA_ERR_WORKSPACE below dsa_workspace_size(
 * DSA_OP_MSA_DECODE, args) (the block scores, 4 * T * Hkv * ceil(max_vis/128)
 * bytes, and two partial attention results per (row, group), 16.5 KB each). */
typedef struct dsa_msa_args {
  dsa_batch batch;               /* rows by request; block_table of 128-token blocks */
  const void* index_keys;        /* device E4M3 [num_blocks, 128, 128]          */
  const void* kv;                /* device E4M3 [num_blocks, 128, 2, Hkv, 128]  */
  int32_t num_blocks;            /* blocks in both pools                        */
  int32_t num_kv_heads;          /* Hkv = GQA groups, 1 .. 8                    */
  int32_t num_q_heads;           /* Hq, multiple of Hkv, Hq / Hkv <= 16         */
  int32_t top_blocks;            /* 1 .. 16                                     */
  const void* q_idx;             /* device bf16 [T, Hkv, 128]                   */
  const void* q;                 /* device bf16 [T, Hq, 128]                    */
  float k_scale, v_scale, sm_scale;
  int32_t* sel_blocks;           /* device int32 [T, Hkv, top_blocks]           */
  float* out;                    /* device fp32 [T, Hq, 128]                    */
  float* lse;                    /* device fp32 [T, Hq] or NULL                 */
  void* workspace;               /* device, 256-byte aligned                    */
  size_t workspace_bytes;
} dsa_msa_args;
dsa_status dsa_msa_decode(const dsa_msa_args* args, hipStream_t stream);

/* Workspace bytes an operation needs for these arguments (0 if none, or if
 * the arguments are invalid).  `args` points to the op's argument struct. */
size_t dsa_workspace_size(int32_t op, const void* args);

const char* dsa_status_str(dsa_status status);
const char* dsa_last_error(void);
int32_t dsa_abi_version(void);

/* dsa_check_debug_flag -- debug builds (the library compiled with
 * DSA_DEBUG=1, libdsa_debug.so) bounds-check the device-resident metadata
 * every kernel reads and note in a device status word what they had to
 * clamp or skip (the survey's failure-detection item: explicit errors, no
 * silent fallback):
 *   DSA_DEBUG_VIS_CLAMPED    a visible count outside [0, max_vis]
 *   DSA_DEBUG_ABSENT_PAGE    a block-table entry outside [0, num_pages)
 *   DSA_DEBUG_ROW_OUTSIDE    a row id >= the pool's rows, or an index past its
 *                            request's block-table row
 *   DSA_DEBUG_REQ_OUTSIDE    a request id outside [0, num_requests)
 * The call waits for the current device, returns the OR of these bits noted
 * since the previous call and clears them.  Release builds return -1 (the
 * checks are compiled out). */
#define DSA_DEBUG_VIS_CLAMPED 1
#define DSA_DEBUG_ABSENT_PAGE 2
#define DSA_DEBUG_ROW_OUTSIDE 4
#define DSA_DEBUG_REQ_OUTSIDE 8
int32_t dsa_check_debug_flag(void);

#ifdef __cplusplus
}
#endif
#endif /* DSA_H */
