/*
 * kvs.h -- C ABI of libkvs: query-aware block-sparse decode attention over a
 * paged KV cache, with a hot-buffer / host-tier variant, for AMD MI355X
 * (gfx950).
 *
 * The method (page "KV 稀疏化", §5 "Quest"): at every decode step, split the
 * KV of a sequence into blocks, keep a compact summary of each block (here
 * the channel-wise min and max of K), use the query and the summaries to
 * pick the top-k blocks, and run exact attention on those blocks only, so a
 * step reads k blocks of K/V instead of all of them.  The attention sink
 * (same page, §2, StreamingLLM) and the newest block (recent window; page
 * "SparDA：把KV選擇提前一層…", §4.2) are always kept.  The hot-buffer variant
 * follows the same wiki page, §7 "HiSparse": a hot buffer in HBM holds the
 * blocks the top-k set is likely to touch, inactive KV lives in host memory,
 * and a swap-in step finds misses, updates the page table and copies the
 * missed KV in before attention.
 *
 * Conventions shared by every call
 * --------------------------------
 *  B  = layout.num_seqs       Hq = layout.num_q_heads   Hkv = num_kv_heads
 *  G  = Hq / Hkv (query heads per KV head; query head h reads KV head h / G)
 *  D  = head_dim  (64 or 128)                S = block_size (16, 32 or 64)
 *  MB = max_blocks (entries per block-table row)   P = num_pages
 *  nb(b) = ceil(seq_lens[b] / S): blocks of sequence b, the last one may be
 *          partial; only token positions t < seq_lens[b] are ever used.
 *
 *  All tensors are dense, row-major (C order), in DEVICE memory unless the
 *  argument says "host"; the library never allocates, frees or keeps any of
 *  them.  Workspaces are caller-owned device buffers of at least the size the
 *  matching *_workspace_size call returns; they need no initial contents.
 *
 *  K pool (paged):    [P][Hkv][S][D] of kv_dtype (token-major tiles); page p
 *                     holds S consecutive tokens of one sequence for every
 *                     KV head.
 *  V pool (paged):    [P][Hkv][S/T][D][T] of kv_dtype, T = min(S, 32): each
 *                     tile is cut into runs of T consecutive tokens, and a
 *                     run is stored channel-major (its T tokens of one
 *                     channel are contiguous), so one 16-channel slice of a
 *                     run is a contiguous 1 KiB (bf16) read.  For S <= 32
 *                     this is the plain channel-major tile [D][S].
 *  fp8 scales:        [P][Hkv][S][D/quant_group] fp32, one per token and
 *                     group of quant_group adjacent channels ("分块稀疏注意力
 *                     与KV Cache量化…", §2.4; symmetric, no zero point).  The
 *                     value of an fp8 element is fp32(decode(code) * scale),
 *                     code in OCP E4M3FN.
 *  block_table:       [B][MB] int32 page ids (the paged layout's "block
 *                     table", page "SparDA…", §4.3).
 *  seq_lens:          [B] int32, tokens per sequence INCLUDING the token being
 *                     decoded (its K/V already written and its block's summary
 *                     rebuilt).  Must lie in [0, MB*S].
 *  sel:               [B][Hkv][k] int32 block ids per (sequence, KV head):
 *                     strictly ascending valid ids, then -1 padding ("SparDA…",
 *                     §6.3: pad ragged masks to one length with invalid values).
 *
 *  Every call only enqueues work on `stream` (a hipStream_t, NULL = the
 *  default stream) and never waits for the device.  Host-visible argument
 *  errors return a non-zero kvs_status before anything is enqueued, with a
 *  message in kvs_last_error().  Data that only the device sees (seq_lens,
 *  table entries, sel entries) is range-checked by the kernels: an offending
 *  item is skipped (a sequence length is clamped to [0, MB*S]) and a bit is
 *  set in the device error word read by kvs_device_errors(); no kernel ever
 *  reads or writes out of bounds.  No call falls back to another code path:
 *  an unsupported shape or dtype returns KVS_ERR_UNSUPPORTED.
 *
 *  Calls on one stream run in order; calls that overlap on different streams
 *  must not share output or workspace buffers.
 */
#ifndef KVS_H
#define KVS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVS_ABI_VERSION 6

typedef enum kvs_status {
  KVS_OK = 0,
  KVS_ERR_INVALID_ARG = 1,   /* null pointer, bad size, inconsistent layout */
  KVS_ERR_UNSUPPORTED = 2,   /* valid but not implemented (dtype, D, S, G)   */
  KVS_ERR_CAPACITY = 3,      /* more blocks requested than hot slots         */
  KVS_ERR_HIP = 4            /* the HIP runtime reported an error            */
} kvs_status;

typedef enum kvs_dtype {
  KVS_F32 = 0,
  KVS_BF16 = 1,
  KVS_FP8_E4M3 = 2           /* OCP E4M3FN, 1 byte per element */
} kvs_dtype;

typedef enum kvs_table_kind {
  /* table = block_table [B][MB] of page ids in [0, P); pools [P][Hkv][S][D] */
  KVS_TABLE_PAGED = 0,
  /* table = hot page table [B][Hkv][MB] of global hot-slot ids in [0, P)
   * (-1 = not resident); one KV head per slot: K pool [P][S][D], V pool
   * [P][S/T][D][T], scales [P][S][D/quant_group]. P is then the total number of
   * hot slots.  Slots hold what kvs_hot_lookup_swapin copied from the host
   * tier: only blocks that no longer receive tokens (see there). */
  KVS_TABLE_HOT = 1
} kvs_table_kind;

typedef struct kvs_layout {
  int32_t num_seqs;      /* B,   >= 0                                   */
  int32_t num_q_heads;   /* Hq,  multiple of num_kv_heads, G <= 16       */
  int32_t num_kv_heads;  /* Hkv, >= 1                                   */
  int32_t head_dim;      /* D:   64 or 128                              */
  int32_t block_size;    /* S:   16, 32 or 64 tokens per page and block */
  int32_t max_blocks;    /* MB:  block-table row length, 1..8192        */
  int32_t num_pages;     /* P:   pages (or hot slots) in the pool, >= 1 */
  int32_t q_dtype;       /* kvs_dtype of q: KVS_F32 or KVS_BF16          */
  int32_t kv_dtype;      /* kvs_dtype of the K/V pools                  */
  int32_t quant_group;   /* channels per fp8 scale (16, 32, 64 or 128,
                            dividing D); 0 unless kv_dtype is fp8       */
} kvs_layout;

/* Supported dtype pairs (q, kv): (F32, F32), (BF16, BF16), (BF16, FP8_E4M3). */

/* ------------------------------------------------------------------------
 * kvs_build_summaries -- per-block channel-wise min/max of K
 *
 * Page "KV 稀疏化", §5 "Quest" (first step: a compact summary per block);
 * run at prefill for every block and at each decode append for the block
 * that received the new token.  For b in [0,B), every KV head g and every
 * block j in [first, first + num_rebuild) ∩ [0, nb(b)), where first =
 * first_block[b] (0 when first_block is NULL):
 *     summaries[b][g][j][0][c] = min_t K[b,g,t,c],
 *     summaries[b][g][j][1][c] = max_t K[b,g,t,c],
 * over the valid tokens t in [j*S, min((j+1)*S, seq_lens[b])), K read through
 * block_table (fp8 elements dequantised first).  Other entries are left
 * untouched.
 *
 *  k_pool       [P][Hkv][S][D] kv_dtype
 *  k_scales     fp8 only: [P][Hkv][S][D/quant_group] fp32, else NULL
 *  block_table  [B][MB] int32;   seq_lens [B] int32
 *  first_block  [B] int32 device array or NULL
 *  num_rebuild  blocks rebuilt per sequence, 0..MB (MB with a NULL
 *               first_block = full prefill build; 1 with first_block[b] =
 *               nb(b)-1 = decode append)
 *  summaries    [B][Hkv][MB][2][D]: bf16 when kv_dtype is bf16 (min/max of
 *               bf16 values is exact in bf16), fp32 otherwise.
 * Errors: INVALID_ARG (null pointer, bad layout, num_rebuild out of range),
 * UNSUPPORTED (dtype/D/S), HIP.  Device flags: KVS_DEVERR_SEQLEN,
 * KVS_DEVERR_TABLE.
 * ---------------------------------------------------------------------- */
kvs_status kvs_build_summaries(const kvs_layout* layout, const void* k_pool,
                               const float* k_scales, const int32_t* block_table,
                               const int32_t* seq_lens, const int32_t* first_block,
                               int32_t num_rebuild, void* summaries, void* stream);

/* Summary kinds ("KV 稀疏化", §5 names min/max and mean as block summaries). */
#define KVS_SUMM_MINMAX 0
#define KVS_SUMM_MEAN   1

/* ------------------------------------------------------------------------
 * kvs_build_summaries_ex -- kvs_build_summaries for either summary kind
 *
 * KVS_SUMM_MINMAX: exactly kvs_build_summaries.  KVS_SUMM_MEAN: per rebuilt
 * block and channel, mean = fp32(sum / n) of K over the block's n valid
 * tokens, the sum in fp64 over ascending token positions and the division
 * in fp64 (fp8 elements dequantised first); summaries is
 * [B][Hkv][MB][D] fp32.  Other arguments and errors as kvs_build_summaries.
 * ---------------------------------------------------------------------- */
kvs_status kvs_build_summaries_ex(const kvs_layout* layout, int32_t summary_kind, const void* k_pool,
                                  const float* k_scales, const int32_t* block_table,
                                  const int32_t* seq_lens, const int32_t* first_block,
                                  int32_t num_rebuild, void* summaries, void* stream);

/* ------------------------------------------------------------------------
 * kvs_select_topk -- query-aware block scores and top-k selection
 *
 * Page "KV 稀疏化", §5 "Quest" (second step: coarse-filter the blocks with the
 * query and the summaries, keep the top-k); §2 and "SparDA…" §4.2 (sink and
 * recent blocks always kept).  The pages do not print the score; the one used
 * is the box upper bound of q.K over the block:
 *     U[b,h,j] = sum_{c=0}^{D-1} max(q[b,h,c]*mn[c], q[b,h,c]*mx[c])
 * accumulated in fp64 in ascending c (every product is exact in fp64, so the
 * result is the correctly ordered fp64 sum), and per KV head the group score
 *     W[b,g,j] = max over the G query heads h of group g of U[b,h,j].
 * Selection per (b,g): if nb(b) <= k every block; otherwise block 0, block
 * nb(b)-1 and the k-2 best of blocks 1..nb(b)-2 under (W descending, block id
 * ascending).  Written to sel ascending, padded with -1.
 *
 *  q            [B][Hq][D] q_dtype
 *  summaries    as written by kvs_build_summaries (same layout)
 *  seq_lens     [B] int32
 *  k            2 <= k <= MB
 *  sel          [B][Hkv][k] int32 output
 *  bounds_out   optional [B][Hkv][MB] fp64 output: W, -inf for j >= nb(b)
 *  workspace    >= kvs_select_workspace_size(layout, k) bytes
 * Two implementations give identical selections.  By default every block's W
 * is computed in exact fp64 and a second kernel selects.  When bounds_out is
 * NULL, q is bf16, MB <= 2048 and B*Hkv*MB >= 65536 (bf16 summaries) or
 * >= 262144 (fp32 summaries, each value split into two bf16 parts), the
 * blocks are instead scored on the matrix cores in fp32 together with a
 * rigorous bound on that rounding, and only the blocks whose fp32 score lies
 * within the bound of the top-k threshold get their W recomputed in exact
 * fp64 to settle the ranking.
 * Errors: INVALID_ARG, UNSUPPORTED, HIP.  Device flags: KVS_DEVERR_SEQLEN.
 * ---------------------------------------------------------------------- */
kvs_status kvs_select_topk(const kvs_layout* layout, const void* q, const void* summaries,
                           const int32_t* seq_lens, int32_t k, int32_t* sel,
                           double* bounds_out, void* workspace, size_t workspace_bytes,
                           void* stream);

/* ------------------------------------------------------------------------
 * kvs_select_topk_append -- kvs_select_topk for a decode step whose newest
 * token has just been appended to the K pool: also rebuilds the summary of
 * every sequence's newest block nb(b)-1 from K (as kvs_build_summaries with
 * first_block = nb(b)-1 and num_rebuild = 1 would).
 *
 * Same computation as kvs_build_summaries followed by kvs_select_topk; the
 * newest block is always selected, so its score never decides the
 * selection.  With bf16 K and bounds_out NULL the rebuild runs as one more
 * workgroup per (sequence, KV head) of the scoring launch, beside the
 * workgroups that score the other blocks (the newest block's own score then
 * uses its summary before or after the rebuild; it is not used).  Otherwise
 * (fp32/fp8 K, or bounds_out requested) the summary is rebuilt first, so
 * bounds_out matches the plain definition on the rebuilt summaries.
 *
 *  k_pool, k_scales, block_table   as for kvs_build_summaries
 *  summaries    in/out, as written by kvs_build_summaries
 *  others       as for kvs_select_topk
 * Errors: as kvs_select_topk and kvs_build_summaries.
 * ---------------------------------------------------------------------- */
kvs_status kvs_select_topk_append(const kvs_layout* layout, const void* q, const void* k_pool,
                                  const float* k_scales, const int32_t* block_table,
                                  const int32_t* seq_lens, void* summaries, int32_t k, int32_t* sel,
                                  double* bounds_out, void* workspace, size_t workspace_bytes,
                                  void* stream);

/* ------------------------------------------------------------------------
 * kvs_append_token -- write the decode token into the paged cache, update
 * its block's summary, and seal a block that has just filled into the host
 * tier
 *
 * Page "KV 稀疏化", §7 "HiSparse": the newest KV is written to the device
 * cache, and KV that is no longer being written sinks to host memory (the
 * tier kvs_hot_lookup_swapin reads back).  For every sequence b with
 * len = seq_lens[b] > 0 (the count includes the new token), token t = len-1
 * goes to block j = t/S, slot s = t%S of page block_table[b][j], for every KV
 * head g:
 *   K pool [page][g][s][c] = k_new[b][g][c]; V pool element (page, g, s, c)
 *   (run s/T, column s%T) = v_new[b][g][c]; fp8: the token's group scales
 *   [page][g][s][:] = k_new_scales / v_new_scales [b][g][:];
 *   summary (b, g, j) = min/max of the block's valid tokens.  It is
 *   computed incrementally: the stored summary must cover tokens jS..t-1
 *   (as kvs_build_summaries or earlier appends leave it); s = 0 starts the
 *   block afresh;
 *   when len % S == 0 and host_k is given, the block's K and V tiles (and
 *   fp8 scales) are copied byte for byte to host tile [b][g][j].
 * Sequences with len == 0 are skipped.
 *
 *  k_new/v_new  [B][Hkv][D] kv_dtype (fp8: E4M3FN codes, quantised by the
 *               caller)
 *  k_new_scales/v_new_scales  fp8 only: [B][Hkv][D/quant_group] fp32
 *  block_table  [B][MB] int32;  k_pool/v_pool/k_scales/v_scales  in/out
 *  host_k/host_v  optional HOST tier [B][Hkv][MB][S][D] (K) and
 *               [B][Hkv][MB][S/T][D][T] (V), pinned with hipHostMalloc (the
 *               layout kvs_hot_lookup_swapin reads); both NULL = no sealing
 *  host_k_scales/host_v_scales  fp8 with a host tier: [B][Hkv][MB][S][D/qg]
 *  summaries    [B][Hkv][MB][2][D] in/out (kvs_build_summaries layout)
 * A page must not be shared by two sequences that append in the same call.
 * Errors: INVALID_ARG (also a host tier that is not pinned), UNSUPPORTED,
 * HIP.  Device flags: KVS_DEVERR_SEQLEN, KVS_DEVERR_TABLE (the sequence is
 * skipped).
 * ---------------------------------------------------------------------- */
typedef struct kvs_append_args {
  const void* k_new;
  const void* v_new;
  const float* k_new_scales;
  const float* v_new_scales;
  const int32_t* block_table;
  void* k_pool;
  void* v_pool;
  float* k_scales;
  float* v_scales;
  void* host_k;
  void* host_v;
  float* host_k_scales;
  float* host_v_scales;
} kvs_append_args;

kvs_status kvs_append_token(const kvs_layout* layout, const kvs_append_args* append,
                            const int32_t* seq_lens, void* summaries, void* stream);

/* ------------------------------------------------------------------------
 * kvs_append_sparse_decode_attn -- kvs_append_token followed by
 * kvs_sparse_decode_attn (paged table) over a given selection, as one call
 *
 * Page "KV 稀疏化", §7 "HiSparse" (the newest KV written to the device
 * cache) and §5 "Quest" (attention over the selected blocks only), for a
 * layer that attends over a selection made elsewhere ("SparDA…" §3.1 and
 * §4.1: deeper layers reuse the mask of the predictor layers).  Results are
 * those of the two calls in a row: the cache, summaries and host tier as
 * kvs_append_token leaves them, out as kvs_sparse_decode_attn returns it on
 * the updated cache.  With bf16 q and K/V, blocks of 32 or 64 tokens and
 * head dim 64 or 128 both run in one launch: the attention takes the new
 * token's K and V from the append arguments (so it does not wait for the
 * write), and one workgroup per (sequence, KV head) writes the token after
 * its attention work; other layouts run the append launch first.
 *
 *  append       as for kvs_append_token; its block_table, k_pool, v_pool,
 *               k_scales and v_scales are also the attention's
 *  summaries, seq_lens  as for kvs_append_token (lengths with the token)
 *  q, sel, k, sm_scale, out, workspace  as for kvs_sparse_decode_attn
 * Errors: as kvs_append_token and kvs_sparse_decode_attn.  Device flags:
 * theirs (a sequence whose length or token page is out of range gets no
 * token, and its attention is that of kvs_sparse_decode_attn).
 * ---------------------------------------------------------------------- */
kvs_status kvs_append_sparse_decode_attn(const kvs_layout* layout, const kvs_append_args* append,
                                         void* summaries, const void* q, const int32_t* seq_lens,
                                         const int32_t* sel, int32_t k, float sm_scale, float* out,
                                         void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * kvs_select_topk_ex -- kvs_select_topk with the selection options of
 * "SparDA…" and an optional token append in the same call
 *
 *  opts->recent_blocks  R >= 1: besides the sink, the R newest blocks are
 *               always kept ("SparDA…" §4.2: the most recent 512 or 1024
 *               tokens are kept by default).  If nb(b) <= k every block;
 *               otherwise block 0, blocks nb-R..nb-1 and the k-1-R best of
 *               blocks 1..nb-R-1.  Needs k >= R + 1.  R = 1 is
 *               kvs_select_topk.
 *  opts->use_ema, ema_alpha, ema_state  score smoothing across decode
 *               steps ("SparDA…" §6.1: 70% of the current score, 30% of
 *               its history).  Per (b, g) and block j < nb(b):
 *                 state[j] = isnan(state[j]) ? W[j]
 *                            : alpha*W[j] + (1-alpha)*state[j]
 *               with each product and the sum rounded to fp64 separately;
 *               blocks are ranked by state[j].  ema_state is
 *               [B][Hkv][MB] fp64 in/out (NaN = no history; reset a row when
 *               its sequence slot is reused); entries j >= nb(b) are left
 *               untouched.  0 <= alpha <= 1.
 *  opts->summary_kind  KVS_SUMM_MINMAX: blocks are scored by the box bound
 *               W on min/max summaries; KVS_SUMM_MEAN: by the mean score
 *               max over the group's heads of sum_c q_c * mean_c (fp64,
 *               ascending c) on mean summaries (kvs_build_summaries_ex).  With
 *               mean summaries an append writes the token and then rebuilds
 *               its block's mean from the pool (a launch each), and scoring is
 *               always the exact path.
 *  opts->accumulate  0, or (kvs_score_blocks only) 1: add this call's
 *               scores to the ones already in `scores` instead of
 *               overwriting them (cross-layer fusion, see kvs_score_blocks);
 *               kvs_select_topk_ex rejects 1 with INVALID_ARG.
 *  opts = NULL  R = 1, no smoothing, min/max summaries, no accumulation.
 *  append       NULL, or the token append of kvs_append_token (same
 *               arguments), done before the blocks are scored.  Without
 *               bounds_out and smoothing it runs inside the scoring launch,
 *               beside the scoring of the other blocks (the newest block is
 *               always kept, so its own score is not used); otherwise as a
 *               launch of its own first.
 *  bounds_out   optional [B][Hkv][MB] fp64: the unsmoothed W.
 *  summaries    in/out when append is given, else only read.
 *  others       as for kvs_select_topk.
 * Matrix-core scoring (see kvs_select_topk) is not used with smoothing.
 * Errors: as kvs_select_topk and kvs_append_token.
 * ---------------------------------------------------------------------- */
typedef struct kvs_select_opts {
  int32_t recent_blocks;
  int32_t use_ema;
  double ema_alpha;
  double* ema_state;
  int32_t summary_kind;  /* KVS_SUMM_MINMAX (the box bound) or KVS_SUMM_MEAN */
  int32_t accumulate;    /* kvs_score_blocks only; see there */
} kvs_select_opts;

kvs_status kvs_select_topk_ex(const kvs_layout* layout, const void* q, void* summaries,
                              const int32_t* seq_lens, int32_t k, const kvs_select_opts* opts,
                              const kvs_append_args* append, int32_t* sel, double* bounds_out,
                              void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * kvs_sparse_decode_attn -- attention over the selected blocks only
 *
 * Page "KV 稀疏化", §5 "Quest" (third step: full attention on the selected
 * blocks); computed tile by tile with a running max and normaliser that are
 * merged across tiles ("分块稀疏注意力与KV Cache量化…", §2.2), fp8 K/V
 * dequantised inside the read (same page, §1.3).  For every query head h of
 * KV head g = h / G, over the token set T = ∪_{j in sel[b][g]} {t : j*S <= t <
 * min((j+1)S, seq_lens[b])}:
 *     s_t = sm_scale * q_h . K_t,  out[b][h] = sum_t softmax(s)_t V_t
 * in fp32 arithmetic; an empty T gives a zero row.
 *
 *  table_kind   KVS_TABLE_PAGED or KVS_TABLE_HOT (see kvs_table_kind)
 *  q            [B][Hq][D] q_dtype
 *  k_pool/v_pool, k_scales/v_scales   per table_kind (V in T-token runs)
 *  table        [B][MB] (paged) or [B][Hkv][MB] (hot) int32
 *  seq_lens     [B] int32
 *  sel          [B][Hkv][k] int32, k >= 1
 *  sm_scale     softmax scale (1/sqrt(D) for standard attention)
 *  out          [B][Hq][D] fp32 output
 *  workspace    >= kvs_attn_workspace_size(layout, k) bytes
 * Errors: INVALID_ARG, UNSUPPORTED, HIP.  Device flags: KVS_DEVERR_SEQLEN,
 * KVS_DEVERR_TABLE (entry out of range or -1: block skipped),
 * KVS_DEVERR_SEL (id >= nb(b), < -1, not ascending or after padding).
 * ---------------------------------------------------------------------- */
kvs_status kvs_sparse_decode_attn(const kvs_layout* layout, int32_t table_kind,
                                  const void* q, const void* k_pool, const void* v_pool,
                                  const float* k_scales, const float* v_scales,
                                  const int32_t* table, const int32_t* seq_lens,
                                  const int32_t* sel, int32_t k, float sm_scale, float* out,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * kvs_sparse_decode_attn_noalloc -- kvs_sparse_decode_attn with no
 * workspace argument, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc)
 *
 * Same computation, arguments, kernels and results as
 * kvs_sparse_decode_attn.  The split partials go to a device array the
 * library holds: KVS_NOALLOC_SCRATCH_BYTES on every GPU it runs on, kept
 * until the process ends.  The call allocates and frees nothing.  Every call
 * on one GPU shares that GPU's array, so calls that overlap on one GPU
 * (concurrent streams, or host threads on the same device) race and give
 * undefined results; calls on one stream are fine.  No contents need to
 * survive between calls (each call writes every partial it reads).
 * Errors: as kvs_sparse_decode_attn, and CAPACITY when the layout's
 * partials (kvs_attn_workspace_size) exceed KVS_NOALLOC_SCRATCH_BYTES; every
 * layout the library accepts needs at most 4.25 MiB.
 * ---------------------------------------------------------------------- */
#define KVS_NOALLOC_SCRATCH_BYTES (8u << 20)

kvs_status kvs_sparse_decode_attn_noalloc(const kvs_layout* layout, int32_t table_kind,
                                          const void* q, const void* k_pool, const void* v_pool,
                                          const float* k_scales, const float* v_scales,
                                          const int32_t* table, const int32_t* seq_lens,
                                          const int32_t* sel, int32_t k, float sm_scale, float* out,
                                          void* stream);

/* ------------------------------------------------------------------------
 * kvs_score_blocks + kvs_select_attn -- the layer-step of kvs_select_topk_ex
 * followed by kvs_sparse_decode_attn, with the top-k done inside the
 * attention launch
 *
 * kvs_score_blocks does everything kvs_select_topk_ex does before the top-k
 * (the optional token append, the block scores of kvs_select_topk, the
 * optional smoothing of opts; opts->recent_blocks is not used here) and
 * writes each block's score -- the smoothed score with smoothing on, else W
 * -- to scores [B][Hkv][MB] fp64 (-inf for j >= nb(b)).  Scores are always
 * the exact fp64 ones.  With an append and neither bounds_out nor smoothing,
 * the append runs inside the scoring launch and the score of each sequence's
 * newest block nb(b)-1 is taken from a summary being updated at the same
 * time: that one entry is unspecified (the block is always kept, so no
 * selection reads it).
 *
 * Cross-layer fusion ("SparDA…" §3.1 and §4.1: a few shallow layers score
 * the history, their scores are fused into one mask, and every deeper layer
 * gathers the K/V that mask names): with opts->accumulate = 1,
 *     scores[b][g][j] = scores[b][g][j] + (this layer's score)
 * for j < nb(b) (one fp64 add, after the smoothing when that is on; -inf
 * beyond nb(b)), so predictor layers 0..P-1 called with accumulate = 0, 1,
 * ..., 1 leave the sum of their scores, added in layer order.  Deeper
 * layers skip scoring: kvs_select_attn on that sum selects once, and
 * kvs_sparse_decode_attn reuses the selection in every further layer.
 *
 * kvs_select_attn selects, per (b, g), the blocks kvs_select_topk_ex would
 * select from those scores (sink, the recent_blocks newest blocks, the best
 * of the rest), writes that selection to sel [B][Hkv][k], and returns the
 * attention of kvs_sparse_decode_attn (paged table) over it.  With bf16 q,
 * bf16 or fp8 K/V, S >= 32 and MB, k <= 2048 every attention workgroup
 * selects its own blocks from the scores, so no separate selection launch or
 * round trip through memory is needed; other shapes run the selection
 * launch first.  Same results either way.
 *
 *  scores       [B][Hkv][MB] fp64, as kvs_score_blocks writes them
 *  k            2 <= k <= MB;  recent_blocks >= 1, k >= recent_blocks + 1
 *  sel          [B][Hkv][k] int32 output
 *  others       as for kvs_sparse_decode_attn (workspace: its size query)
 * Errors: as kvs_select_topk_ex and kvs_sparse_decode_attn.
 * ---------------------------------------------------------------------- */
kvs_status kvs_score_blocks(const kvs_layout* layout, const void* q, void* summaries,
                            const int32_t* seq_lens, const kvs_select_opts* opts,
                            const kvs_append_args* append, double* scores, double* bounds_out,
                            void* stream);

kvs_status kvs_select_attn(const kvs_layout* layout, const void* q, const void* k_pool,
                           const void* v_pool, const float* k_scales, const float* v_scales,
                           const int32_t* block_table, const int32_t* seq_lens,
                           const double* scores, int32_t k, int32_t recent_blocks, int32_t* sel,
                           float sm_scale, float* out, void* workspace, size_t workspace_bytes,
                           void* stream);

/* The paged device cache a sequence's newest block is copied from by the
 * hot-buffer swap-in (kvs_hot_lookup_swapin, kvs_hot_swapin) when the
 * caller passes one: the same pool, scales and block table the decode-token
 * append writes (kvs_append_token), and the sequence lengths after it.  The
 * pool holds layout->num_pages pages. */
typedef struct {
  const void* k_pool;          /* [P][Hkv][S][D] kv_dtype */
  const void* v_pool;          /* [P][Hkv][S/T][D][T] kv_dtype */
  const float* k_scales;       /* [P][Hkv][S][D/qg] fp32, fp8 only (else NULL) */
  const float* v_scales;
  const int32_t* block_table;  /* [B][MB] page ids */
  const int32_t* seq_lens;     /* [B], the appended tokens included */
} kvs_hot_live;

/* ------------------------------------------------------------------------
 * kvs_hot_lookup_swapin -- hot-buffer page-table step and swap-in copy
 *
 * Page "KV 稀疏化", §7 "HiSparse" table: the hot device buffer keeps the KV
 * the current top-k set is likely to touch, inactive KV sits in host memory,
 * and the swap-in step finds the misses on the decode path, updates the page
 * table and copies the KV back; what is resident follows the sparse access
 * set (the selection), not idleness or LRU alone.  Per unit u = b*Hkv + g,
 * with ns = num_slots slots of global ids u*ns + s:
 *   1. every selected block j with page_table[u][j] >= 0 is a hit: its slot's
 *      stamp becomes `step`;
 *   2. the misses are the other selected blocks, ascending -> miss_list[u],
 *      padded with -1, count -> miss_count[u];
 *   3. victims are the slots whose owner is not selected (free slots have
 *      owner -1 and stamp -1), ordered by (stamp ascending, slot ascending);
 *      the r-th miss takes the r-th victim: the old owner's page-table entry
 *      becomes -1, the miss's entry the slot id, owner = miss, stamp = step;
 *   4. each miss's K and V block (and fp8 scales) is copied from the host
 *      tier into its slot.
 * Blocks in the host tier are immutable once written, so eviction needs no
 * write-back.
 *
 * The growing block.  kvs_append_token writes a block to the host tier only
 * when it seals it (full), and a hit is never copied again, so a slot copied
 * from the host tier cannot follow a block that is still receiving tokens
 * (a sequence's newest block in a decode loop that appends).  With `live`
 * non-NULL the swap-in therefore takes each unit's newest block
 * j = (seq_lens[b] - 1) / S from the paged device cache instead: as a miss
 * it is copied from there, and as a hit that is still resident it is copied
 * again, at every call.  A decode step that appends, selects, then calls
 * this and attends through KVS_TABLE_HOT reads every token appended so far;
 * once the block fills, the last such copy holds it whole, as the host tier
 * then does.  Page table, owners, stamps and miss lists are the same as
 * without `live`.  With `live` NULL every block the hot path serves must be
 * final (sealed); the newest block of an appending sequence is not.
 *
 *  layout       num_seqs, num_kv_heads, head_dim, block_size, max_blocks
 *               (page-table row length), kv_dtype, quant_group are used
 *  sel          [B][Hkv][k] int32 (ids < MB), 1 <= k <= num_slots
 *  num_slots    hot slots per unit, 1..4096
 *  step         decode step number, >= 0, larger than any previous step
 *  page_table   [B][Hkv][MB] int32 in/out (global slot id or -1)
 *  slot_owner   [B][Hkv][num_slots] int32 in/out (block id or -1)
 *  slot_stamp   [B][Hkv][num_slots] int64 in/out (-1 when free)
 *  host_k/host_v  HOST [B][Hkv][MB][S][D] (K) and [B][Hkv][MB][S/T][D][T] (V)
 *               kv_dtype, allocated with hipHostMalloc (pinned and mapped;
 *               the kernels read it over the host link); tiles are copied
 *               byte for byte
 *  host_k_scales/host_v_scales  HOST [B][Hkv][MB][S][D/qg] fp32 (fp8 only)
 *  hot_k/hot_v  [B*Hkv*num_slots][S][D] (K) and [B*Hkv*num_slots][S/T][D][T] (V)
 *               kv_dtype (the KVS_TABLE_HOT pools)
 *  hot_k_scales/hot_v_scales  [B*Hkv*num_slots][S][D/qg] fp32 (fp8 only)
 *  miss_list    [B][Hkv][k] int32 output;  miss_count [B][Hkv] int32 output
 *  live         NULL, or the paged cache the newest blocks are copied from
 *               (all its pointers device memory, 16-byte aligned pools; its
 *               pages counted by layout->num_pages)
 * Initial state of a fresh buffer: page_table, slot_owner, slot_stamp all -1.
 * Errors: INVALID_ARG (also when a host pool is not pinned), CAPACITY
 * (k > num_slots), UNSUPPORTED, HIP.  Device flags: KVS_DEVERR_SEL,
 * KVS_DEVERR_TABLE (inconsistent page table / owner state, or a live page
 * id out of range: that block skipped), KVS_DEVERR_SEQLEN (a live length out of
 * [0, MB*S], clamped).
 * ---------------------------------------------------------------------- */
kvs_status kvs_hot_lookup_swapin(const kvs_layout* layout, const int32_t* sel, int32_t k,
                                 int32_t num_slots, int64_t step, int32_t* page_table,
                                 int32_t* slot_owner, int64_t* slot_stamp, const void* host_k,
                                 const void* host_v, const float* host_k_scales,
                                 const float* host_v_scales, void* hot_k, void* hot_v,
                                 float* hot_k_scales, float* hot_v_scales, int32_t* miss_list,
                                 int32_t* miss_count, const kvs_hot_live* live, void* stream);

/* ------------------------------------------------------------------------
 * kvs_hot_lookup + kvs_hot_swapin -- the two halves of kvs_hot_lookup_swapin
 *
 * Same page ("KV 稀疏化", §7 "HiSparse"): the table also notes that misses
 * land on the decode critical path.  Split in two so that a caller can take
 * the page-table step (steps 1-3 above: hits, the miss list, LRU victims)
 * for one layer's hot buffer and run the host-link copy (step 4) on
 * another stream, overlapped with other work ("分块稀疏注意力与KV Cache量化…"
 * §5.3: wider prefetch during decode).  kvs_hot_lookup followed by
 * kvs_hot_swapin with the same page_table, miss_list and miss_count gives
 * exactly kvs_hot_lookup_swapin.
 *
 * kvs_hot_lookup: arguments as kvs_hot_lookup_swapin without the pools; it
 *   leaves page_table, slot_owner, slot_stamp, miss_list and miss_count as
 *   kvs_hot_lookup_swapin does.
 * kvs_hot_swapin: copies, for every unit u, the first miss_count[u] blocks
 *   of miss_list[u] from the host tier into the slot page_table[u][j] gives
 *   them (K and V tiles and fp8 scales, byte for byte), and with `live` the
 *   unit's newest block from the paged cache as described above.  A listed
 *   block whose page-table entry is not one of the unit's slots is skipped
 *   with KVS_DEVERR_TABLE; counts are clamped to [0, k].  It must run after
 *   the kvs_hot_lookup that wrote the list and before anything changes the
 *   page table, after the appends whose tokens it is to carry, and before
 *   the attention that reads the slots.
 * Errors: as kvs_hot_lookup_swapin.
 * ---------------------------------------------------------------------- */
kvs_status kvs_hot_lookup(const kvs_layout* layout, const int32_t* sel, int32_t k, int32_t num_slots,
                          int64_t step, int32_t* page_table, int32_t* slot_owner, int64_t* slot_stamp,
                          int32_t* miss_list, int32_t* miss_count, void* stream);

kvs_status kvs_hot_swapin(const kvs_layout* layout, int32_t k, int32_t num_slots,
                          const int32_t* page_table, const int32_t* miss_list,
                          const int32_t* miss_count, const void* host_k, const void* host_v,
                          const float* host_k_scales, const float* host_v_scales, void* hot_k,
                          void* hot_v, float* hot_k_scales, float* hot_v_scales,
                          const kvs_hot_live* live, void* stream);

/* Workspace bytes needed by kvs_select_topk / kvs_sparse_decode_attn for this
 * layout and k; 0 when the layout or k is invalid. */
size_t kvs_select_workspace_size(const kvs_layout* layout, int32_t k);
size_t kvs_attn_workspace_size(const kvs_layout* layout, int32_t k);

/* 1 when kvs_select_topk (no bounds_out; kvs_select_topk_ex with min/max
 * summaries and no smoothing) scores this layout on the matrix cores and
 * refines only near the threshold; 0 when it computes every block's exact
 * score, as kvs_score_blocks always does.  With 1 the separate selection
 * launch is the cheaper way to select; with 0 kvs_select_attn's in-attention
 * top-k is.  0 also for an invalid layout. */
int32_t kvs_select_uses_matrix_cores(const kvs_layout* layout, int32_t k);

/* Number of key splits the attention kernel uses for this layout and k
 * (each (sequence, KV head) unit's k blocks are spread over that many
 * workgroups whose partial results are merged); 0 when invalid. */
int32_t kvs_attn_num_splits(const kvs_layout* layout, int32_t k);

/* Device error word bits (see each call). */
#define KVS_DEVERR_SEQLEN 0x1u  /* a seq_lens entry outside [0, MB*S]        */
#define KVS_DEVERR_TABLE  0x2u  /* a table entry out of range or inconsistent */
#define KVS_DEVERR_SEL    0x4u  /* a selection entry out of range / order     */

/* Reads the current device's error word (OR of KVS_DEVERR_* bits raised by
 * kernels since the last clear) into *flags after waiting for `stream`; when
 * clear != 0 the word is reset to 0.  Errors: INVALID_ARG, HIP. */
kvs_status kvs_device_errors(uint32_t* flags, int32_t clear, void* stream);

/* Static description of a status code; never NULL. */
const char* kvs_status_string(kvs_status status);

/* Detail message of the last error returned on the calling thread ("" if
 * none); valid until the next call on that thread. */
const char* kvs_last_error(void);

/* KVS_ABI_VERSION of the library. */
int32_t kvs_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVS_H */
