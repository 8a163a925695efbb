/*
 * oracle.h -- plain, single-threaded fp64 CPU oracle for query-aware
 * block-sparse decode attention over a paged KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this code; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark may.  It shares no code, header, table or constant
 * with the HIP library.
 *
 * What it follows (page titles as published):
 *   - "KV 稀疏化" (wiki chapter on KV sparsification), §5 "Quest": per decode
 *     step, split KV into blocks, keep a compact per-block summary
 *     (min/max), coarse-filter the blocks with the query, keep top-k, run
 *     full attention on the kept blocks only.
 *   - same page, §2 (StreamingLLM): the first tokens (attention sink) are
 *     always kept; "SparDA：把KV選擇提前一層…" §4.2: the recent window is
 *     always kept.  Both are forced blocks counted inside k.
 *   - same wiki page, §7 "HiSparse" table: hot device buffer, host inactive
 *     KV, swap-in that finds misses, updates the page table and copies KV in.
 *   - "分块稀疏注意力与KV Cache量化…" §2.2 (tiled softmax with running max
 *     and normaliser) and §2.4 (per-32-channel group scales).
 *
 * The pages do not print the bound; this oracle uses the box bound
 * U = sum_c max(q_c*min_c, q_c*max_c) (the maximum of q.x over the
 * axis-aligned box [min,max]^d that holds every key of the block).
 *
 * Conventions
 *   layout : B sequences, Hq query heads, Hkv KV heads (G = Hq/Hkv, query
 *            head h reads KV head h / G), head dim D, S tokens per block
 *            (= page), max_blocks entries per block-table row, num_pages
 *            pages in the pool.
 *   pools  : the K pool is [num_pages][Hkv][S][D] (token-major tiles), the
 *            V pool [num_pages][Hkv][S/T][D][T] with T = min(S, 32) (runs
 *            of T tokens, each channel-major), both of
 *            kv_dtype (0 = fp32, 1 = bf16 bit patterns, 2 = OCP E4M3FN
 *            codes).  fp8 scales of K and of V are both
 *            [num_pages][Hkv][S][D/quant_group] fp32, one per token and
 *            channel group; the value of an fp8 element is
 *            fp32(decode(code) * scale).
 *   table  : block_table[B][max_blocks], page id of logical block j.
 *   lens   : seq_lens[B], tokens per sequence (0 <= len <= max_blocks*S);
 *            nb = ceil(len / S) blocks, the last one possibly partial.
 *   sel    : [B][Hkv][k] selected block ids, strictly ascending, then -1.
 *
 * Return value of every function: 0 on success, a positive OR_E* code when
 * an argument or an index is out of range.
 */
#ifndef KVS_ORACLE_H
#define KVS_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  OR_OK = 0,
  OR_EARG = 1,      /* bad scalar argument                          */
  OR_ERANGE = 2,    /* index (len, page, block id) out of range      */
  OR_EORDER = 3,    /* selection not strictly ascending / duplicated */
  OR_ECAP = 4       /* more selected blocks than hot slots           */
};

typedef struct {
  int32_t B, Hq, Hkv, D, S, max_blocks, num_pages;
  int32_t kv_dtype;     /* 0 fp32, 1 bf16, 2 e4m3 */
  int32_t quant_group;  /* channels per fp8 scale; 0 unless kv_dtype == 2 */
} or_layout;

/* Element decoders (the oracle's own; pinned against library casts). */
double or_bf16_to_f64(uint16_t bits);
double or_e4m3_to_f64(uint8_t code);                 /* NaN for 0x7F/0xFF */
float  or_e4m3_scaled(uint8_t code, float scale);    /* fp32(decode*scale) */

/* KV cache bytes per token: 2 (K and V) * layers * kv_heads * head_dim *
 * bytes per element ("SparDA…" §1.1 works this out for an 8B model). */
int64_t or_kv_bytes_per_token(int32_t layers, int32_t kv_heads,
                              int32_t head_dim, int32_t bytes_per_elem);

/* Per-block channel min/max of K over valid tokens ("KV 稀疏化" §5).
 * Rebuilds blocks j in [first_block[b], first_block[b]+num_rebuild) ∩
 * [0, nb_b); first_block == NULL means 0.  out is
 * [B][Hkv][max_blocks][2][D] (index 0 = min, 1 = max); entries of blocks
 * that are not rebuilt are left as they are. */
int or_summaries(const or_layout* L, const void* k_pool, const float* k_scales,
                 const int32_t* block_table, const int32_t* seq_lens,
                 const int32_t* first_block, int32_t num_rebuild,
                 double* out);

/* Box upper bound per (b, query head h, block j):
 *   U[b][h][j] = sum_{c=0}^{D-1} max(q[b][h][c]*mn[c], q[b][h][c]*mx[c]),
 * summed in ascending c; and per KV head g the group score
 *   W[b][g][j] = max over the G query heads of group g of U[b][h][j].
 * Entries with j >= nb_b are set to -inf.  q is [B][Hq][D], summ is the
 * or_summaries layout; U is [B][Hq][max_blocks] (may be NULL), W is
 * [B][Hkv][max_blocks]. */
int or_bounds(const or_layout* L, const double* q, const double* summ,
              const int32_t* seq_lens, double* U, double* W);

/* Top-k selection per (b, g) from W: if nb <= k every block; otherwise
 * blocks 0 (sink) and nb-1 (newest) plus the k-2 best of blocks 1..nb-2
 * under the order (W descending, block id ascending).  Output strictly
 * ascending, padded with -1 to k entries.  Requires k >= 2. */
int or_select(const or_layout* L, const double* W, const int32_t* seq_lens,
              int32_t k, int32_t* sel);

/* The same selection with a recent window of `recent` >= 1 newest blocks
 * ("SparDA…" §4.2: besides the sink, the most recent 512 or 1024 tokens
 * are kept by default): if nb <= k every block; otherwise block 0, blocks
 * nb-recent..nb-1 and the k-1-recent best of blocks 1..nb-recent-1 under
 * (W descending, block id ascending).  Requires k >= recent + 1; recent = 1
 * is or_select. */
int or_select_window(const or_layout* L, const double* W, const int32_t* seq_lens,
                     int32_t k, int32_t recent, int32_t* sel);

/* Score smoothing across decode steps ("SparDA…" §6.1: the score a block is
 * ranked by mixes 70% of this step's value with 30% of its history).  Per
 * (b, g) and block j < nb_b:
 *   state[j] = isnan(state[j]) ? W[j] : alpha*W[j] + (1-alpha)*state[j]
 * (each product and the sum rounded to fp64 as written, 1-alpha computed in
 * fp64; NaN marks a block with no history yet), and Wout[j] = state[j];
 * Wout[j] = -inf and state[j] untouched for j >= nb_b.  state and Wout are
 * [B][Hkv][max_blocks]; 0 <= alpha <= 1. */
int or_ema_scores(const or_layout* L, const double* W, const int32_t* seq_lens,
                  double alpha, double* state, double* Wout);

/* Cross-layer score fusion ("SparDA：把KV選擇提前一層…" §3.1 and §4.1: a
 * few shallow layers score the history, their scores are fused into one
 * mask, and every deeper layer gathers the K/V that mask names).  The
 * fused score of (b, g, j) is the sum of the n_layers layers' scores,
 * added left to right in fp64:
 *   out[b][g][j] = (...((W[0][b][g][j] + W[1][b][g][j]) + W[2][b][g][j]) ...)
 * for j < nb_b, -inf beyond.  W is [n_layers][B][Hkv][max_blocks] (each
 * layer's scores as or_bounds / or_ema_scores / or_mean_scores give them),
 * out is [B][Hkv][max_blocks]; n_layers >= 1. */
int or_fuse_scores(const or_layout* L, const double* W, int32_t n_layers,
                   const int32_t* seq_lens, double* out);

/* Softmax attention of every query head over the tokens of its group's
 * selected blocks (t < len only), two passes (max, then sums):
 *   s_t = sm_scale * q_h . K_t ;  out_h = sum_t exp(s_t - m) V_t / sum_t exp(s_t - m)
 * q is [B][Hq][D] fp64, out is [B][Hq][D] fp64; an empty token set gives a
 * zero row.  sel must be strictly ascending valid ids followed by -1. */
int or_sparse_attn(const or_layout* L, const double* q,
                   const void* k_pool, const void* v_pool,
                   const float* k_scales, const float* v_scales,
                   const int32_t* block_table, const int32_t* seq_lens,
                   const int32_t* sel, int32_t k, double sm_scale,
                   double* out);

/* Dense softmax attention over every token t < len (separate code path,
 * no blocks, no selection). */
int or_dense_attn(const or_layout* L, const double* q,
                  const void* k_pool, const void* v_pool,
                  const float* k_scales, const float* v_scales,
                  const int32_t* block_table, const int32_t* seq_lens,
                  double sm_scale, double* out);

/* One hot-buffer step for one (sequence, KV head) unit ("KV 稀疏化" §7):
 *   pt[nb]       logical block -> global hot slot id (slot_base + s) or -1
 *   owner[ns]    slot -> logical block or -1
 *   stamp[ns]    last step the slot was used, -1 when free
 * Rules: every selected block with a slot is a hit and gets stamp = step;
 * the misses are the other selected blocks in ascending order; victims are
 * the slots whose owner is not selected (free slots included), ordered by
 * (stamp ascending, slot ascending); the r-th miss takes the r-th victim,
 * the victim's old block loses its slot.  miss_list[k] gets the misses
 * then -1, *miss_cnt their number.  OR_ECAP when more blocks are selected
 * than there are slots. */
int or_hot_step(int32_t nb, int32_t ns, int32_t k, int64_t step,
                int32_t slot_base, const int32_t* sel, int32_t* pt,
                int32_t* owner, int64_t* stamp, int32_t* miss_list,
                int32_t* miss_cnt);

/* Appends one decode token per sequence ("KV 稀疏化" §7: the newest KV is
 * written to the device cache; a block that is no longer being written
 * sinks to the host tier).  seq_lens[b] counts the new token; for len > 0,
 * t = len-1 goes to block j = t/S, slot s = t%S of page block_table[b][j]:
 *   K[page][g][s][c] = k_new[b][g][c], the V element (page, g, s, c) =
 *   v_new[b][g][c] (V tile [S/T][D][T]), and for fp8 the token's group
 *   scales from k_new_scales / v_new_scales [B][Hkv][D/quant_group];
 * then the summary of block j becomes the min/max over its valid tokens
 * (recomputed from the pool), and when len % S == 0 and host_k is given
 * the block is sealed: its K and V tiles (and scales) are copied byte for
 * byte to host_k/host_v [B][Hkv][max_blocks][tile] (scales
 * [B][Hkv][max_blocks][S][D/quant_group]).  k_new/v_new hold kv_dtype
 * elements (fp8: codes); len == 0 sequences are skipped. */
int or_append_token(const or_layout* L, const void* k_new, const void* v_new,
                    const float* k_new_scales, const float* v_new_scales,
                    const int32_t* block_table, const int32_t* seq_lens,
                    void* k_pool, void* v_pool, float* k_scales, float* v_scales,
                    double* summ, void* host_k, void* host_v,
                    float* host_k_scales, float* host_v_scales);

/* Mean summaries ("KV 稀疏化" §5 lists the mean beside min and max as a
 * block summary): per block and channel, the mean of K over the block's
 * valid tokens, mean = fp32(sum / n) with the sum in fp64 over ascending
 * token positions and the division in fp64.  out is
 * [B][Hkv][max_blocks][D] fp32; block range as for or_summaries. */
int or_summaries_mean(const or_layout* L, const void* k_pool, const float* k_scales,
                      const int32_t* block_table, const int32_t* seq_lens,
                      const int32_t* first_block, int32_t num_rebuild, float* out);

/* Score of a block from its mean: U[b][h][j] = sum_{c=0}^{D-1} q[b][h][c] *
 * mean[c] in fp64, ascending c (an estimate of the block's typical q.k, not
 * a bound); W[b][g][j] = max over the group's heads; -inf for j >= nb_b.
 * U may be NULL. */
int or_mean_scores(const or_layout* L, const double* q, const float* mean,
                   const int32_t* seq_lens, double* U, double* W);

#ifdef __cplusplus
}
#endif

#endif /* KVS_ORACLE_H */
