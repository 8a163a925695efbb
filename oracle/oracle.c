/*
 * oracle.c -- plain fp64 CPU oracle (TEST INFRASTRUCTURE ONLY; see oracle.h).
 *
 * Written for reading, not for speed: one thread, straight loops over the
 * definitions, a library qsort where an ordering is needed.  Build with
 * -ffp-contract=off so that every product and sum is rounded as written.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* element decoders                                                    */
/* ------------------------------------------------------------------ */

/* bfloat16 is the upper half of an IEEE binary32. */
double or_bf16_to_f64(uint16_t bits) {
  uint32_t w = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &w, sizeof f);
  return (double)f;
}

/* OCP 8-bit floating point, E4M3FN variant: 1 sign bit, 4 exponent bits
 * (bias 7), 3 mantissa bits; exponent field 0 is subnormal (m/8 * 2^-6);
 * S.1111.111 is NaN; there is no infinity.  Largest finite value 448. */
double or_e4m3_to_f64(uint8_t code) {
  int sign = (code >> 7) & 1;
  int e = (code >> 3) & 0xF;
  int m = code & 0x7;
  double v;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0)
    v = ldexp((double)m / 8.0, -6);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -v : v;
}

/* Value of a group-quantised fp8 element: the decoded code times its fp32
 * group scale, rounded once to fp32 ("分块稀疏注意力与KV Cache量化…" §2.4:
 * one scale per group of adjacent channels; symmetric, no zero point). */
float or_e4m3_scaled(uint8_t code, float scale) {
  float c = (float)or_e4m3_to_f64(code);
  float v = c * scale;
  return v;
}

int64_t or_kv_bytes_per_token(int32_t layers, int32_t kv_heads,
                              int32_t head_dim, int32_t bytes_per_elem) {
  return (int64_t)2 * layers * kv_heads * head_dim * bytes_per_elem;
}

/* ------------------------------------------------------------------ */
/* addressing helpers                                                  */
/* ------------------------------------------------------------------ */

static int layout_ok(const or_layout* L) {
  if (!L) return 0;
  if (L->B < 0 || L->Hq <= 0 || L->Hkv <= 0 || L->D <= 0 || L->S <= 0) return 0;
  if (L->Hq % L->Hkv != 0) return 0;
  if (L->max_blocks < 0 || L->num_pages < 0) return 0;
  if (L->kv_dtype < 0 || L->kv_dtype > 2) return 0;
  if (L->kv_dtype == 2 && (L->quant_group <= 0 || L->D % L->quant_group != 0)) return 0;
  return 1;
}

/* Element at flat index idx of a pool, with the fp8 scale of (page, g,
 * token s, channel c). */
static double pool_value(const or_layout* L, const void* pool, const float* scales,
                         int64_t idx, int64_t page, int32_t g, int32_t s, int32_t c) {
  if (L->kv_dtype == 0) return (double)((const float*)pool)[idx];
  if (L->kv_dtype == 1) return or_bf16_to_f64(((const uint16_t*)pool)[idx]);
  {
    int32_t groups = L->D / L->quant_group;
    int64_t sidx = ((page * L->Hkv + g) * (int64_t)L->S + s) * groups + c / L->quant_group;
    return (double)or_e4m3_scaled(((const uint8_t*)pool)[idx], scales[sidx]);
  }
}

/* K element (page, kv head g, token s within the page, channel c):
 * token-major tile [S][D]. */
static double kv_value(const or_layout* L, const void* pool, const float* scales,
                       int64_t page, int32_t g, int32_t s, int32_t c) {
  int64_t idx = ((page * L->Hkv + g) * (int64_t)L->S + s) * L->D + c;
  return pool_value(L, pool, scales, idx, page, g, s, c);
}

/* V element (page, kv head g, token s, channel c): the tile is cut into
 * runs of T = min(S, 32) consecutive tokens, each stored channel-major,
 * [S/T][D][T]. */
static double v_value(const or_layout* L, const void* pool, const float* scales,
                      int64_t page, int32_t g, int32_t s, int32_t c) {
  const int32_t T = L->S < 32 ? L->S : 32;
  int64_t idx = (((page * L->Hkv + g) * (int64_t)(L->S / T) + s / T) * L->D + c) * T + s % T;
  return pool_value(L, pool, scales, idx, page, g, s, c);
}

static int32_t num_blocks(const or_layout* L, int32_t len) {
  return (len + L->S - 1) / L->S;
}

static int len_ok(const or_layout* L, int32_t len) {
  return len >= 0 && (int64_t)len <= (int64_t)L->max_blocks * L->S;
}

/* ------------------------------------------------------------------ */
/* summaries                                                           */
/* ------------------------------------------------------------------ */

/* min and max per channel of K over the valid tokens of block j of
 * (sequence b, KV head g), stored in page `page`, into the summary table. */
static void block_min_max(const or_layout* L, const void* k_pool, const float* k_scales,
                          int32_t page, int32_t b, int32_t g, int32_t j, int32_t len,
                          double* out) {
  int32_t t_end = (j + 1) * L->S < len ? (j + 1) * L->S : len;
  double* mn = out + ((((int64_t)b * L->Hkv + g) * L->max_blocks + j) * 2 + 0) * L->D;
  double* mx = mn + L->D;
  for (int32_t c = 0; c < L->D; ++c) {
    double lo = INFINITY, hi = -INFINITY;
    for (int32_t t = j * L->S; t < t_end; ++t) {
      double v = kv_value(L, k_pool, k_scales, page, g, t - j * L->S, c);
      if (v < lo) lo = v;
      if (v > hi) hi = v;
    }
    mn[c] = lo;
    mx[c] = hi;
  }
}

int or_summaries(const or_layout* L, const void* k_pool, const float* k_scales,
                 const int32_t* block_table, const int32_t* seq_lens,
                 const int32_t* first_block, int32_t num_rebuild,
                 double* out) {
  if (!layout_ok(L) || !k_pool || !block_table || !seq_lens || !out) return OR_EARG;
  if (L->kv_dtype == 2 && !k_scales) return OR_EARG;
  if (num_rebuild < 0) return OR_EARG;
  for (int32_t b = 0; b < L->B; ++b) {
    int32_t len = seq_lens[b];
    if (!len_ok(L, len)) return OR_ERANGE;
    int32_t nb = num_blocks(L, len);
    int32_t j0 = first_block ? first_block[b] : 0;
    if (j0 < 0) return OR_ERANGE;
    int64_t j1 = (int64_t)j0 + num_rebuild;
    if (j1 > nb) j1 = nb;
    for (int32_t j = j0; j < j1; ++j) {
      int32_t page = block_table[(int64_t)b * L->max_blocks + j];
      if (page < 0 || page >= L->num_pages) return OR_ERANGE;
      for (int32_t g = 0; g < L->Hkv; ++g) block_min_max(L, k_pool, k_scales, page, b, g, j, len, out);
    }
  }
  return OR_OK;
}

/* ------------------------------------------------------------------ */
/* bounds                                                              */
/* ------------------------------------------------------------------ */

int or_bounds(const or_layout* L, const double* q, const double* summ,
              const int32_t* seq_lens, double* U, double* W) {
  if (!layout_ok(L) || !q || !summ || !seq_lens || !W) return OR_EARG;
  int32_t G = L->Hq / L->Hkv;
  for (int32_t b = 0; b < L->B; ++b) {
    int32_t len = seq_lens[b];
    if (!len_ok(L, len)) return OR_ERANGE;
    int32_t nb = num_blocks(L, len);
    for (int32_t g = 0; g < L->Hkv; ++g) {
      double* w = W + ((int64_t)b * L->Hkv + g) * L->max_blocks;
      for (int32_t j = 0; j < L->max_blocks; ++j) w[j] = -INFINITY;
    }
    for (int32_t h = 0; h < L->Hq; ++h) {
      int32_t g = h / G;
      const double* qh = q + ((int64_t)b * L->Hq + h) * L->D;
      double* w = W + ((int64_t)b * L->Hkv + g) * L->max_blocks;
      double* u = U ? U + ((int64_t)b * L->Hq + h) * L->max_blocks : NULL;
      for (int32_t j = 0; j < L->max_blocks; ++j) {
        if (j >= nb) {
          if (u) u[j] = -INFINITY;
          continue;
        }
        const double* mn = summ + ((((int64_t)b * L->Hkv + g) * L->max_blocks + j) * 2 + 0) * L->D;
        const double* mx = mn + L->D;
        double acc = 0.0;
        for (int32_t c = 0; c < L->D; ++c) {
          double lo = qh[c] * mn[c];
          double hi = qh[c] * mx[c];
          acc = acc + (lo > hi ? lo : hi);
        }
        if (u) u[j] = acc;
        if (acc > w[j]) w[j] = acc;
      }
    }
  }
  return OR_OK;
}

/* ------------------------------------------------------------------ */
/* selection                                                           */
/* ------------------------------------------------------------------ */

typedef struct {
  double w;
  int32_t j;
} cand_t;

/* W descending, then block id ascending. */
static int cand_cmp(const void* pa, const void* pb) {
  const cand_t* a = (const cand_t*)pa;
  const cand_t* b = (const cand_t*)pb;
  if (a->w > b->w) return -1;
  if (a->w < b->w) return 1;
  return (a->j > b->j) - (a->j < b->j);
}

int or_select_window(const or_layout* L, const double* W, const int32_t* seq_lens,
                     int32_t k, int32_t recent, int32_t* sel) {
  if (!layout_ok(L) || !W || !seq_lens || !sel) return OR_EARG;
  if (recent < 1 || k < recent + 1) return OR_EARG;
  cand_t* cands = (cand_t*)malloc(sizeof(cand_t) * (size_t)(L->max_blocks > 0 ? L->max_blocks : 1));
  unsigned char* chosen = (unsigned char*)malloc((size_t)(L->max_blocks > 0 ? L->max_blocks : 1));
  if (!cands || !chosen) {
    free(cands);
    free(chosen);
    return OR_EARG;
  }
  int rc = OR_OK;
  for (int32_t b = 0; b < L->B && rc == OR_OK; ++b) {
    int32_t len = seq_lens[b];
    if (!len_ok(L, len)) {
      rc = OR_ERANGE;
      break;
    }
    int32_t nb = num_blocks(L, len);
    for (int32_t g = 0; g < L->Hkv; ++g) {
      const double* w = W + ((int64_t)b * L->Hkv + g) * L->max_blocks;
      int32_t* out = sel + ((int64_t)b * L->Hkv + g) * k;
      memset(chosen, 0, (size_t)(nb > 0 ? nb : 1));
      if (nb <= k) {
        for (int32_t j = 0; j < nb; ++j) chosen[j] = 1;
      } else {
        /* nb > k >= recent + 1, so the sink and the window do not meet */
        chosen[0] = 1;                                       /* attention sink */
        for (int32_t j = nb - recent; j < nb; ++j) chosen[j] = 1;  /* recent window */
        int32_t n = 0;
        for (int32_t j = 1; j < nb - recent; ++j) {
          cands[n].w = w[j];
          cands[n].j = j;
          ++n;
        }
        qsort(cands, (size_t)n, sizeof(cand_t), cand_cmp);
        for (int32_t i = 0; i < k - 1 - recent; ++i) chosen[cands[i].j] = 1;
      }
      int32_t pos = 0;
      for (int32_t j = 0; j < nb; ++j)
        if (chosen[j]) out[pos++] = j;
      while (pos < k) out[pos++] = -1;
    }
  }
  free(cands);
  free(chosen);
  return rc;
}

int or_select(const or_layout* L, const double* W, const int32_t* seq_lens,
              int32_t k, int32_t* sel) {
  if (k < 2) return OR_EARG;
  return or_select_window(L, W, seq_lens, k, 1, sel);
}

/* ------------------------------------------------------------------ */
/* score smoothing across decode steps                                 */
/* ------------------------------------------------------------------ */

int or_ema_scores(const or_layout* L, const double* W, const int32_t* seq_lens,
                  double alpha, double* state, double* Wout) {
  if (!layout_ok(L) || !W || !seq_lens || !state || !Wout) return OR_EARG;
  if (!(alpha >= 0.0 && alpha <= 1.0)) return OR_EARG;
  const double beta = 1.0 - alpha;  /* the history's weight */
  for (int32_t b = 0; b < L->B; ++b) {
    int32_t len = seq_lens[b];
    if (!len_ok(L, len)) return OR_ERANGE;
    int32_t nb = num_blocks(L, len);
    for (int32_t g = 0; g < L->Hkv; ++g) {
      int64_t row = ((int64_t)b * L->Hkv + g) * L->max_blocks;
      for (int32_t j = 0; j < L->max_blocks; ++j) {
        if (j >= nb) {
          Wout[row + j] = -INFINITY;
          continue;
        }
        double now = W[row + j];
        double hist = state[row + j];
        double s;
        if (isnan(hist)) {
          s = now;  /* a block with no history yet */
        } else {
          double a = alpha * now;
          double h = beta * hist;
          s = a + h;
        }
        state[row + j] = s;
        Wout[row + j] = s;
      }
    }
  }
  return OR_OK;
}

int or_fuse_scores(const or_layout* L, const double* W, int32_t n_layers,
                   const int32_t* seq_lens, double* out) {
  if (!layout_ok(L) || !W || !seq_lens || !out || n_layers < 1) return OR_EARG;
  const int64_t layer_stride = (int64_t)L->B * L->Hkv * L->max_blocks;
  for (int32_t b = 0; b < L->B; ++b) {
    int32_t len = seq_lens[b];
    if (!len_ok(L, len)) return OR_ERANGE;
    int32_t nb = num_blocks(L, len);
    for (int32_t g = 0; g < L->Hkv; ++g) {
      int64_t row = ((int64_t)b * L->Hkv + g) * L->max_blocks;
      for (int32_t j = 0; j < L->max_blocks; ++j) {
        if (j >= nb) {
          out[row + j] = -INFINITY;
          continue;
        }
        double s = W[row + j];  /* the first layer's score */
        for (int32_t l = 1; l < n_layers; ++l) s = s + W[l * layer_stride + row + j];
        out[row + j] = s;
      }
    }
  }
  return OR_OK;
}

/* ------------------------------------------------------------------ */
/* attention                                                           */
/* ------------------------------------------------------------------ */

static double dot_qk(const or_layout* L, const double* qh, const void* k_pool,
                     const float* k_scales, int64_t page, int32_t g, int32_t s) {
  double acc = 0.0;
  for (int32_t c = 0; c < L->D; ++c)
    acc = acc + qh[c] * kv_value(L, k_pool, k_scales, page, g, s, c);
  return acc;
}

/* Validates one unit's selection row: strictly ascending ids in [0, nb)
 * followed only by -1 padding. */
static int check_sel_row(const int32_t* row, int32_t k, int32_t nb) {
  int32_t prev = -1;
  int padding = 0;
  for (int32_t i = 0; i < k; ++i) {
    int32_t j = row[i];
    if (j == -1) {
      padding = 1;
      continue;
    }
    if (padding) return OR_EORDER;
    if (j < 0 || j >= nb) return OR_ERANGE;
    if (j <= prev) return OR_EORDER;
    prev = j;
  }
  return OR_OK;
}

int or_sparse_attn(const or_layout* L, const double* q,
                   const void* k_pool, const void* v_pool,
                   const float* k_scales, const float* v_scales,
                   const int32_t* block_table, const int32_t* seq_lens,
                   const int32_t* sel, int32_t k, double sm_scale,
                   double* out) {
  if (!layout_ok(L) || !q || !k_pool || !v_pool || !block_table || !seq_lens || !sel || !out)
    return OR_EARG;
  if (L->kv_dtype == 2 && (!k_scales || !v_scales)) return OR_EARG;
  if (k < 0) return OR_EARG;
  int32_t G = L->Hq / L->Hkv;
  for (int32_t b = 0; b < L->B; ++b) {
    int32_t len = seq_lens[b];
    if (!len_ok(L, len)) return OR_ERANGE;
    int32_t nb = num_blocks(L, len);
    for (int32_t g = 0; g < L->Hkv; ++g) {
      const int32_t* row = sel + ((int64_t)b * L->Hkv + g) * k;
      int rc = check_sel_row(row, k, nb);
      if (rc != OR_OK) return rc;
      for (int32_t i = 0; i < k; ++i) {
        if (row[i] < 0) continue;
        int32_t page = block_table[(int64_t)b * L->max_blocks + row[i]];
        if (page < 0 || page >= L->num_pages) return OR_ERANGE;
      }
    }
    for (int32_t h = 0; h < L->Hq; ++h) {
      int32_t g = h / G;
      const double* qh = q + ((int64_t)b * L->Hq + h) * L->D;
      const int32_t* row = sel + ((int64_t)b * L->Hkv + g) * k;
      double* o = out + ((int64_t)b * L->Hq + h) * L->D;
      /* pass 1: the maximum score over the selected tokens */
      double m = -INFINITY;
      int64_t count = 0;
      for (int32_t i = 0; i < k; ++i) {
        int32_t j = row[i];
        if (j < 0) continue;
        int32_t page = block_table[(int64_t)b * L->max_blocks + j];
        for (int32_t t = j * L->S; t < (j + 1) * L->S && t < len; ++t) {
          double s = sm_scale * dot_qk(L, qh, k_pool, k_scales, page, g, t - j * L->S);
          if (s > m) m = s;
          ++count;
        }
      }
      for (int32_t c = 0; c < L->D; ++c) o[c] = 0.0;
      if (count == 0) continue;
      /* pass 2: normaliser and weighted sum of V */
      double l = 0.0;
      for (int32_t i = 0; i < k; ++i) {
        int32_t j = row[i];
        if (j < 0) continue;
        int32_t page = block_table[(int64_t)b * L->max_blocks + j];
        for (int32_t t = j * L->S; t < (j + 1) * L->S && t < len; ++t) {
          int32_t s_in = t - j * L->S;
          double p = exp(sm_scale * dot_qk(L, qh, k_pool, k_scales, page, g, s_in) - m);
          l = l + p;
          for (int32_t c = 0; c < L->D; ++c)
            o[c] = o[c] + p * v_value(L, v_pool, v_scales, page, g, s_in, c);
        }
      }
      for (int32_t c = 0; c < L->D; ++c) o[c] = o[c] / l;
    }
  }
  return OR_OK;
}

int or_dense_attn(const or_layout* L, const double* q,
                  const void* k_pool, const void* v_pool,
                  const float* k_scales, const float* v_scales,
                  const int32_t* block_table, const int32_t* seq_lens,
                  double sm_scale, double* out) {
  if (!layout_ok(L) || !q || !k_pool || !v_pool || !block_table || !seq_lens || !out)
    return OR_EARG;
  if (L->kv_dtype == 2 && (!k_scales || !v_scales)) return OR_EARG;
  int32_t G = L->Hq / L->Hkv;
  double* scores = NULL;
  for (int32_t b = 0; b < L->B; ++b) {
    int32_t len = seq_lens[b];
    if (!len_ok(L, len)) {
      free(scores);
      return OR_ERANGE;
    }
    for (int32_t t = 0; t < len; ++t) {
      int32_t page = block_table[(int64_t)b * L->max_blocks + t / L->S];
      if (page < 0 || page >= L->num_pages) {
        free(scores);
        return OR_ERANGE;
      }
    }
    double* grown = (double*)realloc(scores, sizeof(double) * (size_t)(len > 0 ? len : 1));
    if (!grown) {
      free(scores);
      return OR_EARG;
    }
    scores = grown;
    for (int32_t h = 0; h < L->Hq; ++h) {
      int32_t g = h / G;
      const double* qh = q + ((int64_t)b * L->Hq + h) * L->D;
      double* o = out + ((int64_t)b * L->Hq + h) * L->D;
      for (int32_t c = 0; c < L->D; ++c) o[c] = 0.0;
      if (len == 0) continue;
      double m = -INFINITY;
      for (int32_t t = 0; t < len; ++t) {
        int32_t page = block_table[(int64_t)b * L->max_blocks + t / L->S];
        double acc = 0.0;
        for (int32_t c = 0; c < L->D; ++c)
          acc = acc + qh[c] * kv_value(L, k_pool, k_scales, page, g, t % L->S, c);
        scores[t] = sm_scale * acc;
        if (scores[t] > m) m = scores[t];
      }
      double l = 0.0;
      for (int32_t t = 0; t < len; ++t) {
        int32_t page = block_table[(int64_t)b * L->max_blocks + t / L->S];
        double p = exp(scores[t] - m);
        l = l + p;
        for (int32_t c = 0; c < L->D; ++c)
          o[c] = o[c] + p * v_value(L, v_pool, v_scales, page, g, t % L->S, c);
      }
      for (int32_t c = 0; c < L->D; ++c) o[c] = o[c] / l;
    }
  }
  free(scores);
  return OR_OK;
}

/* ------------------------------------------------------------------ */
/* hot buffer step                                                     */
/* ------------------------------------------------------------------ */

typedef struct {
  int64_t stamp;
  int32_t slot;
} victim_t;

/* stamp ascending, then slot ascending */
static int victim_cmp(const void* pa, const void* pb) {
  const victim_t* a = (const victim_t*)pa;
  const victim_t* b = (const victim_t*)pb;
  if (a->stamp < b->stamp) return -1;
  if (a->stamp > b->stamp) return 1;
  return (a->slot > b->slot) - (a->slot < b->slot);
}

int or_hot_step(int32_t nb, int32_t ns, int32_t k, int64_t step,
                int32_t slot_base, const int32_t* sel, int32_t* pt,
                int32_t* owner, int64_t* stamp, int32_t* miss_list,
                int32_t* miss_cnt) {
  if (nb < 0 || ns <= 0 || k < 0 || step < 0 || slot_base < 0) return OR_EARG;
  if (!sel || !pt || !owner || !stamp || !miss_list || !miss_cnt) return OR_EARG;
  int rc = check_sel_row(sel, k, nb);
  if (rc != OR_OK) return rc;
  int32_t n = 0;
  for (int32_t i = 0; i < k; ++i)
    if (sel[i] >= 0) ++n;
  if (n > ns) return OR_ECAP;
  for (int32_t j = 0; j < nb; ++j)
    if (pt[j] != -1 && (pt[j] < slot_base || pt[j] >= slot_base + ns)) return OR_ERANGE;
  for (int32_t s = 0; s < ns; ++s)
    if (owner[s] < -1 || owner[s] >= nb) return OR_ERANGE;

  unsigned char* in_sel = (unsigned char*)calloc((size_t)(nb > 0 ? nb : 1), 1);
  victim_t* vict = (victim_t*)malloc(sizeof(victim_t) * (size_t)ns);
  if (!in_sel || !vict) {
    free(in_sel);
    free(vict);
    return OR_EARG;
  }
  for (int32_t i = 0; i < k; ++i)
    if (sel[i] >= 0) in_sel[sel[i]] = 1;

  /* hits refresh their stamp; misses are collected in ascending order */
  int32_t m = 0;
  for (int32_t i = 0; i < k; ++i) {
    int32_t j = sel[i];
    if (j < 0) continue;
    if (pt[j] >= 0)
      stamp[pt[j] - slot_base] = step;
    else
      miss_list[m++] = j;
  }
  for (int32_t i = m; i < k; ++i) miss_list[i] = -1;
  *miss_cnt = m;

  /* victims: slots not holding a selected block, least recently used first */
  int32_t nv = 0;
  for (int32_t s = 0; s < ns; ++s) {
    if (owner[s] >= 0 && in_sel[owner[s]]) continue;
    vict[nv].stamp = stamp[s];
    vict[nv].slot = s;
    ++nv;
  }
  qsort(vict, (size_t)nv, sizeof(victim_t), victim_cmp);
  for (int32_t r = 0; r < m; ++r) {
    int32_t s = vict[r].slot;
    if (owner[s] >= 0) pt[owner[s]] = -1;
    pt[miss_list[r]] = slot_base + s;
    owner[s] = miss_list[r];
    stamp[s] = step;
  }
  free(in_sel);
  free(vict);
  return OR_OK;
}

/* ------------------------------------------------------------------ */
/* appending the decode token                                          */
/* ------------------------------------------------------------------ */

static size_t elem_bytes(const or_layout* L) {
  return L->kv_dtype == 0 ? 4 : (L->kv_dtype == 1 ? 2 : 1);
}

int or_append_token(const or_layout* L, const void* k_new, const void* v_new,
                    const float* k_new_scales, const float* v_new_scales,
                    const int32_t* block_table, const int32_t* seq_lens,
                    void* k_pool, void* v_pool, float* k_scales, float* v_scales,
                    double* summ, void* host_k, void* host_v,
                    float* host_k_scales, float* host_v_scales) {
  if (!layout_ok(L) || !k_new || !v_new || !block_table || !seq_lens || !k_pool || !v_pool || !summ)
    return OR_EARG;
  const int fp8 = L->kv_dtype == 2;
  if (fp8 && (!k_new_scales || !v_new_scales || !k_scales || !v_scales)) return OR_EARG;
  if ((host_k != NULL) != (host_v != NULL)) return OR_EARG;
  if (host_k && fp8 && (!host_k_scales || !host_v_scales)) return OR_EARG;
  const size_t eb = elem_bytes(L);
  const int32_t S = L->S, D = L->D, T = L->S < 32 ? L->S : 32;
  const int32_t groups = fp8 ? D / L->quant_group : 0;
  for (int32_t b = 0; b < L->B; ++b) {
    int32_t len = seq_lens[b];
    if (!len_ok(L, len)) return OR_ERANGE;
    if (len == 0) continue;  /* nothing to append */
    int32_t t = len - 1, j = t / S, s = t % S;
    int32_t page = block_table[(int64_t)b * L->max_blocks + j];
    if (page < 0 || page >= L->num_pages) return OR_ERANGE;
    for (int32_t g = 0; g < L->Hkv; ++g) {
      int64_t tile = (int64_t)page * L->Hkv + g;  /* (page, head) tile */
      int64_t src = ((int64_t)b * L->Hkv + g) * D;
      for (int32_t c = 0; c < D; ++c) {
        int64_t kd = (tile * S + s) * D + c;                               /* [S][D] */
        int64_t vd = ((tile * (S / T) + s / T) * D + c) * T + s % T;       /* [S/T][D][T] */
        memcpy((char*)k_pool + kd * eb, (const char*)k_new + (src + c) * eb, eb);
        memcpy((char*)v_pool + vd * eb, (const char*)v_new + (src + c) * eb, eb);
      }
      for (int32_t q = 0; q < groups; ++q) {
        k_scales[(tile * S + s) * groups + q] = k_new_scales[((int64_t)b * L->Hkv + g) * groups + q];
        v_scales[(tile * S + s) * groups + q] = v_new_scales[((int64_t)b * L->Hkv + g) * groups + q];
      }
      /* the block's summary over its valid tokens, the new one included */
      block_min_max(L, k_pool, k_scales, page, b, g, j, len, summ);
      /* a block that is now full is sealed: it goes to the host tier */
      if (host_k && len % S == 0) {
        int64_t hb = ((int64_t)b * L->Hkv + g) * L->max_blocks + j;  /* host tile */
        size_t tile_bytes = (size_t)S * D * eb;
        memcpy((char*)host_k + hb * (int64_t)tile_bytes, (const char*)k_pool + tile * (int64_t)tile_bytes, tile_bytes);
        memcpy((char*)host_v + hb * (int64_t)tile_bytes, (const char*)v_pool + tile * (int64_t)tile_bytes, tile_bytes);
        if (fp8) {
          size_t sc = (size_t)S * groups;
          memcpy(host_k_scales + hb * (int64_t)sc, k_scales + tile * (int64_t)sc, sc * sizeof(float));
          memcpy(host_v_scales + hb * (int64_t)sc, v_scales + tile * (int64_t)sc, sc * sizeof(float));
        }
      }
    }
  }
  return OR_OK;
}

/* ------------------------------------------------------------------ */
/* mean summaries                                                      */
/* ------------------------------------------------------------------ */

int or_summaries_mean(const or_layout* L, const void* k_pool, const float* k_scales,
                      const int32_t* block_table, const int32_t* seq_lens,
                      const int32_t* first_block, int32_t num_rebuild, float* out) {
  if (!layout_ok(L) || !k_pool || !block_table || !seq_lens || !out) return OR_EARG;
  if (L->kv_dtype == 2 && !k_scales) return OR_EARG;
  if (num_rebuild < 0) return OR_EARG;
  for (int32_t b = 0; b < L->B; ++b) {
    int32_t len = seq_lens[b];
    if (!len_ok(L, len)) return OR_ERANGE;
    int32_t nb = num_blocks(L, len);
    int32_t j0 = first_block ? first_block[b] : 0;
    if (j0 < 0) return OR_ERANGE;
    int64_t j1 = (int64_t)j0 + num_rebuild;
    if (j1 > nb) j1 = nb;
    for (int32_t j = j0; j < j1; ++j) {
      int32_t page = block_table[(int64_t)b * L->max_blocks + j];
      if (page < 0 || page >= L->num_pages) return OR_ERANGE;
      int32_t t_end = (j + 1) * L->S < len ? (j + 1) * L->S : len;
      int32_t n = t_end - j * L->S;
      for (int32_t g = 0; g < L->Hkv; ++g) {
        float* m = out + (((int64_t)b * L->Hkv + g) * L->max_blocks + j) * L->D;
        for (int32_t c = 0; c < L->D; ++c) {
          double sum = 0.0;
          for (int32_t t = j * L->S; t < t_end; ++t)
            sum = sum + kv_value(L, k_pool, k_scales, page, g, t - j * L->S, c);
          double mean = sum / (double)n;
          m[c] = (float)mean;
        }
      }
    }
  }
  return OR_OK;
}

int or_mean_scores(const or_layout* L, const double* q, const float* mean,
                   const int32_t* seq_lens, double* U, double* W) {
  if (!layout_ok(L) || !q || !mean || !seq_lens || !W) return OR_EARG;
  int32_t G = L->Hq / L->Hkv;
  for (int32_t b = 0; b < L->B; ++b) {
    int32_t len = seq_lens[b];
    if (!len_ok(L, len)) return OR_ERANGE;
    int32_t nb = num_blocks(L, len);
    for (int32_t g = 0; g < L->Hkv; ++g) {
      double* w = W + ((int64_t)b * L->Hkv + g) * L->max_blocks;
      for (int32_t j = 0; j < L->max_blocks; ++j) w[j] = -INFINITY;
    }
    for (int32_t h = 0; h < L->Hq; ++h) {
      int32_t g = h / G;
      const double* qh = q + ((int64_t)b * L->Hq + h) * L->D;
      double* w = W + ((int64_t)b * L->Hkv + g) * L->max_blocks;
      double* u = U ? U + ((int64_t)b * L->Hq + h) * L->max_blocks : NULL;
      for (int32_t j = 0; j < L->max_blocks; ++j) {
        if (j >= nb) {
          if (u) u[j] = -INFINITY;
          continue;
        }
        const float* m = mean + (((int64_t)b * L->Hkv + g) * L->max_blocks + j) * L->D;
        double acc = 0.0;
        for (int32_t c = 0; c < L->D; ++c) acc = acc + qh[c] * (double)m[c];
        if (u) u[j] = acc;
        if (acc > w[j]) w[j] = acc;
      }
    }
  }
  return OR_OK;
}
