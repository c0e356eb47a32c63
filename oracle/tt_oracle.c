/*
 * tt_oracle.c -- plain, slow fp64 CPU oracle for the TwoTower denoiser
 * block-attention step and the confidence unmask that follows it.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  It shares no code,
 * header, table or helper with the GPU library (two_tower_attention_amd/),
 * and the GPU library never calls it.
 *
 * Sources, cited by page title and section:
 *   [REVIEW]  "Nemotron-Labs-TwoTower: Diffusion Language Modeling with
 *             Pretrained Autoregressive Context" (paperfeed.app review),
 *             sections "The idea: freeze the reader, train the writer" and
 *             "Training and sampling".
 *   [SKY]     "NVIDIA's Dual-Tower Diffusion Language Model Explained"
 *             (kongchang.com), sections "The 'Sky Bridges' Between Layers"
 *             and "Generating Text in Parallel Like Solving a Sudoku".
 *   [BOLTED]  "NVIDIA Bolted a Diffusion Model Onto a Frozen LLM ..."
 *             (aibacon.net), section "The two-tower trick".
 *
 * Every function follows the plain definition; no blocking, fusion or
 * reordering beyond it.  Memory layouts are the ones documented for the
 * library's C ABI (row-major):
 *   q                [B, S, Hq, D]
 *   k_blk, v_blk     [B, S, Hkv, D]
 *   k_pages          [P, Hkv, page_size, D]   (token-major)
 *   v_pages          [P, Hkv, D, page_size]   (feature-major inside a page)
 *   page_table       int32 [B, max_pages]
 *   ctx_lens         int32 [B]
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define TTO_OK 0
#define TTO_ERR_ARG (-1)
#define TTO_ERR_PAGE (-2)
#define TTO_ERR_MEM (-3)

/* Decode one stored element exactly to double.  bf16 is the upper half of an
 * IEEE binary32, so widening is a 16-bit left shift of the bit pattern. */
static double elem(const void *base, size_t idx, int is_bf16) {
  if (is_bf16) {
    uint32_t u = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
  }
  return (double)((const float *)base)[idx];
}

/*
 * Block attention for one query row (b, t, h).
 *
 * [REVIEW, "The idea: freeze the reader, train the writer"]: at denoiser
 * layer i the queries of the noisy block attend over keys and values that
 * concatenate the context tower's layer-i cache for the committed past with
 * the denoiser's own keys/values of the current block; attention inside the
 * block is bidirectional.  The printed equation is lost in the extracted
 * text, so the operation is the plain softmax attention over that explicit
 * concatenation (context first, then the S block tokens), with no mask: every
 * block query sees all committed context tokens and all S block tokens.
 * GQA: query head h reads KV head h / (Hq / Hkv).
 *
 * causal != 0 is the context tower ingesting a committed chunk of S tokens
 * ([REVIEW, "The idea: freeze the reader, train the writer"]: the frozen
 * context tower runs causally over clean tokens, and ingests a committed
 * block as one clean forward chunk, updating its caches): chunk position t
 * attends over the committed context and chunk tokens 0..t only, so the
 * concatenation for that row ends at chunk token t.
 */
static int attn_row(int S, int Hq, int Hkv, int D, int page_size, int max_pages,
                    int num_pages, double scale, int is_bf16, const void *q,
                    const void *k_blk, const void *v_blk, const void *k_pages,
                    const void *v_pages, const int32_t *page_table,
                    const int32_t *ctx_lens, int b, int t, int h, int causal, double *out,
                    double *wsum) {
  const int g = Hq / Hkv;
  const int hk = h / g;
  const int L = ctx_lens[b];
  const int Sk = causal ? t + 1 : S;   /* block/chunk tokens in the concatenation */
  const int N = L + Sk;
  if (L < 0 || L > max_pages * page_size) return TTO_ERR_PAGE;

  /* 1. the explicit concatenation Kcat = [K_ctx ; K_blk], Vcat likewise */
  double *kc = (double *)malloc(sizeof(double) * (size_t)N * D);
  double *vc = (double *)malloc(sizeof(double) * (size_t)N * D);
  double *s = (double *)malloc(sizeof(double) * (size_t)N);
  if (!kc || !vc || !s) { free(kc); free(vc); free(s); return TTO_ERR_MEM; }
  for (int j = 0; j < L; ++j) {
    const int page = page_table[(size_t)b * max_pages + j / page_size];
    const int off = j % page_size;
    if (page < 0 || page >= num_pages) { free(kc); free(vc); free(s); return TTO_ERR_PAGE; }
    for (int d = 0; d < D; ++d) {
      kc[(size_t)j * D + d] =
          elem(k_pages, (((size_t)page * Hkv + hk) * page_size + off) * D + d, is_bf16);
      vc[(size_t)j * D + d] =
          elem(v_pages, (((size_t)page * Hkv + hk) * D + d) * page_size + off, is_bf16);
    }
  }
  for (int j = 0; j < Sk; ++j)
    for (int d = 0; d < D; ++d) {
      const size_t src = (((size_t)b * S + j) * Hkv + hk) * D + d;
      kc[(size_t)(L + j) * D + d] = elem(k_blk, src, is_bf16);
      vc[(size_t)(L + j) * D + d] = elem(v_blk, src, is_bf16);
    }

  /* 2. scores s_j = scale * <q, Kcat_j> */
  const size_t qoff = (((size_t)b * S + t) * Hq + h) * D;
  for (int j = 0; j < N; ++j) {
    double acc = 0.0;
    for (int d = 0; d < D; ++d) acc += elem(q, qoff + d, is_bf16) * kc[(size_t)j * D + d];
    s[j] = scale * acc;
  }
  /* 3. softmax: m = max s, p_j = exp(s_j - m), Z = sum p */
  double m = -INFINITY;
  for (int j = 0; j < N; ++j) if (s[j] > m) m = s[j];
  double Z = 0.0;
  for (int j = 0; j < N; ++j) { s[j] = exp(s[j] - m); Z += s[j]; }
  /* 4. O = sum_j (p_j / Z) * Vcat_j */
  double ws = 0.0;
  for (int d = 0; d < D; ++d) out[d] = 0.0;
  for (int j = 0; j < N; ++j) {
    const double w = s[j] / Z;
    ws += w;
    for (int d = 0; d < D; ++d) out[d] += w * vc[(size_t)j * D + d];
  }
  if (wsum) *wsum = ws;
  free(kc); free(vc); free(s);
  return TTO_OK;
}

static int attn_rows(int B, int S, int Hq, int Hkv, int D, int page_size,
                     int max_pages, int num_pages, double scale, int is_bf16,
                     const void *q, const void *k_blk, const void *v_blk,
                     const void *k_pages, const void *v_pages,
                     const int32_t *page_table, const int32_t *ctx_lens,
                     int n_rows, const int32_t *rows, int causal, double *out, double *wsum) {
  if (B < 0 || S < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || D < 1 || page_size < 1 ||
      max_pages < 1)
    return TTO_ERR_ARG;
  const int total = rows ? n_rows : B * S * Hq;
  int err = TTO_OK;
#pragma omp parallel for schedule(dynamic, 1)
  for (int r = 0; r < total; ++r) {
    int b, t, h;
    if (rows) { b = rows[3 * r]; t = rows[3 * r + 1]; h = rows[3 * r + 2]; }
    else { b = r / (S * Hq); t = (r / Hq) % S; h = r % Hq; }
    int e;
    if (b < 0 || b >= B || t < 0 || t >= S || h < 0 || h >= Hq) e = TTO_ERR_ARG;
    else
      e = attn_row(S, Hq, Hkv, D, page_size, max_pages, num_pages, scale, is_bf16, q,
                   k_blk, v_blk, k_pages, v_pages, page_table, ctx_lens, b, t, h, causal,
                   out + (size_t)r * D, wsum ? wsum + r : NULL);
    if (e) {
#pragma omp critical
      err = e;
    }
  }
  return err;
}

/*
 * Block attention over rows.  rows == NULL: all B*S*Hq rows, out is
 * [B, S, Hq, D].  Otherwise rows holds n_rows triples (b, t, h) and out is
 * [n_rows, D].  wsum (optional, per row) receives sum_j p_j / Z.
 */
int tto_block_attn(int B, int S, int Hq, int Hkv, int D, int page_size,
                   int max_pages, int num_pages, double scale, int is_bf16,
                   const void *q, const void *k_blk, const void *v_blk,
                   const void *k_pages, const void *v_pages,
                   const int32_t *page_table, const int32_t *ctx_lens,
                   int n_rows, const int32_t *rows, double *out, double *wsum) {
  return attn_rows(B, S, Hq, Hkv, D, page_size, max_pages, num_pages, scale, is_bf16, q, k_blk,
                   v_blk, k_pages, v_pages, page_table, ctx_lens, n_rows, rows, 0, out, wsum);
}

/* Causal chunk ingest: as tto_block_attn, chunk position t seeing chunk
 * tokens 0..t only (see attn_row). */
int tto_chunk_attn(int B, int S, int Hq, int Hkv, int D, int page_size,
                   int max_pages, int num_pages, double scale, int is_bf16,
                   const void *q, const void *k_blk, const void *v_blk,
                   const void *k_pages, const void *v_pages,
                   const int32_t *page_table, const int32_t *ctx_lens,
                   int n_rows, const int32_t *rows, double *out, double *wsum) {
  return attn_rows(B, S, Hq, Hkv, D, page_size, max_pages, num_pages, scale, is_bf16, q, k_blk,
                   v_blk, k_pages, v_pages, page_table, ctx_lens, n_rows, rows, 1, out, wsum);
}

/*
 * Confidence of one row of logits.
 *
 * [REVIEW, "Training and sampling"] and [SKY, "Generating Text in Parallel
 * Like Solving a Sudoku"]: every masked position is predicted in parallel and
 * the confident predictions are committed.  The pages do not define the
 * confidence; it is read as the greedy prediction's softmax probability at
 * temperature 1:  m = max_v l[v],  id = smallest v with l[v] == m,
 * Z = sum_v exp(l[v] - m),  conf = 1 / Z.
 */
static void row_conf(const float *row, int V, int32_t *id, double *conf) {
  double m = -INFINITY;
  int arg = 0;
  for (int v = 0; v < V; ++v)
    if ((double)row[v] > m) { m = (double)row[v]; arg = v; }
  double Z = 0.0;
  for (int v = 0; v < V; ++v) Z += exp((double)row[v] - m);
  *id = arg;
  *conf = 1.0 / Z;
}

/*
 * Confidence unmask over B sequences of S positions.
 *
 * Only masked positions are candidates: committed tokens stay fixed as
 * anchors ([SKY, "Generating Text in Parallel Like Solving a Sudoku"]).
 * This is the count form of the commit rule: per sequence, the k_eff masked
 * positions with the highest confidence are committed, ties going to the
 * lower position, where k_eff = clamp(k_b, 0, #masked) and k_b is k_commit[b]
 * or, when k_commit is NULL, ceil(#masked / remaining_steps).
 * ids/conf are written for every row; commit[b*S+t] = 1 exactly on the
 * committed positions.
 */
/* Count-form commit over precomputed confidences (shared by the fp32-logits
 * and the LM-head entry points below). */
static int commit_count(int B, int S, const uint8_t *mask, const int32_t *k_commit,
                        int remaining_steps, const double *conf, uint8_t *commit) {
  int *cand = (int *)malloc(sizeof(int) * (size_t)S);
  if (!cand) return TTO_ERR_MEM;
  for (int b = 0; b < B; ++b) {
    int n = 0;
    for (int t = 0; t < S; ++t) {
      commit[(size_t)b * S + t] = 0;
      if (mask[(size_t)b * S + t]) cand[n++] = t;
    }
    long kb = k_commit ? (long)k_commit[b]
                       : ((long)n + remaining_steps - 1) / remaining_steps;
    if (kb < 0) kb = 0;
    if (kb > n) kb = n;
    /* order candidates by (conf descending, position ascending) */
    for (int i = 1; i < n; ++i) {
      const int x = cand[i];
      int j = i - 1;
      while (j >= 0) {
        const double cj = conf[(size_t)b * S + cand[j]], cx = conf[(size_t)b * S + x];
        if (cj > cx || (cj == cx && cand[j] < x)) break;
        cand[j + 1] = cand[j];
        --j;
      }
      cand[j + 1] = x;
    }
    for (int i = 0; i < kb; ++i) commit[(size_t)b * S + cand[i]] = 1;
  }
  free(cand);
  return TTO_OK;
}

int tto_unmask(int B, int S, int V, const float *logits, const uint8_t *mask,
               const int32_t *k_commit, int remaining_steps, int32_t *ids,
               uint8_t *commit, double *conf) {
  if (B < 0 || S < 1 || V < 1) return TTO_ERR_ARG;
  if (!k_commit && remaining_steps < 1) return TTO_ERR_ARG;
#pragma omp parallel for schedule(static)
  for (int r = 0; r < B * S; ++r) row_conf(logits + (size_t)r * V, V, ids + r, conf + r);
  return commit_count(B, S, mask, k_commit, remaining_steps, conf, commit);
}

/*
 * LM head ahead of the unmask.
 *
 * [REVIEW, "Training and sampling"] and [SKY, "Generating Text in Parallel
 * Like Solving a Sudoku"]: the denoiser predicts every masked position of the
 * block, i.e. its final hidden state goes through the model's output head to
 * logits over the vocabulary, and the confidence rule above runs on those
 * logits.  The pages give neither the head's shape nor its weights; the head
 * is read as a plain linear map without bias, logits[r][v] = sum_h
 * hidden[r][h] * weight[v][h] (weight stored one vocabulary row after
 * another), inputs in bf16, evaluated here exactly in fp64.
 *
 * rows (may be NULL = 0..nrows-1) selects which hidden rows to evaluate;
 * logits receives nrows x V values.
 */
int tto_lmhead_logits(int R, int H, int V, const uint16_t *hidden, const uint16_t *weight,
                      const int32_t *rows, int nrows, double *logits) {
  if (R < 0 || H < 1 || V < 1 || nrows < 0) return TTO_ERR_ARG;
  for (int i = 0; i < nrows; ++i) {
    const int r = rows ? rows[i] : i;
    if (r < 0 || r >= R) return TTO_ERR_ARG;
  }
#pragma omp parallel for schedule(static)
  for (long iv = 0; iv < (long)nrows * V; ++iv) {
    const int i = (int)(iv / V), v = (int)(iv % V);
    const int r = rows ? rows[i] : i;
    double acc = 0.0;
    for (int h = 0; h < H; ++h)
      acc += elem(hidden, (size_t)r * H + h, 1) * elem(weight, (size_t)v * H + h, 1);
    logits[iv] = acc;
  }
  return TTO_OK;
}

/* The confidence of one row of fp64 logits (same definition as row_conf). */
static void row_conf_f64(const double *row, int V, int32_t *id, double *conf) {
  double m = -INFINITY;
  int arg = 0;
  for (int v = 0; v < V; ++v)
    if (row[v] > m) { m = row[v]; arg = v; }
  double Z = 0.0;
  for (int v = 0; v < V; ++v) Z += exp(row[v] - m);
  *id = arg;
  *conf = 1.0 / Z;
}

/* Count-form unmask on fp64 logits (the LM head's exact output). */
int tto_unmask_f64(int B, int S, int V, const double *logits, const uint8_t *mask,
                   const int32_t *k_commit, int remaining_steps, int32_t *ids,
                   uint8_t *commit, double *conf) {
  if (B < 0 || S < 1 || V < 1) return TTO_ERR_ARG;
  if (!k_commit && remaining_steps < 1) return TTO_ERR_ARG;
#pragma omp parallel for schedule(static)
  for (int r = 0; r < B * S; ++r) row_conf_f64(logits + (size_t)r * V, V, ids + r, conf + r);
  return commit_count(B, S, mask, k_commit, remaining_steps, conf, commit);
}

/*
 * Threshold form of the commit rule.
 *
 * [REVIEW, "Training and sampling"]: at each step every masked position is
 * predicted and each prediction whose confidence is above gamma (0.8 on the
 * pages) is committed; the number committed per step adapts to the text.
 * [SKY, "Generating Text in Parallel Like Solving a Sudoku"]: commit the
 * positions whose confidence exceeds the threshold, re-mask the rest, run
 * again.  Readings: "above"/"exceeds" is strict (conf > gamma).  The pages
 * do not say what a step does when no masked position clears gamma; here it
 * commits the single most confident masked position (ties to the lower
 * position), so every step makes progress.  Committed positions are never
 * candidates.
 *
 * ids/conf are written for every row (as in tto_unmask); commit[b*S+t] = 1
 * exactly on the committed positions.  nsteps (may be NULL) counts, per
 * sequence, the calls that found at least one masked position.
 */
int tto_unmask_threshold(int B, int S, int V, const float *logits, const uint8_t *mask,
                         double gamma, int32_t *ids, uint8_t *commit, double *conf,
                         int32_t *nsteps) {
  if (B < 0 || S < 1 || V < 1) return TTO_ERR_ARG;
#pragma omp parallel for schedule(static)
  for (int r = 0; r < B * S; ++r) row_conf(logits + (size_t)r * V, V, ids + r, conf + r);

  for (int b = 0; b < B; ++b) {
    int n = 0, n_above = 0, best = -1;
    for (int t = 0; t < S; ++t) {
      const size_t r = (size_t)b * S + t;
      commit[r] = 0;
      if (!mask[r]) continue;
      ++n;
      if (conf[r] > gamma) {
        commit[r] = 1;
        ++n_above;
      }
      /* most confident masked position; strict > keeps the lower one on ties */
      if (best < 0 || conf[r] > conf[(size_t)b * S + best]) best = t;
    }
    if (n > 0 && n_above == 0) commit[(size_t)b * S + best] = 1;
    if (nsteps && n > 0) nsteps[b] += 1;
  }
  return TTO_OK;
}

/* Threads the OpenMP runtime will use (for reporting). */
int tto_num_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Sets the number of OpenMP threads later calls use (n >= 1), for timing the
   oracle on one thread as well as on all of them. */
void tto_set_num_threads(int n) {
#ifdef _OPENMP
  extern void omp_set_num_threads(int);
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
