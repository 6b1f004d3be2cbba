/*
 * echo_oracle.c -- plain, slow CPU oracle for the ECHO decode-step hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file: only the test suite, the smoke check and the CPU-baseline leg
 * of the benchmark use it.  It shares no header, table, constant or helper with
 * the GPU library; every value it needs comes in through its own arguments.
 *
 * Sources (all statements are restated, not quoted):
 *  [P1]  "ECHO: Efficient KV Cache Offloading with Lossless Prefetching for
 *        Serving Native Sparse Attention LLMs (OSDI 2026)", review page on
 *        awesome-system-papers: sections "Problem and motivation" (indexer
 *        scores every past token, the top 2048 are kept), "Key observations"
 *        (observation 2: EMA with smoothing 0.5 of the 2048th score),
 *        "Core method / in-graph per-layer cache management" (free bitmap,
 *        eviction priority, index buffer, two-way host/GPU maps, allocation
 *        by parallel scan, free protects the selected tokens, eviction moves
 *        no data, recall finds misses from the map; metadata 4*N_H + 13*N_G
 *        bytes per layer), "Core method / decode" (EMA threshold prefetch
 *        during scoring under a global counter whose cap grows with context;
 *        exact top-k and recall of every missing selected token).
 *  [P2]  "ECHO: Lossless KV Cache Offloading for Sparse Attention LLMs",
 *        podcast show notes: prediction only decides when to move data; every
 *        missed token is recalled; management state lives in fixed-size
 *        integer tensors.  Source 8 of its list is the DeepSeek-V3.2-Exp
 *        report, whose lightning indexer is
 *        score(s) = sum_j w_j * ReLU(q_j . k_s).
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *  R1  The indexer K is OCP fp8 E4M3FN with scale 1; q is bf16; w is fp32.
 *  R2  Scores are computed in fp64 and rounded once (nearest-even) to fp32;
 *      -0 is replaced by +0.
 *  R3  Top-k order is (score descending, token index ascending); the result
 *      is reported in ascending token order; if ctx <= k every token is kept.
 *  R4  EMA: theta = +inf means "no estimate yet"; the first k-th score seeds
 *      it; afterwards theta <- alpha*s_k + (1-alpha)*theta in fp32 (two
 *      products and one sum, each rounded).  Updated only when ctx >= k.
 *  R5  Prefetch: candidates are tokens with score > theta that have no GPU
 *      slot; request b takes at most cap_b = min(k, ceil(ctx_b/cap_div)) of
 *      them, the first ones in token order, and the free slots
 *      F[off_b + r] (F = ascending free list at step start,
 *      off_b = sum of earlier caps).  Installed with priority t.
 *  R6  Protect: a selected resident token gets priority t.  Misses are listed
 *      in (request, token) order.
 *  R7  Evict: E = occupied slots with priority < t, ordered by
 *      (priority, slot).  n_evict = min(|E|, max(0, |M| + R - n_free)) with
 *      R = sum of caps (reserve for the next step's prefetch).  If
 *      n_free + |E| < |M| the step stops with a capacity error.
 *  R8  Alloc: miss i takes the i-th slot of the ascending free list after
 *      eviction, priority t; its latent row is copied from the host pool.
 *  R9  t (the decode-step counter) advances by one after a successful step.
 *  R10 Append: the step's new token takes host id host_base + ctx of its
 *      request; its indexer key and latent are written there and ctx grows by
 *      one.  It is not placed in the GPU pool.
 *  R11 Attention input: the rows a sparse attention reads are the latents of
 *      the selected tokens in selection order; without offloading they come
 *      straight from the full host copy.  Unused rows (i >= n_sel) are zero.
 *  R12 Request lifecycle: releasing (cancelling) a request gives back the GPU
 *      slot of every token of its host range, clears the range's host-to-GPU
 *      map, resets its EMA threshold to "no estimate" and empties it
 *      (ctx = 0); no bytes move, the host copy stays.  Admitting a request
 *      into an empty batch row sets its host range and length after checking
 *      that the range fits, overlaps no live request and holds no mapped
 *      token; its threshold starts at "no estimate".
 *  R13 Chunked prefill: one request's history of N tokens is fixed while a
 *      chunk of C queries is scored against it (the chunk's own tokens are
 *      not offloaded yet).  Each query keeps its exact top-k.  Its coarse
 *      candidates are the tokens whose 256-bucket key of
 *      fp16(fp32(score - pred)) lies strictly above the bucket where the
 *      count from the top first reaches k (every token if N <= k); pred is
 *      the caller's predicted k-th score for the query (0 if none given).
 *      The union of the candidates is installed first (the transfer that
 *      overlaps the next chunk's scoring), then the rest of the union of the
 *      selections, each at the next ascending free slot, with priority t.
 *      The pool is sized to hold the chunk's union: a prefill chunk evicts
 *      nothing.  Capacity is checked per stage, as each stage's set becomes
 *      known: if the candidates that are not resident exceed the free slots,
 *      nothing changes; if the rest of the union then exceeds what is left,
 *      the candidates stay installed and nothing else changes (the step
 *      counter does not advance).  Both report a capacity error.
 *  R14 Page tables: a request's tokens need not occupy one contiguous host
 *      range.  The host pool is cut into pages of 16 consecutive host ids
 *      (one group of the tiled indexer K), and a request holds a list of
 *      pages: its token s is host id 16 * page[s / 16] + s % 16.  Every map,
 *      score, install, copy and release goes through that translation;
 *      nothing else in the step changes.  Pages of live requests are
 *      distinct: admission checks that the new request's pages are in the
 *      pool, listed once, and shared with no live request (a page shared with
 *      one is a capacity error, like an overlapping range); a decode append
 *      writes into the page its request lists for the new token (the caller
 *      hands out pages) and checks that it exists and is not mapped.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Threads of the scoring loop's OpenMP team (the CPU baseline times the oracle on one
 * thread and on every core).  Returns the previous maximum.  No arithmetic of the
 * method depends on it. */
int orc_set_threads(int n) {
  const int old = omp_get_max_threads();
  if (n > 0) omp_set_num_threads(n);
  return old;
}

#define ORC_OK 0
#define ORC_EINVAL (-1)
#define ORC_ECAPACITY (-4)
#define ORC_EDEVARG (-6)

/* Where each request's tokens live in the host pool (R14).  With a page table
 * (pages != NULL), token s of request b is host id
 * 16 * pages[b * page_stride + s / 16] + s % 16; without one, host_base[b] + s.
 * host_base is written by admission in the contiguous case. */
typedef struct {
  int32_t *host_base;   /* [B], or NULL with a page table */
  const int32_t *pages; /* [B][page_stride], or NULL     */
  int32_t page_stride;
} orc_tokmap;

static int64_t host_id(const orc_tokmap *m, int b, int64_t s) {
  if (m->pages) return 16 * (int64_t)m->pages[(int64_t)b * m->page_stride + s / 16] + s % 16;
  return (int64_t)m->host_base[b] + s;
}

/* Whether request b's first n tokens all have a host id in [0, n_host): every page
 * they use lies in the pool (with a page table), or the range fits (without). */
static int tokens_fit(const orc_tokmap *m, int b, int64_t n, int64_t n_host) {
  if (n < 0) return 0;
  if (!m->pages) return m->host_base[b] >= 0 && (int64_t)m->host_base[b] + n <= n_host;
  if ((n + 15) / 16 > m->page_stride) return 0;
  for (int64_t j = 0; j < (n + 15) / 16; ++j) {
    const int32_t p = m->pages[(int64_t)b * m->page_stride + j];
    if (p < 0 || 16 * (int64_t)p + 16 > n_host) return 0;
  }
  return 1;
}

#define ORC_MODE_EMA 0
#define ORC_MODE_NEG_INF 1
#define ORC_MODE_POS_INF 2

/* ---------------------------------------------------------------- formats */

/* OCP fp8 E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent 0
 * holds subnormals m * 2^-9; 0x7F / 0xFF are NaN; there is no infinity.    */
double orc_e4m3_value(uint8_t code) {
  int sign = (code >> 7) & 1;
  int e = (code >> 3) & 0xF;
  int m = code & 0x7;
  double v;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(1.0 + m / 8.0, e - 7);
  return sign ? -v : v;
}

/* bfloat16 is the upper half of an IEEE binary32. */
double orc_bf16_value(uint16_t code) {
  uint32_t bits = (uint32_t)code << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* ------------------------------------------------------------ metadata */

/* Per-layer management metadata (P1, in-graph cache management): one int32
 * host->GPU entry per host token, and per GPU slot a free byte, an int32
 * priority, an int32 index-buffer entry and an int32 GPU->host entry.     */
int64_t orc_meta_bytes(int64_t n_host, int64_t n_gpu) {
  int64_t per_host = 4;              /* h2g */
  int64_t per_slot = 1 + 4 + 4 + 4;  /* free, prio, idxbuf, g2h */
  return per_host * n_host + per_slot * n_gpu;
}

/* --------------------------------------------------------------- scores */

/* One request: score[s] = sum_j w[j] * max(0, sum_d q[j][d] * K[s][d]),
 * fp64 throughout, one rounding to fp32 at the end (R1, R2).
 * q: bf16 codes [H][D]; w: fp32 [H]; krows: e4m3 codes [ctx][D].           */
void orc_scores(int H, int D, const uint16_t *q, const float *w,
                const uint8_t *krows, int64_t ctx, float *out) {
  double *qd = (double *)malloc(sizeof(double) * (size_t)H * D);
  double kval[256];
  for (int c = 0; c < 256; ++c) kval[c] = orc_e4m3_value((uint8_t)c);
  for (int64_t i = 0; i < (int64_t)H * D; ++i) qd[i] = orc_bf16_value(q[i]);
#pragma omp parallel for schedule(static)
  for (int64_t s = 0; s < ctx; ++s) {
    const uint8_t *k = krows + s * D;
    double r = 0.0;
    for (int j = 0; j < H; ++j) {
      double x = 0.0;
      for (int d = 0; d < D; ++d) x += qd[(int64_t)j * D + d] * kval[k[d]];
      double relu = x > 0.0 ? x : 0.0;
      r += (double)w[j] * relu;
    }
    float f = (float)r;
    if (f == 0.0f) f = 0.0f; /* -0 -> +0 */
    out[s] = f;
  }
  free(qd);
}

/* ---------------------------------------------------------------- top-k */

static const float *g_sort_scores; /* comparator context (single-threaded use) */

static int cmp_score_desc_idx_asc(const void *a, const void *b) {
  int32_t ia = *(const int32_t *)a, ib = *(const int32_t *)b;
  float sa = g_sort_scores[ia], sb = g_sort_scores[ib];
  if (sa > sb) return -1;
  if (sa < sb) return 1;
  return (ia > ib) - (ia < ib);
}

static int cmp_int_asc(const void *a, const void *b) {
  int32_t ia = *(const int32_t *)a, ib = *(const int32_t *)b;
  return (ia > ib) - (ia < ib);
}

/* R3: the min(k, n) tokens that come first under (score desc, index asc),
 * written in ascending index order.  Returns how many were written; if
 * kth_out is not NULL it receives the score of the last one in the
 * (score desc, index asc) order, i.e. the k-th highest score.              */
int orc_topk(const float *scores, int64_t n, int k, int32_t *sel, float *kth_out) {
  int32_t *order = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
  for (int64_t i = 0; i < n; ++i) order[i] = (int32_t)i;
  g_sort_scores = scores;
  qsort(order, (size_t)n, sizeof(int32_t), cmp_score_desc_idx_asc);
  int m = (int)(n < k ? n : k);
  if (kth_out) *kth_out = m > 0 ? scores[order[m - 1]] : NAN;
  memcpy(sel, order, sizeof(int32_t) * (size_t)m);
  qsort(sel, (size_t)m, sizeof(int32_t), cmp_int_asc);
  free(order);
  return m;
}

/* ------------------------------------------------------------------ EMA */

/* R4: one EMA step in fp32.  theta == +inf means "no estimate yet".        */
float orc_ema_update(float theta, float s_k, float alpha) {
  if (isinf(theta) && theta > 0) return s_k;
  float keep = 1.0f - alpha;
  float a = alpha * s_k;
  float b = keep * theta;
  return a + b;
}

/* ------------------------------------------------------ the layer step */

typedef struct {
  int32_t H, D, k, latent;
  int64_t n_host;
  int32_t n_gpu;
  int32_t cap_div;
  float alpha;
} orc_cfg;

typedef struct {
  int32_t *h2g;   /* [n_host], -1 = not on the GPU            */
  int32_t *g2h;   /* [n_gpu],  -1 = free slot                 */
  int32_t *prio;  /* [n_gpu],  step of last use, -1 = free    */
  uint8_t *freef; /* [n_gpu],  1 = free                       */
  float *theta;   /* [B],      EMA of the k-th score          */
  int32_t t;      /* decode-step counter                      */
  uint16_t *pool; /* [n_gpu][latent] bf16 codes, or NULL      */
} orc_state;

typedef struct {
  float *scores;     /* [B][ctx_stride]                          */
  int32_t *sel_tok;  /* [B][k]   selected tokens, ascending       */
  int32_t *sel_slot; /* [B][k]   their GPU slots after the step   */
  int32_t *n_sel;    /* [B]                                        */
  float *kth;        /* [B]      k-th highest score (NaN if none)  */
  int32_t *pf_tok;   /* [B][k]   prefetched tokens, in rank order  */
  int32_t *pf_slot;  /* [B][k]                                     */
  int32_t *n_pf;     /* [B]                                        */
  int32_t *n_cand;   /* [B]      prefetch candidates (before cap)  */
  int32_t *miss_tok; /* [B][k]   missed tokens, ascending          */
  int32_t *n_miss;   /* [B]                                        */
  int32_t *evicted;  /* [n_gpu]  evicted slots in eviction order   */
  int32_t n_evict;
  int32_t n_free_start; /* free slots at step start               */
  int32_t status;
} orc_out;

static void install(const orc_cfg *c, orc_state *st, int64_t h, int32_t g,
                    const uint16_t *host_kv) {
  st->h2g[h] = g;
  st->g2h[g] = (int32_t)h;
  st->freef[g] = 0;
  st->prio[g] = st->t;
  if (st->pool && host_kv)
    memcpy(st->pool + (int64_t)g * c->latent, host_kv + h * c->latent,
           sizeof(uint16_t) * (size_t)c->latent);
}

static int64_t cap_of(const orc_cfg *c, int64_t ctx) {
  int64_t cap = (ctx + c->cap_div - 1) / c->cap_div;
  return cap < c->k ? cap : c->k;
}

static int cmp_prio_slot(const void *a, const void *b) {
  const int64_t *x = (const int64_t *)a, *y = (const int64_t *)b;
  return (*x > *y) - (*x < *y);
}

/* One decode step of one layer for a batch of B requests.
 * q: bf16 [B][H][D]; w: fp32 [B][H]; kidx: e4m3 [n_host][D];
 * host_kv: bf16 [n_host][latent] (may be NULL when st->pool is NULL);
 * map/ctx: request b's token s < ctx[b] is host id host_id(map, b, s);
 * ext_scores: NULL, or [B][ctx_stride] scores to use instead of computing. */
int orc_layer_step(const orc_cfg *c, orc_state *st, int B,
                   const orc_tokmap *map, const int32_t *ctx,
                   const uint16_t *q, const float *w, const uint8_t *kidx,
                   const uint16_t *host_kv, int mode, const float *ext_scores,
                   int64_t ctx_stride, orc_out *o) {
  const int k = c->k;
  const int32_t t = st->t;
  o->status = ORC_OK;
  o->n_evict = 0;

  /* scores (P1 problem statement; R1, R2) */
  for (int b = 0; b < B; ++b) {
    float *sb = o->scores + (int64_t)b * ctx_stride;
    if (ext_scores) {
      memcpy(sb, ext_scores + (int64_t)b * ctx_stride, sizeof(float) * (size_t)ctx[b]);
    } else if (!map->pages) {
      orc_scores(c->H, c->D, q + (int64_t)b * c->H * c->D, w + (int64_t)b * c->H,
                 kidx + (int64_t)map->host_base[b] * c->D, ctx[b], sb);
    } else { /* the request's key rows, gathered in token order */
      uint8_t *rows = (uint8_t *)malloc((size_t)(ctx[b] > 0 ? ctx[b] : 1) * (size_t)c->D);
      for (int64_t s = 0; s < ctx[b]; ++s)
        memcpy(rows + s * c->D, kidx + host_id(map, b, s) * c->D, (size_t)c->D);
      orc_scores(c->H, c->D, q + (int64_t)b * c->H * c->D, w + (int64_t)b * c->H, rows, ctx[b],
                 sb);
      free(rows);
    }
  }

  /* prefetch during scoring (P1 decode; R5) */
  int32_t *F = (int32_t *)malloc(sizeof(int32_t) * (size_t)(c->n_gpu > 0 ? c->n_gpu : 1));
  int64_t nF = 0;
  for (int32_t g = 0; g < c->n_gpu; ++g)
    if (st->freef[g]) F[nF++] = g;
  o->n_free_start = (int32_t)nF;
  int64_t off = 0, reserve = 0;
  for (int b = 0; b < B; ++b) {
    int64_t cap = cap_of(c, ctx[b]);
    reserve += cap;
    float th = INFINITY;
    int active = 0;
    if (mode == ORC_MODE_EMA) {
      th = st->theta[b];
      active = !(isinf(th) && th > 0);
    } else if (mode == ORC_MODE_NEG_INF) {
      th = -INFINITY;
      active = 1;
    }
    int32_t r = 0, ncand = 0;
    if (active) {
      const float *sb = o->scores + (int64_t)b * ctx_stride;
      for (int64_t s = 0; s < ctx[b]; ++s) {
        int64_t h = host_id(map, b, s);
        if (sb[s] > th && st->h2g[h] == -1) {
          ++ncand;
          if (r < cap && off + r < nF) {
            int32_t g = F[off + r];
            install(c, st, h, g, host_kv);
            o->pf_tok[(int64_t)b * k + r] = (int32_t)s;
            o->pf_slot[(int64_t)b * k + r] = g;
            ++r;
          }
        }
      }
    }
    o->n_pf[b] = r;
    o->n_cand[b] = ncand;
    off += cap;
  }

  /* exact top-k (P1 decode; R3) and EMA (P1 observation 2; R4) */
  for (int b = 0; b < B; ++b) {
    const float *sb = o->scores + (int64_t)b * ctx_stride;
    float kth;
    int m = orc_topk(sb, ctx[b], k, o->sel_tok + (int64_t)b * k, &kth);
    o->n_sel[b] = m;
    o->kth[b] = kth;
    if (mode == ORC_MODE_EMA && ctx[b] >= k)
      st->theta[b] = orc_ema_update(st->theta[b], kth, c->alpha);
  }

  /* protect the selected tokens and list the misses (P1 cache management; R6) */
  int64_t n_miss_all = 0;
  for (int b = 0; b < B; ++b) {
    int32_t nm = 0;
    for (int i = 0; i < o->n_sel[b]; ++i) {
      int32_t s = o->sel_tok[(int64_t)b * k + i];
      int64_t h = host_id(map, b, s);
      int32_t g = st->h2g[h];
      o->sel_slot[(int64_t)b * k + i] = g;
      if (g >= 0)
        st->prio[g] = t;
      else
        o->miss_tok[(int64_t)b * k + nm++] = s;
    }
    o->n_miss[b] = nm;
    n_miss_all += nm;
  }

  /* evict (P1 cache management; R7): no bytes move */
  int64_t n_free = 0, nE = 0;
  int64_t *E = (int64_t *)malloc(sizeof(int64_t) * (size_t)(c->n_gpu > 0 ? c->n_gpu : 1));
  for (int32_t g = 0; g < c->n_gpu; ++g) {
    if (st->freef[g])
      ++n_free;
    else if (st->prio[g] < t)
      E[nE++] = ((int64_t)st->prio[g] << 32) | (int64_t)g; /* prio >= 0 here */
  }
  if (n_free + nE < n_miss_all) {
    o->status = ORC_ECAPACITY;
    free(E);
    free(F);
    return o->status;
  }
  qsort(E, (size_t)nE, sizeof(int64_t), cmp_prio_slot);
  int64_t want = n_miss_all + reserve - n_free;
  if (want < 0) want = 0;
  int64_t n_evict = want < nE ? want : nE;
  for (int64_t i = 0; i < n_evict; ++i) {
    int32_t g = (int32_t)(E[i] & 0xFFFFFFFF);
    st->h2g[st->g2h[g]] = -1;
    st->g2h[g] = -1;
    st->freef[g] = 1;
    st->prio[g] = -1;
    o->evicted[i] = g;
  }
  o->n_evict = (int32_t)n_evict;

  /* allocate and recall (P1 cache management; R8) */
  nF = 0;
  for (int32_t g = 0; g < c->n_gpu; ++g)
    if (st->freef[g]) F[nF++] = g;
  int64_t i = 0;
  for (int b = 0; b < B; ++b) {
    for (int j = 0; j < o->n_miss[b]; ++j, ++i) {
      int32_t s = o->miss_tok[(int64_t)b * k + j];
      int64_t h = host_id(map, b, s);
      install(c, st, h, F[i], host_kv);
    }
    for (int j = 0; j < o->n_sel[b]; ++j) {
      int64_t h = host_id(map, b, o->sel_tok[(int64_t)b * k + j]);
      o->sel_slot[(int64_t)b * k + j] = st->h2g[h];
    }
  }
  st->t = t + 1; /* R9 */
  free(E);
  free(F);
  return ORC_OK;
}

/* Decode append and writeback, [P1] "Core method / in-graph per-layer cache
 * management" (the KV of every token is backed up to the host pool when it is
 * generated, and the indexer K stays on the GPU) and "Design trade-offs" (every
 * new token is written back).  Reading R10: for request b the new token takes
 * host id h = host_id(map, b, ctx[b]); key row kidx[h] = k_new[b] (D bytes) and
 * latent host_kv[h] = lat_new[b] (`latent` values); with `advance`, ctx[b] grows
 * by one.  The requests are checked first, in order: no room (ctx[b] = max_ctx,
 * the id outside the pool -- past n_host, or with a page table the new token's
 * page slot past page_stride or its page outside the pool -- or, without a page
 * table, h inside
 * another request's range [host_base[o], host_base[o] + ctx[o]] counting that
 * request's own new token) gives ORC_ECAPACITY, a host id some slot already maps
 * (h2g[h] != -1) gives ORC_EDEVARG; the first such request decides and nothing
 * is written.  With a page table the page is the caller's choice (R14).
 * A batch row with ctx[b] = 0 is empty (never admitted, or released): it takes
 * no token, is not checked, does not grow, and its stale host_base occupies no
 * range in the other requests' checks. */
int orc_append(int B, int D, int latent, int64_t n_host, int32_t max_ctx,
               const orc_tokmap *map, int32_t *ctx, const int32_t *h2g,
               const uint8_t *k_new, const uint16_t *lat_new, uint8_t *kidx,
               uint16_t *host_kv, int advance) {
  for (int b = 0; b < B; ++b) {
    if (ctx[b] == 0) continue; /* an empty row */
    if (ctx[b] < 0 || ctx[b] >= max_ctx) return ORC_ECAPACITY;
    if (map->pages) { /* the page listed for the new token: in the table, in the pool */
      const int64_t j = ctx[b] / 16;
      if (j >= map->page_stride) return ORC_ECAPACITY;
      const int32_t p = map->pages[(int64_t)b * map->page_stride + j];
      if (p < 0 || 16 * (int64_t)p + 16 > n_host) return ORC_ECAPACITY;
    } else if (!tokens_fit(map, b, (int64_t)ctx[b] + 1, n_host)) {
      return ORC_ECAPACITY;
    }
    const int64_t h = host_id(map, b, ctx[b]);
    if (!map->pages) {
      const int32_t *hb = map->host_base;
      for (int o = 0; o < B; ++o) {
        if (o == b || ctx[o] == 0) continue;
        if (h >= hb[o] && h < (int64_t)hb[o] + ctx[o] + 1) return ORC_ECAPACITY;
      }
    }
    if (h2g[h] != -1) return ORC_EDEVARG;
  }
  for (int b = 0; b < B; ++b) {
    if (ctx[b] == 0) continue;
    const int64_t h = host_id(map, b, ctx[b]);
    memcpy(kidx + h * D, k_new + (int64_t)b * D, (size_t)D);
    if (host_kv)
      memcpy(host_kv + h * latent, lat_new + (int64_t)b * latent, (size_t)latent * 2);
  }
  if (advance)
    for (int b = 0; b < B; ++b)
      if (ctx[b] != 0) ctx[b] += 1;
  return ORC_OK;
}

/* Attention input without offloading, [P1] "Core method / decode" (after the
 * exact top-k every selected token's KV must be present before the sparse
 * attention runs; "lossless" means the attention sees exactly these rows) and
 * [P2] (prediction only decides when data moves, never which data is read).
 * Reading R11: out[b][i] = host_kv[host_id(map, b, sel_tok[b][i])] (`latent`
 * values) for i < n_sel[b], zero for n_sel[b] <= i < k.  sel_tok is [B][k]. */
void orc_gather(int B, int k, int latent, const orc_tokmap *map, const int32_t *sel_tok,
                const int32_t *n_sel, const uint16_t *host_kv, uint16_t *out) {
  for (int b = 0; b < B; ++b) {
    for (int i = 0; i < k; ++i) {
      uint16_t *o = out + ((int64_t)b * k + i) * latent;
      if (i < n_sel[b]) {
        const int64_t h = host_id(map, b, sel_tok[(int64_t)b * k + i]);
        memcpy(o, host_kv + h * latent, (size_t)latent * 2);
      } else {
        memset(o, 0, (size_t)latent * 2);
      }
    }
  }
}

/* Request cancellation, [P1] "Systemic flaws" (the paper leaves request
 * cancellation open) and "Limitations and future work" (final top-k and
 * attention input must stay equal to the no-offload baseline under request
 * cancellation), with the state of "Core method / in-graph per-layer cache
 * management".  Reading R12: for every request b with mask[b] != 0, each host
 * id h = host_id(map, b, s), s < ctx[b], that maps a slot g gives it
 * back (g2h[g] = -1, free[g] = 1, prio[g] = -1) and h2g[h] becomes -1; then
 * theta[b] = +inf, and with `commit` ctx[b] = 0 (the batch row is shared by all
 * layers: it is emptied with the last one).  A masked request whose tokens do not
 * fit (ctx < 0, ctx > max_ctx, an id outside the pool: host_base < 0 or past
 * n_host, or a page outside the pool or past page_stride) gives ORC_EDEVARG,
 * checked for all masked requests before anything changes.  The host pages stay
 * the caller's (R14). */
int orc_release(int B, int64_t n_host, int32_t max_ctx, const orc_tokmap *map, int32_t *ctx,
                const int32_t *mask, int32_t *h2g, int32_t *g2h, int32_t *prio, uint8_t *freef,
                float *theta, int commit) {
  for (int b = 0; b < B; ++b) {
    if (!mask[b]) continue;
    if (ctx[b] < 0 || ctx[b] > max_ctx || !tokens_fit(map, b, ctx[b], n_host))
      return ORC_EDEVARG;
  }
  for (int b = 0; b < B; ++b) {
    if (!mask[b]) continue;
    for (int32_t s = 0; s < ctx[b]; ++s) {
      const int64_t h = host_id(map, b, s);
      const int32_t g = h2g[h];
      if (g >= 0) {
        g2h[g] = -1;
        freef[g] = 1;
        prio[g] = -1;
      }
      h2g[h] = -1;
    }
    theta[b] = INFINITY;
    if (commit) ctx[b] = 0;
  }
  return ORC_OK;
}

/* Request admission, the other half of R12.  Request b (an empty batch row)
 * takes len tokens.  Without a page table they are the host range
 * [base, base + len); with one (R14) they are the first len ids of the pages the
 * caller listed in row b of the table, and base is not used.  Checks, in order:
 * b outside [0, B), len outside [0, max_ctx], or (without a page table) base < 0
 * or base + len > n_host give ORC_EINVAL; a row still in use (ctx[b] != 0) gives
 * ORC_EDEVARG; with a page table, more pages than page_stride, a page outside
 * the pool or a page listed twice gives ORC_EDEVARG; a range meeting the range of
 * another request o with ctx[o] > 0 (with a page table: a page that one of o's
 * tokens uses) gives ORC_ECAPACITY; a host id of the new tokens that some slot
 * still maps gives ORC_EDEVARG.  Nothing changes on an error.  Otherwise
 * theta[b] = +inf, and with `commit` (the last layer) ctx[b] = len and, without a
 * page table, host_base[b] = base. */
int orc_admit(int B, int64_t n_host, int32_t max_ctx, const orc_tokmap *map, int32_t *ctx,
              const int32_t *h2g, float *theta, int b, int32_t base, int32_t len, int commit) {
  if (b < 0 || b >= B || len < 0 || len > max_ctx) return ORC_EINVAL;
  if (!map->pages && (base < 0 || (int64_t)base + len > n_host)) return ORC_EINVAL;
  if (ctx[b] != 0) return ORC_EDEVARG;
  const int64_t np = ((int64_t)len + 15) / 16;
  if (map->pages) {
    if (np > map->page_stride) return ORC_EDEVARG;
    const int32_t *row = map->pages + (int64_t)b * map->page_stride;
    for (int64_t j = 0; j < np; ++j) {
      if (row[j] < 0 || 16 * (int64_t)row[j] + 16 > n_host) return ORC_EDEVARG;
      for (int64_t i = 0; i < j; ++i)
        if (row[i] == row[j]) return ORC_EDEVARG;
    }
    for (int o = 0; o < B; ++o) {
      if (o == b || ctx[o] <= 0) continue;
      const int32_t *ro = map->pages + (int64_t)o * map->page_stride;
      for (int64_t i = 0; i < ((int64_t)ctx[o] + 15) / 16; ++i)
        for (int64_t j = 0; j < np; ++j)
          if (ro[i] == row[j]) return ORC_ECAPACITY;
    }
    for (int32_t s = 0; s < len; ++s)
      if (h2g[16 * (int64_t)row[s / 16] + s % 16] != -1) return ORC_EDEVARG;
  } else {
    for (int o = 0; o < B; ++o) {
      if (o == b || ctx[o] <= 0) continue;
      const int64_t lo = map->host_base[o], hi = (int64_t)map->host_base[o] + ctx[o];
      if ((int64_t)base < hi && lo < (int64_t)base + len) return ORC_ECAPACITY;
    }
    for (int32_t s = 0; s < len; ++s)
      if (h2g[(int64_t)base + s] != -1) return ORC_EDEVARG;
  }
  theta[b] = INFINITY;
  if (commit) {
    if (!map->pages) map->host_base[b] = base;
    ctx[b] = len;
  }
  return ORC_OK;
}

/* ------------------------------------------------------ chunked prefill */

/* IEEE binary16 bits of an fp32 value, round to nearest, ties to even
 * (magnitudes from 65520 up become infinity).  Written from the format: a
 * normal half has 10 fraction bits, exponent bias 15; a subnormal is m*2^-24.
 * NaN gives 0x7E00. */
uint16_t orc_f16_bits(float x) {
  const uint16_t sign = signbit(x) ? 0x8000 : 0;
  double a = fabs((double)x);
  if (isnan(x)) return 0x7E00;
  if (a >= 65536.0) return sign | 0x7C00;
  int e;
  frexp(a, &e); /* a = f * 2^e, f in [0.5, 1): the leading bit is 2^(e-1) */
  e -= 1;
  if (a == 0.0) return sign;
  double quantum = e < -14 ? ldexp(1.0, -24) : ldexp(1.0, e - 10);
  double m = nearbyint(a / quantum); /* exact quotient, ties to even */
  if (e < -14) return sign | (uint16_t)m; /* m = 1024 is the smallest normal */
  return sign | (uint16_t)(((e + 15) << 10) + (int)m - 1024);
}

/* The 256 coarse buckets: the top byte of an order key of the half bits
 * (larger value, larger key; -0 counts as +0). */
int orc_f16_bucket(uint16_t u) {
  if (u == 0x8000) u = 0;
  const uint16_t key = (u & 0x8000) ? (uint16_t)~u : (uint16_t)(u | 0x8000);
  return key >> 8;
}

/* Coarse bucket of a score, shifted by the predicted k-th score: the
 * difference is taken in fp32, then rounded to half precision. */
static int coarse_bucket(float score, float pred) {
  const float d = score - pred;
  return orc_f16_bucket(orc_f16_bits(d));
}

typedef struct {
  float *scores;     /* [C][N]                                         */
  int32_t *sel;      /* [C][k]  each query's top-k, ascending           */
  int32_t *n_sel;    /* [C]                                             */
  float *kth;        /* [C]     k-th highest score                      */
  int32_t *beta;     /* [C]     boundary bucket, -1 if N <= k           */
  int32_t *n_qcand;  /* [C]     coarse candidates of each query         */
  int32_t *cand;     /* [N]     union of the candidates, ascending      */
  int32_t *uni;      /* [N]     union of the selections, ascending      */
  int32_t *pf_h;     /* [N]     candidate installs: host id, slot       */
  int32_t *pf_g;
  int32_t *miss_h;   /* [N]     remaining installs: host id, slot       */
  int32_t *miss_g;
  int32_t n_cand, n_uni, n_pf, n_miss;
} orc_prefill_out;

/* One prefill chunk, [P1] "Core method / prefill" (query chunks; chunk i's
 * identified candidates move while chunk i+1 is scored; a 256-bucket coarse
 * histogram keeps the strictly-high buckets and leaves the threshold bucket
 * for later; subtracting the predicted k-th score refines the buckets near
 * the boundary; the exact fetch afterwards covers what was missed) and
 * "Core method / prefetch inside the indexer pipeline" (prefill splits the
 * indexer's work by query chunk).  Reading R13.
 * q: bf16 [C][H][D]; w: fp32 [C][H]; kidx: e4m3 [n_host][D]; the history is
 * host ids hb .. hb+N-1; pred: [C] or NULL; ext_scores: [C][N] or NULL.
 * Returns ORC_OK or ORC_ECAPACITY (outputs up to the unions still set; after
 * a capacity error in the second stage the first stage's installs stand). */
int orc_prefill_chunk(const orc_cfg *c, orc_state *st, int C, int32_t hb, int64_t N,
                      const uint16_t *q, const float *w, const uint8_t *kidx, const float *pred,
                      const uint16_t *host_kv, const float *ext_scores, orc_prefill_out *o) {
  const int k = c->k;
  /* scores, one query at a time */
  for (int i = 0; i < C; ++i) {
    float *row = o->scores + (int64_t)i * N;
    if (ext_scores)
      memcpy(row, ext_scores + (int64_t)i * N, sizeof(float) * (size_t)N);
    else
      orc_scores(c->H, c->D, q + (int64_t)i * c->H * c->D, w + (int64_t)i * c->H,
                 kidx + (int64_t)hb * c->D, N, row);
  }
  uint8_t *cflag = (uint8_t *)calloc((size_t)(N > 0 ? N : 1), 1);
  uint8_t *uflag = (uint8_t *)calloc((size_t)(N > 0 ? N : 1), 1);
  for (int i = 0; i < C; ++i) {
    const float *row = o->scores + (int64_t)i * N;
    /* coarse candidates */
    int32_t nq = 0;
    if (N <= k) {
      o->beta[i] = -1;
      for (int64_t s = 0; s < N; ++s) cflag[s] = 1;
      nq = (int32_t)N;
    } else {
      const float p = pred ? pred[i] : 0.0f;
      int64_t hist[256] = {0};
      for (int64_t s = 0; s < N; ++s) hist[coarse_bucket(row[s], p)] += 1;
      int beta = 255;
      int64_t above = 0; /* tokens in buckets higher than beta */
      while (above + hist[beta] < k) above += hist[beta--];
      o->beta[i] = beta;
      for (int64_t s = 0; s < N; ++s)
        if (coarse_bucket(row[s], p) > beta) {
          cflag[s] = 1;
          ++nq;
        }
    }
    o->n_qcand[i] = nq;
    /* exact top-k */
    int32_t *sel = o->sel + (int64_t)i * k;
    o->n_sel[i] = orc_topk(row, N, k, sel, &o->kth[i]);
    for (int j = 0; j < o->n_sel[i]; ++j) uflag[sel[j]] = 1;
  }
  o->n_cand = o->n_uni = 0;
  for (int64_t s = 0; s < N; ++s) {
    if (cflag[s]) o->cand[o->n_cand++] = (int32_t)s;
    if (uflag[s]) o->uni[o->n_uni++] = (int32_t)s;
  }
  free(cflag);
  free(uflag);
  o->n_pf = o->n_miss = 0;
  int32_t *F = (int32_t *)malloc(sizeof(int32_t) * (size_t)(c->n_gpu > 0 ? c->n_gpu : 1));
  int32_t nF = 0;
  for (int32_t g = 0; g < c->n_gpu; ++g)
    if (st->freef[g]) F[nF++] = g;
  const int32_t t = st->t;
  int32_t next = 0;
  int64_t need = 0; /* each stage checks its own set against the free slots left */
  for (int32_t j = 0; j < o->n_cand; ++j)
    if (st->h2g[(int64_t)hb + o->cand[j]] == -1) ++need;
  if (need > nF) {
    free(F);
    return ORC_ECAPACITY;
  }
  for (int32_t j = 0; j < o->n_cand; ++j) { /* the early transfer */
    const int64_t h = (int64_t)hb + o->cand[j];
    if (st->h2g[h] >= 0) {
      st->prio[st->h2g[h]] = t;
    } else {
      const int32_t g = F[next++];
      install(c, st, h, g, host_kv);
      o->pf_h[o->n_pf] = (int32_t)h;
      o->pf_g[o->n_pf++] = g;
    }
  }
  need = 0;
  for (int32_t j = 0; j < o->n_uni; ++j)
    if (st->h2g[(int64_t)hb + o->uni[j]] == -1) ++need;
  if (need > nF - next) {
    free(F);
    return ORC_ECAPACITY;
  }
  for (int32_t j = 0; j < o->n_uni; ++j) { /* the exact fetch */
    const int64_t h = (int64_t)hb + o->uni[j];
    if (st->h2g[h] >= 0) {
      st->prio[st->h2g[h]] = t;
    } else {
      const int32_t g = F[next++];
      install(c, st, h, g, host_kv);
      o->miss_h[o->n_miss] = (int32_t)h;
      o->miss_g[o->n_miss++] = g;
    }
  }
  free(F);
  st->t = t + 1;
  return ORC_OK;
}
