/*
 * A walk over every entry point of the CPU oracle, built with AddressSanitizer
 * and UndefinedBehaviorSanitizer (tests/test_oracle_sanitize.py compiles and
 * runs it on the host).  It includes the oracle's source, so the whole oracle is
 * instrumented; the inputs are seeded and small: contiguous and paged requests,
 * an empty batch row, decode steps in all three threshold modes under eviction
 * pressure, appends, the attention-input gather, release and admission into the
 * released row, prefill chunks with and without predicted k-th scores, and the
 * degenerate sizes (no request, a context shorter than k, an empty history).
 * Every call must return a status the oracle documents; the sanitizers abort on
 * any out-of-bounds access, use after free, leak or undefined operation.
 */
#include "../oracle/echo_oracle.c"

#include <stdio.h>

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void) { /* xorshift64* */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}
static float rnd_unit(void) { return (float)(rnd() >> 8) / 16777216.0f * 2.0f - 1.0f; }
static uint16_t rnd_bf16(void) {
  const float f = rnd_unit();
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(u >> 16);
}
static uint8_t rnd_e4m3(void) { /* any finite code */
  uint8_t c;
  do c = (uint8_t)rnd(); while ((c & 0x7F) == 0x7F);
  return c;
}

/* what the walk reached: steps that ended cleanly, evictions, prefetches, misses */
static long n_ok, n_evicted, n_prefetched, n_missed;

#define CHECK(cond, what)                                       \
  do {                                                          \
    if (!(cond)) {                                              \
      fprintf(stderr, "FAILED: %s (line %d)\n", what, __LINE__); \
      exit(1);                                                  \
    }                                                           \
  } while (0)

typedef struct {
  orc_cfg c;
  orc_state st;
  int32_t max_ctx;
  int B;
  uint8_t *kidx;
  uint16_t *host_kv;
} rig;

static void rig_init(rig *r, int B, int64_t n_host, int32_t n_gpu, int32_t max_ctx) {
  r->c.H = 8;
  r->c.D = 32;
  r->c.k = 16;
  r->c.latent = 8;
  r->c.n_host = n_host;
  r->c.n_gpu = n_gpu;
  r->c.cap_div = 8;
  r->c.alpha = 0.5f;
  r->B = B;
  r->max_ctx = max_ctx;
  r->st.h2g = (int32_t *)malloc(sizeof(int32_t) * (size_t)n_host);
  r->st.g2h = (int32_t *)malloc(sizeof(int32_t) * (size_t)n_gpu);
  r->st.prio = (int32_t *)malloc(sizeof(int32_t) * (size_t)n_gpu);
  r->st.freef = (uint8_t *)malloc((size_t)n_gpu);
  r->st.theta = (float *)malloc(sizeof(float) * (size_t)(B > 0 ? B : 1));
  r->st.pool = (uint16_t *)calloc((size_t)n_gpu * r->c.latent, sizeof(uint16_t));
  r->st.t = 0;
  for (int64_t h = 0; h < n_host; ++h) r->st.h2g[h] = -1;
  for (int32_t g = 0; g < n_gpu; ++g) {
    r->st.g2h[g] = -1;
    r->st.prio[g] = -1;
    r->st.freef[g] = 1;
  }
  for (int b = 0; b < B; ++b) r->st.theta[b] = INFINITY;
  r->kidx = (uint8_t *)malloc((size_t)n_host * r->c.D);
  r->host_kv = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)n_host * r->c.latent);
  for (int64_t i = 0; i < n_host * r->c.D; ++i) r->kidx[i] = rnd_e4m3();
  for (int64_t i = 0; i < n_host * r->c.latent; ++i) r->host_kv[i] = rnd_bf16();
}

static void rig_free(rig *r) {
  free(r->st.h2g);
  free(r->st.g2h);
  free(r->st.prio);
  free(r->st.freef);
  free(r->st.theta);
  free(r->st.pool);
  free(r->kidx);
  free(r->host_kv);
}

/* one decode step with fresh queries; returns the status */
static int rig_step(rig *r, const orc_tokmap *map, const int32_t *ctx, int mode) {
  const int B = r->B, H = r->c.H, D = r->c.D, k = r->c.k;
  const int64_t stride = r->max_ctx > 0 ? r->max_ctx : 1;
  const int Bn = B > 0 ? B : 1;
  uint16_t *q = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)Bn * H * D);
  float *w = (float *)malloc(sizeof(float) * (size_t)Bn * H);
  for (int i = 0; i < B * H * D; ++i) q[i] = rnd_bf16();
  for (int i = 0; i < B * H; ++i) w[i] = rnd_unit();
  orc_out o;
  o.scores = (float *)calloc((size_t)(Bn * stride), sizeof(float));
  o.sel_tok = (int32_t *)calloc((size_t)Bn * k, sizeof(int32_t));
  o.sel_slot = (int32_t *)calloc((size_t)Bn * k, sizeof(int32_t));
  o.n_sel = (int32_t *)calloc((size_t)Bn, sizeof(int32_t));
  o.kth = (float *)calloc((size_t)Bn, sizeof(float));
  o.pf_tok = (int32_t *)calloc((size_t)Bn * k, sizeof(int32_t));
  o.pf_slot = (int32_t *)calloc((size_t)Bn * k, sizeof(int32_t));
  o.n_pf = (int32_t *)calloc((size_t)Bn, sizeof(int32_t));
  o.n_cand = (int32_t *)calloc((size_t)Bn, sizeof(int32_t));
  o.miss_tok = (int32_t *)calloc((size_t)Bn * k, sizeof(int32_t));
  o.n_miss = (int32_t *)calloc((size_t)Bn, sizeof(int32_t));
  o.evicted = (int32_t *)calloc((size_t)r->c.n_gpu, sizeof(int32_t));
  const int rc = orc_layer_step(&r->c, &r->st, B, map, ctx, q, w, r->kidx, r->host_kv, mode,
                                NULL, stride, &o);
  CHECK(rc == ORC_OK || rc == ORC_ECAPACITY || rc == ORC_EDEVARG, "layer step status");
  CHECK(rc == o.status, "layer step status echoed");
  if (rc == ORC_OK) {
    ++n_ok;
    n_evicted += o.n_evict;
  }
  for (int b = 0; b < B && rc == ORC_OK; ++b) {
    n_prefetched += o.n_pf[b];
    n_missed += o.n_miss[b];
    CHECK(o.n_sel[b] >= 0 && o.n_sel[b] <= k, "n_sel in range");
    for (int i = 1; i < o.n_sel[b]; ++i)
      CHECK(o.sel_tok[(int64_t)b * k + i - 1] < o.sel_tok[(int64_t)b * k + i], "ascending");
  }
  /* the attention input of the selection */
  uint16_t *att = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)Bn * k * r->c.latent);
  orc_gather(B, k, r->c.latent, map, o.sel_tok, o.n_sel, r->host_kv, att);
  free(att);
  free(q);
  free(w);
  free(o.scores);
  free(o.sel_tok);
  free(o.sel_slot);
  free(o.n_sel);
  free(o.kth);
  free(o.pf_tok);
  free(o.pf_slot);
  free(o.n_pf);
  free(o.n_cand);
  free(o.miss_tok);
  free(o.n_miss);
  free(o.evicted);
  return rc;
}

static int rig_append(rig *r, const orc_tokmap *map, int32_t *ctx) {
  const int B = r->B, Bn = B > 0 ? B : 1;
  uint8_t *kn = (uint8_t *)malloc((size_t)Bn * r->c.D);
  uint16_t *ln = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)Bn * r->c.latent);
  for (int i = 0; i < B * r->c.D; ++i) kn[i] = rnd_e4m3();
  for (int i = 0; i < B * r->c.latent; ++i) ln[i] = rnd_bf16();
  const int rc = orc_append(B, r->c.D, r->c.latent, r->c.n_host, r->max_ctx, map, ctx,
                            r->st.h2g, kn, ln, r->kidx, r->host_kv, 1);
  CHECK(rc == ORC_OK || rc == ORC_ECAPACITY || rc == ORC_EDEVARG, "append status");
  free(kn);
  free(ln);
  return rc;
}

static void decode_walk(int paged) {
  const int B = 3;
  rig r;
  rig_init(&r, B, 1024, 96, 200);
  int32_t base[3] = {0, 256, 512};
  int32_t ctx[3] = {100, 37, 0}; /* the last row is empty */
  const int stride = 14;         /* pages per request (200 tokens fit 13) */
  int32_t *pages = NULL;
  orc_tokmap map = {base, NULL, 0};
  if (paged) {
    /* pages of the 64-page pool in a scrambled order, each listed once */
    pages = (int32_t *)malloc(sizeof(int32_t) * B * stride);
    int32_t perm[64];
    for (int i = 0; i < 64; ++i) perm[i] = i;
    for (int i = 63; i > 0; --i) {
      const int j = (int)(rnd() % (uint32_t)(i + 1));
      const int32_t x = perm[i];
      perm[i] = perm[j];
      perm[j] = x;
    }
    for (int i = 0; i < B * stride; ++i) pages[i] = perm[i];
    map.host_base = NULL;
    map.pages = pages;
    map.page_stride = stride;
  }
  const int modes[3] = {ORC_MODE_EMA, ORC_MODE_NEG_INF, ORC_MODE_POS_INF};
  for (int s = 0; s < 9; ++s) {
    rig_step(&r, &map, ctx, modes[s % 3]);
    rig_append(&r, &map, ctx);
  }
  /* release request 1, append around the empty row, admit a new request there */
  int32_t mask[3] = {0, 1, 0};
  int rc = orc_release(B, r.c.n_host, r.max_ctx, &map, ctx, mask, r.st.h2g, r.st.g2h, r.st.prio,
                       r.st.freef, r.st.theta, 1);
  CHECK(rc == ORC_OK && ctx[1] == 0, "release");
  rig_step(&r, &map, ctx, ORC_MODE_EMA);
  rig_append(&r, &map, ctx);
  if (paged) {
    /* the released pages of row 1 go to the new request, which admits 20 tokens */
    rc = orc_admit(B, r.c.n_host, r.max_ctx, &map, ctx, r.st.h2g, r.st.theta, 1, 0, 20, 1);
  } else {
    rc = orc_admit(B, r.c.n_host, r.max_ctx, &map, ctx, r.st.h2g, r.st.theta, 1, 768, 20, 1);
  }
  CHECK(rc == ORC_OK && ctx[1] == 20, "admit");
  /* a request whose tokens collide with a live one is refused and changes nothing */
  if (!paged) {
    rc = orc_admit(B, r.c.n_host, r.max_ctx, &map, ctx, r.st.h2g, r.st.theta, 2, 0, 16, 1);
    CHECK(rc == ORC_ECAPACITY && ctx[2] == 0, "overlapping admission refused");
  }
  for (int s = 0; s < 4; ++s) {
    rig_step(&r, &map, ctx, modes[s % 3]);
    rig_append(&r, &map, ctx);
  }
  /* a pool too small for one request's selection: the capacity error */
  rig small;
  rig_init(&small, 2, 256, 8, 64);
  int32_t sb[2] = {0, 64}, sc[2] = {60, 50};
  orc_tokmap sm = {sb, NULL, 0};
  CHECK(rig_step(&small, &sm, sc, ORC_MODE_EMA) == ORC_ECAPACITY, "capacity error");
  rig_free(&small);
  /* no request at all */
  rig none;
  rig_init(&none, 0, 64, 8, 1);
  orc_tokmap nm = {NULL, NULL, 0};
  CHECK(rig_step(&none, &nm, NULL, ORC_MODE_EMA) == ORC_OK, "empty batch");
  rig_free(&none);
  rig_free(&r);
  free(pages);
}

static void prefill_walk(void) {
  rig r;
  rig_init(&r, 1, 1024, 400, 300);
  const int C = 4, H = r.c.H, D = r.c.D, k = r.c.k;
  const int64_t Ns[3] = {300, 12, 0}; /* above k, below k, an empty history */
  for (int v = 0; v < 3; ++v) {
    const int64_t N = Ns[v];
    const int64_t Nn = N > 0 ? N : 1;
    uint16_t *q = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)C * H * D);
    float *w = (float *)malloc(sizeof(float) * (size_t)C * H);
    float pred[4];
    for (int i = 0; i < C * H * D; ++i) q[i] = rnd_bf16();
    for (int i = 0; i < C * H; ++i) w[i] = rnd_unit();
    for (int i = 0; i < C; ++i) pred[i] = rnd_unit();
    orc_prefill_out o;
    o.scores = (float *)calloc((size_t)(C * Nn), sizeof(float));
    o.sel = (int32_t *)calloc((size_t)C * k, sizeof(int32_t));
    o.n_sel = (int32_t *)calloc((size_t)C, sizeof(int32_t));
    o.kth = (float *)calloc((size_t)C, sizeof(float));
    o.beta = (int32_t *)calloc((size_t)C, sizeof(int32_t));
    o.n_qcand = (int32_t *)calloc((size_t)C, sizeof(int32_t));
    o.cand = (int32_t *)calloc((size_t)Nn, sizeof(int32_t));
    o.uni = (int32_t *)calloc((size_t)Nn, sizeof(int32_t));
    o.pf_h = (int32_t *)calloc((size_t)Nn, sizeof(int32_t));
    o.pf_g = (int32_t *)calloc((size_t)Nn, sizeof(int32_t));
    o.miss_h = (int32_t *)calloc((size_t)Nn, sizeof(int32_t));
    o.miss_g = (int32_t *)calloc((size_t)Nn, sizeof(int32_t));
    for (int withpred = 0; withpred < 2; ++withpred) {
      const int rc = orc_prefill_chunk(&r.c, &r.st, C, 64, N, q, w, r.kidx,
                                       withpred ? pred : NULL, r.host_kv, NULL, &o);
      CHECK(rc == ORC_OK || rc == ORC_ECAPACITY, "prefill status");
      CHECK(o.n_uni >= 0 && o.n_uni <= N && o.n_cand >= 0 && o.n_cand <= N, "prefill sizes");
    }
    free(q);
    free(w);
    free(o.scores);
    free(o.sel);
    free(o.n_sel);
    free(o.kth);
    free(o.beta);
    free(o.n_qcand);
    free(o.cand);
    free(o.uni);
    free(o.pf_h);
    free(o.pf_g);
    free(o.miss_h);
    free(o.miss_g);
  }
  rig_free(&r);
}

static void small_calls(void) {
  /* top-k with ties, with k above the length, and on nothing */
  float s[10] = {1, 3, 3, 2, 3, -1, 0, 3, 2, 1};
  int32_t sel[16];
  float kth;
  CHECK(orc_topk(s, 10, 4, sel, &kth) == 4 && kth == 3.0f, "top-k with ties");
  CHECK(orc_topk(s, 10, 16, sel, &kth) == 10, "k above the length");
  CHECK(orc_topk(s, 0, 4, sel, &kth) == 0, "empty top-k");
  /* the threshold update, from "no estimate" and from a value */
  CHECK(orc_ema_update(INFINITY, 2.0f, 0.5f) == 2.0f, "EMA seed");
  CHECK(orc_ema_update(2.0f, 4.0f, 0.5f) == 3.0f, "EMA step");
  /* every half-precision rounding path, and both decoders on every code */
  for (int i = 0; i < 4096; ++i) {
    const float x = ldexpf(rnd_unit(), (int)(rnd() % 48) - 30);
    CHECK(orc_f16_bucket(orc_f16_bits(x)) >= 0, "f16 bucket");
  }
  CHECK(orc_f16_bits(NAN) == 0x7E00 && orc_f16_bits(1e9f) == 0x7C00, "f16 specials");
  double acc = 0.0;
  for (int c = 0; c < 256; ++c) {
    const double v = orc_e4m3_value((uint8_t)c);
    if (!isnan(v)) acc += v;
  }
  for (int c = 0; c < 65536; c += 7) {
    const double v = orc_bf16_value((uint16_t)c);
    if (isfinite(v)) acc += v * 0.0;
  }
  CHECK(acc == 0.0, "the e4m3 codes sum to zero (symmetric)");
  CHECK(orc_meta_bytes(1000, 100) == 4 * 1000 + 13 * 100, "metadata bytes");
}

int main(void) {
  orc_set_threads(2);
  small_calls();
  decode_walk(0);
  decode_walk(1);
  prefill_walk();
  printf("oracle sanitizer walk: ok (%ld steps, %ld evicted, %ld prefetched, %ld missed)\n",
         n_ok, n_evicted, n_prefetched, n_missed);
  return 0;
}
