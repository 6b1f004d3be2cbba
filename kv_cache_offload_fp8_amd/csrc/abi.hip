// C ABI entry points (include/echo.h): host-side validation and the launch
// sequence of each call.  No entry point allocates, frees or synchronizes.
#include <math.h>
#include <string.h>

#include <mutex>

#include "kernels.h"
#include "prefill.h"

using namespace echo;

// Scratch of echo_topk_noalloc: a file-scope device array, one copy on every GPU
// the library runs on, held until the process ends.  In host code the name is only
// a stand-in; the device address comes from hipGetSymbolAddress (per device, in
// static_scratch below) and is what kernels and fills receive.
constexpr int64_t kStaticScratchBytes = 32LL << 20;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];


namespace {

int check_dims(const echo_dims_t *d) {
  if (!d) return ECHO_EINVAL;
  if (d->n_heads < 1 || d->head_dim < 1 || d->top_k < 1 || d->latent_dim < 1 || d->n_host < 1 ||
      d->n_gpu < 1 || d->max_batch < 1 || d->max_ctx < 1 || d->prefetch_cap_div < 1 ||
      d->q_ring < 1)
    return ECHO_EINVAL;
  if (!(d->ema_alpha > 0.0f && d->ema_alpha <= 1.0f)) return ECHO_EINVAL;
  if (d->n_host >= (1LL << 31) || d->max_ctx > (1 << 30) || d->n_gpu > (1 << 30))
    return ECHO_EINVAL;
  if (d->n_host % 16 != 0) return ECHO_EINVAL;
  if (d->n_heads > kHeadsPad || d->head_dim > kDimPad || d->head_dim % 32 != 0 ||
      d->top_k > 4096 || d->max_batch > kMaxBatch || (d->latent_dim * 2) % 16 != 0)
    return ECHO_EUNSUPPORTED;
  return ECHO_OK;
}

// The management kernel keeps all of its workgroups (one per 4096 slots, plus the
// copy workgroups) resident for its grid barrier, and the scoring kernel all of its
// workgroups for the look-back and the copy queue: each grid must fit what the
// compute units hold at once, by the runtime's occupancy query.
int check_launch(const echo_dims_t *d) {
  const int64_t atiles = ((int64_t)d->n_gpu + kSlotTile - 1) / kSlotTile;
  int gs = 1, gc = 1;
  index_grid(*d, true, &gs, &gc);
  const int64_t copy_blocks = 2 * (int64_t)gc * kScoreWaves / 16;  // 16-wave workgroups
  if (atiles + copy_blocks > (int64_t)manage_resident_per_cu() * device_cus())
    return ECHO_EUNSUPPORTED;
  if ((int64_t)gs + gc > (int64_t)score_resident_per_cu() * device_cus())
    return ECHO_EUNSUPPORTED;
  return ECHO_OK;
}

struct PublicLayout {
  int64_t scores, sel_tok, sel_slot, n_sel, kth, pf_tok, pf_slot, n_pf, n_cand, miss_tok, n_miss,
      recall_h, recall_g, counters, status, internal, total, internal_bytes;
};

PublicLayout public_layout(const echo_dims_t &d) {
  PublicLayout L;
  int64_t off = 0;
  auto take = [&](int64_t bytes) {
    int64_t o = off;
    off = align256(off + bytes);
    return o;
  };
  const int64_t B = d.max_batch, C = d.max_ctx, K = d.top_k;
  L.scores = take(B * C * 4);
  L.sel_tok = take(B * K * 4);
  L.sel_slot = take(B * K * 4);
  L.n_sel = take(B * 4);
  L.kth = take(B * 4);
  L.pf_tok = take(B * K * 4);
  L.pf_slot = take(B * K * 4);
  L.n_pf = take(B * 4);
  L.n_cand = take(B * 4);
  L.miss_tok = take(B * K * 4);
  L.n_miss = take(B * 4);
  L.recall_h = take(B * K * 4);
  L.recall_g = take(B * K * 4);
  L.counters = take(ECHO_NCOUNTERS * 4);
  L.status = take(4);
  L.internal_bytes = scratch_layout(d, nullptr, nullptr);
  L.internal = take(L.internal_bytes);
  L.total = off;
  return L;
}

bool ws_ok(const echo_ws_t *ws) {
  return ws && ws->scores && ws->sel_tok && ws->sel_slot && ws->n_sel && ws->kth && ws->pf_tok &&
         ws->pf_slot && ws->n_pf && ws->n_cand && ws->miss_tok && ws->n_miss && ws->recall_h &&
         ws->recall_g && ws->counters && ws->status && ws->internal;
}

bool batch_ok(const echo_dims_t &d, const echo_batch_t *b) {
  if (!b || b->batch < 0 || b->batch > d.max_batch) return false;
  if (b->batch > 0 && !b->ctx_len) return false;
  if (b->page_table) return b->page_stride >= 1;
  return b->batch == 0 || b->host_base;
}

bool layer_ok(const echo_layer_t *l, bool need_theta) {
  if (!l) return false;
  const echo_layer_meta_t &m = l->meta;
  if (!m.h2g || !m.g2h || !m.prio || !m.idxbuf || !m.free_flags) return false;
  if (!l->k_index || !l->gpu_kv || !l->host_kv || !l->q || !l->w || !l->ctl) return false;
  if (((uintptr_t)l->q & 15) != 0 || ((uintptr_t)l->k_index & 15) != 0 ||
      ((uintptr_t)l->gpu_kv & 15) != 0 || ((uintptr_t)l->host_kv & 15) != 0)
    return false;  // 16-byte vector loads and stores
  if (need_theta && !l->theta) return false;
  return true;
}

StepArgs make_args(const echo_dims_t &d, const echo_layer_t *l, const echo_batch_t *bt,
                   const echo_ws_t &ws, int mode) {
  StepArgs a;
  memset(&a, 0, sizeof a);
  a.H = d.n_heads;
  a.D = d.head_dim;
  a.K = d.top_k;
  a.latent = d.latent_dim;
  a.n_gpu = d.n_gpu;
  a.max_ctx = d.max_ctx;
  a.q_ring = d.q_ring;
  a.cap_div = d.prefetch_cap_div;
  a.max_batch = d.max_batch;
  a.n_host = d.n_host;
  a.alpha = d.ema_alpha;
  if (bt) {
    a.B = bt->batch;
    a.host_base = bt->host_base;
    a.ctx_len = bt->ctx_len;
    a.pages = bt->page_table;
    a.page_stride = bt->page_table ? bt->page_stride : 0;
  }
  if (l) {
    a.h2g = l->meta.h2g;
    a.g2h = l->meta.g2h;
    a.prio = l->meta.prio;
    a.idxbuf = l->meta.idxbuf;
    a.freef = l->meta.free_flags;
    a.kidx = l->k_index;
    a.gpu_kv = l->gpu_kv;
    a.host_kv = l->host_kv;
    a.q = l->q;
    a.w = l->w;
    a.theta = l->theta;
    a.guard = l->guard;
    a.ctl = l->ctl;
  }
  a.stats = nullptr;  // only the layer step adds to the running totals
  a.scores_in = ws.scores;
  a.score_stride = d.max_ctx;
  a.theta_upd = nullptr;
  a.guard_upd = nullptr;
  a.mode = mode;
  int gs = 1, gc = 1;
  index_grid(d, mode != ECHO_THETA_POS_INF, &gs, &gc);
  a.score_blocks = gs;
  a.score_waves = gs * kScoreWaves;
  a.copy_waves = gc * kScoreWaves;
  a.ws = ws;
  scratch_layout(d, ws.internal, &a.sc);
  return a;
}

// Device address of `scratch` on the current device, looked up once per device
// with that device current and kept for the process's lifetime.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

int static_scratch(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ECHO_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return ECHO_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ECHO_OK;
}

// The part of the internal scratch that the top-k call uses (request table,
// counters, selection bitmap, boundary-bin candidates), plus the workspace counter
// words, laid out from `base`; with base == nullptr only measures it.  The other
// Scratch pointers stay null.
int64_t topk_scratch_layout(const echo_dims_t &d, uint8_t *base, Scratch *s,
                            int32_t **counters) {
  int64_t off = 0;
  auto take = [&](int64_t bytes) -> uint8_t * {
    uint8_t *p = base ? base + off : nullptr;
    off = align256(off + bytes);
    return p;
  };
  const int64_t B = d.max_batch, C = d.max_ctx;
  Scratch t;
  memset(&t, 0, sizeof t);
  t.bw = (int32_t)((C + 63) / 64 * 2);
  t.max_tiles = (int32_t)(B * ((C + kScoreTile - 1) / kScoreTile));
  t.req = (ReqInfo *)take(B * sizeof(ReqInfo));
  t.misc = (int32_t *)take(M_NMISC * 4);
  int32_t *cnt = (int32_t *)take(ECHO_NCOUNTERS * 4);
  t.tbits = (uint32_t *)take(B * t.bw * 4);
  t.tcand_key = (uint32_t *)take(B * C * 4);
  t.tcand_idx = (int32_t *)take(B * C * 4);
  if (s) *s = t;
  if (counters) *counters = cnt;
  return off;
}

#define LAUNCH(x)                           \
  do {                                      \
    if ((x) != hipSuccess) return ECHO_EHIP; \
  } while (0)

// ------------------------------------------------------------ prefill workspace
struct PrefillLayout {
  int64_t scores, sel, n_sel, kth, beta, n_qcand, cand, uni, pf_h, pf_g, miss_h, miss_g, counts,
      status, internal, qhi, qlo, wsc, cflag, uflag, seg, tmp, hist, total;
};

int64_t round_seg(int64_t n) { return (n + kPfSeg - 1) / kPfSeg * kPfSeg; }

bool prefill_layout(const echo_dims_t *d, int32_t max_chunk, PrefillLayout *L) {
  if (check_dims(d) != ECHO_OK || max_chunk < 1 || max_chunk > 4096 || d->max_ctx > (1 << 22))
    return false;
  int64_t off = 0;
  auto take = [&](int64_t bytes) {
    const int64_t o = off;
    off += (bytes + 255) / 256 * 256;
    return o;
  };
  const int64_t C = max_chunk, N = d->max_ctx, K = d->top_k;
  L->scores = take(C * N * 4);
  L->sel = take(C * K * 4);
  L->n_sel = take(C * 4);
  L->kth = take(C * 4);
  L->beta = take(C * 4);
  L->n_qcand = take(C * 4);
  L->cand = take(N * 4);
  L->uni = take(N * 4);
  L->pf_h = take(N * 4);
  L->pf_g = take(N * 4);
  L->miss_h = take(N * 4);
  L->miss_g = take(N * 4);
  L->counts = take(ECHO_PF_NCOUNTS * 4);
  L->status = take(4);
  L->internal = off;
  L->qhi = take(C * kHeadsPad * kDimPad);
  L->qlo = take(C * kHeadsPad * kDimPad);
  L->wsc = take(C * kHeadsPad * 4);
  L->cflag = take(round_seg(N));
  L->uflag = take(round_seg(N));
  L->seg = take((round_seg(N) / kPfSeg + 1) * 4);
  L->tmp = take((int64_t)d->n_gpu * 4);
  L->hist = take(C * 256 * 4);
  L->total = off;
  return true;
}

bool prefill_ws_ok(const echo_prefill_ws_t *w) {
  return w && w->max_chunk >= 1 && w->scores && w->sel && w->n_sel && w->kth && w->beta &&
         w->n_qcand && w->cand && w->uni && w->pf_h && w->pf_g && w->miss_h && w->miss_g &&
         w->counts && w->status && w->internal;
}

void fill_prefill_ws(const echo_dims_t &d, const echo_prefill_ws_t *w, PrefillArgs *p) {
  PrefillLayout L;
  prefill_layout(&d, w->max_chunk, &L);
  uint8_t *in = w->internal;
  p->scores = w->scores;
  p->sel = w->sel;
  p->n_sel = w->n_sel;
  p->kth = w->kth;
  p->beta = w->beta;
  p->n_qcand = w->n_qcand;
  p->cand = w->cand;
  p->uni = w->uni;
  p->pf_h = w->pf_h;
  p->pf_g = w->pf_g;
  p->miss_h = w->miss_h;
  p->miss_g = w->miss_g;
  p->counts = w->counts;
  p->status = w->status;
  p->qhi = in + (L.qhi - L.internal);
  p->qlo = in + (L.qlo - L.internal);
  p->wsc = (float *)(in + (L.wsc - L.internal));
  p->cflag = in + (L.cflag - L.internal);
  p->uflag = in + (L.uflag - L.internal);
  p->seg = (int32_t *)(in + (L.seg - L.internal));
  p->tmp = (int32_t *)(in + (L.tmp - L.internal));
  p->hist = (uint32_t *)(in + (L.hist - L.internal));
}

int prefill_args(const echo_dims_t *dims, const echo_layer_t *layer,
                 const echo_prefill_chunk_t *c, const echo_prefill_ws_t *pws, StepArgs *a,
                 PrefillArgs *p) {
  int rc = check_dims(dims);
  if (rc != ECHO_OK) return rc;
  if (!layer_ok(layer, false) || !prefill_ws_ok(pws) || !c) return ECHO_EINVAL;
  PrefillLayout L;
  if (!prefill_layout(dims, pws->max_chunk, &L)) return ECHO_EINVAL;
  if (c->queries < 1 || c->queries > pws->max_chunk || c->hist_len < 1 ||
      c->hist_len > dims->max_ctx || c->host_base < 0 || c->host_base % 16 != 0 ||
      (int64_t)c->host_base + c->hist_len > dims->n_host || !c->q || !c->w ||
      ((uintptr_t)c->q & 15) != 0)
    return ECHO_EINVAL;
  *a = make_args(*dims, layer, nullptr, echo_ws_t(), ECHO_THETA_POS_INF);
  memset(p, 0, sizeof *p);
  fill_prefill_ws(*dims, pws, p);
  p->C = c->queries;
  p->N = c->hist_len;
  p->hb = c->host_base;
  p->q = c->q;
  p->w = c->w;
  p->pred = c->pred;
  p->qblocks = (c->queries + kPfQBlock - 1) / kPfQBlock;
  const int nch = (c->hist_len + 63) / 64;
  // About one scoring workgroup per compute unit (a workgroup fills a compute unit's
  // registers, so a grid of several rounds waits at every round for its slowest
  // wave); token splits a multiple of the 8 XCDs.
  int ts = (device_cus() + p->qblocks - 1) / p->qblocks;
  ts = (ts + 7) / 8 * 8;
  const int tmax = (nch + 7) / 8 * 8;
  p->tsplits = ts < 8 ? 8 : (ts > tmax ? tmax : ts);
  return ECHO_OK;
}

// The scoring launch's workgroups all resident (see check_launch).
int check_score_launch(const StepArgs &a) {
  const int64_t grid = (int64_t)a.score_blocks + a.copy_waves / kScoreWaves;
  return grid > (int64_t)score_resident_per_cu() * device_cus() ? ECHO_EUNSUPPORTED : ECHO_OK;
}

int run_indexer(const StepArgs &a, int extra_roles, hipStream_t s) {
  const int rc = check_score_launch(a);
  if (rc != ECHO_OK) return rc;
  LAUNCH(launch_begin(a, BEGIN_REQ | BEGIN_Q | BEGIN_CLR_INDEX | BEGIN_CLR_TOPK | extra_roles, s));
  LAUNCH(launch_score(a, s));
  return ECHO_OK;
}

}  // namespace

extern "C" {

int64_t echo_meta_bytes(int64_t n_host, int64_t n_gpu) {
  if (n_host < 0 || n_gpu < 0) return -1;
  return 4 * n_host + (1 + 4 + 4 + 4) * n_gpu;  // h2g | free, prio, idxbuf, g2h
}

size_t echo_ws_bytes(const echo_dims_t *dims) {
  if (check_dims(dims) != ECHO_OK) return 0;
  return (size_t)public_layout(*dims).total;
}

int echo_ws_bind(const echo_dims_t *dims, void *base, size_t bytes, echo_ws_t *ws) {
  int rc = check_dims(dims);
  if (rc != ECHO_OK) return rc;
  if (!base || !ws || ((uintptr_t)base & 255) != 0) return ECHO_EINVAL;
  const PublicLayout L = public_layout(*dims);
  if (bytes < (size_t)L.total) return ECHO_EINVAL;
  uint8_t *p = (uint8_t *)base;
  ws->scores = (float *)(p + L.scores);
  ws->sel_tok = (int32_t *)(p + L.sel_tok);
  ws->sel_slot = (int32_t *)(p + L.sel_slot);
  ws->n_sel = (int32_t *)(p + L.n_sel);
  ws->kth = (float *)(p + L.kth);
  ws->pf_tok = (int32_t *)(p + L.pf_tok);
  ws->pf_slot = (int32_t *)(p + L.pf_slot);
  ws->n_pf = (int32_t *)(p + L.n_pf);
  ws->n_cand = (int32_t *)(p + L.n_cand);
  ws->miss_tok = (int32_t *)(p + L.miss_tok);
  ws->n_miss = (int32_t *)(p + L.n_miss);
  ws->recall_h = (int32_t *)(p + L.recall_h);
  ws->recall_g = (int32_t *)(p + L.recall_g);
  ws->counters = (int32_t *)(p + L.counters);
  ws->status = (int32_t *)(p + L.status);
  ws->internal = p + L.internal;
  ws->internal_bytes = (size_t)L.internal_bytes;
  return ECHO_OK;
}

int echo_meta_init(const echo_dims_t *dims, const echo_layer_t *layer, hipStream_t stream) {
  int rc = check_dims(dims);
  if (rc != ECHO_OK) return rc;
  if (!layer || !layer->meta.h2g || !layer->meta.g2h || !layer->meta.prio || !layer->meta.idxbuf ||
      !layer->meta.free_flags || !layer->theta || !layer->ctl)
    return ECHO_EINVAL;
  echo_ws_t none;
  memset(&none, 0, sizeof none);
  StepArgs a = make_args(*dims, layer, nullptr, none, ECHO_THETA_POS_INF);
  a.stats = layer->stats;
  LAUNCH(launch_meta_init(a, stream));
  return ECHO_OK;
}

int echo_ws_reset(const echo_dims_t *dims, const echo_ws_t *ws, hipStream_t stream) {
  int rc = check_dims(dims);
  if (rc != ECHO_OK) return rc;
  if (!ws_ok(ws)) return ECHO_EINVAL;
  LAUNCH(launch_ws_reset(*ws, stream));
  return ECHO_OK;
}

int echo_indexer_prefetch(const echo_dims_t *dims, const echo_layer_t *layer,
                          const echo_batch_t *batch, const echo_ws_t *ws, int theta_mode,
                          hipStream_t stream) {
  int rc = check_dims(dims);
  if (rc != ECHO_OK) return rc;
  if (theta_mode < ECHO_THETA_EMA || theta_mode > ECHO_THETA_POS_INF) return ECHO_EINVAL;
  if (!layer_ok(layer, theta_mode == ECHO_THETA_EMA) || !batch_ok(*dims, batch) || !ws_ok(ws))
    return ECHO_EINVAL;
  const StepArgs a = make_args(*dims, layer, batch, *ws, theta_mode);
  return run_indexer(a, 0, stream);
}

int echo_indexer_begin(const echo_dims_t *dims, const echo_layer_t *layer,
                       const echo_batch_t *batch, const echo_ws_t *ws, int theta_mode,
                       hipStream_t stream) {
  int rc = check_dims(dims);
  if (rc != ECHO_OK) return rc;
  if (theta_mode < ECHO_THETA_EMA || theta_mode > ECHO_THETA_POS_INF) return ECHO_EINVAL;
  if (!layer_ok(layer, theta_mode == ECHO_THETA_EMA) || !batch_ok(*dims, batch) || !ws_ok(ws))
    return ECHO_EINVAL;
  const StepArgs a = make_args(*dims, layer, batch, *ws, theta_mode);
  LAUNCH(launch_begin(a, BEGIN_REQ | BEGIN_Q | BEGIN_CLR_INDEX | BEGIN_CLR_TOPK, stream));
  return ECHO_OK;
}

int echo_indexer_score(const echo_dims_t *dims, const echo_layer_t *layer,
                       const echo_batch_t *batch, const echo_ws_t *ws, int theta_mode,
                       hipStream_t stream) {
  int rc = check_dims(dims);
  if (rc != ECHO_OK) return rc;
  if (theta_mode < ECHO_THETA_EMA || theta_mode > ECHO_THETA_POS_INF) return ECHO_EINVAL;
  if (!layer_ok(layer, theta_mode == ECHO_THETA_EMA) || !batch_ok(*dims, batch) || !ws_ok(ws))
    return ECHO_EINVAL;
  const StepArgs a = make_args(*dims, layer, batch, *ws, theta_mode);
  rc = check_score_launch(a);
  if (rc != ECHO_OK) return rc;
  LAUNCH(launch_score(a, stream));
  return ECHO_OK;
}

int echo_topk(const echo_dims_t *dims, const float *scores, int64_t score_stride,
              const echo_batch_t *batch, const echo_ws_t *ws, float *theta, hipStream_t stream) {
  int rc = check_dims(dims);
  if (rc != ECHO_OK) return rc;
  if (!scores || score_stride < dims->max_ctx || !batch_ok(*dims, batch) || !ws_ok(ws))
    return ECHO_EINVAL;
  StepArgs a = make_args(*dims, nullptr, batch, *ws, ECHO_THETA_POS_INF);
  a.scores_in = scores;
  a.score_stride = score_stride;
  a.theta_upd = theta;
  LAUNCH(launch_begin(a, BEGIN_REQ | BEGIN_CLR_TOPK, stream));
  LAUNCH(launch_topk(a, false, stream));
  return ECHO_OK;
}

int echo_topk_noalloc(const echo_dims_t *dims, const float *scores, int64_t score_stride,
                      const echo_batch_t *batch, int32_t *sel_tok, int32_t *n_sel, float *kth,
                      float *theta, int32_t *status, hipStream_t stream) {
  int rc = check_dims(dims);
  if (rc != ECHO_OK) return rc;
  if (!scores || score_stride < dims->max_ctx || !batch_ok(*dims, batch) || !sel_tok ||
      !n_sel || !kth || !status)
    return ECHO_EINVAL;
  if (topk_scratch_layout(*dims, nullptr, nullptr, nullptr) > kStaticScratchBytes)
    return ECHO_ESCRATCH;
  void *base = nullptr;
  rc = static_scratch(&base);
  if (rc != ECHO_OK) return rc;
  echo_ws_t ws;
  memset(&ws, 0, sizeof ws);
  ws.sel_tok = sel_tok;
  ws.n_sel = n_sel;
  ws.kth = kth;
  ws.status = status;
  StepArgs a = make_args(*dims, nullptr, batch, ws, ECHO_THETA_POS_INF);
  topk_scratch_layout(*dims, (uint8_t *)base, &a.sc, &a.ws.counters);
  a.scores_in = scores;
  a.score_stride = score_stride;
  a.theta_upd = theta;
  // the array keeps the previous call's contents: the counters start at zero (fill
  // kernels, not memset nodes); everything else is written before it is read
  LAUNCH(launch_fill_zero((uint32_t *)a.sc.misc, M_NMISC, stream));
  LAUNCH(launch_fill_zero((uint32_t *)a.ws.counters, ECHO_NCOUNTERS, stream));
  LAUNCH(launch_begin(a, BEGIN_REQ | BEGIN_CLR_TOPK, stream));
  LAUNCH(launch_topk(a, false, stream));
  return ECHO_OK;
}

int echo_cache_alloc_evict(const echo_dims_t *dims, const echo_layer_t *layer,
                           const echo_batch_t *batch, const echo_ws_t *ws, hipStream_t stream) {
  int rc = check_dims(dims);
  if (rc != ECHO_OK) return rc;
  if (!layer_ok(layer, false) || !batch_ok(*dims, batch) || !ws_ok(ws)) return ECHO_EINVAL;
  rc = check_launch(dims);
  if (rc != ECHO_OK) return rc;
  const StepArgs a = make_args(*dims, layer, batch, *ws, ECHO_THETA_POS_INF);
  LAUNCH(launch_begin(a, BEGIN_REQ | BEGIN_CLR_MANAGE, stream));
  LAUNCH(launch_protect(a, stream));
  LAUNCH(launch_manage(a, false, false, stream));
  return ECHO_OK;
}

int echo_recall(const echo_dims_t *dims, const echo_layer_t *layer, const echo_ws_t *ws,
                hipStream_t stream) {
  int rc = check_dims(dims);
  if (rc != ECHO_OK) return rc;
  if (!layer_ok(layer, false) || !ws_ok(ws)) return ECHO_EINVAL;
  const StepArgs a = make_args(*dims, layer, nullptr, *ws, ECHO_THETA_POS_INF);
  LAUNCH(launch_recall(a, stream));
  return ECHO_OK;
}

int echo_gather(const echo_dims_t *dims, const echo_layer_t *layer, const echo_batch_t *batch,
                const echo_ws_t *ws, uint16_t *out, hipStream_t stream) {
  int rc = check_dims(dims);
  if (rc != ECHO_OK) return rc;
  if (!layer_ok(layer, false) || !batch_ok(*dims, batch) || !ws_ok(ws)) return ECHO_EINVAL;
  if (batch->batch == 0) return ECHO_OK;
  if (!out || ((uintptr_t)out & 15) != 0) return ECHO_EINVAL;
  const StepArgs a = make_args(*dims, layer, batch, *ws, ECHO_THETA_POS_INF);
  LAUNCH(launch_gather(a, out, stream));
  return ECHO_OK;
}

int echo_append(const echo_dims_t *dims, const echo_layer_t *layer, const echo_batch_t *batch,
                const uint8_t *k_new, const uint16_t *latent_new, const echo_ws_t *ws,
                int advance, hipStream_t stream) {
  int rc = check_dims(dims);
  if (rc != ECHO_OK) return rc;
  if (!layer_ok(layer, false) || !ws_ok(ws) || !batch_ok(*dims, batch)) return ECHO_EINVAL;
  if (batch->batch == 0) return ECHO_OK;
  if (!k_new || !latent_new || ((uintptr_t)latent_new & 15) != 0) return ECHO_EINVAL;
  const StepArgs a = make_args(*dims, layer, batch, *ws, ECHO_THETA_POS_INF);
  LAUNCH(launch_append(a, k_new, latent_new, const_cast<int32_t *>(batch->ctx_len),
                       advance ? 1 : 0, stream));
  return ECHO_OK;
}

int echo_release(const echo_dims_t *dims, const echo_layer_t *layer, const echo_batch_t *batch,
                 const int32_t *mask, int commit, const echo_ws_t *ws, hipStream_t stream) {
  int rc = check_dims(dims);
  if (rc != ECHO_OK) return rc;
  if (!layer_ok(layer, true) || !ws_ok(ws) || !batch_ok(*dims, batch)) return ECHO_EINVAL;
  if (batch->batch == 0) return ECHO_OK;
  if (!mask) return ECHO_EINVAL;
  const StepArgs a = make_args(*dims, layer, batch, *ws, ECHO_THETA_POS_INF);
  LAUNCH(launch_release(a, mask, const_cast<int32_t *>(batch->ctx_len), commit ? 1 : 0, stream));
  return ECHO_OK;
}

int echo_admit(const echo_dims_t *dims, const echo_layer_t *layer, const echo_batch_t *batch,
               int32_t b, int32_t base, int32_t len, int commit, const echo_ws_t *ws,
               hipStream_t stream) {
  int rc = check_dims(dims);
  if (rc != ECHO_OK) return rc;
  if (!layer_ok(layer, true) || !ws_ok(ws) || !batch_ok(*dims, batch)) return ECHO_EINVAL;
  if (b < 0 || b >= batch->batch || len < 0 || len > dims->max_ctx) return ECHO_EINVAL;
  if (!batch->page_table && (base < 0 || (int64_t)base + len > dims->n_host)) return ECHO_EINVAL;
  const StepArgs a = make_args(*dims, layer, batch, *ws, ECHO_THETA_POS_INF);
  LAUNCH(launch_admit(a, b, base, len, const_cast<int32_t *>(batch->host_base),
                      const_cast<int32_t *>(batch->ctx_len), commit ? 1 : 0, stream));
  return ECHO_OK;
}

size_t echo_prefill_ws_bytes(const echo_dims_t *dims, int32_t max_chunk) {
  PrefillLayout L;
  if (!prefill_layout(dims, max_chunk, &L)) return 0;
  return (size_t)L.total;
}

int echo_prefill_ws_bind(const echo_dims_t *dims, int32_t max_chunk, void *base, size_t bytes,
                         echo_prefill_ws_t *pws) {
  PrefillLayout L;
  if (!prefill_layout(dims, max_chunk, &L)) return ECHO_EINVAL;
  if (!base || !pws || ((uintptr_t)base & 255) != 0 || bytes < (size_t)L.total)
    return ECHO_EINVAL;
  uint8_t *p = (uint8_t *)base;
  pws->max_chunk = max_chunk;
  pws->scores = (float *)(p + L.scores);
  pws->sel = (int32_t *)(p + L.sel);
  pws->n_sel = (int32_t *)(p + L.n_sel);
  pws->kth = (float *)(p + L.kth);
  pws->beta = (int32_t *)(p + L.beta);
  pws->n_qcand = (int32_t *)(p + L.n_qcand);
  pws->cand = (int32_t *)(p + L.cand);
  pws->uni = (int32_t *)(p + L.uni);
  pws->pf_h = (int32_t *)(p + L.pf_h);
  pws->pf_g = (int32_t *)(p + L.pf_g);
  pws->miss_h = (int32_t *)(p + L.miss_h);
  pws->miss_g = (int32_t *)(p + L.miss_g);
  pws->counts = (int32_t *)(p + L.counts);
  pws->status = (int32_t *)(p + L.status);
  pws->internal = p + L.internal;
  pws->internal_bytes = (size_t)(L.total - L.internal);
  return ECHO_OK;
}

int echo_prefill_ws_reset(const echo_dims_t *dims, const echo_prefill_ws_t *pws,
                          hipStream_t stream) {
  if (check_dims(dims) != ECHO_OK || !prefill_ws_ok(pws)) return ECHO_EINVAL;
  LAUNCH(launch_fill_zero((uint32_t *)pws->counts, ECHO_PF_NCOUNTS, stream));
  LAUNCH(launch_fill_zero((uint32_t *)pws->status, 1, stream));
  LAUNCH(launch_fill_zero((uint32_t *)pws->internal, (int64_t)(pws->internal_bytes / 4), stream));
  return ECHO_OK;
}

int echo_prefill_score(const echo_dims_t *dims, const echo_layer_t *layer,
                       const echo_prefill_chunk_t *chunk, const echo_prefill_ws_t *pws,
                       hipStream_t stream) {
  StepArgs a;
  PrefillArgs p;
  const int rc = prefill_args(dims, layer, chunk, pws, &a, &p);
  if (rc != ECHO_OK) return rc;
  LAUNCH(launch_prefill_score(a, p, stream));
  return ECHO_OK;
}

int echo_prefill_early(const echo_dims_t *dims, const echo_layer_t *layer,
                       const echo_prefill_chunk_t *chunk, const echo_prefill_ws_t *pws,
                       hipStream_t stream) {
  StepArgs a;
  PrefillArgs p;
  const int rc = prefill_args(dims, layer, chunk, pws, &a, &p);
  if (rc != ECHO_OK) return rc;
  LAUNCH(launch_prefill_early(a, p, stream));
  return ECHO_OK;
}

int echo_prefill_select(const echo_dims_t *dims, const echo_layer_t *layer,
                        const echo_prefill_chunk_t *chunk, const echo_prefill_ws_t *pws,
                        hipStream_t stream) {
  StepArgs a;
  PrefillArgs p;
  const int rc = prefill_args(dims, layer, chunk, pws, &a, &p);
  if (rc != ECHO_OK) return rc;
  LAUNCH(launch_prefill_exact(a, p, stream));
  return ECHO_OK;
}

int echo_prefill_copy(const echo_dims_t *dims, const echo_layer_t *layer,
                      const echo_prefill_ws_t *pws, int list, hipStream_t stream) {
  if (check_dims(dims) != ECHO_OK) return ECHO_EINVAL;
  if (!layer_ok(layer, false) || !prefill_ws_ok(pws) || (list != 0 && list != 1))
    return ECHO_EINVAL;
  StepArgs a = make_args(*dims, layer, nullptr, echo_ws_t(), ECHO_THETA_POS_INF);
  PrefillArgs p;
  memset(&p, 0, sizeof p);
  fill_prefill_ws(*dims, pws, &p);
  LAUNCH(launch_prefill_copy(a, p, list, stream));
  return ECHO_OK;
}

int echo_step_advance(const echo_layer_t *layer, const echo_ws_t *ws, hipStream_t stream) {
  if (!layer || !layer->ctl || !ws || !ws->status) return ECHO_EINVAL;
  StepArgs a;
  memset(&a, 0, sizeof a);
  a.ctl = layer->ctl;
  a.ws = *ws;
  LAUNCH(launch_step_advance(a, stream));
  return ECHO_OK;
}

int echo_layer_step(const echo_dims_t *dims, const echo_layer_t *layer, const echo_batch_t *batch,
                    const echo_ws_t *ws, int theta_mode, hipStream_t stream) {
  int rc = check_dims(dims);
  if (rc != ECHO_OK) return rc;
  if (theta_mode < ECHO_THETA_EMA || theta_mode > ECHO_THETA_POS_INF) return ECHO_EINVAL;
  if (!layer_ok(layer, theta_mode == ECHO_THETA_EMA) || !batch_ok(*dims, batch) || !ws_ok(ws))
    return ECHO_EINVAL;
  rc = check_launch(dims);
  if (rc != ECHO_OK) return rc;
  StepArgs a = make_args(*dims, layer, batch, *ws, theta_mode);
  a.theta_upd = theta_mode == ECHO_THETA_EMA ? layer->theta : nullptr;
  a.guard_upd = layer->guard;
  a.stats = layer->stats;
  a.copy_handoff = 1;  // the prefetch copy runs on through top-k and management
  rc = run_indexer(a, BEGIN_CLR_MANAGE, stream);
  if (rc != ECHO_OK) return rc;
  if (a.B > 0 && select_manage_blocks(a) <= manage_resident_per_cu() * device_cus()) {
    // one launch: the prefetch copy runs on from selection into management
    LAUNCH(launch_select_manage(a, stream));
  } else {
    LAUNCH(launch_topk(a, true, stream));
    LAUNCH(launch_manage(a, true, true, stream));
  }
  return ECHO_OK;
}

int echo_kindex_pack(const echo_dims_t *dims, const uint8_t *rows, uint8_t *tiled,
                     int64_t n_rows, hipStream_t stream) {
  int rc = check_dims(dims);
  if (rc != ECHO_OK) return rc;
  if (!rows || !tiled || n_rows < 0 || n_rows % 16 != 0) return ECHO_EINVAL;
  const int64_t bytes = n_rows * dims->head_dim;
  if ((const uint8_t *)tiled < rows + bytes && rows < (const uint8_t *)tiled + bytes &&
      n_rows > 0)
    return ECHO_EINVAL;
  if (((uintptr_t)rows & 15) != 0 || ((uintptr_t)tiled & 15) != 0) return ECHO_EINVAL;
  LAUNCH(launch_kindex_pack(rows, tiled, n_rows, dims->head_dim, stream));
  return ECHO_OK;
}

int echo_check_invariants(const echo_dims_t *dims, const echo_layer_t *layer,
                          const echo_batch_t *batch, const echo_ws_t *ws, int32_t *report,
                          hipStream_t stream) {
  int rc = check_dims(dims);
  if (rc != ECHO_OK) return rc;
  if (!layer_ok(layer, false) || !ws_ok(ws) || !report) return ECHO_EINVAL;
  if (batch && !batch_ok(*dims, batch)) return ECHO_EINVAL;
  const StepArgs a = make_args(*dims, layer, batch, *ws, ECHO_THETA_POS_INF);
  LAUNCH(launch_check_invariants(a, batch && batch->batch > 0 ? 1 : 0, report, stream));
  return ECHO_OK;
}

const char *echo_status_string(int code) {
  switch (code) {
    case ECHO_OK: return "ok";
    case ECHO_EINVAL: return "invalid argument";
    case ECHO_EHIP: return "kernel launch failed";
    case ECHO_EUNSUPPORTED: return "unsupported shape";
    case ECHO_ECAPACITY: return "GPU pool too small for the missed tokens";
    case ECHO_ETIMEOUT: return "cross-workgroup wait timed out";
    case ECHO_EDEVARG: return "device-side batch arguments out of range or overlapping";
    case ECHO_ECORRUPT: return "cache-management state violates an invariant";
    case ECHO_ESCRATCH: return "the call needs more than the library's static scratch";
    default: return "unknown status";
  }
}

}  // extern "C"
