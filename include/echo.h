/*
 * echo.h -- C ABI of the MI355X (gfx950) decode-step hot path of ECHO's lossless
 * KV-cache offloading for sparse-attention (DeepSeek Sparse Attention) models.
 *
 * Source: "ECHO: Efficient KV Cache Offloading with Lossless Prefetching for
 * Serving Native Sparse Attention LLMs (OSDI 2026)", review page on
 * awesome-system-papers (cited below as "the ECHO review"), and the podcast show
 * notes "ECHO: Lossless KV Cache Offloading for Sparse Attention LLMs".  The
 * pages give no API; the calls below follow their problem statement: every
 * structure is a fixed-size preallocated device tensor, there is no per-layer
 * CPU control, the whole step can be captured in one graph, and allocation,
 * eviction and recall are separate operations (review, "Core method / in-graph
 * per-layer cache management").
 *
 * Conventions shared by every call
 *  - Every pointer inside the structs is a device address, except where a field
 *    says otherwise.  `host_kv` is pinned, mapped host memory: its device-visible
 *    address (with unified addressing, the host pointer returned by hipHostMalloc).
 *  - The caller allocates and owns all memory.  The library never allocates,
 *    frees or synchronizes; each call validates its arguments on the host, enqueues
 *    kernels on `stream` and returns.  Every call can be captured in a hipGraph.
 *  - Host-side return codes: ECHO_OK, or ECHO_EINVAL (bad argument or shape; nothing
 *    was enqueued), ECHO_EUNSUPPORTED (a shape this library has no kernel for, or
 *    a launch whose workgroups wait on each other -- scoring with prefetch,
 *    management -- and would not all fit on the compute units at once by the
 *    runtime's occupancy query), or ECHO_EHIP (a launch failed).  Those waits also
 *    give up after 1 s (ECHO_ETIMEOUT below), so work of another process holding
 *    compute units for longer ends the step with an error, never a hang.
 *  - Errors found on the device (capacity, bad device-side lengths, a stuck wait)
 *    are written to `ws->status`: the first error wins and stays until
 *    echo_ws_reset.  Once it is set, every later kernel of every call is a no-op,
 *    and the metadata stays consistent (mutual maps, free flags, priorities).
 *    Read it after your own synchronization.
 *  - Token identities: without a page table, request b of a batch owns host ids
 *    host_base[b] .. host_base[b] + ctx_len[b] - 1; ranges of different requests
 *    must not overlap, and every host_base is a multiple of 16 (both checked on
 *    the device: ECHO_EDEVARG).  With a page table (echo_batch_t.page_table), the
 *    host pool is cut into pages of 16 host ids and token s of request b is host
 *    id 16 * page_table[b * page_stride + s / 16] + s % 16; the pages a request
 *    uses must lie in the pool (checked on the device: ECHO_EDEVARG) and must not
 *    be shared with another live request (checked by echo_admit).
 *  - The indexer K cache is kept in the tiled layout that the gfx950 fp8 MFMA
 *    consumes (see echo_kindex_pack): host ids are grouped by 16, and group g
 *    holds bytes [16*g*D, 16*(g+1)*D), D = head_dim.
 */
#ifndef ECHO_H
#define ECHO_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------ status codes */
enum {
  ECHO_OK = 0,
  ECHO_EINVAL = -1,       /* argument or shape check failed                    */
  ECHO_EHIP = -2,         /* a kernel launch failed                            */
  ECHO_EUNSUPPORTED = -3, /* shape with no kernel in this library              */
  ECHO_ECAPACITY = -4,    /* device: free + evictable slots < missed tokens    */
  ECHO_ETIMEOUT = -5,     /* device: a cross-workgroup wait exceeded 1 s       */
  ECHO_EDEVARG = -6,      /* device: ctx_len/host_base out of range or overlap */
  ECHO_ECORRUPT = -7,     /* device: echo_check_invariants found a violation   */
  ECHO_ESCRATCH = -8      /* the shape needs more than the static scratch      */
};

/* Prefetch threshold modes.  EMA: the threshold is the exponential moving
 * average of past k-th scores (ECHO review, "Core method / decode"; smoothing
 * from "Key observations", observation 2).  NEG_INF admits every non-resident
 * token (up to the cap); POS_INF disables prefetch.  The selected set and the
 * gathered KV do not depend on the mode: that is the losslessness property. */
enum { ECHO_THETA_EMA = 0, ECHO_THETA_NEG_INF = 1, ECHO_THETA_POS_INF = 2 };

/* Indices into echo_ws_t.counters (int32, written by the step's kernels). */
enum {
  ECHO_CNT_MISS = 0,      /* selected tokens that were not resident (all requests) */
  ECHO_CNT_EVICT = 1,     /* slots evicted this step                               */
  ECHO_CNT_FREE = 2,      /* free slots after prefetch, before eviction            */
  ECHO_CNT_EVICTABLE = 3, /* occupied slots with priority < t                      */
  ECHO_CNT_FREE_END = 4,  /* free slots after allocation                           */
  ECHO_CNT_PREFETCH = 5,  /* tokens prefetched this step (all requests)            */
  ECHO_CNT_SHORTCUT = 6,  /* requests whose top-k came from the guard candidates   */
  ECHO_NCOUNTERS = 16
};

/* Running totals of one layer (echo_layer_t.stats, uint64), added to by
 * echo_layer_step (a step that ends with a device error may have added part of
 * its counts; STEPS counts completed steps) and cleared by echo_meta_init.  They
 * measure how useful the prefetch is (ECHO review, "Key observations",
 * observation 2, and "Limitations and future work": the wasted prefetch traffic
 * and the final recall count are worth recording). */
enum {
  ECHO_STAT_STEPS = 0,       /* layer steps counted                                     */
  ECHO_STAT_SELECTED = 1,    /* selected tokens                                         */
  ECHO_STAT_MISSED = 2,      /* selected tokens not resident after prefetch (recalled)  */
  ECHO_STAT_PREFETCHED = 3,  /* tokens prefetched while scoring                         */
  ECHO_STAT_PF_SELECTED = 4, /* of those, tokens selected by the same step's top-k      */
  ECHO_STAT_CANDIDATES = 5,  /* prefetch candidates before the cap                      */
  ECHO_STAT_EVICTED = 6,     /* slots evicted                                           */
  ECHO_STAT_WORDS = 8
};

/* Words of per-layer control state (echo_layer_t.ctl). */
enum {
  ECHO_CTL_STEP = 0,  /* decode-step counter t of this layer                        */
  ECHO_CTL_NFREE = 1, /* length of the ascending free list kept in meta.idxbuf       */
  ECHO_CTL_WORDS = 4
};

/* Counts written by the chunked-prefill calls (echo_prefill_ws_t.counts). */
enum {
  ECHO_PF_CNT_CAND = 0,  /* tokens in the union of the coarse candidates             */
  ECHO_PF_CNT_UNION = 1, /* tokens in the union of the exact selections              */
  ECHO_PF_CNT_EARLY = 2, /* candidates installed early (pf_h / pf_g)                 */
  ECHO_PF_CNT_LATE = 3,  /* the rest of the union installed after the exact select   */
  ECHO_PF_NCOUNTS = 8
};

/* Shapes.  Supported by this library: 1 <= n_heads <= 64; head_dim in {32, 64, 96,
 * 128}; 1 <= top_k <= 4096; latent_dim*2 a multiple of 16 bytes; n_host < 2^31
 * and a multiple of 16;
 * 1 <= n_gpu < 2^31; 1 <= max_batch <= 64; 1 <= max_ctx < 2^31; prefetch_cap_div
 * >= 1; q_ring >= 1; 0 < ema_alpha <= 1. */
typedef struct {
  int32_t n_heads;          /* H: indexer heads                                     */
  int32_t head_dim;         /* D: indexer dimension (bytes per fp8 K row)          */
  int32_t top_k;            /* k: tokens selected per request (2048 in DSA)        */
  int32_t latent_dim;       /* MLA latent elements per token (576 bf16)            */
  int64_t n_host;           /* N_H: host pool tokens                               */
  int32_t n_gpu;            /* N_G: GPU pool slots per layer                       */
  int32_t max_batch;        /* largest batch any call will use                     */
  int32_t max_ctx;          /* largest context any request will have               */
  float ema_alpha;          /* EMA smoothing: theta <- a*s_k + (1-a)*theta (0.5)   */
  int32_t prefetch_cap_div; /* per-request prefetch cap = min(k, ceil(ctx/div))    */
  int32_t q_ring;           /* query slots in echo_layer_t.q, used as t mod q_ring */
} echo_dims_t;

/* Per-layer cache-management metadata (ECHO review, "Core method / in-graph
 * per-layer cache management"): a free bitmap (one byte per slot), an eviction
 * priority (the step of last use), an index buffer (the ascending free list) and
 * the two maps.  Total 4*n_host + 13*n_gpu bytes (echo_meta_bytes). */
typedef struct {
  int32_t *h2g;        /* [n_host]  GPU slot of each host token, -1 if not resident */
  int32_t *g2h;        /* [n_gpu]   host token held by each slot, -1 if free        */
  int32_t *prio;       /* [n_gpu]   step of last use, -1 if free                    */
  int32_t *idxbuf;     /* [n_gpu]   ascending free slots, first ctl[NFREE] valid     */
  uint8_t *free_flags; /* [n_gpu]   1 = free                                         */
} echo_layer_meta_t;

/* One layer's tensors.  k_index, gpu_kv, host_kv and q must be 16-byte aligned
 * (ECHO_EINVAL otherwise).
 *
 * Between calls, a layer's whole cache-management state is in meta (five
 * arrays), gpu_kv, theta, guard, ctl and stats; the workspace carries nothing
 * from one step to the next, and the maps hold indices, not addresses.  The ECHO
 * review ("Critical analysis / systemic flaws") notes that the full host copy of
 * the cache is not a persistence mechanism: a byte copy of these buffers is one.
 * Written back, at the same or other addresses and with any workspace, the
 * following steps give bit-identical results. */
typedef struct {
  echo_layer_meta_t meta;
  const uint8_t *k_index;  /* n_host*head_dim bytes: indexer K, OCP fp8 E4M3FN, in the
                              tiled layout of echo_kindex_pack, resident in HBM     */
  uint16_t *gpu_kv;        /* [n_gpu][latent_dim] bf16 GPU pool                      */
  const uint16_t *host_kv; /* [n_host][latent_dim] bf16 host pool (mapped, pinned)   */
  const uint16_t *q;       /* [q_ring][batch][n_heads][head_dim] bf16 queries        */
  const float *w;          /* [batch][n_heads] fp32 head weights                     */
  float *theta;            /* [max_batch] EMA threshold, +inf = no estimate yet       */
  float *guard;            /* [max_batch] last step's k-th score, +inf = none; may be
                              NULL.  Only a shortcut for the exact top-k (tokens near or
                              above it are collected while scoring, and if at least k
                              are, the full-score passes are skipped); results never
                              depend on it. */
  int32_t *ctl;            /* [ECHO_CTL_WORDS] step counter and free-list length      */
  uint64_t *stats;         /* [ECHO_STAT_WORDS] running totals, or NULL (not kept)   */
} echo_layer_t;

/* The batch.  Where a request's tokens live is either one contiguous host range
 * (host_base) or a page table: the ECHO review leaves request cancellation and
 * host-pool exhaustion open ("Systemic flaws"), and pages let a new request use
 * any free host pages, holes left by released requests included.  A page is 16
 * host ids, one group of the tiled indexer K (echo_kindex_pack).  The lifecycle
 * calls (echo_append, echo_release, echo_admit) write ctx_len (and, echo_admit
 * without a page table, host_base) through although they are declared const for
 * the step calls. */
typedef struct {
  int32_t batch;             /* B, host value, 0 <= B <= max_batch                  */
  const int32_t *host_base;  /* [B] device: first host id of each request; not used
                                (may be NULL) with a page table                      */
  const int32_t *ctx_len;    /* [B] device: context length, 0 <= ctx <= max_ctx      */
  const int32_t *page_table; /* [B][page_stride] device, or NULL: host page of each
                                16-token page of each request's context              */
  int32_t page_stride;       /* host value, >= 1 with a page table: entries per row  */
} echo_batch_t;

/* Workspace: one caller-allocated device buffer carved by echo_ws_bind.  The
 * named arrays are outputs of the step that the caller may read. */
typedef struct {
  float *scores;      /* [max_batch][max_ctx] indexer scores                        */
  int32_t *sel_tok;   /* [max_batch][top_k] selected tokens, ascending              */
  int32_t *sel_slot;  /* [max_batch][top_k] their GPU slots after the step           */
  int32_t *n_sel;     /* [max_batch] min(top_k, ctx)                                */
  float *kth;         /* [max_batch] k-th highest score of the step                 */
  int32_t *pf_tok;    /* [max_batch][top_k] prefetched tokens, in rank order        */
  int32_t *pf_slot;   /* [max_batch][top_k] their slots                             */
  int32_t *n_pf;      /* [max_batch] prefetched tokens                              */
  int32_t *n_cand;    /* [max_batch] prefetch candidates before the cap             */
  int32_t *miss_tok;  /* [max_batch][top_k] selected tokens that were not resident   */
  int32_t *n_miss;    /* [max_batch]                                                */
  int32_t *recall_h;  /* [max_batch*top_k] recall list: host ids, (request, token)   */
  int32_t *recall_g;  /* [max_batch*top_k] recall list: destination slots           */
  int32_t *counters;  /* [ECHO_NCOUNTERS]                                           */
  int32_t *status;    /* [1] sticky device status                                   */
  uint8_t *internal;  /* scratch used between the step's kernels                    */
  size_t internal_bytes;
} echo_ws_t;

/* ------------------------------------------------------------- sizing */

/* Bytes of per-layer metadata: 4*n_host + 13*n_gpu (ECHO review, "Core method /
 * in-graph per-layer cache management": about 10 MB per layer at 2M host and
 * 200K GPU tokens).  Pure function; returns -1 for negative sizes. */
int64_t echo_meta_bytes(int64_t n_host, int64_t n_gpu);

/* Bytes of the workspace buffer for these dims (0 if dims are invalid). */
size_t echo_ws_bytes(const echo_dims_t *dims);

/* Carve `base` (device, `bytes` >= echo_ws_bytes, 256-byte aligned) into *ws.
 * Host-only; returns ECHO_EINVAL on a bad argument. */
int echo_ws_bind(const echo_dims_t *dims, void *base, size_t bytes, echo_ws_t *ws);

/* ------------------------------------------------------------- init */

/* Reset one layer: every slot free (free=1, prio=-1, g2h=-1), h2g=-1 for every
 * host token, idxbuf = 0..n_gpu-1, theta = guard = +inf for max_batch requests,
 * step 0, and the running totals (if kept) zero. */
int echo_meta_init(const echo_dims_t *dims, const echo_layer_t *layer, hipStream_t stream);

/* Clear the workspace (status, counters and internal scratch). */
int echo_ws_reset(const echo_dims_t *dims, const echo_ws_t *ws, hipStream_t stream);

/* Write indexer K rows into the tiled layout the scoring kernel reads.
 * `rows` is [n_rows][D] row-major fp8 (device), `tiled` receives the same
 * n_rows*D bytes (device, may not alias `rows`), n_rows a multiple of 16.
 * Byte d of host id h goes to
 *     16*D*(h/16) + 8*D*((d%32)/16) + 256*(d/32) + 16*(h%16) + d%16,
 * so that for every 16-token group one 16-byte load per lane, 64 lanes wide,
 * reads 1 KB (for D = 128) of contiguous memory holding exactly the MFMA
 * operand bytes of those lanes: lane c*16 + r gets dims 32c + 16j .. +15 of
 * token r in load j (j = 0, 1).  The layout is a permutation inside each group
 * of 16 rows; the scores do not depend on it.  Returns ECHO_EINVAL for a bad
 * argument (nothing enqueued). */
int echo_kindex_pack(const echo_dims_t *dims, const uint8_t *rows, uint8_t *tiled,
                     int64_t n_rows, hipStream_t stream);

/* ------------------------------------------------------ the hot path */

/* The two halves of echo_indexer_prefetch, for callers that time or schedule
 * them apart (same passages, same arguments): echo_indexer_begin enqueues the
 * query prologue (request table, fp8 query split, cleared per-call state) and
 * echo_indexer_score the scoring + prefetch kernel, which must follow it on the
 * same stream with the same arguments and nothing between them that uses the
 * workspace.  Errors: as echo_indexer_prefetch. */
int echo_indexer_begin(const echo_dims_t *dims, const echo_layer_t *layer,
                       const echo_batch_t *batch, const echo_ws_t *ws, int theta_mode,
                       hipStream_t stream);
int echo_indexer_score(const echo_dims_t *dims, const echo_layer_t *layer,
                       const echo_batch_t *batch, const echo_ws_t *ws, int theta_mode,
                       hipStream_t stream);

/* Steps a0-a2: query prologue, lightning-indexer scoring
 * score[b,s] = sum_j w[b,j] * max(0, q[b,j,:] . K[host_base[b]+s,:]) for s < ctx_len[b]
 * (DeepSeek Sparse Attention's indexer, which the ECHO review's "Problem and
 * motivation" names; fp8 K, bf16 q, fp32 accumulation), and, while scoring
 * proceeds, EMA-threshold prefetch (ECHO review, "Core method / decode" and
 * "Core method / prefetch inside the indexer pipeline"): tokens with
 * score > theta that have no slot are taken in token order, at most
 * min(top_k, ceil(ctx/prefetch_cap_div)) per request, into the free slots
 * idxbuf[off_b + r] (off_b = sum of earlier requests' caps), with priority t,
 * and their latent rows are read from the host pool.  Writes ws->scores,
 * pf_tok/pf_slot/n_pf/n_cand and counters[PREFETCH]. */
int echo_indexer_prefetch(const echo_dims_t *dims, const echo_layer_t *layer,
                          const echo_batch_t *batch, const echo_ws_t *ws, int theta_mode,
                          hipStream_t stream);

/* Step a3: exact top-k per request of `scores` ([batch][score_stride] fp32,
 * device; may be ws->scores or any caller buffer): the min(top_k, ctx) tokens
 * that come first under (score descending, token ascending), written in
 * ascending token order to ws->sel_tok, with ws->n_sel and ws->kth (ECHO review,
 * "Core method / decode").  If `theta` is not NULL, requests with ctx >= top_k
 * update their EMA threshold theta[b] (seeded by the first k-th score).
 * Scores must be finite. */
int echo_topk(const echo_dims_t *dims, const float *scores, int64_t score_stride,
              const echo_batch_t *batch, const echo_ws_t *ws, float *theta,
              hipStream_t stream);

/* Steps a4-a6 for the tokens in ws->sel_tok (ECHO review, "Core method /
 * in-graph per-layer cache management"): protect every resident selected token
 * (priority t) and list the misses in (request, token) order; evict the
 * n_evict = min(|E|, max(0, misses + R - free)) occupied slots with the lowest
 * (priority, slot) among those with priority < t (R = sum of prefetch caps; no
 * data moves); give miss i the i-th free slot in ascending order; rebuild the
 * free list in idxbuf.  Writes sel_slot, miss_tok, n_miss, recall_h/recall_g
 * and counters.  Sets ECHO_ECAPACITY if free + evictable < misses. */
int echo_cache_alloc_evict(const echo_dims_t *dims, const echo_layer_t *layer,
                           const echo_batch_t *batch, const echo_ws_t *ws, hipStream_t stream);

/* Step a7: copy every row in the recall list from the host pool to the GPU pool
 * (a kernel reading mapped host memory directly; ECHO review, "Core method /
 * in-graph per-layer cache management"). */
int echo_recall(const echo_dims_t *dims, const echo_layer_t *layer, const echo_ws_t *ws,
                hipStream_t stream);

/* Advance the layer's step counter t by one (skipped if ws->status is set). */
int echo_step_advance(const echo_layer_t *layer, const echo_ws_t *ws, hipStream_t stream);

/* Attention input: out[b][i] = the GPU-pool row (latent bf16 values) of request
 * b's i-th selected token, gpu_kv[ws->sel_slot[b][i]], for i < ws->n_sel[b], and
 * zero rows for n_sel[b] <= i < k.  The ECHO review ("Core method / decode") runs
 * the sparse attention only after the exact top-k and the recall of every
 * missing selected token, so these rows equal what the attention would read with
 * no offloading at all.  out: device, [batch][k][latent] bf16, 16-byte aligned,
 * caller-owned.  Call after the layer's step; a no-op if ws->status is set.
 * Errors: ECHO_EINVAL (host checks). */
int echo_gather(const echo_dims_t *dims, const echo_layer_t *layer, const echo_batch_t *batch,
                const echo_ws_t *ws, uint16_t *out, hipStream_t stream);

/* Decode append and writeback: the step's new token joins every request's
 * context.  The ECHO review ("Core method / in-graph per-layer cache
 * management") keeps the indexer K resident on the GPU and backs each token's KV
 * up to the host pool when it is generated, so eviction moves no data; its
 * "Design trade-offs" section counts that writeback of every new token.
 *   batch    the batch; the new token of request b is its token ctx_len[b], at host
 *            id host_base[b] + ctx_len[b] or, with a page table, in the page that
 *            row b lists for it (the caller hands out pages); with advance != 0
 *            the call then adds one to batch->ctx_len[b] (written through)
 *   k_new  [batch][D]       device: the token's indexer key, e4m3, row-major; it is
 *                           written into layer->k_index in the tiled layout
 *   latent_new [batch][latent] device, 16-byte aligned: the token's bf16 latent,
 *                           written into layer->host_kv (mapped pinned host memory)
 * layer->k_index and layer->host_kv are written through although the layer
 * struct declares them const for the other calls.  Call it once per layer after
 * that layer's step, with advance != 0 only for the last layer of the step.  The
 * token is not placed in the GPU pool (it becomes resident when prefetched or
 * recalled).  Errors: ECHO_EINVAL (host checks; batch 0 is a no-op).  Device:
 * ECHO_ECAPACITY if a request has no room (ctx_len = max_ctx; the id at or past
 * n_host; with a page table, a page slot past page_stride or a listed page outside
 * the pool; without one, the id inside another request's range including its own
 * new token), ECHO_EDEVARG if a slot already maps the host id; the lowest such
 * request decides, and nothing is written.  A row with ctx_len 0 is empty
 * (released, or never admitted): it takes no token, does not grow, and its stale
 * host_base takes no part in the other requests' room checks. */
int echo_append(const echo_dims_t *dims, const echo_layer_t *layer, const echo_batch_t *batch,
                const uint8_t *k_new, const uint16_t *latent_new, const echo_ws_t *ws,
                int advance, hipStream_t stream);

/* Request release (cancellation) between decode steps.  The ECHO review leaves
 * request cancellation open ("Systemic flaws") and asks that top-k and attention
 * input stay equal to the no-offload baseline when requests are cancelled
 * ("Limitations and future work"); the state is that of "Core method / in-graph
 * per-layer cache management".  For every request b with mask[b] != 0, each host
 * id of its tokens (its range, or the ids its pages give its ctx_len[b] tokens)
 * that holds a GPU slot gives it back (g2h = -1, free = 1, prio = -1), those h2g
 * rows become -1, theta[b] (and guard[b]) become +inf; no bytes move, and host
 * pages stay the caller's to reuse.  Then the ascending free list (meta.idxbuf,
 * ctl[ECHO_CTL_NFREE]) is rebuilt.  With commit != 0, batch->ctx_len[b] of every
 * released request becomes 0 (written through).
 *   mask [batch]: device int32
 * Call it between steps, once per layer, with commit != 0 only for the last
 * layer (the batch row is shared by the layers).  Errors:
 * ECHO_EINVAL (host checks; batch 0 is a no-op).  Device: ECHO_EDEVARG if a
 * masked request's tokens do not fit (ctx_len outside [0, max_ctx]; host_base < 0
 * or the range past n_host; with a page table, more pages than page_stride or a
 * page outside the pool); all are checked first and nothing changes.  A no-op
 * while ws->status holds an error. */
int echo_release(const echo_dims_t *dims, const echo_layer_t *layer, const echo_batch_t *batch,
                 const int32_t *mask, int commit, const echo_ws_t *ws, hipStream_t stream);

/* Request admission into an empty batch row b (the other half of the lifecycle
 * above): theta[b] = guard[b] = +inf (no estimate yet) and, with commit != 0,
 * row b takes len tokens: without a page table the host ids [base, base + len)
 * (host_base[b] = base), with one the first len ids of the pages the caller has
 * written into row b of the page table (base is not used); ctx_len[b] = len.  The
 * caller has written (or will append) those tokens' indexer keys and host latents.
 * Errors: ECHO_EINVAL (host checks: b outside [0, batch), len outside
 * [0, max_ctx]; without a page table base < 0 or base + len > n_host; nothing
 * enqueued).  Device, in this order: ECHO_EDEVARG if ctx_len[b] != 0 (the row is
 * in use: release it first); with a page table, ECHO_EDEVARG if the len tokens
 * need more pages than page_stride, or one of their pages lies outside the pool or
 * is listed twice; ECHO_ECAPACITY if the range meets the range of another request
 * with ctx_len > 0 (with a page table: one of their pages is a page another live
 * request's tokens use); ECHO_EDEVARG if some slot still maps a host id of the
 * new tokens.  Nothing is written on an error; a no-op while ws->status holds an
 * error.  One call per layer, with commit != 0 only for the last, like
 * echo_release. */
int echo_admit(const echo_dims_t *dims, const echo_layer_t *layer, const echo_batch_t *batch,
               int32_t b, int32_t base, int32_t len, int commit, const echo_ws_t *ws,
               hipStream_t stream);

/* echo_topk for callers that cannot allocate: code under graph capture, tight
 * serving loops, harnesses that forbid device allocation.  It computes exactly
 * what echo_topk computes (same selection, k-th scores and threshold update, same
 * kernels), but takes its outputs as plain device arrays instead of a workspace
 * and keeps its internal scratch (request table, selection bitmap, boundary-bin
 * candidates, counters) in a static device array of the library, 32 MiB on each
 * GPU, held until the process ends.  The call allocates nothing.
 *   scores   [batch][score_stride] fp32, device, score_stride >= max_ctx
 *   sel_tok  [batch][top_k] int32, device: selected tokens, ascending
 *   n_sel    [batch] int32, device: min(top_k, ctx)
 *   kth      [batch] fp32, device: k-th highest score
 *   theta    [batch] fp32, device, or NULL: EMA thresholds updated as echo_topk does
 *   status   [1] int32, device: sticky status of the call, like echo_ws_t.status
 *            (a device-side batch error sets it; while it is set the call changes
 *            nothing); the caller clears it.
 * The scratch needs 64 bytes per request for the request table, about
 * max_ctx / 8 bytes per request for the bitmap and 8 * max_ctx bytes per request
 * for the candidates (each region rounded up to 256 bytes), plus a few hundred
 * bytes: up to 32 requests of 100,000 tokens fit.  Larger dims return
 * ECHO_ESCRATCH with nothing enqueued.  Every call on a GPU uses that GPU's one
 * array: calls that overlap on one GPU (other streams, other threads) race and
 * give wrong results; calls ordered on one stream do not.  Errors: ECHO_EINVAL
 * (host checks), ECHO_ESCRATCH, ECHO_EHIP. */
int echo_topk_noalloc(const echo_dims_t *dims, const float *scores, int64_t score_stride,
                      const echo_batch_t *batch, int32_t *sel_tok, int32_t *n_sel, float *kth,
                      float *theta, int32_t *status, hipStream_t stream);

/* Steps a0-a8 for one layer and one decode step, in order, on `stream`: indexer
 * + prefetch, top-k with the EMA update (mode EMA only), protect/evict/alloc,
 * recall, and the step-counter advance.  The ECHO review's "Core method / decode"
 * gives the order (prefetch while the indexer scores, exact top-k, then recall of
 * every selected token that is still missing, before the sparse attention);
 * "Core method / in-graph per-layer cache management" keeps every layer's
 * management on the GPU inside the captured graph, with no per-layer CPU
 * control; "Core method / prefetch inside the indexer pipeline" overlaps the
 * prefetch transfers with scoring.  Here the prefetch copy also runs on through
 * top-k and management and is complete when the call's last kernel ends.  The
 * results equal those of echo_indexer_prefetch, echo_topk (theta updated in mode
 * EMA), echo_cache_alloc_evict, echo_recall and echo_step_advance called in
 * turn.  Errors: as those calls; ECHO_EUNSUPPORTED if the indexer launch cannot
 * keep all of its workgroups resident. */
int echo_layer_step(const echo_dims_t *dims, const echo_layer_t *layer,
                    const echo_batch_t *batch, const echo_ws_t *ws, int theta_mode,
                    hipStream_t stream);

/* ------------------------------------------------------- chunked prefill */

/* One prefill chunk: C queries scored against one request's history of N tokens
 * (host ids host_base .. host_base + N - 1, indexer K resident in the layer's
 * tiled K).  The chunk's own tokens are not part of the history. */
typedef struct {
  int32_t queries;   /* C, host value, 1 <= C <= max_chunk                          */
  int32_t host_base; /* host value, a multiple of 16, host_base + N <= n_host      */
  int32_t hist_len;  /* N, host value, 1 <= N <= max_ctx                            */
  const uint16_t *q; /* [C][n_heads][head_dim] bf16, device, 16-byte aligned        */
  const float *w;    /* [C][n_heads] fp32 head weights, device                      */
  const float *pred; /* [C] device: predicted k-th score per query, or NULL (0)     */
} echo_prefill_chunk_t;

/* Prefill workspace: one caller-allocated device buffer carved by
 * echo_prefill_ws_bind.  The named arrays are outputs the caller may read. */
typedef struct {
  int32_t max_chunk;
  float *scores;     /* [max_chunk][N] indexer scores of the last chunk (row stride N) */
  int32_t *sel;      /* [max_chunk][top_k] each query's top-k, ascending               */
  int32_t *n_sel;    /* [max_chunk] min(top_k, N)                                      */
  float *kth;        /* [max_chunk] each query's k-th highest score                    */
  int32_t *beta;     /* [max_chunk] boundary bucket, -1 if N <= top_k                  */
  int32_t *n_qcand;  /* [max_chunk] coarse candidates of each query                    */
  int32_t *cand;     /* [max_ctx] union of the candidates, ascending tokens            */
  int32_t *uni;      /* [max_ctx] union of the selections, ascending tokens            */
  int32_t *pf_h;     /* [max_ctx] early installs: host ids, in candidate order         */
  int32_t *pf_g;     /* [max_ctx] their slots                                          */
  int32_t *miss_h;   /* [max_ctx] later installs: host ids, in union order             */
  int32_t *miss_g;   /* [max_ctx] their slots                                          */
  int32_t *counts;   /* [ECHO_PF_NCOUNTS]                                              */
  int32_t *status;   /* [1] sticky device status of the prefill calls                  */
  uint8_t *internal; /* scratch between the calls (must start zeroed: bind + reset)    */
  size_t internal_bytes;
} echo_prefill_ws_t;

/* Bytes of a prefill workspace for chunks of up to max_chunk queries (0 if the
 * dims or max_chunk are invalid: 1 <= max_chunk <= 4096, max_ctx <= 2^22). */
size_t echo_prefill_ws_bytes(const echo_dims_t *dims, int32_t max_chunk);

/* Carve `base` (device, >= echo_prefill_ws_bytes, 256-byte aligned) into *pws.
 * Host-only.  The buffer must then be cleared with echo_prefill_ws_reset. */
int echo_prefill_ws_bind(const echo_dims_t *dims, int32_t max_chunk, void *base, size_t bytes,
                         echo_prefill_ws_t *pws);

/* Clear status, counts and internal flags (fill kernels, no memset nodes). */
int echo_prefill_ws_reset(const echo_dims_t *dims, const echo_prefill_ws_t *pws,
                          hipStream_t stream);

/* Chunked prefill, part 1: scores and coarse candidates.  The ECHO
 * review ("Core method / prefill"): chunk i's identified candidates move while
 * chunk i+1 is scored; a 256-bucket coarse histogram keeps the strictly-high
 * buckets and leaves the threshold bucket to the exact selection; subtracting a
 * predicted k-th score refines the buckets near the boundary.  "Core method /
 * prefetch inside the indexer pipeline": prefill splits the indexer's work by
 * query chunk.  Per query i the call writes scores[i][0..N) (the decode
 * formula), beta[i] = the bucket of fp16(score - pred[i]) at which the count from
 * the top first reaches top_k (-1 if N <= top_k) and n_qcand[i]; cand = the
 * ascending union of the tokens above their query's boundary (every token if
 * N <= top_k).  The prefill calls are no-ops while pws->status holds an error.
 * Errors: ECHO_EINVAL (host checks), ECHO_EUNSUPPORTED. */
int echo_prefill_score(const echo_dims_t *dims, const echo_layer_t *layer,
                       const echo_prefill_chunk_t *chunk, const echo_prefill_ws_t *pws,
                       hipStream_t stream);

/* Chunked prefill, part 2: the early install (same passages).  In cand order, a
 * resident token gets priority t (the layer's step counter) and the others take
 * the lowest free slots (meta.idxbuf, ascending), listed in pf_h / pf_g.  Copy
 * them with echo_prefill_copy(list 0), on another stream if wanted, while the
 * exact selection and the next chunk's scoring run; the next chunk's
 * echo_prefill_early rewrites the list, so order it after that copy.  Device:
 * ECHO_ECAPACITY if the candidates without a slot exceed the free slots
 * (nothing installed). */
int echo_prefill_early(const echo_dims_t *dims, const echo_layer_t *layer,
                       const echo_prefill_chunk_t *chunk, const echo_prefill_ws_t *pws,
                       hipStream_t stream);

/* Chunked prefill, part 3: the exact fetch.  Per query, the top_k tokens by
 * (score desc, token asc), written ascending into sel[i], with n_sel[i] and
 * kth[i] (pass kth as the next chunk's pred); uni = their ascending union.  In
 * uni order a resident token gets priority t and the others take the next free
 * slots after the early installs (miss_h / miss_g; copy them with
 * echo_prefill_copy(list 1)).  Then t advances and the ascending free list is
 * rebuilt.  The chunk must be the one given to echo_prefill_score and
 * echo_prefill_early, and the next chunk's echo_prefill_select rewrites list 1,
 * so order it after that list's copy.  Device:
 * ECHO_ECAPACITY if the rest of the union exceeds the free slots left (the early
 * installs stand; t does not advance).  A prefill chunk evicts nothing. */
int echo_prefill_select(const echo_dims_t *dims, const echo_layer_t *layer,
                        const echo_prefill_chunk_t *chunk, const echo_prefill_ws_t *pws,
                        hipStream_t stream);

/* Copy the host rows of install list 0 (early) or 1 (later) into the GPU pool,
 * reading mapped host memory directly.  Order it after the call that wrote the
 * list (echo_prefill_early for list 0, echo_prefill_select for list 1). */
int echo_prefill_copy(const echo_dims_t *dims, const echo_layer_t *layer,
                      const echo_prefill_ws_t *pws, int list, hipStream_t stream);

/* ------------------------------------------------------------- diagnostics */

/* Indices into the report of echo_check_invariants: violations of each kind, then
 * two counts. */
enum {
  ECHO_INV_H2G = 0,       /* host ids whose h2g entry is neither -1 nor a slot mapping back */
  ECHO_INV_G2H = 1,       /* slots whose g2h entry is neither -1 nor a host id mapping back */
  ECHO_INV_FREE = 2,      /* slots where "free", "g2h = -1" and "prio = -1" disagree         */
  ECHO_INV_PRIO = 3,      /* occupied slots with a priority outside [0, t)                  */
  ECHO_INV_FREE_LIST = 4, /* free-list entries not free or not ascending, plus one if its
                             length differs from the number of free slots                  */
  ECHO_INV_SELECTED = 5,  /* selected tokens (batch given) not resident at their reported
                             slot with priority t - 1                                      */
  ECHO_INV_RESIDENT = 6,  /* count: host ids that hold a slot                               */
  ECHO_INV_OCCUPIED = 7,  /* count: slots that are not free                                 */
  ECHO_INV_WORDS = 8
};

/* Debug check of one layer's cache-management state (ECHO review, "Core method /
 * in-graph per-layer cache management": free bitmap, priorities, index buffer and
 * the two maps; "Systemic flaws": correctness depends on the order of
 * allocation, protection, map updates and transfers).  Checks that h2g and g2h
 * are mutual inverses, that free <=> g2h = -1 <=> prio = -1, that every occupied
 * slot's priority lies in [0, t) with t = ctl[ECHO_CTL_STEP], and that
 * idxbuf[0 .. ctl[ECHO_CTL_NFREE]) is the ascending list of all free slots.  With
 * `batch` not NULL it also checks the last step's selection in ws (sel_tok,
 * n_sel, sel_slot): every selected token holds the reported slot, with priority
 * t - 1; pass it only right after a step that ended with status 0.
 *   report: device int32 [ECHO_INV_WORDS], caller-owned, overwritten.
 * If any violation is counted, or the resident and occupied counts differ,
 * ws->status becomes ECHO_ECORRUPT (unless an earlier error holds it).  Reads the
 * state only, and runs whatever the status.  Errors: ECHO_EINVAL (host checks). */
int echo_check_invariants(const echo_dims_t *dims, const echo_layer_t *layer,
                          const echo_batch_t *batch, const echo_ws_t *ws, int32_t *report,
                          hipStream_t stream);

/* Static string for a status code. */
const char *echo_status_string(int code);

#ifdef __cplusplus
}
#endif

#endif /* ECHO_H */
