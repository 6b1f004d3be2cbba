// Kernel arguments and launcher declarations (internal).
#pragma once

#include "common.h"

namespace echo {

// Everything a step's kernels read, passed by value as one kernel argument.
struct StepArgs {
  // dims
  int32_t H, D, K, latent, n_gpu, max_ctx, q_ring, cap_div, max_batch;
  int64_t n_host;
  float alpha;
  // batch (B is a host value baked into the launch)
  int32_t B;
  const int32_t *host_base, *ctx_len;
  const int32_t *pages;  // [B][page_stride] host page of each 16-token page, or null
  int32_t page_stride;
  // layer
  int32_t *h2g, *g2h, *prio, *idxbuf;
  uint8_t *freef;
  const uint8_t *kidx;
  uint16_t *gpu_kv;
  const uint16_t *host_kv;
  const uint16_t *q;
  const float *w;
  float *theta;   // prefetch threshold state (read by the prologue)
  float *guard;   // last k-th score per request (selection guard), or null
  int32_t *ctl;
  uint64_t *stats;  // running totals of the layer (echo_layer_step only), or null
  // scores read by the top-k passes
  const float *scores_in;
  int64_t score_stride;
  float *theta_upd;  // EMA state to update in the top-k epilogue, or null
  float *guard_upd;  // selection guard to refresh in the top-k epilogue, or null
  int32_t mode;
  // launch shapes, fixed by the dims so that a captured graph stays valid
  int32_t score_blocks;  // indexer workgroups that score (the rest copy)
  int32_t score_waves;   // score_blocks * kScoreWaves
  int32_t copy_waves;    // copy workgroups * kScoreWaves
  int32_t copy_handoff;  // 1: the copy continues in the top-k and management kernels
  // workspace
  echo_ws_t ws;
  Scratch sc;
};

// Host id of token s of request b: through the page table (a page is 16 host ids,
// one tiled-K group), or in the contiguous range that starts at `base`.
__device__ inline int64_t token_host(const StepArgs &a, int b, int32_t base, int32_t s) {
  if (a.pages) return 16LL * a.pages[(int64_t)b * a.page_stride + (s >> 4)] + (s & 15);
  return (int64_t)base + s;
}

// Whether host page p lies in the pool (all 16 of its ids below n_host).
__device__ inline bool page_in_pool(const StepArgs &a, int32_t p) {
  return p >= 0 && 16LL * p + 16 <= a.n_host;
}

// Threads of the one-workgroup admission kernels.
constexpr int kListThreads = 1024;

// Workgroup roles by XCD.  MI355X deals consecutive workgroup ids to its eight XCDs
// in turn.  When the grid has room, the nc copy workgroups take ids 0, 8, 16, ...,
// so that all of them sit on one XCD and only that XCD's L2 carries the
// long-latency host reads, while the workgroups that stream HBM run on the other
// seven (measured in the capacity layer step: the scoring kernel 96-98 us with its
// 32 copy workgroups on one XCD; the decode step 2.3% faster than with them
// spread over all eight).  Otherwise the last nc ids copy.  Returns true for a
// copy workgroup; *idx is its rank among the copy workgroups, or among the others.
__device__ inline bool xcd_copy_role(int bid, int grid, int nc, int *idx) {
  if (nc > 0 && 8 * (nc - 1) < grid) {
    if ((bid & 7) == 0 && (bid >> 3) < nc) {
      *idx = bid >> 3;
      return true;
    }
    const int below = (bid + 7) >> 3;  // copy ids 0, 8, .. below bid
    *idx = bid - (below < nc ? below : nc);
    return false;
  }
  const int first = grid - nc;
  *idx = bid >= first ? bid - first : bid;
  return bid >= first;
}

// begin-kernel roles
enum {
  BEGIN_REQ = 1,         // request table, scoring jobs, reserve
  BEGIN_Q = 2,           // fp8 hi/lo split of the query
  BEGIN_CLR_INDEX = 4,   // look-back states, prefetch outputs
  BEGIN_CLR_TOPK = 8,    // shortcut counter
  BEGIN_CLR_MANAGE = 16  // eviction histogram, look-back states, barriers, counters
};

// Scoring and copying workgroups of the indexer launch for these dims (together at
// most one per compute unit, so that all of them are resident at once); without
// prefetch there are no copy workgroups.
void index_grid(const echo_dims_t &d, bool with_copy, int *score_blocks, int *copy_blocks);
// Compute units of the current device (cached per device).
int device_cus();
// Workgroups of the launches whose workgroups wait on each other (the scoring kernel's
// look-back and copy queue; the grid barriers of selection + management and of
// management) that one compute unit holds at once, the least over their variants, from
// the runtime's occupancy query (cached per device; 0 if one does not fit).  Such a
// launch is made only when its grid fits that many per compute unit.
int score_resident_per_cu();
int manage_resident_per_cu();

hipError_t launch_begin(const StepArgs &a, int roles, hipStream_t s);
hipError_t launch_score(const StepArgs &a, hipStream_t s);
hipError_t launch_topk(const StepArgs &a, bool protect, hipStream_t s);
hipError_t launch_protect(const StepArgs &a, hipStream_t s);
hipError_t launch_manage(const StepArgs &a, bool recall, bool advance, hipStream_t s);
// top-k (with protection), management (recall, step advance) and the prefetch copy
// in one launch of select_manage_blocks(a) workgroups, all resident
int select_manage_blocks(const StepArgs &a);
hipError_t launch_select_manage(const StepArgs &a, hipStream_t s);
hipError_t launch_gather(const StepArgs &a, uint16_t *out, hipStream_t s);
hipError_t launch_append(const StepArgs &a, const uint8_t *k_new, const uint16_t *lat_new,
                         int32_t *ctx_io, int advance, hipStream_t s);
hipError_t launch_release(const StepArgs &a, const int32_t *mask, int32_t *ctx_io, int commit,
                          hipStream_t s);
hipError_t launch_admit(const StepArgs &a, int b, int32_t base, int32_t len, int32_t *hb_io,
                        int32_t *ctx_io, int commit, hipStream_t s);
hipError_t launch_recall(const StepArgs &a, hipStream_t s);
hipError_t launch_step_advance(const StepArgs &a, hipStream_t s);
hipError_t launch_meta_init(const StepArgs &a, hipStream_t s);
hipError_t launch_ws_reset(const echo_ws_t &ws, hipStream_t s);
hipError_t launch_fill_zero(uint32_t *p, int64_t n_words, hipStream_t s);
hipError_t launch_check_invariants(const StepArgs &a, int check_sel, int32_t *report,
                                   hipStream_t s);
hipError_t launch_kindex_pack(const uint8_t *rows, uint8_t *tiled, int64_t n_rows, int D,
                              hipStream_t s);

}  // namespace echo
