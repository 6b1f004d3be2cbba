// Chunked-prefill kernel arguments and launchers (internal).
#pragma once

#include "kernels.h"

namespace echo {

// One chunked-prefill call: the chunk (host values and device inputs), the
// prefill workspace, and the scoring grid.
struct PrefillArgs {
  int32_t C, N, hb;            // queries, history tokens, first host id of the history
  const uint16_t *q;           // [C][H][D] bf16
  const float *w;              // [C][H]
  const float *pred;           // [C] or null
  float *scores;               // [max_chunk][N] (row stride N)
  int32_t *sel, *n_sel;        // [max_chunk][K], [max_chunk]
  float *kth;                  // [max_chunk]
  int32_t *beta, *n_qcand;     // [max_chunk]
  int32_t *cand, *uni;         // [max_ctx]
  int32_t *pf_h, *pf_g, *miss_h, *miss_g;  // [max_ctx]
  int32_t *counts, *status;
  uint8_t *qhi, *qlo;          // [max_chunk][kHeadsPad][kDimPad]
  float *wsc;                  // [max_chunk][kHeadsPad]
  uint8_t *cflag, *uflag;      // [max_ctx rounded up to kPfSeg]
  int32_t *seg;                // [max_ctx / kPfSeg + 1]
  int32_t *tmp;                // [n_gpu] free-list buffer
  uint32_t *hist;              // [max_chunk][256] coarse-bucket histogram per query
  int32_t qblocks, tsplits;    // scoring grid: query blocks x token splits
};
constexpr int kPfSeg = 4096;   // list entries per workgroup of the ordered passes
constexpr int ECHO_PF_CNT_LEFT = 5;  // internal count: free slots left after a chunk
constexpr int kPfWaves = 8;    // waves per prefill scoring workgroup
constexpr int kPfQ = 2;        // queries per prefill scoring wave
constexpr int kPfQBlock = kPfWaves * kPfQ;  // queries per prefill scoring workgroup

hipError_t launch_prefill_score(const StepArgs &a, const PrefillArgs &p, hipStream_t s);
hipError_t launch_prefill_early(const StepArgs &a, const PrefillArgs &p, hipStream_t s);
hipError_t launch_prefill_exact(const StepArgs &a, const PrefillArgs &p, hipStream_t s);
hipError_t launch_prefill_copy(const StepArgs &a, const PrefillArgs &p, int list, hipStream_t s);

}  // namespace echo
