// Invariant check of one layer's cache-management state (a debug call).
//
// The ECHO review ("Core method / in-graph per-layer cache management") keeps a
// free bitmap, an eviction priority, an index buffer and the two maps between
// host tokens and GPU slots, all updated inside the graph; its "Systemic flaws"
// section notes that correctness then rests on the order of slot allocation,
// protection, map updates and transfers.  This kernel checks the state those
// steps must leave behind:
//   - the maps are mutual inverses (h2g[h] = g  <=>  g2h[g] = h);
//   - a slot is free  <=>  g2h = -1  <=>  prio = -1, and free flags are 0 or 1;
//   - an occupied slot's priority is a past step, 0 <= prio < t;
//   - the index buffer's first ctl[NFREE] entries are exactly the free slots, in
//     ascending order;
//   - optionally (batch given), every token of the last step's selection is
//     resident, at the slot the step reported, with priority t - 1.
// Violations are counted per kind in a caller buffer; any violation (or resident
// host ids and occupied slots that do not count the same) sets the sticky status
// to ECHO_ECORRUPT.
//
// Three launches: clear the report, one grid-stride pass over host ids, slots,
// the free list and the selection (block-reduced counts, one atomic per block
// and kind), and a one-thread finish.  Reads only; runs whatever the status.
#include "kernels.h"

namespace echo {

constexpr int kCheckThreads = 256;
constexpr int kCheckBlocks = 1024;

__global__ void k_inv_clear(int32_t *report) {
  if (threadIdx.x < ECHO_INV_WORDS) report[threadIdx.x] = 0;
}

__global__ __launch_bounds__(kCheckThreads) void k_inv_scan(StepArgs a, int check_sel,
                                                            int32_t *report) {
  __shared__ int s_cnt[ECHO_INV_WORDS];
  const int tid = threadIdx.x;
  if (tid < ECHO_INV_WORDS) s_cnt[tid] = 0;
  __syncthreads();
  int c[ECHO_INV_WORDS];
#pragma unroll
  for (int i = 0; i < ECHO_INV_WORDS; ++i) c[i] = 0;
  const int64_t i0 = (int64_t)blockIdx.x * kCheckThreads + tid;
  const int64_t step = (int64_t)gridDim.x * kCheckThreads;
  const int t = a.ctl[ECHO_CTL_STEP];
  // host ids: a slot, if any, must map back
  for (int64_t h = i0; h < a.n_host; h += step) {
    const int32_t g = a.h2g[h];
    if (g >= 0) {
      ++c[ECHO_INV_RESIDENT];
      if (g >= a.n_gpu || a.g2h[g] != (int32_t)h) ++c[ECHO_INV_H2G];
    } else if (g != -1) {
      ++c[ECHO_INV_H2G];
    }
  }
  // slots: flags, maps and priorities agree
  for (int64_t g = i0; g < a.n_gpu; g += step) {
    const int f = a.freef[g];
    const int32_t m = a.g2h[g], p = a.prio[g];
    const bool free_ok = (f == 1 && m == -1 && p == -1) || (f == 0 && m >= 0 && p >= 0);
    if (!free_ok) ++c[ECHO_INV_FREE];
    if (f == 0) {
      ++c[ECHO_INV_OCCUPIED];
      if (p < 0 || p >= t) ++c[ECHO_INV_PRIO];
    }
    if (m >= 0 && ((int64_t)m >= a.n_host || a.h2g[m] != (int32_t)g)) ++c[ECHO_INV_G2H];
    else if (m < -1) ++c[ECHO_INV_G2H];
  }
  // the ascending free list
  int32_t nfree = a.ctl[ECHO_CTL_NFREE];
  nfree = nfree < 0 ? 0 : (nfree > a.n_gpu ? a.n_gpu : nfree);
  for (int64_t i = i0; i < nfree; i += step) {
    const int32_t e = a.idxbuf[i];
    const bool ok = e >= 0 && e < a.n_gpu && a.freef[e] == 1 && (i == 0 || a.idxbuf[i - 1] < e);
    if (!ok) ++c[ECHO_INV_FREE_LIST];
  }
  // the last step's selection
  if (check_sel) {
    const int64_t n = (int64_t)a.B * a.K;
    for (int64_t j = i0; j < n; j += step) {
      const int b = (int)(j / a.K), i = (int)(j - (int64_t)b * a.K);
      int ns = a.ws.n_sel[b];
      ns = ns < 0 ? 0 : (ns > a.K ? a.K : ns);
      if (i >= ns) continue;
      const int32_t s = a.ws.sel_tok[j];
      bool ok = s >= 0 && s < a.ctx_len[b] && (!a.pages || s < 16 * a.page_stride);
      const int64_t h = ok ? token_host(a, b, a.pages ? 0 : a.host_base[b], s) : -1;
      ok = ok && h >= 0 && h < a.n_host;
      if (ok) {
        const int32_t g = a.h2g[h];
        ok = g >= 0 && g < a.n_gpu && g == a.ws.sel_slot[j] && a.prio[g] == t - 1;
      }
      if (!ok) ++c[ECHO_INV_SELECTED];
    }
  }
#pragma unroll
  for (int i = 0; i < ECHO_INV_WORDS; ++i) {
    const int v = wave_sum(c[i]);
    if (lane_id() == 0 && v) atomicAdd(&s_cnt[i], v);
  }
  __syncthreads();
  if (tid < ECHO_INV_WORDS && s_cnt[tid]) atomicAdd(&report[tid], s_cnt[tid]);
}

__global__ void k_inv_finish(StepArgs a, int32_t *report) {
  if (threadIdx.x != 0) return;
  // the free list must be as long as the free slots are many
  const int32_t nfree = a.ctl[ECHO_CTL_NFREE];
  const int64_t want = (int64_t)a.n_gpu - report[ECHO_INV_OCCUPIED];
  if ((int64_t)nfree != want) report[ECHO_INV_FREE_LIST] += 1;
  bool bad = report[ECHO_INV_RESIDENT] != report[ECHO_INV_OCCUPIED];
  for (int i = 0; i < ECHO_INV_RESIDENT; ++i) bad |= report[i] != 0;
  if (bad) fail(a.ws.status, ECHO_ECORRUPT);
}

hipError_t launch_check_invariants(const StepArgs &a, int check_sel, int32_t *report,
                                   hipStream_t s) {
  hipLaunchKernelGGL(k_inv_clear, dim3(1), dim3(64), 0, s, report);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_inv_scan, dim3(kCheckBlocks), dim3(kCheckThreads), 0, s, a, check_sel,
                     report);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_inv_finish, dim3(1), dim3(64), 0, s, a, report);
  return hipGetLastError();
}

}  // namespace echo
