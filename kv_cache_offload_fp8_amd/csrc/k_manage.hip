// Allocation, recall, step advance and initialisation.
//
// Allocation (ECHO review, "Core method / in-graph per-layer cache
// management": free slots are found by a parallel scan, and a counter hands
// them out): one pass over the free bitmap in 4096-slot work items, ranked with
// a decoupled look-back, so miss i (in request, token order) receives the i-th
// free slot in ascending order and the leftover free slots are written back in
// ascending order to the index buffer for the next step's prefetch.  Recall
// (same section: a GPU kernel reads host memory directly) copies every missed
// row from mapped pinned host memory into the GPU pool.
#include "kernels.h"

namespace echo {

__global__ __launch_bounds__(256) void k_alloc(StepArgs a) {
  __shared__ int s_tau, s_E;
  __shared__ int s_wcnt[4];
  __shared__ int s_moff[kMaxBatch + 1];
  if (failed(a.ws.status)) return;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  if (tid == 0) s_tau = atomicAdd(&a.sc.misc[M_TICKET_ALLOC], 1);
  if (wid == 0) {  // exclusive prefix of the per-request miss counts
    const int v = lane < a.B ? a.ws.n_miss[lane] : 0;
    const int incl = wave_incl_scan(v);
    if (lane < a.B) s_moff[lane] = incl - v;
    if (lane == kWave - 1) s_moff[a.B] = incl;
  }
  __syncthreads();
  const int tau = s_tau;
  if (tau >= a.sc.atiles) return;
  const int nmiss = s_moff[a.B];
  const int t = a.ctl[ECHO_CTL_STEP];
  const int g0 = tau * kSlotTile + wid * (kSlotTile / 4);

  uint64_t masks[16];
  int wc = 0;
#pragma unroll
  for (int it = 0; it < 16; ++it) {
    const int g = g0 + it * kWave + lane;
    const bool fr = g < a.n_gpu && a.freef[g] != 0;
    masks[it] = __ballot(fr);
    wc += __popcll(masks[it]);
  }
  if (lane == 0) s_wcnt[wid] = wc;
  __syncthreads();
  const int c = s_wcnt[0] + s_wcnt[1] + s_wcnt[2] + s_wcnt[3];
  int base = 0;
  for (int i = 0; i < wid; ++i) base += s_wcnt[i];
  if (wid == 0) {
    const int E = lookback(a.sc.astate, tau, 0, c, a.ws.status);
    if (lane == 0) s_E = E;
  }
  __syncthreads();
  base += s_E;
#pragma unroll
  for (int it = 0; it < 16; ++it) {
    const uint64_t m = masks[it];
    if ((m >> lane) & 1ull) {
      const int g = g0 + it * kWave + lane;
      const int rank = base + __popcll(m & lanemask_lt());
      if (rank < nmiss) {
        int b = 0;
        for (int i = 1; i < a.B; ++i)
          if (s_moff[i] <= rank) b = i;
        const int j = rank - s_moff[b];
        const int s = a.ws.miss_tok[(int64_t)b * a.K + j];
        const int i = a.sc.miss_i[(int64_t)b * a.K + j];
        const int64_t h = (int64_t)a.sc.req[b].base + s;
        a.h2g[h] = g;
        a.g2h[g] = (int32_t)h;
        a.freef[g] = 0;
        a.prio[g] = t;
        a.ws.sel_slot[(int64_t)b * a.K + i] = g;
        a.ws.recall_h[rank] = (int32_t)h;
        a.ws.recall_g[rank] = g;
      } else {
        a.idxbuf[rank - nmiss] = g;
      }
    }
    base += __popcll(m);
  }
  if (tau == a.sc.atiles - 1 && tid == 0) {
    const int total = s_E + c;
    a.ctl[ECHO_CTL_NFREE] = total > nmiss ? total - nmiss : 0;
    a.ws.counters[ECHO_CNT_FREE_END] = total > nmiss ? total - nmiss : 0;
    if (total < nmiss) fail(a.ws.status, ECHO_ECAPACITY);
  }
}

hipError_t launch_alloc(const StepArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(k_alloc, dim3(a.sc.atiles), dim3(256), 0, s, a);
  return hipGetLastError();
}

// Recall: rows of 16-byte chunks, four loads in flight per thread.
constexpr int kRecallBlocks = 1024;

__global__ __launch_bounds__(256) void k_recall(StepArgs a, int advance) {
  if (failed(a.ws.status)) return;
  const int n = a.ws.counters[ECHO_CNT_MISS];
  const int cpr = a.latent * 2 / 16;
  const int64_t total = (int64_t)n * cpr;
  const uint4 *src = (const uint4 *)a.host_kv;
  uint4 *dst = (uint4 *)a.gpu_kv;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i0 = (int64_t)blockIdx.x * 256 + threadIdx.x; i0 < total; i0 += 4 * stride) {
    uint4 v[4];
    int hh[4], gg[4], cc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t i = i0 + u * stride;
      hh[u] = -1;
      if (i < total) {
        const int r = (int)(i / cpr);
        cc[u] = (int)(i - (int64_t)r * cpr);
        hh[u] = a.ws.recall_h[r];
        gg[u] = a.ws.recall_g[r];
        v[u] = src[(int64_t)hh[u] * cpr + cc[u]];
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (hh[u] >= 0) dst[(int64_t)gg[u] * cpr + cc[u]] = v[u];
  }
  if (advance && blockIdx.x == 0 && threadIdx.x == 0) a.ctl[ECHO_CTL_STEP] += 1;
}

hipError_t launch_recall(const StepArgs &a, bool advance, hipStream_t s) {
  hipLaunchKernelGGL(k_recall, dim3(kRecallBlocks), dim3(256), 0, s, a, advance ? 1 : 0);
  return hipGetLastError();
}

__global__ void k_step_advance(int32_t *ctl, const int32_t *status) {
  if (threadIdx.x == 0 && !failed(status)) ctl[ECHO_CTL_STEP] += 1;
}

hipError_t launch_step_advance(const StepArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(k_step_advance, dim3(1), dim3(64), 0, s, a.ctl, a.ws.status);
  return hipGetLastError();
}

// Fresh layer: every slot free, no token resident, no EMA estimate, step 0.
__global__ __launch_bounds__(256) void k_meta_init(StepArgs a) {
  const int64_t i0 = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t step = (int64_t)gridDim.x * 256;
  for (int64_t i = i0; i < a.n_host; i += step) a.h2g[i] = -1;
  for (int64_t i = i0; i < a.n_gpu; i += step) {
    a.g2h[i] = -1;
    a.prio[i] = -1;
    a.idxbuf[i] = (int32_t)i;
    a.freef[i] = 1;
  }
  for (int64_t i = i0; i < a.max_batch; i += step) {
    a.theta[i] = __builtin_huge_valf();
    if (a.guard) a.guard[i] = __builtin_huge_valf();
  }
  if (i0 == 0) {
    a.ctl[ECHO_CTL_STEP] = 0;
    a.ctl[ECHO_CTL_NFREE] = a.n_gpu;
    for (int w = 2; w < ECHO_CTL_WORDS; ++w) a.ctl[w] = 0;
  }
}

hipError_t launch_meta_init(const StepArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(k_meta_init, dim3(1024), dim3(256), 0, s, a);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_fill_zero(uint32_t *p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = 0;
}

hipError_t launch_ws_reset(const echo_ws_t &ws, hipStream_t s) {
  hipLaunchKernelGGL(k_fill_zero, dim3(1), dim3(256), 0, s, (uint32_t *)ws.status, (int64_t)1);
  hipLaunchKernelGGL(k_fill_zero, dim3(1), dim3(256), 0, s, (uint32_t *)ws.counters,
                     (int64_t)ECHO_NCOUNTERS);
  hipLaunchKernelGGL(k_fill_zero, dim3(1024), dim3(256), 0, s, (uint32_t *)ws.internal,
                     (int64_t)(ws.internal_bytes / 4));
  return hipGetLastError();
}

}  // namespace echo
