// Eviction, allocation and recall in one kernel, alone or fused with top-k for
// the layer step; standalone recall, step advance and initialisation.  The
// per-tile body (what eviction, allocation and recall compute, after the ECHO
// review's "Core method / in-graph per-layer cache management") is in manage.h.
//
// MI355X mapping.  One 1024-thread workgroup per 4096 slots (4 contiguous slots
// per thread), all resident at once.  Each workgroup histograms the age bin
// (priority - t + 4096, clamped at 0) of its evictable slots in LDS and merges it
// into a global histogram; after one grid barrier every workgroup finds the
// boundary bin itself.  Bins 1..4095 hold one priority each, so the boundary
// bin's slots are ranked by slot id alone with a decoupled look-back over the
// workgroups; only a boundary in the clamped bin 0 (slots idle for 4096 steps or
// more) needs the exact (priority, slot) select, done by one workgroup between
// two more barriers.  A second look-back over the workgroups ranks the free
// slots for the allocation; after a last barrier the workgroups split the recall
// list evenly and copy its rows.
//
// In the layer step the same management workgroups run inside one launch with
// the per-request top-k workgroups (they wait for a count of finished
// selections) and with copy workgroups that finish the step's prefetch copy from
// the launch's start to its end.
#include "manage.h"

namespace echo {

template <bool RECALL, bool ADVANCE>
__global__ __launch_bounds__(kSelThreads) void k_manage(StepArgs a) {
  // the status is looked at after the first reads are issued (one round trip)
  const int32_t st0 = __hip_atomic_load(a.ws.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int blk = blockIdx.x, nblk = a.sc.atiles;
  if (blk >= nblk) {
    if (st0 == 0) manage_copy(a, blk - nblk);
    return;
  }
  __shared__ ManageLds L;
  manage_block<RECALL, ADVANCE>(a, blk, st0, L);
}

// Top-k, protection, management and the rest of the prefetch copy of a layer step
// in one launch: workgroups [0, B) select (one request each), [B, B + atiles)
// manage the slots once every selection is done, and the rest copy prefetched
// rows from the launch's start to its end.  Compared with two launches, the copy
// does not stop and restart between selection and management.  Every workgroup
// is resident (the launch is used only when they fit one per compute unit).
template <bool RECALL, bool ADVANCE>
__global__ __launch_bounds__(kSelThreads) void k_select_manage(StepArgs a) {
  // a workgroup selects or manages, never both: their shared memory overlaps
  __shared__ union {
    TopkLds t;
    ManageLds m;
  } L;
  const int32_t st0 = __hip_atomic_load(a.ws.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int blk = blockIdx.x;
  if (blk < a.B) {
    topk_block<true>(a, blk, st0, L.t);
    return;
  }
  const int mb = blk - a.B, nblk = a.sc.atiles;
  if (mb >= nblk) {
    // small batches until every management workgroup has reached the recall: top-k
    // and management are chains of memory round trips, and host reads in flight
    // lengthen every one of them (measured: the layer step 264-266 us with full
    // batches throughout, 258 us with small ones during top-k; small ones through
    // management as well took the capacity decode step from 14.24 to 14.12 ms)
    if (st0 == 0) manage_copy(a, mb - nblk, &a.sc.misc[M_BAR3], nblk);
    return;
  }
  if (st0 != 0) return;
  // priorities, miss lists and counts of every request are final once all the
  // selecting workgroups have counted themselves done
  if (!wait_count(&a.sc.misc[M_TOPK_DONE], a.B, a.ws.status)) return;
  manage_block<RECALL, ADVANCE>(a, mb, 0, L.m);
}

int manage_resident_per_cu() {
  static int cache[64] = {0};  // per device: 0 not asked yet, -1 none fits, else the count
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cache[dev] == 0) {
    const void *fns[] = {reinterpret_cast<const void *>(&k_select_manage<true, true>),
                         reinterpret_cast<const void *>(&k_manage<true, true>),
                         reinterpret_cast<const void *>(&k_manage<true, false>),
                         reinterpret_cast<const void *>(&k_manage<false, true>),
                         reinterpret_cast<const void *>(&k_manage<false, false>)};
    int m = 1 << 30;
    for (const void *f : fns) {
      int n = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, f, kSelThreads, 0) != hipSuccess) n = 0;
      m = n < m ? n : m;
    }
    cache[dev] = m > 0 ? m : -1;
  }
  return cache[dev] > 0 ? cache[dev] : 0;
}

// Workgroups of the fused launch: selection + management + copy.
int select_manage_blocks(const StepArgs &a) {
  return a.B + a.sc.atiles + 2 * a.copy_waves / (kSelThreads / kWave);
}

hipError_t launch_select_manage(const StepArgs &a, hipStream_t s) {
  const dim3 grid(select_manage_blocks(a)), block(kSelThreads);
  hipLaunchKernelGGL((k_select_manage<true, true>), grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_manage(const StepArgs &a, bool recall, bool advance, hipStream_t s) {
  // the first atiles workgroups manage slots (all resident, they meet at barriers);
  // with a copy hand-off, more workgroups finish the prefetch copy beside them
  const int extra = a.copy_handoff ? 2 * a.copy_waves / (kSelThreads / kWave) : 0;
  const dim3 grid(a.sc.atiles + extra), block(kSelThreads);
  if (recall && advance)
    hipLaunchKernelGGL((k_manage<true, true>), grid, block, 0, s, a);
  else if (recall)
    hipLaunchKernelGGL((k_manage<true, false>), grid, block, 0, s, a);
  else if (advance)
    hipLaunchKernelGGL((k_manage<false, true>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((k_manage<false, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

// Standalone recall: rows of 16-byte chunks, four loads in flight per thread.
// The host link saturates with about 128-512 KB in flight and slows down with
// several MB (measured: a 1 MB transfer at 48-50 GB/s with 32 workgroups, 39 GB/s
// with 1024), so a small grid walks the list.  No load or store sits under a
// branch: threads past the last piece copy the last piece again.
constexpr int kRecallBlocks = 32;

__global__ __launch_bounds__(256) void k_recall(StepArgs a) {
  if (failed(a.ws.status)) return;
  const int n = a.ws.counters[ECHO_CNT_MISS];
  if (n <= 0) return;
  const int cpr = a.latent * 2 / 16;
  const int64_t total = (int64_t)n * cpr;
  const v4i *src = (const v4i *)a.host_kv;
  v4i *dst = (v4i *)a.gpu_kv;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i0 = (int64_t)blockIdx.x * 256 + threadIdx.x; i0 < total; i0 += 4 * stride) {
    v4i v[4];
    int64_t d[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t i = i0 + u * stride < total ? i0 + u * stride : total - 1;
      const int r = (int)(i / cpr);
      const int c = (int)(i - (int64_t)r * cpr);
      d[u] = (int64_t)a.ws.recall_g[r] * cpr + c;
      v[u] = src[(int64_t)a.ws.recall_h[r] * cpr + c];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) dst[d[u]] = v[u];
  }
}

hipError_t launch_recall(const StepArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(k_recall, dim3(kRecallBlocks), dim3(256), 0, s, a);
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
  if (a.stats && i0 < ECHO_STAT_WORDS) a.stats[i0] = 0;
}

hipError_t launch_meta_init(const StepArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(k_meta_init, dim3(1024), dim3(256), 0, s, a);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_fill_zero(uint32_t *p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = 0;
}

hipError_t launch_fill_zero(uint32_t *p, int64_t n_words, hipStream_t s) {
  hipLaunchKernelGGL(k_fill_zero, dim3(n_words > 256 * 1024 ? 1024 : 64), dim3(256), 0, s, p,
                     n_words);
  return hipGetLastError();
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
