// Eviction, allocation and recall in one kernel, alone or fused with top-k for
// the layer step; standalone recall, step advance and initialisation.
//
// Eviction (ECHO review, "Core method / in-graph per-layer cache management":
// low-priority entries are evicted after the selected tokens are protected)
// takes the n_evict occupied slots with the lowest (priority, slot) among those
// with priority < t.  Allocation (same section: free slots are found by a
// parallel scan and a counter hands them out) gives miss i the i-th free slot in
// ascending order and writes the remaining free slots, ascending, to the index
// buffer for the next step's prefetch.  Recall (same section: a GPU kernel reads
// host memory directly) copies every missed row from mapped pinned host memory
// into the GPU pool.
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
#include "topk.h"

namespace echo {

__device__ static inline int evict_bin(int prio, int t) {
  const int64_t v = (int64_t)prio - (int64_t)t + kBins;
  return v < 0 ? 0 : (v > kBins - 1 ? kBins - 1 : (int)v);
}

__device__ static inline void evict_slot(const StepArgs &a, int g) {
  const int h = a.g2h[g];
  if (h >= 0 && (int64_t)h < a.n_host) a.h2g[h] = -1;
  a.g2h[g] = -1;
  a.freef[g] = 1;
  a.prio[g] = -1;
}

typedef int v4i __attribute__((ext_vector_type(4)));

// Copy `n` rows (host ids hs[i] -> slots gs[i], both in LDS) with the whole block,
// four 16-byte loads in flight per thread.
__device__ static void copy_rows(const StepArgs &a, const int32_t *hs, const int32_t *gs, int n) {
  if (n <= 0) return;
  const int cpr = a.latent * 2 / 16;
  const v4i *src = (const v4i *)a.host_kv;
  v4i *dst = (v4i *)a.gpu_kv;
  const int total = n * cpr;
  // no load or store under a branch (each would wait for the one before): threads
  // past the last piece copy the last piece again, the same bytes to the same place
  for (int i0 = threadIdx.x; i0 < total; i0 += 4 * kSelThreads) {
    v4i v0, v1, v2, v3;
    int64_t d0, d1, d2, d3;
#define ECHO_ROW_LOAD(u, v, d)                                         \
    {                                                                  \
      const int i = i0 + (u) * kSelThreads;                            \
      const int ic = i < total ? i : total - 1;                        \
      const int e = ic / cpr, c = ic - e * cpr;                        \
      d = (int64_t)gs[e] * cpr + c;                                    \
      v = src[(int64_t)hs[e] * cpr + c];                               \
    }
    ECHO_ROW_LOAD(0, v0, d0) ECHO_ROW_LOAD(1, v1, d1) ECHO_ROW_LOAD(2, v2, d2)
    ECHO_ROW_LOAD(3, v3, d3)
#undef ECHO_ROW_LOAD
    dst[d0] = v0;
    dst[d1] = v1;
    dst[d2] = v2;
    dst[d3] = v3;
  }
}

// Eviction, allocation, recall and the step counter for slot tile `blk` of
// a.sc.atiles (all of them resident: they meet at grid barriers).  st0: the
// status word, read at the kernel's start.
template <bool RECALL, bool ADVANCE>
__device__ static void manage_block(const StepArgs &a, int blk, int32_t st0) {
  __shared__ uint32_t s_hist[kBins];
  __shared__ int32_t s_rh[kSlotTile], s_rg[kSlotTile];
  __shared__ int sh[kSelThreads / kWave + 1];
  __shared__ int s_moff[kMaxBatch + 1];
  __shared__ int s_bin, s_below, s_E;
  const int tid = threadIdx.x;
  const int nblk = a.sc.atiles;
  const int t = a.ctl[ECHO_CTL_STEP];
  if (st0 != 0) return;
  const int g0 = blk * kSlotTile + tid * 4;

  // ---- phase 1: free count, age histogram of the evictable slots
  bool fr[4];
  int pr[4];
  for (int i = tid; i < kBins; i += kSelThreads) s_hist[i] = 0;
  if (tid < kWave) {  // exclusive prefix of the per-request miss counts
    const int v = tid < a.B ? a.ws.n_miss[tid] : 0;
    const int incl = wave_incl_scan(v);
    if (tid < a.B) s_moff[tid] = incl - v;
    if (tid == kWave - 1) s_moff[a.B] = incl;
  }
  __syncthreads();
  int nfree = 0, nev = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int g = g0 + u;
    fr[u] = false;
    pr[u] = t;
    if (g < a.n_gpu) {
      fr[u] = a.freef[g] != 0;
      pr[u] = fr[u] ? t : a.prio[g];
    }
    if (fr[u]) ++nfree;
    if (g < a.n_gpu && !fr[u] && pr[u] < t) {
      ++nev;
      atomicAdd(&s_hist[evict_bin(pr[u], t)], 1u);
    }
  }
  int tot;
  block_excl_scan<kSelThreads>((nfree << 16) | nev, sh, &tot);  // per block: < 2^13 each
  for (int i = tid; i < kBins; i += kSelThreads)
    if (s_hist[i]) atomicAdd(&a.sc.ehist[i], s_hist[i]);
  if (tid == 0) {
    atomicAdd(&a.ws.counters[ECHO_CNT_FREE], tot >> 16);
    atomicAdd(&a.ws.counters[ECHO_CNT_EVICTABLE], tot & 0xFFFF);
  }
  if (!grid_sync(&a.sc.misc[M_BAR0], nblk, a.ws.status)) return;

  // ---- phase 2: eviction
  const int nmiss = __hip_atomic_load(&a.ws.counters[ECHO_CNT_MISS], __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
  const int F = __hip_atomic_load(&a.ws.counters[ECHO_CNT_FREE], __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
  const int nE = __hip_atomic_load(&a.ws.counters[ECHO_CNT_EVICTABLE], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
  if ((int64_t)F + nE < nmiss) {
    if (tid == 0) fail(a.ws.status, ECHO_ECAPACITY);
    return;
  }
  const int64_t want = (int64_t)nmiss + a.sc.misc[M_RESERVE] - F;
  const int n_evict = (int)(want <= 0 ? 0 : (want < nE ? want : nE));
  if (blk == 0 && tid == 0) {
    a.ws.counters[ECHO_CNT_EVICT] = n_evict;
    if (a.stats && n_evict > 0) atomicAdd((unsigned long long *)&a.stats[ECHO_STAT_EVICTED],
                                          (unsigned long long)n_evict);
  }
  bool ev[4] = {false, false, false, false};
  if (n_evict > 0) {
    find_boundary<true>(a.sc.ehist, n_evict, &s_bin, &s_below, sh);
    const int bstar = s_bin;
    const int need = n_evict - s_below;
    if (bstar > 0) {
      // boundary bin = one priority: rank its slots by slot id across workgroups
      int nb = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool evictable = g0 + u < a.n_gpu && !fr[u] && pr[u] < t;
        const int bin = evictable ? evict_bin(pr[u], t) : kBins;
        ev[u] = bin < bstar;
        if (bin == bstar) ++nb;
      }
      int btot;
      int rank = block_excl_scan<kSelThreads>(nb, sh, &btot);
      if (tid < kWave) {
        const int E = lookback(a.sc.estate, blk, 0, btot, a.ws.status);
        if (tid == 0) s_E = E;
      }
      __syncthreads();
      rank += s_E;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool evictable = g0 + u < a.n_gpu && !fr[u] && pr[u] < t;
        if (evictable && evict_bin(pr[u], t) == bstar) {
          if (rank < need) ev[u] = true;
          ++rank;
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (ev[u]) {
          evict_slot(a, g0 + u);
          fr[u] = true;
        }
    } else {
      // boundary in the clamped bin: exact (priority, slot) select of its slots
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool evictable = g0 + u < a.n_gpu && !fr[u] && pr[u] < t;
        if (evictable && evict_bin(pr[u], t) == 0) {
          const int pos = atomicAdd(&a.sc.ecnt[0], 1);
          a.sc.ecand_key[pos] = (uint32_t)pr[u];
          a.sc.ecand_idx[pos] = g0 + u;
        }
      }
      if (!grid_sync(&a.sc.misc[M_BAR1], nblk, a.ws.status)) return;
      if (blk == 0) {
        const int c = __hip_atomic_load(&a.sc.ecnt[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        uint64_t P;
        int pos;
        block_select(a.sc.ecand_key, a.sc.ecand_idx, c, need, &P, &pos);
        for (int i = tid; i < c; i += kSelThreads) {
          const uint32_t k = a.sc.ecand_key[i];
          const int32_t g = a.sc.ecand_idx[i];
          if (composite_selected(k, g, P, pos)) evict_slot(a, g);
        }
      }
      if (!grid_sync(&a.sc.misc[M_BAR2], nblk, a.ws.status)) return;
      // no bin lies below bin 0; slots of higher bins stay
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int g = g0 + u;
        const bool evictable = g < a.n_gpu && !fr[u] && pr[u] < t;
        if (evictable && evict_bin(pr[u], t) == 0 && a.freef[g])
          fr[u] = true;  // evicted by workgroup 0 (made visible by the barrier's fences)
      }
    }
  }

  // ---- phase 3: allocation in ascending slot order
  int nf = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) nf += fr[u] ? 1 : 0;
  int ftot;
  int rank = block_excl_scan<kSelThreads>(nf, sh, &ftot);
  if (tid < kWave) {
    const int E = lookback(a.sc.astate, blk, 0, ftot, a.ws.status);
    if (tid == 0) s_E = E;
  }
  __syncthreads();
  const int E = s_E;
  rank += E;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    if (!fr[u]) continue;
    const int g = g0 + u;
    if (rank < nmiss) {
      int b = 0;
      for (int i = 1; i < a.B; ++i)
        if (s_moff[i] <= rank) b = i;
      const int j = rank - s_moff[b];
      const int s = a.ws.miss_tok[(int64_t)b * a.K + j];
      const int i = a.sc.miss_i[(int64_t)b * a.K + j];
      const int64_t h = token_host(a, b, a.sc.req[b].base, s);
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
    ++rank;
  }
  if (blk == nblk - 1 && tid == 0) {
    const int total = E + ftot;
    const int left = total > nmiss ? total - nmiss : 0;
    a.ctl[ECHO_CTL_NFREE] = left;
    a.ws.counters[ECHO_CNT_FREE_END] = left;
    if (total < nmiss) fail(a.ws.status, ECHO_ECAPACITY);
  }

  // ---- phase 4: recall.  Misses take the lowest free slots, so the workgroups
  // that allocated them are few; after a barrier every workgroup copies an equal
  // share of the whole recall list instead.
  if (RECALL && nmiss > 0) {
    if (!grid_sync(&a.sc.misc[M_BAR3], nblk, a.ws.status)) return;
    const int r0 = (int)((int64_t)nmiss * blk / nblk);
    const int r1 = (int)((int64_t)nmiss * (blk + 1) / nblk);
    for (int r = r0 + tid; r < r1; r += kSelThreads) {
      s_rh[r - r0] = __hip_atomic_load(&a.ws.recall_h[r], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
      s_rg[r - r0] = __hip_atomic_load(&a.ws.recall_g[r], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    copy_rows(a, s_rh, s_rg, r1 - r0);
  }
  if (ADVANCE) {
    __syncthreads();
    if (tid == 0) {
      const int done = __hip_atomic_fetch_add(&a.sc.misc[M_DONE], 1, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
      if (done == nblk - 1 && !failed(a.ws.status)) {
        a.ctl[ECHO_CTL_STEP] = t + 1;
        if (a.stats) atomicAdd((unsigned long long *)&a.stats[ECHO_STAT_STEPS], 1ull);
      }
    }
  }
}

// copy workgroup w of a management launch: finish the step's prefetch copy, two
// waves per copy wave (small batches while *slow < slow_target, if given)
__device__ static void manage_copy(const StepArgs &a, int w, const int32_t *slow = nullptr,
                                   int slow_target = 0) {
  const int g = w * (kSelThreads / kWave) + (int)threadIdx.x / kWave;
  copy_worker(a, a.sc.req, g % a.copy_waves, g / a.copy_waves, 2, nullptr, 0, slow, slow_target);
}

template <bool RECALL, bool ADVANCE>
__global__ __launch_bounds__(kSelThreads) void k_manage(StepArgs a) {
  // the status is looked at after the first reads are issued (one round trip)
  const int32_t st0 = __hip_atomic_load(a.ws.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int blk = blockIdx.x, nblk = a.sc.atiles;
  if (blk >= nblk) {
    if (st0 == 0) manage_copy(a, blk - nblk);
    return;
  }
  manage_block<RECALL, ADVANCE>(a, blk, st0);
}

// Top-k, protection, management and the rest of the prefetch copy of a layer step
// in one launch: workgroups [0, B) select (one request each), [B, B + atiles)
// manage the slots once every selection is done, and the rest copy prefetched
// rows from the launch's start to its end.  Compared with two launches, the copy
// does not stop and restart between selection and management.  Every workgroup
// is resident (the launch is used only when they fit one per compute unit).
template <bool RECALL, bool ADVANCE>
__global__ __launch_bounds__(kSelThreads) void k_select_manage(StepArgs a) {
  const int32_t st0 = __hip_atomic_load(a.ws.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int blk = blockIdx.x;
  if (blk < a.B) {
    topk_block<true>(a, blk, st0);
    return;
  }
  const int mb = blk - a.B, nblk = a.sc.atiles;
  if (mb >= nblk) {
    // small batches until every selection is done: top-k is latency-bound and the
    // host reads in flight slow its memory round trips (measured: the layer step
    // 264-266 us with full batches throughout, 258 us with this)
    if (st0 == 0) manage_copy(a, mb - nblk, &a.sc.misc[M_TOPK_DONE], a.B);
    return;
  }
  if (st0 != 0) return;
  // priorities, miss lists and counts of every request are final once all the
  // selecting workgroups have counted themselves done
  if (!wait_count(&a.sc.misc[M_TOPK_DONE], a.B, a.ws.status)) return;
  manage_block<RECALL, ADVANCE>(a, mb, 0);
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
