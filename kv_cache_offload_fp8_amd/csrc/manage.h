// Eviction, allocation and recall of one slot tile (internal): the body shared by
// the management kernel, the fused top-k + management kernel and the fused
// layer-step kernel.
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
#pragma once

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

// Copy `n` rows (host ids hs[i] -> slots gs[i], both in LDS) with the whole block of
// NT threads, four 16-byte loads in flight per thread.
template <int NT>
__device__ static void copy_rows(const StepArgs &a, const int32_t *hs, const int32_t *gs, int n) {
  if (n <= 0) return;
  const int cpr = a.latent * 2 / 16;
  const v4i *src = (const v4i *)a.host_kv;
  v4i *dst = (v4i *)a.gpu_kv;
  const int total = n * cpr;
  // no load or store under a branch (each would wait for the one before): threads
  // past the last piece copy the last piece again, the same bytes to the same place
  for (int i0 = threadIdx.x; i0 < total; i0 += 4 * NT) {
    v4i v0, v1, v2, v3;
    int64_t d0, d1, d2, d3;
#define ECHO_ROW_LOAD(u, v, d)                                         \
    {                                                                  \
      const int i = i0 + (u) * NT;                                     \
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

// Shared memory of manage_block.
struct ManageLds {
  uint32_t hist[kBins];
  int32_t rh[kSlotTile], rg[kSlotTile];
  int sh[kMaxSelWaves + 1];
  int moff[kMaxBatch + 1];
  int bin, below, E;
  SelectLds sel_lds;
};

// Eviction, allocation, recall and the step counter for slot tile `blk` of
// a.sc.atiles (all of them resident: they meet at grid barriers), by a workgroup
// of NT threads, SPT = kSlotTile / NT contiguous slots per thread.  st0: the
// status word, read at the kernel's start.
template <bool RECALL, bool ADVANCE, int NT = kSelThreads>
__device__ static void manage_block(const StepArgs &a, int blk, int32_t st0, ManageLds &L) {
  constexpr int SPT = kSlotTile / NT;
  uint32_t *const s_hist = L.hist;
  int32_t *const s_rh = L.rh;
  int32_t *const s_rg = L.rg;
  int *const sh = L.sh;
  int *const s_moff = L.moff;
  const int tid = threadIdx.x;
  const int nblk = a.sc.atiles;
  const int t = a.ctl[ECHO_CTL_STEP];
  if (st0 != 0) return;
  const int g0 = blk * kSlotTile + tid * SPT;

  // ---- phase 1: free count, age histogram of the evictable slots
  bool fr[SPT];
  int pr[SPT];
  for (int i = tid; i < kBins; i += NT) s_hist[i] = 0;
  if (tid < kWave) {  // exclusive prefix of the per-request miss counts
    const int v = tid < a.B ? a.ws.n_miss[tid] : 0;
    const int incl = wave_incl_scan(v);
    if (tid < a.B) s_moff[tid] = incl - v;
    if (tid == kWave - 1) s_moff[a.B] = incl;
  }
  __syncthreads();
  int nfree = 0, nev = 0;
#pragma unroll
  for (int u = 0; u < SPT; ++u) {
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
  block_excl_scan<NT>((nfree << 16) | nev, sh, &tot);  // per block: < 2^13 each
  for (int i = tid; i < kBins; i += NT)
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
  bool ev[SPT];
#pragma unroll
  for (int u = 0; u < SPT; ++u) ev[u] = false;
  if (n_evict > 0) {
    find_boundary<true, NT>(a.sc.ehist, n_evict, &L.bin, &L.below, sh);
    const int bstar = L.bin;
    const int need = n_evict - L.below;
    if (bstar > 0) {
      // boundary bin = one priority: rank its slots by slot id across workgroups
      int nb = 0;
#pragma unroll
      for (int u = 0; u < SPT; ++u) {
        const bool evictable = g0 + u < a.n_gpu && !fr[u] && pr[u] < t;
        const int bin = evictable ? evict_bin(pr[u], t) : kBins;
        ev[u] = bin < bstar;
        if (bin == bstar) ++nb;
      }
      int btot;
      int rank = block_excl_scan<NT>(nb, sh, &btot);
      if (tid < kWave) {
        const int E = lookback(a.sc.estate, blk, 0, btot, a.ws.status);
        if (tid == 0) L.E = E;
      }
      __syncthreads();
      rank += L.E;
#pragma unroll
      for (int u = 0; u < SPT; ++u) {
        const bool evictable = g0 + u < a.n_gpu && !fr[u] && pr[u] < t;
        if (evictable && evict_bin(pr[u], t) == bstar) {
          if (rank < need) ev[u] = true;
          ++rank;
        }
      }
#pragma unroll
      for (int u = 0; u < SPT; ++u)
        if (ev[u]) {
          evict_slot(a, g0 + u);
          fr[u] = true;
        }
    } else {
      // boundary in the clamped bin: exact (priority, slot) select of its slots
#pragma unroll
      for (int u = 0; u < SPT; ++u) {
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
        block_select<NT>(a.sc.ecand_key, a.sc.ecand_idx, c, need, &P, &pos, L.sel_lds);
        for (int i = tid; i < c; i += NT) {
          const uint32_t k = a.sc.ecand_key[i];
          const int32_t g = a.sc.ecand_idx[i];
          if (composite_selected(k, g, P, pos)) evict_slot(a, g);
        }
      }
      if (!grid_sync(&a.sc.misc[M_BAR2], nblk, a.ws.status)) return;
      // no bin lies below bin 0; slots of higher bins stay
#pragma unroll
      for (int u = 0; u < SPT; ++u) {
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
  for (int u = 0; u < SPT; ++u) nf += fr[u] ? 1 : 0;
  int ftot;
  int rank = block_excl_scan<NT>(nf, sh, &ftot);
  if (tid < kWave) {
    const int E = lookback(a.sc.astate, blk, 0, ftot, a.ws.status);
    if (tid == 0) L.E = E;
  }
  __syncthreads();
  const int E = L.E;
  rank += E;
#pragma unroll
  for (int u = 0; u < SPT; ++u) {
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
    for (int r = r0 + tid; r < r1; r += NT) {
      s_rh[r - r0] = __hip_atomic_load(&a.ws.recall_h[r], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
      s_rg[r - r0] = __hip_atomic_load(&a.ws.recall_g[r], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    copy_rows<NT>(a, s_rh, s_rg, r1 - r0);
  } else if (tid == 0) {
    // no recall: count the arrival anyway, since the prefetch copy beside this
    // launch keeps its batches small until the count reaches nblk
    __hip_atomic_fetch_add(&a.sc.misc[M_BAR3], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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


}  // namespace echo
