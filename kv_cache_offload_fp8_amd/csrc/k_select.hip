// Exact selection: top-k per request, and the eviction victims of a layer.
//
// Both are "take the n smallest composite keys (key, index)" problems:
//  - top-k (ECHO review, "Core method / decode": the exact top-k after the
//    indexer): key = ~order(score), so ascending keys are descending scores, and
//    the token index breaks ties toward the lower index;
//  - eviction (review, "Core method / in-graph per-layer cache management":
//    take low-priority slots after protecting the selected tokens): key = the
//    slot's priority (its step of last use), ties toward the lower slot.
// Pass 1 builds a 4096-bin histogram of a monotone bin function of the key in
// LDS, merged into a global histogram with one atomic per non-empty bin and
// workgroup.  Pass 2 finds the bin that holds the n-th key, marks every element
// of lower bins directly, and appends the elements of that bin to a candidate
// list.  A single workgroup then resolves the candidates exactly with an MSD
// radix select on the 64-bit composite (11-bit digits, LDS histograms), which
// stops as soon as the boundary digit's bucket is taken whole.  For top-k the
// bins split the observed key range [min, max] evenly (the scoring kernel
// records the range per request); for eviction, bin = priority - t + 4096
// (clamped), so the last 4095 steps get one bin each.
#include "kernels.h"

namespace echo {

constexpr int kResolveThreads = 1024;

// ------------------------------------------------------- shared pieces

// Boundary bin of a global histogram: the first bin whose inclusive cumulative
// count reaches `need` (1 <= need <= total).  Block of 256 threads, 16 bins each.
__device__ static void find_boundary(const uint32_t *hist, int need, int *s_bin, int *s_below,
                                     int *sh) {
  const int tid = threadIdx.x;
  if (tid == 0) {  // defaults, overwritten by the thread that holds the crossing
    *s_bin = kBins - 1;
    *s_below = 0;
  }
  uint32_t loc[16];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    loc[i] = hist[tid * 16 + i];
    sum += (int)loc[i];
  }
  int tot;
  const int excl = block_excl_scan<256>(sum, sh, &tot);
  if (excl < need && excl + sum >= need) {
    int cum = excl;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (cum < need && cum + (int)loc[i] >= need) {
        *s_bin = tid * 16 + i;
        *s_below = cum;
      }
      cum += (int)loc[i];
    }
  }
  __syncthreads();
}

// MSD radix select of the `need` smallest composites x = (key << 32) | idx among
// `c` candidates (keys and indices in global memory).  On return, candidate x is
// selected iff (x >> *pos) <= *P.  Block of kResolveThreads.
__device__ static void block_select(const uint32_t *ckey, const int32_t *cidx, int c, int need,
                                    uint64_t *P_out, int *pos_out) {
  __shared__ uint32_t s_hist[2048];
  __shared__ int sh[kResolveThreads / kWave + 1];
  __shared__ uint64_t shu[kResolveThreads / kWave];
  __shared__ int s_q, s_below;
  const int tid = threadIdx.x;
  if (need >= c) {  // everything
    *P_out = ~0ull;
    *pos_out = 0;
    return;
  }
  uint64_t mn = ~0ull, mx = 0;
  for (int i = tid; i < c; i += kResolveThreads) {
    const uint64_t x = ((uint64_t)ckey[i] << 32) | (uint32_t)cidx[i];
    mn = x < mn ? x : mn;
    mx = x > mx ? x : mx;
  }
  mn = block_min_u64<kResolveThreads>(mn, shu);
  mx = block_max_u64<kResolveThreads>(mx, shu);
  const uint64_t diff = mn ^ mx;
  int pos = diff ? 64 - __clzll((long long)diff) : 0;
  uint64_t P = pos < 64 ? (mn >> pos) : 0;
  int rem = need;
  while (pos > 0) {
    const int d = pos < 11 ? pos : 11;
    const int npos = pos - d;
    const int nb = 1 << d;
    for (int i = tid; i < 2048; i += kResolveThreads) s_hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < c; i += kResolveThreads) {
      const uint64_t x = ((uint64_t)ckey[i] << 32) | (uint32_t)cidx[i];
      if ((pos >= 64 ? 0 : (x >> pos)) == P)
        atomicAdd(&s_hist[(x >> npos) & (uint64_t)(nb - 1)], 1u);
    }
    __syncthreads();
    const int h0 = (int)s_hist[2 * tid], h1 = (int)s_hist[2 * tid + 1];
    int tot;
    const int excl = block_excl_scan<kResolveThreads>(h0 + h1, sh, &tot);
    if (excl < rem && excl + h0 + h1 >= rem) {
      if (excl + h0 >= rem) {
        s_q = 2 * tid;
        s_below = excl;
      } else {
        s_q = 2 * tid + 1;
        s_below = excl + h0;
      }
    }
    __syncthreads();
    const int q = s_q;
    rem -= s_below;
    P = (P << d) | (uint64_t)q;
    pos = npos;
    const int inbucket = (int)s_hist[q];
    __syncthreads();
    if (inbucket == rem) break;
  }
  *P_out = P;
  *pos_out = pos;
}

__device__ static inline bool composite_selected(uint32_t key, int32_t idx, uint64_t P, int pos) {
  const uint64_t x = ((uint64_t)key << 32) | (uint32_t)idx;
  return (pos >= 64 ? 0 : (x >> pos)) <= P;
}

// ------------------------------------------------------------------ top-k

// True when request b's exact top-k lies among the candidates collected above the
// selection guard while scoring: at least k were found and all of them fit the list.
__device__ static inline bool guard_covers(const StepArgs &a, int b) {
  if (!a.sc.req[b].use_guard) return false;
  return a.sc.gcand_ovf[b] == 0 && a.sc.gcand_n[b] >= a.K;
}

// Key range per request, for callers that pass their own scores.
__global__ __launch_bounds__(256) void k_topk_minmax(StepArgs a) {
  __shared__ uint32_t s_mn[4], s_mx[4];
  if (failed(a.ws.status)) return;
  const int b = blockIdx.y;
  const int ctx = a.sc.req[b].ctx;
  const int c0 = blockIdx.x * kSelChunk;
  if (c0 >= ctx || guard_covers(a, b)) return;
  const float *sc = a.scores_in + (int64_t)b * a.score_stride;
  uint32_t mn = 0xFFFFFFFFu, mx = 0;
  const int end = min(ctx, c0 + kSelChunk);
  for (int s = c0 + threadIdx.x; s < end; s += 256) {
    const uint32_t k = topk_key(sc[s]);
    mn = min(mn, k);
    mx = max(mx, k);
  }
  mn = wave_min_u32(mn);
  mx = wave_max_u32(mx);
  if (lane_id() == 0) {
    s_mn[threadIdx.x / 64] = mn;
    s_mx[threadIdx.x / 64] = mx;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    atomicMin(&a.sc.kmin[b], min(min(s_mn[0], s_mn[1]), min(s_mn[2], s_mn[3])));
    atomicMax(&a.sc.kmax[b], max(max(s_mx[0], s_mx[1]), max(s_mx[2], s_mx[3])));
  }
}

__global__ __launch_bounds__(256) void k_topk_hist(StepArgs a) {
  __shared__ uint32_t h[kBins];
  if (failed(a.ws.status)) return;
  const int b = blockIdx.y;
  const int ctx = a.sc.req[b].ctx;
  const int c0 = blockIdx.x * kSelChunk;
  if (ctx <= a.K || c0 >= ctx || guard_covers(a, b)) return;
  for (int i = threadIdx.x; i < kBins; i += 256) h[i] = 0;
  __syncthreads();
  const uint32_t kmin = a.sc.kmin[b];
  const int shift = bin_shift(kmin, a.sc.kmax[b]);
  const float *sc = a.scores_in + (int64_t)b * a.score_stride;
  const int end = min(ctx, c0 + kSelChunk);
  for (int s = c0 + threadIdx.x; s < end; s += 256)
    atomicAdd(&h[min((topk_key(sc[s]) - kmin) >> shift, (uint32_t)(kBins - 1))], 1u);
  __syncthreads();
  uint32_t *gh = a.sc.thist + (int64_t)b * kBins;
  for (int i = threadIdx.x; i < kBins; i += 256)
    if (h[i]) atomicAdd(&gh[i], h[i]);
}

__global__ __launch_bounds__(256) void k_topk_collect(StepArgs a) {
  __shared__ int sh[8];
  __shared__ int s_bin, s_below;
  if (failed(a.ws.status)) return;
  const int b = blockIdx.y;
  const int ctx = a.sc.req[b].ctx;
  const int c0 = blockIdx.x * kSelChunk;
  if (ctx <= a.K || c0 >= ctx || guard_covers(a, b)) return;
  find_boundary(a.sc.thist + (int64_t)b * kBins, a.K, &s_bin, &s_below, sh);
  const uint32_t bstar = (uint32_t)s_bin;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    a.sc.tbelow[b] = s_below;
    a.sc.tbin[b] = s_bin;
  }
  const uint32_t kmin = a.sc.kmin[b];
  const int shift = bin_shift(kmin, a.sc.kmax[b]);
  const float *sc = a.scores_in + (int64_t)b * a.score_stride;
  uint64_t *bits = (uint64_t *)(a.sc.tbits + (int64_t)b * a.sc.bw);
  const int l = lane_id(), w = threadIdx.x / kWave;
  const int end = min(ctx, c0 + kSelChunk);
  for (int s0 = c0 + w * kWave; s0 < end; s0 += 256) {
    const int s = s0 + l;
    const bool valid = s < end;
    const uint32_t key = valid ? topk_key(sc[s]) : 0u;
    const uint32_t bin = (key - kmin) >> shift;
    const bool take = valid && bin < bstar;
    const bool cand = valid && bin == bstar;
    const uint64_t m = __ballot(take);
    if (l == 0) bits[s0 / 64] = m;
    const uint64_t cm = __ballot(cand);
    if (cm) {
      int basepos = 0;
      if (l == 0) basepos = atomicAdd(&a.sc.tcand_n[b], __popcll(cm));
      basepos = __shfl(basepos, 0);
      if (cand) {
        const int pos = basepos + __popcll(cm & lanemask_lt());
        a.sc.tcand_key[(int64_t)b * a.max_ctx + pos] = key;
        a.sc.tcand_idx[(int64_t)b * a.max_ctx + pos] = s;
      }
    }
  }
}

// Protect the selected tokens of request b (held in LDS) and list its misses in
// token order (review, "Core method / in-graph per-layer cache management":
// recall first looks the selected tokens up in the map).
__device__ static void protect_request(const StepArgs &a, int b, const int32_t *s_sel, int n,
                                       int *sh) {
  const int t = a.ctl[ECHO_CTL_STEP];
  const int base = a.sc.req[b].base;
  int off = 0;
  for (int i0 = 0; i0 < n; i0 += kResolveThreads) {
    const int i = i0 + threadIdx.x;
    const bool valid = i < n && s_sel[i] >= 0;
    int s = 0, g = -1;
    if (valid) {
      s = s_sel[i];
      const int64_t h = (int64_t)base + s;
      if (h >= 0 && h < a.n_host) g = a.h2g[h];
      if (g >= a.n_gpu) g = -1;
      if (g >= 0) a.prio[g] = t;
      a.ws.sel_slot[(int64_t)b * a.K + i] = g;
    }
    const int miss = (valid && g < 0) ? 1 : 0;
    int tot;
    const int pos = off + block_excl_scan<kResolveThreads>(miss, sh, &tot);
    if (miss) {
      a.ws.miss_tok[(int64_t)b * a.K + pos] = s;
      a.sc.miss_i[(int64_t)b * a.K + pos] = i;
    }
    off += tot;
  }
  if (threadIdx.x == 0) {
    a.ws.n_miss[b] = off;
    atomicAdd(&a.ws.counters[ECHO_CNT_MISS], off);
  }
}

template <bool PROTECT>
__global__ __launch_bounds__(kResolveThreads) void k_topk_resolve(StepArgs a) {
  __shared__ int32_t s_sel[4096];
  __shared__ int sh[kResolveThreads / kWave + 1];
  __shared__ uint64_t shu[kResolveThreads / kWave];
  if (failed(a.ws.status)) return;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int ctx = a.sc.req[b].ctx;
  const int K = a.K;
  const int nsel = ctx < K ? ctx : K;
  float kth;
  if (ctx <= K) {
    for (int i = tid; i < ctx; i += kResolveThreads) {
      s_sel[i] = i;
      a.ws.sel_tok[(int64_t)b * K + i] = i;
    }
    kth = ctx > 0 ? score_of_key(a.sc.kmax[b]) : __builtin_nanf("");
  } else {
    uint32_t *bits = a.sc.tbits + (int64_t)b * a.sc.bw;
    const int nwords = (ctx + 31) / 32;
    const uint32_t *ckey;
    const int32_t *cidx;
    int c, need;
    if (guard_covers(a, b)) {  // candidates collected while scoring; nothing marked yet
      // gather the work items' fixed slots into one list
      const ReqInfo r = a.sc.req[b];
      uint32_t *dkey = a.sc.tcand_key + (int64_t)b * a.max_ctx;
      int32_t *didx = a.sc.tcand_idx + (int64_t)b * a.max_ctx;
      const int per = (r.ntiles + kResolveThreads - 1) / kResolveThreads;
      const int t0 = min(r.ntiles, tid * per), t1 = min(r.ntiles, t0 + per);
      int mine = 0;
      for (int ti = t0; ti < t1; ++ti) mine += a.sc.gcand_cnt[r.tile0 + ti];
      int tot;
      int p = block_excl_scan<kResolveThreads>(mine, sh, &tot);
      for (int ti = t0; ti < t1; ++ti) {
        const int tau = r.tile0 + ti;
        const int n = a.sc.gcand_cnt[tau];
        for (int j = 0; j < n; ++j, ++p) {
          dkey[p] = a.sc.gcand_key[(int64_t)tau * kGuardSlots + j];
          didx[p] = a.sc.gcand_idx[(int64_t)tau * kGuardSlots + j];
        }
      }
      __threadfence();
      __syncthreads();
      ckey = dkey;
      cidx = didx;
      c = tot;
      need = K;
      for (int wi = tid; wi < nwords; wi += kResolveThreads) bits[wi] = 0u;
      if (tid == 0) atomicAdd(&a.ws.counters[ECHO_CNT_SHORTCUT], 1);
    } else {  // histogram path: lower bins already marked, boundary bin listed
      ckey = a.sc.tcand_key + (int64_t)b * a.max_ctx;
      cidx = a.sc.tcand_idx + (int64_t)b * a.max_ctx;
      c = a.sc.tcand_n[b];
      need = K - a.sc.tbelow[b];
    }
    uint64_t P;
    int pos;
    block_select(ckey, cidx, c, need, &P, &pos);
    __threadfence();
    __syncthreads();
    uint64_t kmax_sel = 0;
    for (int i = tid; i < c; i += kResolveThreads) {
      const uint32_t k = ckey[i];
      const int32_t s = cidx[i];
      if (composite_selected(k, s, P, pos)) {
        atomicOr(&bits[s >> 5], 1u << (s & 31));
        kmax_sel = k > kmax_sel ? k : kmax_sel;
      }
    }
    kmax_sel = block_max_u64<kResolveThreads>(kmax_sel, shu);
    kth = score_of_key((uint32_t)kmax_sel);
    __threadfence();
    __syncthreads();
    // ordered extraction of the selection bitmap
    const int per = (nwords + kResolveThreads - 1) / kResolveThreads;
    const int w0 = tid * per, w1 = min(nwords, w0 + per);
    int cnt = 0;
    for (int wi = w0; wi < w1; ++wi)
      cnt += __popc(__hip_atomic_load(&bits[wi], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    int tot;
    int p = block_excl_scan<kResolveThreads>(cnt, sh, &tot);
    for (int wi = w0; wi < w1; ++wi) {
      uint32_t x = __hip_atomic_load(&bits[wi], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      while (x) {
        const int bit = __ffs(x) - 1;
        x &= x - 1;
        const int s = wi * 32 + bit;
        if (p < K) {
          s_sel[p] = s;
          a.ws.sel_tok[(int64_t)b * K + p] = s;
        }
        ++p;
      }
    }
  }
  if (tid == 0) {
    a.ws.n_sel[b] = nsel;
    a.ws.kth[b] = kth;
    if (a.theta_upd && ctx >= K && ctx > 0) {
      const float th = a.theta_upd[b];
      const float keep = __fsub_rn(1.0f, a.alpha);
      a.theta_upd[b] = (isinf(th) && th > 0) ? kth
                                              : __fadd_rn(__fmul_rn(a.alpha, kth),
                                                          __fmul_rn(keep, th));
    }
    if (a.guard_upd) a.guard_upd[b] = ctx > K ? kth : __builtin_huge_valf();
  }
  if (PROTECT) {
    __syncthreads();
    protect_request(a, b, s_sel, nsel, sh);
  }
}

__global__ __launch_bounds__(kResolveThreads) void k_protect(StepArgs a) {
  __shared__ int32_t s_sel[4096];
  __shared__ int sh[kResolveThreads / kWave + 1];
  if (failed(a.ws.status)) return;
  const int b = blockIdx.x;
  int n = a.ws.n_sel[b];
  n = n < 0 ? 0 : (n > a.K ? a.K : n);
  for (int i = threadIdx.x; i < n; i += kResolveThreads) {
    int s = a.ws.sel_tok[(int64_t)b * a.K + i];
    s_sel[i] = (s < 0 || s >= a.sc.req[b].ctx) ? -1 : s;
  }
  __syncthreads();
  protect_request(a, b, s_sel, n, sh);
}

hipError_t launch_topk_minmax(const StepArgs &a, hipStream_t s) {
  dim3 grid((a.max_ctx + kSelChunk - 1) / kSelChunk, a.B);
  if (a.B == 0) return hipSuccess;
  hipLaunchKernelGGL(k_topk_minmax, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}
hipError_t launch_topk_hist(const StepArgs &a, hipStream_t s) {
  dim3 grid((a.max_ctx + kSelChunk - 1) / kSelChunk, a.B);
  if (a.B == 0) return hipSuccess;
  hipLaunchKernelGGL(k_topk_hist, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}
hipError_t launch_topk_collect(const StepArgs &a, hipStream_t s) {
  dim3 grid((a.max_ctx + kSelChunk - 1) / kSelChunk, a.B);
  if (a.B == 0) return hipSuccess;
  hipLaunchKernelGGL(k_topk_collect, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}
hipError_t launch_topk_resolve(const StepArgs &a, bool protect, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  if (protect)
    hipLaunchKernelGGL(k_topk_resolve<true>, dim3(a.B), dim3(kResolveThreads), 0, s, a);
  else
    hipLaunchKernelGGL(k_topk_resolve<false>, dim3(a.B), dim3(kResolveThreads), 0, s, a);
  return hipGetLastError();
}
hipError_t launch_protect(const StepArgs &a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  hipLaunchKernelGGL(k_protect, dim3(a.B), dim3(kResolveThreads), 0, s, a);
  return hipGetLastError();
}

// --------------------------------------------------------------- eviction

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

__global__ __launch_bounds__(256) void k_evict_hist(StepArgs a) {
  __shared__ uint32_t h[kBins];
  __shared__ int s_free[4], s_ev[4];
  if (failed(a.ws.status)) return;
  const int t = a.ctl[ECHO_CTL_STEP];
  for (int i = threadIdx.x; i < kBins; i += 256) h[i] = 0;
  __syncthreads();
  const int g0 = blockIdx.x * kSlotTile;
  const int end = min(a.n_gpu, g0 + kSlotTile);
  int nfree = 0, nev = 0;
  for (int g = g0 + threadIdx.x; g < end; g += 256) {
    if (a.freef[g]) {
      ++nfree;
    } else {
      const int p = a.prio[g];
      if (p < t) {
        ++nev;
        atomicAdd(&h[evict_bin(p, t)], 1u);
      }
    }
  }
  nfree = wave_sum(nfree);
  nev = wave_sum(nev);
  if (lane_id() == 0) {
    s_free[threadIdx.x / 64] = nfree;
    s_ev[threadIdx.x / 64] = nev;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kBins; i += 256)
    if (h[i]) atomicAdd(&a.sc.ehist[i], h[i]);
  if (threadIdx.x == 0) {
    atomicAdd(&a.ws.counters[ECHO_CNT_FREE], s_free[0] + s_free[1] + s_free[2] + s_free[3]);
    atomicAdd(&a.ws.counters[ECHO_CNT_EVICTABLE], s_ev[0] + s_ev[1] + s_ev[2] + s_ev[3]);
  }
}

// n_evict = min(|E|, max(0, misses + reserve - free)); capacity error if
// free + |E| < misses.  Lower bins are evicted here, the boundary bin is listed.
__device__ static inline int evict_count(const StepArgs &a, bool *cap_err) {
  const int nmiss = a.ws.counters[ECHO_CNT_MISS];
  const int nfree = a.ws.counters[ECHO_CNT_FREE];
  const int nE = a.ws.counters[ECHO_CNT_EVICTABLE];
  const int64_t want = (int64_t)nmiss + a.sc.misc[M_RESERVE] - nfree;
  *cap_err = (int64_t)nfree + nE < nmiss;
  const int64_t w = want < 0 ? 0 : want;
  return (int)(w < nE ? w : nE);
}

__global__ __launch_bounds__(256) void k_evict_collect(StepArgs a) {
  __shared__ int sh[8];
  __shared__ int s_bin, s_below;
  if (failed(a.ws.status)) return;
  bool cap_err;
  const int nev = evict_count(a, &cap_err);
  if (cap_err) {
    if (threadIdx.x == 0) fail(a.ws.status, ECHO_ECAPACITY);
    return;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) a.ws.counters[ECHO_CNT_EVICT] = nev;
  if (nev == 0) return;
  find_boundary(a.sc.ehist, nev, &s_bin, &s_below, sh);
  const int bstar = s_bin;
  if (blockIdx.x == 0 && threadIdx.x == 0) a.sc.ecnt[1] = s_below;
  const int t = a.ctl[ECHO_CTL_STEP];
  const int g0 = blockIdx.x * kSlotTile;
  const int end = min(a.n_gpu, g0 + kSlotTile);
  const int l = lane_id();
  for (int gb = g0 + (threadIdx.x / kWave) * kWave; gb < end; gb += 256) {
    const int g = gb + l;
    bool cand = false;
    int p = 0;
    if (g < end && !a.freef[g]) {
      p = a.prio[g];
      if (p < t) {
        const int bin = evict_bin(p, t);
        if (bin < bstar)
          evict_slot(a, g);
        else if (bin == bstar)
          cand = true;
      }
    }
    const uint64_t cm = __ballot(cand);
    if (cm) {
      int basepos = 0;
      if (l == 0) basepos = atomicAdd(&a.sc.ecnt[0], __popcll(cm));
      basepos = __shfl(basepos, 0);
      if (cand) {
        const int pos = basepos + __popcll(cm & lanemask_lt());
        a.sc.ecand_key[pos] = (uint32_t)p;
        a.sc.ecand_idx[pos] = g;
      }
    }
  }
}

__global__ __launch_bounds__(kResolveThreads) void k_evict_resolve(StepArgs a) {
  if (failed(a.ws.status)) return;
  const int nev = a.ws.counters[ECHO_CNT_EVICT];
  const int need = nev - a.sc.ecnt[1];
  const int c = a.sc.ecnt[0];
  if (nev <= 0 || need <= 0) return;
  uint64_t P;
  int pos;
  block_select(a.sc.ecand_key, a.sc.ecand_idx, c, need, &P, &pos);
  for (int i = threadIdx.x; i < c; i += kResolveThreads) {
    const uint32_t k = a.sc.ecand_key[i];
    const int32_t g = a.sc.ecand_idx[i];
    if (composite_selected(k, g, P, pos)) evict_slot(a, g);
  }
}

hipError_t launch_evict_hist(const StepArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(k_evict_hist, dim3(a.sc.atiles), dim3(256), 0, s, a);
  return hipGetLastError();
}
hipError_t launch_evict_collect(const StepArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(k_evict_collect, dim3(a.sc.atiles), dim3(256), 0, s, a);
  return hipGetLastError();
}
hipError_t launch_evict_resolve(const StepArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(k_evict_resolve, dim3(1), dim3(kResolveThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace echo
