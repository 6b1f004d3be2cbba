// Block-level selection primitives shared by the top-k and eviction kernels
// (internal).  Every function is called by all threads of a 1024-thread block.
#pragma once

#include "kernels.h"

namespace echo {

constexpr int kSelThreads = 1024;

// First bin of a kBins histogram whose inclusive cumulative count reaches `need`
// (1 <= need <= total) and the count below it.  ATOMIC: read the bins with
// device-scope atomic loads (a histogram other workgroups updated in this launch).
template <bool ATOMIC>
__device__ inline void find_boundary(const uint32_t *hist, int need, int *s_bin, int *s_below,
                                     int *sh) {
  constexpr int PER = kBins / kSelThreads;
  const int tid = threadIdx.x;
  if (tid == 0) {  // defaults, overwritten by the thread that holds the crossing
    *s_bin = kBins - 1;
    *s_below = 0;
  }
  uint32_t loc[PER];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const uint32_t *p = hist + tid * PER + i;
    loc[i] = ATOMIC ? __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : *p;
    sum += (int)loc[i];
  }
  int tot;
  const int excl = block_excl_scan<kSelThreads>(sum, sh, &tot);
  if (excl < need && excl + sum >= need) {
    int cum = excl;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (cum < need && cum + (int)loc[i] >= need) {
        *s_bin = tid * PER + i;
        *s_below = cum;
      }
      cum += (int)loc[i];
    }
  }
  __syncthreads();
}

// MSD radix select of the `need` smallest composites x = (key << 32) | idx among
// `c` candidates, candidate i being get(i) (unique composites).  On return,
// candidate x is selected iff (x >> *pos) <= *P.
template <class Get>
__device__ inline void block_select_by(Get get, int c, int need, uint64_t *P_out, int *pos_out) {
  __shared__ uint32_t s_hist[2048];
  __shared__ int sh[kSelThreads / kWave + 1];
  __shared__ uint64_t shu[kSelThreads / kWave];
  __shared__ int s_q, s_below;
  const int tid = threadIdx.x;
  if (need >= c) {  // everything
    *P_out = ~0ull;
    *pos_out = 0;
    return;
  }
  uint64_t mn = ~0ull, mx = 0;
  for (int i = tid; i < c; i += kSelThreads) {
    const uint64_t x = get(i);
    mn = x < mn ? x : mn;
    mx = x > mx ? x : mx;
  }
  mn = block_min_u64<kSelThreads>(mn, shu);
  mx = block_max_u64<kSelThreads>(mx, shu);
  const uint64_t diff = mn ^ mx;
  int pos = diff ? 64 - __clzll((long long)diff) : 0;
  uint64_t P = pos < 64 ? (mn >> pos) : 0;
  int rem = need;
  while (pos > 0) {
    const int d = pos < 11 ? pos : 11;
    const int npos = pos - d;
    const int nb = 1 << d;
    for (int i = tid; i < 2048; i += kSelThreads) s_hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < c; i += kSelThreads) {
      const uint64_t x = get(i);
      if ((pos >= 64 ? 0 : (x >> pos)) == P)
        atomicAdd(&s_hist[(x >> npos) & (uint64_t)(nb - 1)], 1u);
    }
    __syncthreads();
    const int h0 = (int)s_hist[2 * tid], h1 = (int)s_hist[2 * tid + 1];
    int tot;
    const int excl = block_excl_scan<kSelThreads>(h0 + h1, sh, &tot);
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

// The same over keys and indices in global memory.
__device__ inline void block_select(const uint32_t *ckey, const int32_t *cidx, int c, int need,
                                    uint64_t *P_out, int *pos_out) {
  block_select_by([=](int i) { return ((uint64_t)ckey[i] << 32) | (uint32_t)cidx[i]; }, c, need,
                  P_out, pos_out);
}

__device__ inline bool composite_selected(uint32_t key, int32_t idx, uint64_t P, int pos) {
  const uint64_t x = ((uint64_t)key << 32) | (uint32_t)idx;
  return (pos >= 64 ? 0 : (x >> pos)) <= P;
}

}  // namespace echo
