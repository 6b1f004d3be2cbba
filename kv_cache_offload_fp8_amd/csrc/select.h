// Block-level selection primitives shared by the top-k and eviction kernels
// (internal).  Every function is called by all NT threads of a block (1024 in the
// top-k, management and prefill kernels, 512 in the fused layer-step kernel), and
// takes its shared memory from the caller, so that a kernel whose workgroups
// change roles can lay the roles' memory over each other.
#pragma once

#include "kernels.h"

namespace echo {

constexpr int kSelThreads = 1024;
constexpr int kMaxSelWaves = kSelThreads / kWave;  // per-wave slots of the block reductions

// Shared memory of block_select_by.
struct SelectLds {
  uint32_t hist[2048];
  int sh[kMaxSelWaves + 1];
  uint64_t shu[kMaxSelWaves];
  int q, below;
};

// First bin of a kBins histogram whose inclusive cumulative count reaches `need`
// (1 <= need <= total) and the count below it.  ATOMIC: read the bins with
// device-scope atomic loads (a histogram other workgroups updated in this launch).
template <bool ATOMIC, int NT = kSelThreads>
__device__ inline void find_boundary(const uint32_t *hist, int need, int *s_bin, int *s_below,
                                     int *sh) {
  constexpr int PER = kBins / NT;
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
  const int excl = block_excl_scan<NT>(sum, sh, &tot);
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
template <int NT, class Get>
__device__ inline void block_select_by(Get get, int c, int need, uint64_t *P_out, int *pos_out,
                                       SelectLds &L) {
  constexpr int PERB = 2048 / NT;  // digit bins per thread in the scan
  const int tid = threadIdx.x;
  if (need >= c) {  // everything
    *P_out = ~0ull;
    *pos_out = 0;
    return;
  }
  uint64_t mn = ~0ull, mx = 0;
  for (int i = tid; i < c; i += NT) {
    const uint64_t x = get(i);
    mn = x < mn ? x : mn;
    mx = x > mx ? x : mx;
  }
  mn = block_min_u64<NT>(mn, L.shu);
  mx = block_max_u64<NT>(mx, L.shu);
  const uint64_t diff = mn ^ mx;
  int pos = diff ? 64 - __clzll((long long)diff) : 0;
  uint64_t P = pos < 64 ? (mn >> pos) : 0;
  int rem = need;
  while (pos > 0) {
    const int d = pos < 11 ? pos : 11;
    const int npos = pos - d;
    const int nb = 1 << d;
    for (int i = tid; i < 2048; i += NT) L.hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < c; i += NT) {
      const uint64_t x = get(i);
      if ((pos >= 64 ? 0 : (x >> pos)) == P)
        atomicAdd(&L.hist[(x >> npos) & (uint64_t)(nb - 1)], 1u);
    }
    __syncthreads();
    int h[PERB], hs = 0;
#pragma unroll
    for (int u = 0; u < PERB; ++u) {
      h[u] = (int)L.hist[PERB * tid + u];
      hs += h[u];
    }
    int tot;
    const int excl = block_excl_scan<NT>(hs, L.sh, &tot);
    if (excl < rem && excl + hs >= rem) {
      int cum = excl;
#pragma unroll
      for (int u = 0; u < PERB; ++u) {
        if (cum < rem && cum + h[u] >= rem) {
          L.q = PERB * tid + u;
          L.below = cum;
        }
        cum += h[u];
      }
    }
    __syncthreads();
    const int q = L.q;
    rem -= L.below;
    P = (P << d) | (uint64_t)q;
    pos = npos;
    const int inbucket = (int)L.hist[q];
    __syncthreads();
    if (inbucket == rem) break;
  }
  *P_out = P;
  *pos_out = pos;
}

// The same over keys and indices in global memory.
template <int NT = kSelThreads>
__device__ inline void block_select(const uint32_t *ckey, const int32_t *cidx, int c, int need,
                                    uint64_t *P_out, int *pos_out, SelectLds &L) {
  block_select_by<NT>([=](int i) { return ((uint64_t)ckey[i] << 32) | (uint32_t)cidx[i]; }, c,
                      need, P_out, pos_out, L);
}

__device__ inline bool composite_selected(uint32_t key, int32_t idx, uint64_t P, int pos) {
  const uint64_t x = ((uint64_t)key << 32) | (uint32_t)idx;
  return (pos >= 64 ? 0 : (x >> pos)) <= P;
}

}  // namespace echo
