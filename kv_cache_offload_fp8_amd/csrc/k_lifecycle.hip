// Request lifecycle: release (cancel) and admission between decode steps.
//
// The ECHO review lists request cancellation among what the paper leaves open
// ("Systemic flaws") and asks that top-k and attention input stay equal to the
// no-offload baseline when requests are cancelled ("Limitations and future
// work").  With the per-layer state of "Core method / in-graph per-layer cache
// management", releasing request b means: every token of its host range that
// holds a GPU slot gives it back (g2h = -1, free = 1, priority = -1), the range's
// host-to-GPU map rows become -1, its EMA threshold returns to "no estimate"
// and its context becomes empty.  No bytes move: the host copy of every token
// stays where it is.  The ascending free list that the next step's prefetch
// hands out is rebuilt from the free flags.  Admission puts a new request into
// an empty batch row after checking its host range against the live requests
// and the map.
#include "kernels.h"

namespace echo {

constexpr int kReleaseThreads = 256;
constexpr int kReleaseBlocksX = 64;  // workgroups per released request

// Every workgroup checks every masked request (the same data, so every
// workgroup reaches the same verdict); the first one reports it.
__global__ __launch_bounds__(kReleaseThreads) void k_release_free(StepArgs a,
                                                                  const int32_t *mask) {
  __shared__ int s_bad;
  const int tid = threadIdx.x;
  const int32_t st0 = __hip_atomic_load(a.ws.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (tid < kWave) {
    bool bad = false;
    if (tid < a.B && mask[tid]) {
      const int32_t n = a.ctx_len[tid], hb = a.host_base[tid];
      bad = n < 0 || n > a.max_ctx || hb < 0 || (int64_t)hb + n > a.n_host;
    }
    const uint64_t any = __ballot(bad);
    if (tid == 0) {
      s_bad = any != 0;
      if (any && blockIdx.x == 0 && blockIdx.y == 0 && st0 == 0) fail(a.ws.status, ECHO_EDEVARG);
    }
  }
  __syncthreads();
  if (st0 != 0 || s_bad) return;
  const int b = blockIdx.y;
  if (!mask[b]) return;
  const int64_t base = a.host_base[b];
  const int32_t n = a.ctx_len[b];
  for (int32_t s = blockIdx.x * kReleaseThreads + tid; s < n;
       s += kReleaseBlocksX * kReleaseThreads) {
    const int64_t h = base + s;
    const int32_t g = a.h2g[h];
    if (g >= 0 && g < a.n_gpu) {
      a.g2h[g] = -1;
      a.freef[g] = 1;
      a.prio[g] = -1;
    }
    a.h2g[h] = -1;
  }
}

// After the slots are back: thresholds, empty rows (with `commit`: the batch
// row is shared by the layers and is emptied with the last), and the ascending free list
// (idxbuf[0 .. nfree)) rebuilt by a block scan over the free flags.
__global__ __launch_bounds__(kListThreads) void k_release_finish(StepArgs a, const int32_t *mask,
                                                                 int32_t *ctx_io, int commit) {
  __shared__ int sh[kListThreads / kWave + 1];
  if (failed(a.ws.status)) return;  // also set by k_release_free's range check
  const int tid = threadIdx.x;
  if (tid < a.B && mask[tid]) {
    a.theta[tid] = __builtin_huge_valf();
    if (a.guard) a.guard[tid] = __builtin_huge_valf();
    if (commit) ctx_io[tid] = 0;
  }
  rebuild_free_list(a, sh);
}

hipError_t launch_release(const StepArgs &a, const int32_t *mask, int32_t *ctx_io, int commit,
                          hipStream_t s) {
  hipLaunchKernelGGL(k_release_free, dim3(kReleaseBlocksX, a.B), dim3(kReleaseThreads), 0, s, a,
                     mask);
  hipLaunchKernelGGL(k_release_finish, dim3(1), dim3(kListThreads), 0, s, a, mask, ctx_io,
                     commit);
  return hipGetLastError();
}

// Admission of request b with host range [base, base + len) (checked on the host
// against n_host and max_ctx).  Checks, in this order: the row is empty
// (EDEVARG otherwise), no live request's range meets the new one (ECAPACITY),
// no token of the range is mapped (EDEVARG).  Nothing is written on an error;
// otherwise the threshold resets and, with `commit`, the batch row is written.
__global__ __launch_bounds__(kListThreads) void k_admit(StepArgs a, int b, int32_t base,
                                                        int32_t len, int32_t *hb_io,
                                                        int32_t *ctx_io, int commit) {
  __shared__ int s_code;
  if (failed(a.ws.status)) return;
  const int tid = threadIdx.x;
  if (tid < kWave) {
    int code = 0;  // lane o: does request o block the admission?
    if (tid < a.B) {
      const int32_t n = ctx_io[tid];
      if (tid == b) {
        if (n != 0) code = ECHO_EDEVARG;
      } else if (n > 0) {
        const int64_t lo = hb_io[tid], hi = lo + n;
        if ((int64_t)base < hi && lo < (int64_t)base + len) code = ECHO_ECAPACITY;
      }
    }
    // the row check comes first, then overlaps
    const uint64_t row = __ballot(tid == b && code != 0);
    const uint64_t ovl = __ballot(code != 0);
    if (tid == 0) s_code = row ? ECHO_EDEVARG : (ovl ? ECHO_ECAPACITY : 0);
  }
  __syncthreads();
  int code = s_code;
  if (code == 0) {
    int stale = 0;
    for (int32_t s = tid; s < len; s += kListThreads) stale |= a.h2g[(int64_t)base + s] != -1;
    if (__syncthreads_or(stale)) code = ECHO_EDEVARG;
  }
  if (tid != 0) return;
  if (code != 0) {
    fail(a.ws.status, code);
    return;
  }
  if (commit) {
    hb_io[b] = base;
    ctx_io[b] = len;
  }
  a.theta[b] = __builtin_huge_valf();
  if (a.guard) a.guard[b] = __builtin_huge_valf();
}

hipError_t launch_admit(const StepArgs &a, int b, int32_t base, int32_t len, int32_t *hb_io,
                        int32_t *ctx_io, int commit, hipStream_t s) {
  hipLaunchKernelGGL(k_admit, dim3(1), dim3(kListThreads), 0, s, a, b, base, len, hb_io, ctx_io,
                     commit);
  return hipGetLastError();
}

}  // namespace echo
