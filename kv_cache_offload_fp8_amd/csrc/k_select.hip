// Top-k and protection kernels (the per-request body is in topk.h).
#include "topk.h"

namespace echo {

template <bool PROTECT>
__global__ __launch_bounds__(kSelThreads) void k_topk(StepArgs a) {
  // the status is looked at after the first reads are issued (one round trip)
  const int32_t st0 = __hip_atomic_load(a.ws.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if ((int)blockIdx.x >= a.B) {  // copy workgroup: prefetched rows, until selection ends
    if (st0 != 0) return;
    copy_worker(a, a.sc.req,
                ((int)blockIdx.x - a.B) * (kSelThreads / kWave) + (int)threadIdx.x / kWave, 0, 1,
                &a.sc.misc[M_TOPK_DONE], a.B);
    return;
  }
  __shared__ TopkLds L;
  topk_block<PROTECT>(a, blockIdx.x, st0, L);
}

__global__ __launch_bounds__(kSelThreads) void k_protect(StepArgs a) {
  __shared__ int32_t s_sel[4096];
  __shared__ int sh[kSelThreads / kWave + 1];
  if (failed(a.ws.status)) return;
  const int b = blockIdx.x;
  int n = a.ws.n_sel[b];
  n = n < 0 ? 0 : (n > a.K ? a.K : n);
  for (int i = threadIdx.x; i < n; i += kSelThreads) {
    int s = a.ws.sel_tok[(int64_t)b * a.K + i];
    s_sel[i] = (s < 0 || s >= a.sc.req[b].ctx) ? -1 : s;
  }
  __syncthreads();
  protect_request(a, b, s_sel, n, sh);
}

hipError_t launch_topk(const StepArgs &a, bool protect, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  // copy workgroups continue the indexer's prefetch copy (one wave per copy wave)
  const int extra = a.copy_handoff ? a.copy_waves / (kSelThreads / kWave) : 0;
  const dim3 grid(a.B + extra);
  if (protect)
    hipLaunchKernelGGL(k_topk<true>, grid, dim3(kSelThreads), 0, s, a);
  else
    hipLaunchKernelGGL(k_topk<false>, grid, dim3(kSelThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_protect(const StepArgs &a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  hipLaunchKernelGGL(k_protect, dim3(a.B), dim3(kSelThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace echo
