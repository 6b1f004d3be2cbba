// Decode append: the step's new token joins each request's context.
//
// The ECHO review ("Core method / in-graph per-layer cache management") keeps the
// indexer K resident on the GPU and backs every token's KV up to the host pool
// when it is generated, which is why eviction never copies data back; its
// "Design trade-offs" section counts that writeback (every new token) as the
// price of the full host copy.  Per layer and request this kernel writes the new
// token's indexer key into the tiled K at host id host_base + ctx and its latent
// into the mapped host pool at the same id; with `advance` it then grows
// ctx_len by one (once per decode step, after the last layer).  With a page table
// the new token's host id comes from the page its request lists for it (the caller
// hands out pages; distinct pages per request are the admission's check).  The token is not
// placed in the GPU pool: it becomes resident like any other token, when the
// threshold prefetch or the exact recall selects it.
#include "kernels.h"

namespace echo {

constexpr int kAppendThreads = 1024;

__global__ __launch_bounds__(kAppendThreads) void k_append(StepArgs a, const uint8_t *k_new,
                                                           const uint16_t *lat_new,
                                                           int32_t *ctx_io, int advance) {
  __shared__ int32_t s_ctx[kMaxBatch], s_base[kMaxBatch];
  __shared__ int64_t s_h[kMaxBatch];  // the new token's host id
  __shared__ int s_bad;
  const int tid = threadIdx.x;
  const int32_t st0 = __hip_atomic_load(a.ws.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (tid < a.B) {
    s_ctx[tid] = ctx_io[tid];
    s_base[tid] = a.pages ? 0 : a.host_base[tid];
  }
  if (tid == 0) s_bad = 0;
  __syncthreads();
  if (st0 != 0) return;
  // Checks, lane b for request b: room below max_ctx and n_host, no collision with
  // another request's range (counting that request's own new token), and a host id
  // that no slot maps yet.  The lowest failing request decides the status.  A row
  // with ctx 0 is empty (released or never admitted): it is not checked, takes no
  // token, and its stale host_base blocks nobody.
  if (tid < kWave) {
    int code = 0;
    const int s = tid < a.B ? s_ctx[tid] : 0;
    int64_t h = -1;
    if (tid < a.B && s != 0) {
      if (s < 0 || s >= a.max_ctx) {
        code = ECHO_ECAPACITY;
      } else if (a.pages) {
        // the page the request lists for its new token: in the table and in the pool
        const int32_t p = (s >> 4) < a.page_stride
                              ? a.pages[(int64_t)tid * a.page_stride + (s >> 4)] : -1;
        if (!page_in_pool(a, p)) code = ECHO_ECAPACITY;
        else h = 16LL * p + (s & 15);
      } else {
        h = (int64_t)s_base[tid] + s;
        if (s_base[tid] < 0 || h >= a.n_host) code = ECHO_ECAPACITY;
        // another live request's range, counting its own new token
        for (int o = 0; o < a.B && code == 0; ++o)
          if (o != tid && s_ctx[o] != 0 && h >= s_base[o] && h < (int64_t)s_base[o] + s_ctx[o] + 1)
            code = ECHO_ECAPACITY;
      }
      if (code == 0 && a.h2g[h] != -1) code = ECHO_EDEVARG;
    }
    if (tid < a.B) s_h[tid] = h;
    const uint64_t bad = __ballot(code != 0);
    if (bad) {
      const int c = __shfl(code, __ffsll((unsigned long long)bad) - 1);
      if (tid == 0) {
        fail(a.ws.status, c);
        s_bad = 1;
      }
    }
  }
  __syncthreads();
  if (s_bad) return;
  // the keys, one byte per thread, at their place in the tiled layout
  uint8_t *kidx = const_cast<uint8_t *>(a.kidx);
  const int D = a.D;
  for (int i = tid; i < a.B * D; i += kAppendThreads) {
    const int b = i / D, d = i - b * D;
    if (s_ctx[b] == 0) continue;
    const int64_t h = s_h[b];
    const int64_t off = 16LL * D * (h >> 4) + 8LL * D * ((d & 31) >> 4) + 256LL * (d >> 5) +
                        16 * (h & 15) + (d & 15);
    kidx[off] = k_new[i];
  }
  // the latents, 16 bytes per thread, into mapped host memory
  const int cpr = a.latent * 2 / 16;
  const uint4 *src = (const uint4 *)lat_new;
  uint4 *dst = (uint4 *)const_cast<uint16_t *>(a.host_kv);
  for (int i = tid; i < a.B * cpr; i += kAppendThreads) {
    const int b = i / cpr, c = i - b * cpr;
    if (s_ctx[b] == 0) continue;
    const int64_t h = s_h[b];
    dst[h * cpr + c] = src[i];
  }
  if (advance && tid < a.B && s_ctx[tid] != 0) ctx_io[tid] = s_ctx[tid] + 1;
}

hipError_t launch_append(const StepArgs &a, const uint8_t *k_new, const uint16_t *lat_new,
                         int32_t *ctx_io, int advance, hipStream_t s) {
  hipLaunchKernelGGL(k_append, dim3(1), dim3(kAppendThreads), 0, s, a, k_new, lat_new, ctx_io,
                     advance);
  return hipGetLastError();
}

}  // namespace echo
