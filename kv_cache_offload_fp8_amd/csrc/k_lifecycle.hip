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
// and the map.  With a page table a request's tokens live on pages of 16 host
// ids anywhere in the pool: release walks its tokens through the table (the
// pages stay the caller's to hand out again) and admission checks that the new
// request's pages lie in the pool, are listed once and belong to no live request
// (a bitmap over the pool's pages), which is what lets a new request fill the
// holes that released ones leave.
#include "kernels.h"

namespace echo {

constexpr int kReleaseThreads = 256;
constexpr int kReleaseBlocksX = 64;  // workgroups per released request
constexpr int kCheckGrid = 64;       // workgroups of the page checks

// Every masked request's tokens must fit: its context in [0, max_ctx] and its
// range in the pool, or (page table) its pages in the table and in the pool.  Any
// failure sets ECHO_EDEVARG, which turns the rest of the release into a no-op.
__global__ __launch_bounds__(kReleaseThreads) void k_release_check(StepArgs a,
                                                                   const int32_t *mask) {
  if (failed(a.ws.status)) return;
  const int tid = threadIdx.x;
  bool bad = false;
  if (blockIdx.x == 0 && tid < a.B && mask[tid]) {
    const int32_t n = a.ctx_len[tid];
    if (n < 0 || n > a.max_ctx) bad = true;
    else if (a.pages) bad = (n + 15) / 16 > a.page_stride;
    else bad = a.host_base[tid] < 0 || (int64_t)a.host_base[tid] + n > a.n_host;
  }
  if (a.pages) {
    const int64_t total = (int64_t)a.B * a.page_stride;
    for (int64_t i = (int64_t)blockIdx.x * kReleaseThreads + tid; i < total;
         i += (int64_t)gridDim.x * kReleaseThreads) {
      const int b = (int)(i / a.page_stride);
      const int j = (int)(i - (int64_t)b * a.page_stride);
      const int32_t n = a.ctx_len[b];
      if (mask[b] && n > 0 && n <= a.max_ctx && j < (n + 15) / 16 && !page_in_pool(a, a.pages[i]))
        bad = true;
    }
  }
  if (bad) fail(a.ws.status, ECHO_EDEVARG);
}

__global__ __launch_bounds__(kReleaseThreads) void k_release_free(StepArgs a,
                                                                  const int32_t *mask) {
  if (failed(a.ws.status)) return;  // an earlier error, or what k_release_check found
  const int tid = threadIdx.x;
  const int b = blockIdx.y;
  if (!mask[b]) return;
  const int32_t base = a.pages ? 0 : a.host_base[b];
  const int32_t n = a.ctx_len[b];
  for (int32_t s = blockIdx.x * kReleaseThreads + tid; s < n;
       s += kReleaseBlocksX * kReleaseThreads) {
    const int64_t h = token_host(a, b, base, s);
    const int32_t g = a.h2g[h];
    if (g >= 0 && g < a.n_gpu) {
      a.g2h[g] = -1;
      a.freef[g] = 1;
      a.prio[g] = -1;
    }
    a.h2g[h] = -1;
  }
}

// After the slots are back: thresholds and empty rows (with `commit`: the batch
// row is shared by the layers and is emptied with the last).
__global__ void k_release_finish(StepArgs a, const int32_t *mask, int32_t *ctx_io, int commit) {
  if (failed(a.ws.status)) return;  // also set by k_release_free's range check
  const int tid = threadIdx.x;
  if (tid < a.B && mask[tid]) {
    a.theta[tid] = __builtin_huge_valf();
    if (a.guard) a.guard[tid] = __builtin_huge_valf();
    if (commit) ctx_io[tid] = 0;
  }
}

// The ascending free list (idxbuf[0 .. nfree)) rebuilt from the free flags, because
// the next step's prefetch hands out idxbuf[off + rank]: one 1024-thread workgroup
// per slot tile of kSlotTile slots (4 per thread).  k_free_count stores each tile's
// free count; k_free_write sums the counts of the tiles before its own, ranks its
// free slots with a block scan and writes them; the last tile writes nfree.  (One
// workgroup scanning all 110,000 slots took about 41 us; two launches of 27 take a
// few.)
constexpr int kFreeThreads = 1024;
constexpr int kFreeSpt = kSlotTile / kFreeThreads;

__global__ __launch_bounds__(kFreeThreads) void k_free_count(StepArgs a) {
  __shared__ int sh[kFreeThreads / kWave + 1];
  if (failed(a.ws.status)) return;
  const int64_t g0 = (int64_t)blockIdx.x * kSlotTile + (int64_t)threadIdx.x * kFreeSpt;
  int n = 0;
#pragma unroll
  for (int u = 0; u < kFreeSpt; ++u)
    if (g0 + u < a.n_gpu && a.freef[g0 + u]) ++n;
  int tot;
  block_excl_scan<kFreeThreads>(n, sh, &tot);
  if (threadIdx.x == 0) ((int32_t *)a.sc.astate)[blockIdx.x] = tot;
}

__global__ __launch_bounds__(kFreeThreads) void k_free_write(StepArgs a) {
  __shared__ int sh[kFreeThreads / kWave + 1];
  if (failed(a.ws.status)) return;
  const int tid = threadIdx.x, blk = blockIdx.x;
  const int32_t *cnt = (const int32_t *)a.sc.astate;
  int before = 0;  // free slots in the tiles before this one
  for (int i = tid; i < blk; i += kFreeThreads) before += cnt[i];
  int total_before;
  block_excl_scan<kFreeThreads>(before, sh, &total_before);
  const int64_t g0 = (int64_t)blk * kSlotTile + (int64_t)tid * kFreeSpt;
  bool fr[kFreeSpt];
  int n = 0;
#pragma unroll
  for (int u = 0; u < kFreeSpt; ++u) {
    fr[u] = g0 + u < a.n_gpu && a.freef[g0 + u] != 0;
    n += fr[u] ? 1 : 0;
  }
  int tot;
  int r = total_before + block_excl_scan<kFreeThreads>(n, sh, &tot);
#pragma unroll
  for (int u = 0; u < kFreeSpt; ++u)
    if (fr[u]) a.idxbuf[r++] = (int32_t)(g0 + u);
  if (blk == (int)gridDim.x - 1 && tid == 0) a.ctl[ECHO_CTL_NFREE] = total_before + tot;
}

hipError_t launch_release(const StepArgs &a, const int32_t *mask, int32_t *ctx_io, int commit,
                          hipStream_t s) {
  hipLaunchKernelGGL(k_release_check, dim3(kCheckGrid), dim3(kReleaseThreads), 0, s, a, mask);
  hipLaunchKernelGGL(k_release_free, dim3(kReleaseBlocksX, a.B), dim3(kReleaseThreads), 0, s, a,
                     mask);
  hipLaunchKernelGGL(k_release_finish, dim3(1), dim3(kMaxBatch), 0, s, a, mask, ctx_io, commit);
  hipLaunchKernelGGL(k_free_count, dim3(a.sc.atiles), dim3(kFreeThreads), 0, s, a);
  hipLaunchKernelGGL(k_free_write, dim3(a.sc.atiles), dim3(kFreeThreads), 0, s, a);
  return hipGetLastError();
}

// Admission with a page table, before k_admit: the row is empty (EDEVARG
// otherwise), the new tokens need at most page_stride pages (EDEVARG), and the
// page bitmap is cleared.
__global__ __launch_bounds__(kListThreads) void k_admit_pages_begin(StepArgs a, int b, int32_t len,
                                                                    const int32_t *ctx_io) {
  if (failed(a.ws.status)) return;
  const int tid = threadIdx.x;
  if (tid == 0 && (ctx_io[b] != 0 || (len + 15) / 16 > a.page_stride))
    fail(a.ws.status, ECHO_EDEVARG);
  const int64_t words = (a.n_host / 16 + 31) / 32;
  for (int64_t i = tid; i < words; i += kListThreads) a.sc.pgbits[i] = 0;
}

// The new request's pages: each in the pool and listed once (EDEVARG), marked in
// the bitmap.
__global__ __launch_bounds__(kReleaseThreads) void k_admit_pages_mark(StepArgs a, int b,
                                                                      int32_t len) {
  if (failed(a.ws.status)) return;
  const int np = (len + 15) / 16;
  bool bad = false;
  for (int j = blockIdx.x * kReleaseThreads + threadIdx.x; j < np;
       j += gridDim.x * kReleaseThreads) {
    const int32_t p = a.pages[(int64_t)b * a.page_stride + j];
    if (!page_in_pool(a, p)) {
      bad = true;
    } else {
      const uint32_t bit = 1u << (p & 31);
      if (atomicOr(&a.sc.pgbits[p >> 5], bit) & bit) bad = true;  // listed twice
    }
  }
  if (bad) fail(a.ws.status, ECHO_EDEVARG);
}

// No page of a live request's tokens is one of the new request's (ECAPACITY).
__global__ __launch_bounds__(kReleaseThreads) void k_admit_pages_overlap(StepArgs a, int b,
                                                                         const int32_t *ctx_io) {
  if (failed(a.ws.status)) return;
  const int64_t total = (int64_t)a.B * a.page_stride;
  bool hit = false;
  for (int64_t i = (int64_t)blockIdx.x * kReleaseThreads + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * kReleaseThreads) {
    const int o = (int)(i / a.page_stride);
    const int j = (int)(i - (int64_t)o * a.page_stride);
    const int32_t n = ctx_io[o];
    if (o == b || n <= 0 || j >= (n + 15) / 16) continue;
    const int32_t p = a.pages[i];
    if (page_in_pool(a, p) && ((a.sc.pgbits[p >> 5] >> (p & 31)) & 1u)) hit = true;
  }
  if (hit) fail(a.ws.status, ECHO_ECAPACITY);
}

// Admission of request b with len tokens: the host range [base, base + len)
// (checked on the host against n_host and max_ctx), or the pages of row b of the
// page table (checked by the three kernels above).  Checks here, in this order:
// without a page table, the row is empty (EDEVARG otherwise) and no live request's
// range meets the new one (ECAPACITY); in both cases, no new token is mapped
// (EDEVARG).  Nothing is written on an error; otherwise the threshold resets and,
// with `commit`, the batch row is written.
__global__ __launch_bounds__(kListThreads) void k_admit(StepArgs a, int b, int32_t base,
                                                        int32_t len, int32_t *hb_io,
                                                        int32_t *ctx_io, int commit) {
  __shared__ int s_code;
  if (failed(a.ws.status)) return;
  const int tid = threadIdx.x;
  if (tid < kWave) {
    int code = 0;  // lane o: does request o block the admission?
    if (!a.pages && tid < a.B) {
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
    for (int32_t s = tid; s < len; s += kListThreads)
      stale |= a.h2g[token_host(a, b, base, s)] != -1;
    if (__syncthreads_or(stale)) code = ECHO_EDEVARG;
  }
  if (tid != 0) return;
  if (code != 0) {
    fail(a.ws.status, code);
    return;
  }
  if (commit) {
    if (!a.pages) hb_io[b] = base;
    ctx_io[b] = len;
  }
  a.theta[b] = __builtin_huge_valf();
  if (a.guard) a.guard[b] = __builtin_huge_valf();
}

hipError_t launch_admit(const StepArgs &a, int b, int32_t base, int32_t len, int32_t *hb_io,
                        int32_t *ctx_io, int commit, hipStream_t s) {
  if (a.pages) {
    hipLaunchKernelGGL(k_admit_pages_begin, dim3(1), dim3(kListThreads), 0, s, a, b, len, ctx_io);
    hipLaunchKernelGGL(k_admit_pages_mark, dim3(kCheckGrid), dim3(kReleaseThreads), 0, s, a, b,
                       len);
    hipLaunchKernelGGL(k_admit_pages_overlap, dim3(kCheckGrid), dim3(kReleaseThreads), 0, s, a,
                       b, ctx_io);
  }
  hipLaunchKernelGGL(k_admit, dim3(1), dim3(kListThreads), 0, s, a, b, base, len, hb_io, ctx_io,
                     commit);
  return hipGetLastError();
}

}  // namespace echo
