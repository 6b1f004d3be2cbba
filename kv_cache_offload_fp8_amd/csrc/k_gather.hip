// Attention input: the latents of every request's selected tokens, gathered from
// the GPU pool in selection order.
//
// The ECHO review ("Core method / decode") runs the sparse attention only after
// the exact top-k and the recall of every missing selected token: losslessness
// means the attention reads exactly the rows it would read with no offloading.
// This kernel produces that input, out[b][i] = gpu_kv[sel_slot[b][i]] for
// i < n_sel[b] and zero rows after, in the dense [B][k][latent] layout a sparse
// attention kernel takes.  It streams HBM: 2 x 1152 B per selected token (pool
// read, output write), eight 16-byte pieces per thread in flight, with enough
// workgroups that each thread makes one round (the slot lookups, then the row
// reads: two round trips), and no load or store under a branch.  (Measured on
// 65,536 rows: 24.9 us with eight pieces, 26.2 us with four in two or three
// rounds, 25.8 and 30.6 us with twelve and sixteen.)
#include "kernels.h"

namespace echo {

constexpr int kGatherBlocks = 4096;
constexpr int kGatherPieces = 8;  // 16-byte pieces per thread per round, all in flight

__global__ __launch_bounds__(256) void k_gather(StepArgs a, uint16_t *out) {
  if (failed(a.ws.status)) return;
  typedef int v4 __attribute__((ext_vector_type(4)));
  const int cpr = a.latent * 2 / 16;
  const int64_t rows = (int64_t)a.B * a.K;
  const int64_t total = rows * cpr;
  const v4 *src = (const v4 *)a.gpu_kv;
  v4 *dst = (v4 *)out;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i0 = (int64_t)blockIdx.x * 256 + threadIdx.x; i0 < total;
       i0 += kGatherPieces * stride) {
    v4 v[kGatherPieces];
    int64_t d[kGatherPieces];
#pragma unroll
    for (int u = 0; u < kGatherPieces; ++u) {
      // pieces past the end repeat the last piece (same bytes, same place)
      const int64_t i = i0 + u * stride < total ? i0 + u * stride : total - 1;
      const int64_t row = i / cpr;
      const int c = (int)(i - row * cpr);
      const int b = (int)(row / a.K), r = (int)(row - (int64_t)b * a.K);
      const int g = a.ws.sel_slot[row];
      const bool ok = r < a.ws.n_sel[b] && g >= 0 && g < a.n_gpu;
      const v4 x = src[(int64_t)(ok ? g : 0) * cpr + c];
      const v4 z = {0, 0, 0, 0};
      v[u] = ok ? x : z;
      d[u] = i;
    }
#pragma unroll
    for (int u = 0; u < kGatherPieces; ++u) dst[d[u]] = v[u];
  }
}

hipError_t launch_gather(const StepArgs &a, uint16_t *out, hipStream_t s) {
  const int64_t total = (int64_t)a.B * a.K * (a.latent * 2 / 16);
  // enough workgroups for one round per thread: the slot lookups and the row reads
  // then each take one round trip
  int64_t grid = (total + kGatherPieces * 256 - 1) / (kGatherPieces * 256);
  if (grid > kGatherBlocks) grid = kGatherBlocks;
  if (grid < 1) return hipSuccess;
  hipLaunchKernelGGL(k_gather, dim3((unsigned)grid), dim3(256), 0, s, a, out);
  return hipGetLastError();
}

}  // namespace echo
