// Prefetch-row copy shared by the indexer, top-k and management kernels
// (internal).
//
// The indexer publishes every prefetched row by rank as a self-validating 64-bit
// entry (1 << 63 | host id << 31 | slot, relaxed device-scope atomics), and each
// request's last work item publishes its final count.  The copy wave that
// consumes an entry clears it, so the list is all zero again when the step ends
// (and after echo_ws_reset), without a bulk clear per step.  Copy waves read the rows from mapped host memory into the GPU pool.
// Wave w of the NW copy waves owns the 4-rank blocks x = w + i*NW (block x is
// ranks 4*(x / B) .. +3 of request x % B), in increasing i: small blocks spread
// the rows that are ready at any moment over many waves.  Inside a layer
// step the copy is spread over the step's kernels: the indexer's and the top-k
// kernel's copy waves stop once their kernel's own workgroups are done and save
// (i, ranks done) per wave; the next kernel's copy waves resume from there, and
// the management kernel's finish everything.  Host reads then use the host link
// during selection and management too, not only during scoring, and they never
// run on a compute unit that streams K (host reads issued from a compute unit
// hold up that unit's HBM loads).
#pragma once

#include "kernels.h"

namespace echo {

typedef int v4i_c __attribute__((ext_vector_type(4)));

constexpr int kCopyLoads = 8;  // 16-byte loads in flight per lane per round (unrolled below)
constexpr int kCopyRowsStoppable = 4;  // rows per batch of a wave that hands over

// Copy the n <= 64 rows whose host id / slot lanes 0..n-1 hold, 8 KB at a time:
// eight 16-byte host reads per lane in flight, then the eight HBM writes.
__device__ inline void copy_batch(const StepArgs &a, int my_h, int my_g, int n) {
  const int lane = lane_id();
  const int cpr = a.latent * 2 / 16;
  const v4i_c *src = (const v4i_c *)a.host_kv;
  v4i_c *dst = (v4i_c *)a.gpu_kv;
  const int nchunks = n * cpr;
  for (int c0 = 0; c0 < nchunks; c0 += kCopyLoads * kWave) {
    v4i_c v0, v1, v2, v3, v4, v5, v6, v7;
    int64_t d0, d1, d2, d3, d4, d5, d6, d7;
    // chunk u of this lane: host offset (row h, piece c) -> pool offset (slot g, piece c)
#define ECHO_COPY_LOAD(u, v, d)                                          \
    {                                                                    \
      const int ci = c0 + (u) * kWave + lane;                            \
      const int cc = ci < nchunks ? ci : nchunks - 1;                    \
      const int e = cc / cpr;                                            \
      const int hh = __shfl(my_h, e), gg = __shfl(my_g, e);              \
      d = ci < nchunks ? (int64_t)gg * cpr + (cc - e * cpr) : -1;        \
      if (ci < nchunks) v = src[(int64_t)hh * cpr + (cc - e * cpr)];     \
    }
    ECHO_COPY_LOAD(0, v0, d0) ECHO_COPY_LOAD(1, v1, d1) ECHO_COPY_LOAD(2, v2, d2)
    ECHO_COPY_LOAD(3, v3, d3) ECHO_COPY_LOAD(4, v4, d4) ECHO_COPY_LOAD(5, v5, d5)
    ECHO_COPY_LOAD(6, v6, d6) ECHO_COPY_LOAD(7, v7, d7)
#undef ECHO_COPY_LOAD
    if (d0 >= 0) dst[d0] = v0;
    if (d1 >= 0) dst[d1] = v1;
    if (d2 >= 0) dst[d2] = v2;
    if (d3 >= 0) dst[d3] = v3;
    if (d4 >= 0) dst[d4] = v4;
    if (d5 >= 0) dst[d5] = v5;
    if (d6 >= 0) dst[d6] = v6;
    if (d7 >= 0) dst[d7] = v7;
  }
}

// Copy wave `w` of NW (= a.copy_waves), as part `q` of `m` waves that share its
// blocks (blocks i_cur + q, i_cur + q + m, ...; part 0 resumes the saved partial
// block).  With `stop` set, the wave leaves before its next batch once *stop
// reaches `stop_target`, saving its progress (m must be 1); otherwise it copies
// every row it owns.
__device__ inline void copy_worker(const StepArgs &a, const ReqInfo *req, int w, int q, int m,
                                   const int32_t *stop, int stop_target) {
  const int lane = lane_id();
  const int NW = a.copy_waves;
  const int nbk = (a.K + kCopyRows - 1) / kCopyRows;
  const int64_t nblocks = (int64_t)a.B * nbk;
  int32_t *st = a.sc.cstate + 2 * w;
  int i = st[0] + q;
  int done = q == 0 ? st[1] : 0;  // ranks of the current block already copied
  for (; (int64_t)w + (int64_t)i * NW < nblocks; i += m, done = 0) {
    const int64_t x = (int64_t)w + (int64_t)i * NW;
    const int b = (int)(x % a.B), r0 = (int)(x / a.B) * kCopyRows;
    const ReqInfo &r = req[b];
    if (!r.active || r0 >= r.cap) continue;
    uint64_t t0 = wall_clock64();
    int nap = 1;  // polls back off while nothing is ready: idle waves must not flood memory
    while (true) {
      if (stop && __hip_atomic_load(stop, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >=
                      stop_target) {
        if (lane == 0) {  // hand the rest to the next kernel of the step
          st[0] = i;
          st[1] = done;
        }
        return;
      }
      const int rank = r0 + done + lane;
      uint64_t e = 0;
      if (lane < kCopyRows - done && rank < a.K)
        e = __hip_atomic_load(&a.sc.pfq[(int64_t)b * a.K + rank], __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT);
      const uint64_t fin =
          __hip_atomic_load(&a.sc.pfn[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      int need = kCopyRows;  // ranks of this block the request fills
      if (fin >> 32) need = max(0, min(kCopyRows, (int)(uint32_t)fin - r0));
      if (done >= need) break;
      const uint64_t have = __ballot(lane < kCopyRows - done && (e >> 63) != 0);
      // A wave that may be told to stop takes at most four rows at a time: its reads
      // then finish soon after the stop even with the link saturated (512 waves x
      // 4 rows in flight still cover the link's latency).
      const int ready = min(min(__ffsll((unsigned long long)~have) - 1, need - done),
                            stop ? kCopyRowsStoppable : kCopyRows);
      if (ready > 0) {
        const int my_h = lane < ready ? (int)((e >> 31) & 0x7FFFFFFFull) : 0;
        const int my_g = lane < ready ? (int)(e & 0x7FFFFFFFull) : 0;
        copy_batch(a, my_h, my_g, ready);
        // consumed: clear the entry, so the list is empty again at the end of the step
        if (lane < ready)
          __hip_atomic_store(&a.sc.pfq[(int64_t)b * a.K + rank], 0ull, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        done += ready;
        t0 = wall_clock64();
        nap = 1;
        continue;
      }
      for (int z = 0; z < nap; ++z) __builtin_amdgcn_s_sleep(8);  // 512 cycles each
      nap = nap < 8 ? 2 * nap : 8;
      if (failed(a.ws.status)) return;
      if ((long long)(wall_clock64() - t0) > kSpinLimit) {
        if (lane == 0) fail(a.ws.status, ECHO_ETIMEOUT);
        return;
      }
    }
  }
  if (stop && lane == 0) {  // everything owned is copied
    st[0] = i;
    st[1] = 0;
  }
}

}  // namespace echo
