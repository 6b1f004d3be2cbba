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
constexpr int kCopyRowsStoppable = 2;  // rows per batch of a wave that hands over

// Copy the n (1 <= n <= 64) rows whose host id / slot lanes 0..n-1 hold, 8 KB
// at a time: eight 16-byte host reads per lane in flight, then the eight HBM
// writes, non-temporal: the rows are not read again in the step, and dirty lines
// left in L2 would lengthen the write-back of every device-scope fence that the
// selection and management workgroups make meanwhile (measured: the capacity
// decode step 0.6% shorter).  No load or store sits under a branch (the compiler would wait for
// each one before the next): a lane past the last piece reads and writes the
// last piece again, the same bytes to the same place.
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
      d = (int64_t)gg * cpr + (cc - e * cpr);                            \
      v = src[(int64_t)hh * cpr + (cc - e * cpr)];                       \
    }
    ECHO_COPY_LOAD(0, v0, d0) ECHO_COPY_LOAD(1, v1, d1) ECHO_COPY_LOAD(2, v2, d2)
    ECHO_COPY_LOAD(3, v3, d3) ECHO_COPY_LOAD(4, v4, d4) ECHO_COPY_LOAD(5, v5, d5)
    ECHO_COPY_LOAD(6, v6, d6) ECHO_COPY_LOAD(7, v7, d7)
#undef ECHO_COPY_LOAD
    __builtin_nontemporal_store(v0, &dst[d0]);
    __builtin_nontemporal_store(v1, &dst[d1]);
    __builtin_nontemporal_store(v2, &dst[d2]);
    __builtin_nontemporal_store(v3, &dst[d3]);
    __builtin_nontemporal_store(v4, &dst[d4]);
    __builtin_nontemporal_store(v5, &dst[d5]);
    __builtin_nontemporal_store(v6, &dst[d6]);
    __builtin_nontemporal_store(v7, &dst[d7]);
  }
}

// What a copy wave reads before a batch, in one round trip: the stop and slow
// counters, the entries of the block's ranks not yet copied (lane l: rank
// r0 + done + l) and the request's final count.
struct CopyView {
  int sv, sl;
  uint64_t e, fin;
};

__device__ inline CopyView copy_view(const StepArgs &a, const int32_t *stop, int b, int r0,
                                     int done, const int32_t *slow = nullptr) {
  const int lane = lane_id();
  const int rank = r0 + done + lane;
  const bool mine = lane < kCopyRows - done && rank < a.K;
  const int r_any = r0 + done < a.K ? r0 + done : a.K - 1;
  CopyView v;
  v.sv = 0;
  v.sl = 0x7FFFFFFF;
  if (stop) v.sv = __hip_atomic_load(stop, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (slow) v.sl = __hip_atomic_load(slow, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // every lane loads (lanes past the block reread its first entry): no branch
  v.e = __hip_atomic_load(&a.sc.pfq[(int64_t)b * a.K + (mine ? rank : r_any)], __ATOMIC_RELAXED,
                          __HIP_MEMORY_SCOPE_AGENT);
  v.e = mine ? v.e : 0;
  v.fin = __hip_atomic_load(&a.sc.pfn[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return v;
}

// Copy wave `w` of NW (= a.copy_waves), as part `q` of `m` waves that share its
// blocks (blocks i_cur + q, i_cur + q + m, ...; part 0 resumes the saved partial
// block).  With `stop` set, the wave leaves before its next batch once *stop
// reaches `stop_target`, saving its progress (m must be 1); otherwise it copies
// every row it owns.  With `slow` set, batches stay as small as a stoppable
// wave's while *slow is below `slow_target` (fewer host reads in flight while
// latency-bound work runs beside the copy).  A batch that completes its block
// reads the next block's entries before its own host reads, so that round trip
// overlaps the copy; a complete block is left without reading it again.  The stop
// counter is read again after such a batch, since a batch can outlast the stop by
// several microseconds (the host-link queue): with the value read before it, a
// wave took one more batch, and the kernel ended up to 18 us after its scoring
// workgroups (now about 10).  The loop keeps to register
// arithmetic otherwise (block -> request and rank stepped without division, each
// request's cap in a lane register): a batch is about one host-link round trip.
__device__ inline void copy_worker(const StepArgs &a, const ReqInfo *req, int w, int q, int m,
                                   const int32_t *stop, int stop_target,
                                   const int32_t *slow = nullptr, int slow_target = 0) {
  const int lane = lane_id();
  w = __builtin_amdgcn_readfirstlane(w);  // one wave, one copy worker
  const int NW = a.copy_waves, B = a.B;
  const int nbk = (a.K + kCopyRows - 1) / kCopyRows;
  const int nblocks = B * nbk;  // B <= 64 and K <= 4096 (host checks): no overflow
  // lane b: the ranks request b may fill this step (0 if it prefetches nothing)
  const int lcap = lane < B ? (req[lane].active ? req[lane].cap : 0) : 0;
  int32_t *st = a.sc.cstate + 2 * w;
  int i = st[0] + q;
  int done = q == 0 ? st[1] : 0;  // ranks of the current block already copied
  // block x = w + i * NW is ranks r0 = (x / B) * kCopyRows.. of request b = x % B;
  // a step of m blocks adds m * NW to x
  int x = w + i * NW;
  int b = x % B, g = x / B;
  const int step = m * NW, db = step % B, dg = step / B;
  auto advance = [&]() {
    i += m;
    x += step;
    b += db;
    g += dg;
    if (b >= B) {
      b -= B;
      ++g;
    }
  };
  uint64_t t0 = 0;  // start of the current wait for entries (0: not waiting)
  int nap = 1;  // polls back off while nothing is ready: idle waves must not flood memory
  bool ahead = false;  // `view` already holds block i's entries (read during the last batch)
  CopyView view = {0, 0x7FFFFFFF, 0, 0};
  while (x < nblocks) {
    const int r0 = g * kCopyRows;
    if (r0 >= __builtin_amdgcn_readlane(lcap, b)) {
      advance();
      done = 0;
      ahead = false;
      continue;
    }
    if (!ahead) view = copy_view(a, stop, b, r0, done, slow);
    else if (stop) view.sv = __hip_atomic_load(stop, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    ahead = false;
    if (stop && view.sv >= stop_target) {
      if (lane == 0) {  // hand the rest to the next kernel of the step
        st[0] = i;
        st[1] = done;
      }
      return;
    }
    int need = kCopyRows;  // ranks of this block the request fills
    if (view.fin >> 32) need = max(0, min(kCopyRows, (int)(uint32_t)view.fin - r0));
    if (done >= need) {
      advance();
      done = 0;
      continue;
    }
    const uint64_t have = __ballot(lane < kCopyRows - done && (view.e >> 63) != 0);
    // A wave that may be told to stop takes at most two rows at a time: its reads
    // then finish soon after the stop, and the copy keeps few host reads in flight
    // (host reads in flight slow the scoring waves' HBM stream on every compute
    // unit, not only their own).
    const int ready = min(min(__ffsll((unsigned long long)~have) - 1, need - done),
                          (stop || view.sl < slow_target) ? kCopyRowsStoppable : kCopyRows);
    if (ready > 0) {
      const int rank = r0 + done + lane;
      const int cb = b, d0 = done;
      const int my_h = lane < ready ? (int)((view.e >> 31) & 0x7FFFFFFFull) : 0;
      const int my_g = lane < ready ? (int)(view.e & 0x7FFFFFFFull) : 0;
      done += ready;
      if (done >= need) {  // block complete (need < kCopyRows only once the count is final)
        advance();
        done = 0;
        if (x < nblocks) {
          view = copy_view(a, stop, b, g * kCopyRows, 0, slow);
          ahead = true;
        }
      }
      copy_batch(a, my_h, my_g, ready);
      // consumed: clear the entries, so the list is empty again at the end of the
      // step (lanes past them clear the first one again, without a branch)
      __hip_atomic_store(&a.sc.pfq[(int64_t)cb * a.K + (lane < ready ? rank : r0 + d0)], 0ull,
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      t0 = 0;
      nap = 1;
      continue;
    }
    if (t0 == 0) t0 = wall_clock64();
    for (int z = 0; z < nap; ++z) __builtin_amdgcn_s_sleep(8);  // 512 cycles each
    nap = nap < 8 ? 2 * nap : 8;
    if (failed(a.ws.status)) return;
    if ((long long)(wall_clock64() - t0) > kSpinLimit) {
      if (lane == 0) fail(a.ws.status, ECHO_ETIMEOUT);
      return;
    }
  }
  if (stop && lane == 0) {  // everything owned is copied
    st[0] = i;
    st[1] = 0;
  }
}

}  // namespace echo
