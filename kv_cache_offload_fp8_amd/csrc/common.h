// Internal device primitives and the workspace layout shared by the kernels.
// Nothing here is part of the public ABI (include/echo.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "echo.h"

namespace echo {

// ----------------------------------------------------------------- sizes
constexpr int kWave = 64;
constexpr int kHeadsPad = 64;     // indexer heads padded to 4 groups of 16 (MFMA rows)
constexpr int kDimPad = 128;      // indexer dim padded to one 16x16x128 fp8 MFMA k-step
constexpr int kScoreTile = 256;   // tokens per scoring work item (one wave, 4 x 64)
constexpr int kGuardSlots = 32;   // selection-guard candidates kept per work item
constexpr int kScoreWaves = 8;    // waves per indexer workgroup (scoring or copying)
constexpr int kCopyBlocks = 64;   // indexer workgroups that only copy prefetched rows
constexpr int kCopyRows = 4;      // prefetch ranks a copy wave takes at a time
constexpr uint32_t kGuardUlps = 1u << 18;  // selection guard margin: ~3% below last k-th score
constexpr int kBins = 4096;       // first-level histogram bins
constexpr int kSelChunk = 8192;   // tokens per block in the top-k histogram/collect passes
constexpr int kSlotTile = 4096;   // slots per block in the eviction and allocation passes
constexpr int kMaxBatch = 64;
constexpr long long kSpinLimit = 100000000LL;  // 1 s of the 100 MHz constant clock

// internal counters (Scratch::misc)
enum {
  M_SLOTS = 0,        // scoring jobs (sum over requests of their waves)
  M_TOTAL_TILES = 2,  // scoring work items of the batch
  M_RESERVE = 3,      // sum of the prefetch caps
  M_BAR0 = 4,         // grid-barrier arrival counters of the management kernel
  M_BAR1 = 5,
  M_BAR2 = 6,
  M_DONE = 7,         // management workgroups finished
  M_BAR3 = 8,
  M_SCORE_DONE = 9,   // indexer scoring workgroups finished (copy hand-off)
  M_TOPK_DONE = 10,   // top-k workgroups finished (copy hand-off)
  M_NMISC = 16
};

// lookback state: flag in the high word, value in the low word
constexpr uint64_t kFlagA = 1ull << 32;  // aggregate of this tile only
constexpr uint64_t kFlagP = 2ull << 32;  // inclusive prefix

struct ReqInfo {
  int32_t ctx;     // context length (0 if the request's arguments were rejected)
  int32_t base;    // first host id (a multiple of 16)
  int32_t cap;     // prefetch cap min(k, ceil(ctx/div))
  int32_t off;     // sum of earlier caps: first free-list position of this request
  int32_t tile0;   // first scoring work item of this request
  int32_t ntiles;  // scoring work items of this request
  int32_t active;  // prefetch enabled for this request in this step
  float theta;     // prefetch threshold
  int32_t use_guard;   // collect selection candidates with key <= guard_key
  uint32_t guard_key;  // top-k key of (last k-th score - margin), saturated
  int32_t wb;      // scoring waves given to this request
  int32_t slot0;   // first scoring job of this request
  int32_t pad[4];
};

// Carved internal scratch.  Every region starts 256-byte aligned.
struct Scratch {
  uint8_t *qhi, *qlo;     // [max_batch][64][128] fp8 split of the scaled query, zero-padded
  float *wsc;             // [max_batch][64] head weights / query scale, zero-padded
  ReqInfo *req;           // [max_batch]
  int32_t *misc;          // [M_NMISC]
  uint64_t *tstate;       // [max_tiles] scoring look-back states
  uint32_t *tcand_key;    // [max_batch][max_ctx] boundary-bin candidates of the top-k
  int32_t *tcand_idx;     // [max_batch][max_ctx]
  uint32_t *tbits;        // [max_batch][bw] selection bitmap
  uint32_t *gcand_key;    // [max_tiles][kGuardSlots] candidates above the selection guard
  int32_t *gcand_idx;     // [max_tiles][kGuardSlots]
  int32_t *gcand_cnt;     // [max_tiles] candidates found in each work item
  uint64_t *pfq;          // [max_batch][top_k] prefetch rows by rank: 1<<63 | h<<31 | slot
  uint64_t *pfn;          // [max_batch] 1<<32 | prefetched count, once final
  int32_t *cstate;        // [kCopyBlocks * kScoreWaves][2] copy-wave progress (block, done)
  int32_t *miss_i;        // [max_batch][top_k] position of each miss in sel_tok
  uint32_t *ehist;        // [kBins]
  uint32_t *ecand_key;    // [n_gpu]
  int32_t *ecand_idx;     // [n_gpu]
  int32_t *ecnt;          // [4]: candidates of the rare exact eviction path
  uint64_t *estate;       // [alloc tiles] eviction-rank look-back states
  uint64_t *astate;       // [alloc tiles] free-list look-back states
  uint32_t *pgbits;       // [n_host / 512] one bit per host page (admission with pages)
  int32_t max_tiles, bw, atiles, pad_;
};

inline int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

// Lays out the internal scratch for `d`; with base == nullptr only measures it.
inline int64_t scratch_layout(const echo_dims_t &d, uint8_t *base, Scratch *s) {
  int64_t off = 0;
  auto take = [&](int64_t bytes) -> uint8_t * {
    uint8_t *p = base ? base + off : nullptr;
    off = align256(off + bytes);
    return p;
  };
  const int64_t B = d.max_batch, C = d.max_ctx, K = d.top_k, G = d.n_gpu;
  const int32_t max_tiles = (int32_t)(B * ((C + kScoreTile - 1) / kScoreTile));
  const int32_t bw = (int32_t)((C + 63) / 64 * 2);  // whole 64-bit groups
  const int32_t atiles = (int32_t)((G + kSlotTile - 1) / kSlotTile);
  Scratch t;
  t.qhi = take(B * kHeadsPad * kDimPad);
  t.qlo = take(B * kHeadsPad * kDimPad);
  t.wsc = (float *)take(B * kHeadsPad * 4);
  t.req = (ReqInfo *)take(B * sizeof(ReqInfo));
  t.misc = (int32_t *)take(M_NMISC * 4);
  t.tstate = (uint64_t *)take((int64_t)max_tiles * 8);
  t.tcand_key = (uint32_t *)take(B * C * 4);
  t.tcand_idx = (int32_t *)take(B * C * 4);
  t.tbits = (uint32_t *)take(B * bw * 4);
  t.gcand_key = (uint32_t *)take((int64_t)max_tiles * kGuardSlots * 4);
  t.gcand_idx = (int32_t *)take((int64_t)max_tiles * kGuardSlots * 4);
  t.gcand_cnt = (int32_t *)take((int64_t)max_tiles * 4);
  t.pfq = (uint64_t *)take(B * K * 8);
  t.pfn = (uint64_t *)take(B * 8);
  t.cstate = (int32_t *)take(2 * kCopyBlocks * kScoreWaves * 4);
  t.miss_i = (int32_t *)take(B * K * 4);
  t.ehist = (uint32_t *)take(kBins * 4);
  t.ecand_key = (uint32_t *)take(G * 4);
  t.ecand_idx = (int32_t *)take(G * 4);
  t.ecnt = (int32_t *)take(16);
  t.estate = (uint64_t *)take((int64_t)atiles * 8);
  t.astate = (uint64_t *)take((int64_t)atiles * 8);
  t.pgbits = (uint32_t *)take((d.n_host / 16 + 31) / 32 * 4);
  t.max_tiles = max_tiles;
  t.bw = bw;
  t.atiles = atiles;
  t.pad_ = 0;
  if (s) *s = t;
  return off;
}

// ------------------------------------------------------------- status
__device__ inline bool failed(const int32_t *status) {
  return __hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
}
__device__ inline void fail(int32_t *status, int code) {
  int expected = 0;
  __hip_atomic_compare_exchange_strong(status, &expected, code, __ATOMIC_RELAXED,
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------- wave / block
__device__ inline int lane_id() { return threadIdx.x & (kWave - 1); }
__device__ inline uint64_t lanemask_lt() { return (1ull << lane_id()) - 1ull; }

// v summed over the four lanes l, l^16, l^32, l^48, returned in all four: first
// the pairs 16 apart, then 32 apart.  gfx950's lane-swap instructions do the
// exchange in the vector ALU (v_permlane16_swap swaps rows 1 and 3 of its first
// operand with rows 0 and 2 of its second, v_permlane32_swap the upper half of
// the first with the lower half of the second; with both operands v, the two
// results hold v and its partner in every lane), where a cross-lane shuffle
// goes through the LDS crossbar and waits for its return.
__device__ inline float sum_lane_groups16(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float v16 = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
  const uint32_t w = __float_as_uint(v16);
  const auto r32 = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
}

__device__ inline int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ inline uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o));
  return v;
}
__device__ inline uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
  return v;
}
__device__ inline uint64_t wave_min_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint64_t x = __shfl_xor(v, o);
    v = x < v ? x : v;
  }
  return v;
}
__device__ inline uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint64_t x = __shfl_xor(v, o);
    v = x > v ? x : v;
  }
  return v;
}
__device__ inline int wave_incl_scan(int v) {
  const int l = lane_id();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int x = __shfl_up(v, o);
    if (l >= o) v += x;
  }
  return v;
}

// Exclusive block scan of one int per thread.  `sh` needs NT/64 + 1 ints of
// shared memory.  Returns the exclusive prefix; *total receives the block sum.
template <int NT>
__device__ inline int block_excl_scan(int v, int *sh, int *total) {
  constexpr int NW = NT / kWave;
  const int l = lane_id(), w = threadIdx.x / kWave;
  int incl = wave_incl_scan(v);
  if (l == kWave - 1) sh[w] = incl;
  __syncthreads();
  if (w == 0) {
    int x = l < NW ? sh[l] : 0;
    int xs = wave_incl_scan(x);
    if (l < NW) sh[l] = xs - x;
    if (l == NW - 1) sh[NW] = xs;
  }
  __syncthreads();
  int r = sh[w] + incl - v;
  *total = sh[NW];
  __syncthreads();
  return r;
}

template <int NT>
__device__ inline uint64_t block_min_u64(uint64_t v, uint64_t *sh) {
  constexpr int NW = NT / kWave;
  v = wave_min_u64(v);
  if (lane_id() == 0) sh[threadIdx.x / kWave] = v;
  __syncthreads();
  uint64_t r = sh[0];
  for (int i = 1; i < NW; ++i) r = sh[i] < r ? sh[i] : r;
  __syncthreads();
  return r;
}
template <int NT>
__device__ inline uint64_t block_max_u64(uint64_t v, uint64_t *sh) {
  constexpr int NW = NT / kWave;
  v = wave_max_u64(v);
  if (lane_id() == 0) sh[threadIdx.x / kWave] = v;
  __syncthreads();
  uint64_t r = sh[0];
  for (int i = 1; i < NW; ++i) r = sh[i] > r ? sh[i] : r;
  __syncthreads();
  return r;
}

// ------------------------------------------------------ decoupled look-back
// Called by one whole wave.  Work item `tau` of a segment that starts at item
// `seg0` publishes its own count `c` (lb_publish; the segment's first item
// publishes it as its inclusive prefix), and later walks back over earlier items
// of the same segment (aggregates until an inclusive prefix is found), publishes
// its inclusive prefix and gets its exclusive prefix (lb_resolve).  A caller may
// do other work between the two calls, so that the items before it have
// published by the time it resolves.  Callers guarantee that every earlier item
// is owned by a resident wave that publishes it without waiting on a later item,
// so the wait always ends; a 1 s guard turns a broken invariant into
// ECHO_ETIMEOUT instead of a hang.  Only the state words cross workgroups, as
// relaxed device-scope atomics: no cache flush is needed.
__device__ inline void lb_publish(uint64_t *st, int tau, int seg0, int c) {
  if (lane_id() == 0)
    __hip_atomic_store(&st[tau], (tau == seg0 ? kFlagP : kFlagA) | (uint32_t)c, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// Second half of the look-back: item `tau` (whose count `c` lb_publish has
// published) sums the aggregates of the items before it back to the nearest
// inclusive prefix, publishes its own inclusive prefix and returns the exclusive
// one.  Only the states up to that nearest prefix are waited for.
__device__ inline int lb_resolve(uint64_t *st, int tau, int seg0, int c, int32_t *status) {
  if (tau == seg0) return 0;
  const int l = lane_id();
  int E = 0;
  int j = tau - 1;
  const uint64_t t0 = wall_clock64();
  bool timed_out = false;
  while (true) {
    const int idx = j - l;
    uint64_t v = idx >= seg0 ? __hip_atomic_load(&st[idx], __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT)
                             : kFlagP;
    uint64_t pm;
    while (true) {
      const uint64_t fm = __ballot((v >> 32) != 0);
      pm = __ballot((v >> 32) == 2);
      // lanes that matter: up to the nearest inclusive prefix, or all of them
      const uint64_t need = pm ? ((pm & (0 - pm)) << 1) - 1 : ~0ull;
      if ((fm & need) == need) break;
      if (((v >> 32) == 0) && ((need >> l) & 1ull))
        v = __hip_atomic_load(&st[idx], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (__any((long long)(wall_clock64() - t0) > kSpinLimit) || failed(status)) {
        timed_out = true;  // or another workgroup already failed: stop waiting
        break;
      }
    }
    if (timed_out) break;
    const int val = (int)(uint32_t)v;
    if (pm) {
      const int first = __ffsll((unsigned long long)pm) - 1;
      E += wave_sum(l <= first ? val : 0);
      break;
    }
    E += wave_sum(val);
    j -= kWave;
  }
  if (timed_out) {
    if (l == 0) fail(status, ECHO_ETIMEOUT);
  }
  if (l == 0)
    __hip_atomic_store(&st[tau], kFlagP | (uint32_t)(E + c), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  return E;
}

// Non-blocking form of lb_resolve, in two halves so that the state loads of one
// chunk are consumed only at the next: lb_try_load reads the 64 states before
// `tau` (lane l: item tau - 1 - l); lb_try_finish returns false if one of them,
// up to the nearest inclusive prefix, is not published yet (nothing is written
// then).  Otherwise it completes the look-back like lb_resolve and returns true.
// Every lane loads (lanes before the segment read its first state) and the value
// is not looked at here: a select right after the load would wait for it, and
// for every load issued before it, on the spot.  lb_try_finish masks those lanes.
__device__ inline uint64_t lb_try_load(const uint64_t *st, int tau, int seg0) {
  const int idx = tau - 1 - lane_id();
  return __hip_atomic_load(&st[idx >= seg0 ? idx : seg0], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline bool lb_try_finish(uint64_t *st, int tau, int seg0, int c, uint64_t v,
                                     int32_t *status, int &E) {
  if (tau == seg0) {
    E = 0;
    return true;
  }
  if (tau - 1 - lane_id() < seg0) v = kFlagP;  // before the segment: an inclusive prefix of 0
  const uint64_t fm = __ballot((v >> 32) != 0);
  const uint64_t pm = __ballot((v >> 32) == 2);
  const uint64_t need = pm ? ((pm & (0 - pm)) << 1) - 1 : ~0ull;
  if ((fm & need) != need) return false;
  if (!pm) {  // 64 published aggregates and no prefix yet: walk on (nothing waits long)
    E = lb_resolve(st, tau, seg0, c, status);
    return true;
  }
  const int l = lane_id();
  const int first = __ffsll((unsigned long long)pm) - 1;
  E = wave_sum(l <= first ? (int)(uint32_t)v : 0);
  if (l == 0)
    __hip_atomic_store(&st[tau], kFlagP | (uint32_t)(E + c), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

__device__ inline int lookback(uint64_t *st, int tau, int seg0, int c, int32_t *status) {
  lb_publish(st, tau, seg0, c);
  return lb_resolve(st, tau, seg0, c, status);
}

// ------------------------------------------------------------ grid barrier
// Barrier over the `nblocks` workgroups of a launch that are all resident
// (grids no larger than one workgroup per compute unit).  `ctr` is zero at
// launch and used once.  Returns false, in every workgroup, if the status is
// set meanwhile or the wait exceeds 1 s (which then sets ECHO_ETIMEOUT).
__device__ inline bool grid_sync(int32_t *ctr, int nblocks, int32_t *status) {
  __shared__ int s_ok;
  __syncthreads();
  if (threadIdx.x == 0) {
    __threadfence();
    __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int ok = 1;
    const uint64_t t0 = wall_clock64();
    while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < nblocks) {
      if (failed(status)) {
        ok = 0;
        break;
      }
      if ((long long)(wall_clock64() - t0) > kSpinLimit) {
        fail(status, ECHO_ETIMEOUT);
        ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    __threadfence();
    s_ok = ok;
  }
  __syncthreads();
  return s_ok != 0;
}

// Wait, as a whole workgroup, until *ctr reaches `target` (counted by other
// workgroups of the launch, each after a fence): false if the status fails
// meanwhile or the wait exceeds the spin limit (then ECHO_ETIMEOUT).
__device__ inline bool wait_count(int32_t *ctr, int target, int32_t *status) {
  __shared__ int s_ok;
  __syncthreads();
  if (threadIdx.x == 0) {
    int ok = 1;
    const uint64_t t0 = wall_clock64();
    while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      if (failed(status)) {
        ok = 0;
        break;
      }
      if ((long long)(wall_clock64() - t0) > kSpinLimit) {
        fail(status, ECHO_ETIMEOUT);
        ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    __threadfence();
    s_ok = ok;
  }
  __syncthreads();
  return s_ok != 0;
}

// ------------------------------------------------------------ key orders
// Order-preserving map of a finite fp32 value to uint32 (-0 treated as +0).
__device__ inline uint32_t f32_order(float f) {
  uint32_t u = __float_as_uint(f == 0.0f ? 0.0f : f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ inline float f32_from_order(uint32_t o) {
  uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __uint_as_float(u);
}
// Top-k keys ascend as scores descend.
__device__ inline uint32_t topk_key(float score) { return ~f32_order(score); }
__device__ inline float score_of_key(uint32_t key) { return f32_from_order(~key); }

// Histogram shift so that (key - kmin) >> shift < kBins for every key <= kmax.
__device__ inline int bin_shift(uint32_t kmin, uint32_t kmax) {
  uint32_t range = kmax - kmin;
  int bits = range ? 32 - __clz(range) : 0;
  return bits > 12 ? bits - 12 : 0;
}

}  // namespace echo
