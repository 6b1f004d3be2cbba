// Exact top-k per request and the protection of the selected tokens (internal):
// the body shared by the top-k kernel and the fused top-k + management kernel.
//
// Top-k (ECHO review, "Core method / decode": the exact top-2048 after the
// indexer) takes the min(k, ctx) tokens that come first under (score
// descending, token ascending), listed in ascending token order.  Keys are
// key = ~order(score), so ascending keys are descending scores.  One 1024-thread
// workgroup handles one request:
//  - guard path: when the scoring kernel kept at least k tokens at or above a
//    guard just below the previous step's k-th score (and no work item
//    overflowed its slots), the exact top-k is among them.  They are gathered in
//    token order into LDS, the k-th smallest key is found with four 8-bit radix
//    passes over LDS, and one ordered scan writes the selection: every key below
//    it, then the first keys equal to it (lowest token ids, since the list is in
//    token order);
//  - full path: a 4096-bin histogram over the request's observed key range finds
//    the bin holding the k-th key; lower bins are marked in a bitmap, the
//    boundary bin is listed and resolved exactly by an MSD radix select on the
//    64-bit composite (key << 32 | token), and the bitmap is read out in order.
// Protection (review, "Core method / in-graph per-layer cache management":
// recall first looks the selected tokens up in the map) then sets priority t on
// every resident selected token and lists the misses in token order.
#pragma once

#include "copy.h"
#include "select.h"

namespace echo {


constexpr int kGuardLds = 8192;  // guard candidates the LDS path holds

// Shared memory of topk_block (and of the helpers it calls).
struct TopkLds {
  uint32_t key[kGuardLds];  // guard keys, or the full path's histogram
  int32_t idx[kGuardLds];
  int32_t sel[4096];
  int sh[kMaxSelWaves + 1];
  uint64_t shu[kMaxSelWaves];
  int bin, below, cnt;
  uint32_t h256[256];  // lds_kth_key
  int s2[2];
  SelectLds sel_lds;
};

// k-th smallest of `c` keys in LDS (1 <= need <= c): the key kb and how many keys
// equal to kb belong to the selection.  h256, s2: 256 + 2 words of shared memory.
template <int NT>
__device__ static void lds_kth_key(const uint32_t *keys, int c, int need, uint32_t *kb_out,
                                   int *rem_out, uint32_t *h256, int *s2) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0;
  int rem = need;
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < 256; i += NT) h256[i] = 0;
    __syncthreads();
    for (int i = tid; i < c; i += NT) {
      const uint32_t k = keys[i];
      const bool match = pass == 0 ? true : ((k >> (shift + 8)) == prefix);
      if (match) atomicAdd(&h256[(k >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < kWave) {
      uint32_t v[4];
      int sum = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        v[u] = h256[tid * 4 + u];
        sum += (int)v[u];
      }
      const int incl = wave_incl_scan(sum);
      int cum = incl - sum;
      if (cum < rem && incl >= rem) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (cum < rem && cum + (int)v[u] >= rem) {
            s2[0] = tid * 4 + u;
            s2[1] = cum;
          }
          cum += (int)v[u];
        }
      }
    }
    __syncthreads();
    rem -= s2[1];
    prefix = (prefix << 8) | (uint32_t)s2[0];
    __syncthreads();
  }
  *kb_out = prefix;
  *rem_out = rem;
}

// Protect the selected tokens of request b (held in LDS) and list its misses in
// token order.  Returns the number of misses (in every thread).
template <int NT = kSelThreads>
__device__ static int protect_request(const StepArgs &a, int b, const int32_t *s_sel, int n,
                                      int *sh) {
  const int t = a.ctl[ECHO_CTL_STEP];
  const int base = a.sc.req[b].base;
  int off = 0;
  for (int i0 = 0; i0 < n; i0 += NT) {
    const int i = i0 + threadIdx.x;
    const bool valid = i < n && s_sel[i] >= 0;
    int s = 0, g = -1;
    if (valid) {
      s = s_sel[i];
      const int64_t h = token_host(a, b, base, s);
      if (h >= 0 && h < a.n_host) g = a.h2g[h];
      if (g >= a.n_gpu) g = -1;
      if (g >= 0) a.prio[g] = t;
      a.ws.sel_slot[(int64_t)b * a.K + i] = g;
    }
    const int miss = (valid && g < 0) ? 1 : 0;
    int tot;
    const int pos = off + block_excl_scan<NT>(miss, sh, &tot);
    if (miss) {
      a.ws.miss_tok[(int64_t)b * a.K + pos] = s;
      a.sc.miss_i[(int64_t)b * a.K + pos] = i;
    }
    off += tot;
  }
  if (threadIdx.x == 0) {
    a.ws.n_miss[b] = off;
    atomicAdd(&a.ws.counters[ECHO_CNT_MISS], off);
  }
  return off;
}

// Running totals of request b's step (a.stats): selected, missed, prefetched and
// candidate counts, and how many of the prefetched tokens the step selected.  The
// prefetch list pf_tok (final when the scoring kernel ended) and the selection s_sel
// (in LDS) are both in ascending token order; each prefetched token is looked up in
// the selection by binary search.
template <int NT>
__device__ static void add_step_stats(const StepArgs &a, int b, const int32_t *s_sel, int nsel,
                                      int nmiss, int *sh) {
  const int npf = a.ws.n_pf[b];
  const int ncand = a.ws.n_cand[b];
  const int32_t *pf = a.ws.pf_tok + (int64_t)b * a.K;
  int found = 0;
  for (int i = threadIdx.x; i < npf; i += NT) {
    const int s = pf[i];
    int lo = 0, hi = nsel;  // first position whose token is >= s
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (s_sel[mid] < s) lo = mid + 1;
      else hi = mid;
    }
    found += (lo < nsel && s_sel[lo] == s) ? 1 : 0;
  }
  int tot;
  block_excl_scan<NT>(found, sh, &tot);
  if (threadIdx.x == 0) {
    unsigned long long *st = (unsigned long long *)a.stats;
    atomicAdd(&st[ECHO_STAT_SELECTED], (unsigned long long)nsel);
    atomicAdd(&st[ECHO_STAT_MISSED], (unsigned long long)nmiss);
    atomicAdd(&st[ECHO_STAT_PREFETCHED], (unsigned long long)npf);
    atomicAdd(&st[ECHO_STAT_PF_SELECTED], (unsigned long long)tot);
    atomicAdd(&st[ECHO_STAT_CANDIDATES], (unsigned long long)ncand);
  }
}

// Top-k of request b, its threshold / guard updates and (PROTECT) the protection
// of its selection, by one workgroup of NT threads; at the end the workgroup adds
// one to misc[M_TOPK_DONE].  st0: the status word, read at the kernel's start.
template <bool PROTECT, int NT = kSelThreads>
__device__ static void topk_block(const StepArgs &a, int b, int32_t st0, TopkLds &L) {
  uint32_t *const s_key = L.key;
  int32_t *const s_idx = L.idx;
  int32_t *const s_sel = L.sel;
  int *const sh = L.sh;
  uint64_t *const shu = L.shu;
  const int tid = threadIdx.x, lane = lane_id(), wid = tid / kWave;
  const ReqInfo r = a.sc.req[b];
  if (st0 != 0) return;
  const int ctx = r.ctx;
  const int K = a.K;
  const int nsel = ctx < K ? ctx : K;
  const float *sc = a.scores_in + (int64_t)b * a.score_stride;
  int32_t *sel_out = a.ws.sel_tok + (int64_t)b * K;
  float kth;
  if (ctx <= K) {
    uint64_t mx = 0;
    for (int i = tid; i < ctx; i += NT) {
      s_sel[i] = i;
      sel_out[i] = i;
      const uint64_t k = topk_key(sc[i]);
      mx = k > mx ? k : mx;
    }
    mx = block_max_u64<NT>(mx, shu);
    kth = ctx > 0 ? score_of_key((uint32_t)mx) : __builtin_nanf("");
  } else {
    // ---- guard path availability: per-item candidate counts of this request
    const int per = (r.ntiles + NT - 1) / NT;
    const int t0 = min(r.ntiles, tid * per), t1 = min(r.ntiles, t0 + per);
    int mine = 0, ovf = 0;
    if (r.use_guard) {
      for (int ti = t0; ti < t1; ++ti) {
        const int n = a.sc.gcand_cnt[r.tile0 + ti];
        mine += n < kGuardSlots ? n : kGuardSlots;
        ovf |= n > kGuardSlots;
      }
    }
    int tot;
    int p = block_excl_scan<NT>(mine, sh, &tot);
    const bool any_ovf = __syncthreads_or(ovf) != 0;
    if (r.use_guard && !any_ovf && tot >= K && tot <= kGuardLds) {
      for (int ti = t0; ti < t1; ++ti) {
        const int tau = r.tile0 + ti;
        const int n = a.sc.gcand_cnt[tau];
        for (int j = 0; j < n; ++j, ++p) {
          s_key[p] = a.sc.gcand_key[(int64_t)tau * kGuardSlots + j];
          s_idx[p] = a.sc.gcand_idx[(int64_t)tau * kGuardSlots + j];
        }
      }
      __syncthreads();
      uint32_t kb;
      int rem;
      lds_kth_key<NT>(s_key, tot, K, &kb, &rem, L.h256, L.s2);
      // ordered write-out: keys below kb, then the first `rem` keys equal to kb
      int c_lt = 0, c_eq = 0;
      for (int i0 = 0; i0 < tot; i0 += NT) {
        const int i = i0 + tid;
        const bool v = i < tot;
        const uint32_t k = v ? s_key[i] : 0xFFFFFFFFu;
        const bool lt = v && k < kb, eq = v && k == kb;
        int rt;
        const int ex = block_excl_scan<NT>((lt ? 1 << 16 : 0) | (eq ? 1 : 0), sh, &rt);
        const int eq_before = c_eq + (ex & 0xFFFF);
        if (lt || (eq && eq_before < rem)) {
          const int pos = c_lt + (ex >> 16) + min(eq_before, rem);
          s_sel[pos] = s_idx[i];
          sel_out[pos] = s_idx[i];
        }
        c_lt += rt >> 16;
        c_eq += rt & 0xFFFF;
      }
      kth = score_of_key(kb);
      if (tid == 0) atomicAdd(&a.ws.counters[ECHO_CNT_SHORTCUT], 1);
    } else {
      // ---- full path
      uint32_t *bits = a.sc.tbits + (int64_t)b * a.sc.bw;
      uint32_t *ckey = a.sc.tcand_key + (int64_t)b * a.max_ctx;
      int32_t *cidx = a.sc.tcand_idx + (int64_t)b * a.max_ctx;
      uint64_t mn = ~0ull, mx = 0;
      for (int s = tid; s < ctx; s += NT) {
        const uint64_t k = topk_key(sc[s]);
        mn = k < mn ? k : mn;
        mx = k > mx ? k : mx;
      }
      mn = block_min_u64<NT>(mn, shu);
      mx = block_max_u64<NT>(mx, shu);
      const uint32_t kmin = (uint32_t)mn;
      const int shift = bin_shift(kmin, (uint32_t)mx);
      uint32_t *hist = s_key;
      for (int i = tid; i < kBins; i += NT) hist[i] = 0;
      if (tid == 0) L.cnt = 0;
      __syncthreads();
      for (int s = tid; s < ctx; s += NT)
        atomicAdd(&hist[min((topk_key(sc[s]) - kmin) >> shift, (uint32_t)(kBins - 1))], 1u);
      __syncthreads();
      find_boundary<false, NT>(hist, K, &L.bin, &L.below, sh);
      const uint32_t bstar = (uint32_t)L.bin;
      const int below = L.below;
      for (int s0 = wid * kWave; s0 < ctx; s0 += NT) {
        const int s = s0 + lane;
        const bool valid = s < ctx;
        const uint32_t key = valid ? topk_key(sc[s]) : 0u;
        const uint32_t bin = min((key - kmin) >> shift, (uint32_t)(kBins - 1));
        const uint64_t m = __ballot(valid && bin < bstar);
        if (lane == 0) {
          bits[s0 / 32] = (uint32_t)m;
          bits[s0 / 32 + 1] = (uint32_t)(m >> 32);
        }
        const bool cand = valid && bin == bstar;
        const uint64_t cm = __ballot(cand);
        if (cm) {
          int basepos = 0;
          if (lane == 0) basepos = atomicAdd(&L.cnt, __popcll(cm));
          basepos = __shfl(basepos, 0);
          if (cand) {
            const int pos = basepos + __popcll(cm & lanemask_lt());
            ckey[pos] = key;
            cidx[pos] = s;
          }
        }
      }
      __threadfence_block();
      __syncthreads();
      const int c = L.cnt;
      uint64_t P;
      int pos;
      block_select<NT>(ckey, cidx, c, K - below, &P, &pos, L.sel_lds);
      __threadfence_block();
      __syncthreads();
      uint64_t kmax_sel = 0;
      for (int i = tid; i < c; i += NT) {
        const uint32_t k = ckey[i];
        const int32_t s = cidx[i];
        if (composite_selected(k, s, P, pos)) {
          atomicOr(&bits[s >> 5], 1u << (s & 31));
          kmax_sel = k > kmax_sel ? k : kmax_sel;
        }
      }
      kmax_sel = block_max_u64<NT>(kmax_sel, shu);
      kth = score_of_key((uint32_t)kmax_sel);
      __threadfence_block();
      __syncthreads();
      // ordered extraction of the selection bitmap
      const int nwords = (ctx + 31) / 32;
      const int wper = (nwords + NT - 1) / NT;
      const int w0 = tid * wper, w1 = min(nwords, w0 + wper);
      int cnt = 0;
      for (int wi = w0; wi < w1; ++wi)
        cnt += __popc(__hip_atomic_load(&bits[wi], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      int rt;
      int q = block_excl_scan<NT>(cnt, sh, &rt);
      for (int wi = w0; wi < w1; ++wi) {
        uint32_t x = __hip_atomic_load(&bits[wi], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        while (x) {
          const int bit = __ffs(x) - 1;
          x &= x - 1;
          const int s = wi * 32 + bit;
          if (q < K) {
            s_sel[q] = s;
            sel_out[q] = s;
          }
          ++q;
        }
      }
    }
  }
  if (tid == 0) {
    a.ws.n_sel[b] = nsel;
    a.ws.kth[b] = kth;
    if (a.theta_upd && ctx >= K && ctx > 0) {
      const float th = a.theta_upd[b];
      const float keep = __fsub_rn(1.0f, a.alpha);
      a.theta_upd[b] = (isinf(th) && th > 0) ? kth
                                              : __fadd_rn(__fmul_rn(a.alpha, kth),
                                                          __fmul_rn(keep, th));
    }
    if (a.guard_upd) a.guard_upd[b] = ctx > K ? kth : __builtin_huge_valf();
  }
  if (PROTECT) {
    __syncthreads();
    const int nmiss = protect_request<NT>(a, b, s_sel, nsel, sh);
    if (a.stats) add_step_stats<NT>(a, b, s_sel, nsel, nmiss, sh);
  }
  // done: the fence makes this workgroup's selection, priorities and miss list
  // visible before the count (management waits for it in the fused kernel)
  __syncthreads();
  if (tid == 0) {
    __threadfence();
    __hip_atomic_fetch_add(&a.sc.misc[M_TOPK_DONE], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace echo
