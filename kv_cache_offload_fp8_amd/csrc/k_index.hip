// Step prologue and the fused lightning-indexer + prefetch kernel.
//
// Scoring follows DeepSeek Sparse Attention's lightning indexer, which the ECHO
// review ("Problem and motivation") names as the component that rates every past
// token before the top-2048 selection:
//     score[b,s] = sum_j w[b,j] * max(0, q[b,j,:] . K[host_base[b]+s,:]).
// Prefetch follows the review's "Core method / decode" and "Core method /
// prefetch inside the indexer pipeline": as soon as a block of tokens is scored,
// the ones above the EMA threshold that have no GPU slot are fetched from host
// memory, without waiting for the exact top-k; a per-request cap that grows with
// the context bounds the volume.
//
// MI355X mapping.  The heads x tokens contraction runs on the gfx950 fp8 MFMA
// (v_mfma_f32_16x16x128_f8f6f4): one instruction multiplies 16 heads by 16
// tokens over all 128 dims, and K feeds it straight from HBM with no
// conversion.  q arrives in bf16; the prologue scales each head by a power of
// two (max |q| lands in [128, 256)) and splits it into q_hi = e4m3(q') and
// q_lo = e4m3(q' - q_hi).  For every element with |q'| >= 2^-2 the split is
// exact (a bf16 significand has 8 bits, q_hi keeps 4, the remainder has at most
// 4 and lies on the e4m3 grid); the weights absorb the inverse scale exactly
// (ReLU is positively homogeneous).  Products of two fp8 values are exact; the
// instruction sums neighbouring products in a window about 2^-15 of the largest
// one before the fp32 accumulation (measured on this chip), which bounds the
// score error by a small multiple of 2^-15 * sum_j |w_j| sum_d |q_jd k_d|.
// Two MFMAs per 16 heads x 16 tokens (hi, lo) run as fast as the bf16 path's
// four, and the fp8->bf16 widening they replace costs 8 cycles per pair of bytes.
// Each wave owns 64 tokens at a time: it streams their K rows straight from HBM
// into MFMA operand registers (no LDS staging: every K byte is used by exactly
// one lane), applies ReLU and the head weights in registers, and reduces the 64
// heads with two
// cross-lane adds.  A workgroup holds seven scoring waves and one copy wave.
// Each scoring wave is an independent worker: it takes 256-token work items from
// an atomic ticket (the next ticket is fetched while the current item streams),
// keeps the next 64 tokens' K loads in flight while it computes, ranks its
// prefetch candidates in token order with a decoupled look-back over the work
// items of the request, installs them in the maps and hands (host row, slot)
// pairs to the copy wave through an LDS ring.  The copy wave reads those rows
// from mapped host memory and writes them to the GPU pool, so the PCIe latency
// never stalls the HBM stream -- the MI355X form of the pages' dedicated
// prefetch role inside the indexer pipeline.  Scoring waves also collect the
// tokens whose score clears a guard just below the previous step's k-th score;
// when at least k of them do, the exact top-k needs only those candidates.
#include "kernels.h"

namespace echo {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ begin

__device__ static void build_request_table(const StepArgs &a, int roles) {
  // one wave: lane b handles request b
  const int l = threadIdx.x;
  if (l >= kWave) return;
  const bool in = l < a.B;
  int ctx = in ? a.ctx_len[l] : 0;
  int base = in ? a.host_base[l] : 0;
  bool bad = in && (ctx < 0 || ctx > a.max_ctx || base < 0 ||
                    (int64_t)base + (int64_t)ctx > a.n_host);
  // disjoint host ranges
  for (int o = 0; o < kWave; ++o) {
    int c2 = __shfl(ctx, o), b2 = __shfl(base, o);
    if (in && o != l && o < a.B && ctx > 0 && c2 > 0 && base < b2 + c2 && b2 < base + ctx)
      bad = true;
  }
  const bool any_bad = __any(bad);
  if (any_bad) {
    if (l == 0) fail(a.ws.status, ECHO_EDEVARG);
    ctx = 0;
  }
  if (!in) ctx = 0;
  int cap = (int)min((int64_t)a.K, ((int64_t)ctx + a.cap_div - 1) / a.cap_div);
  int ntiles = (ctx + kScoreTile - 1) / kScoreTile;
  int cap_incl = wave_incl_scan(cap);
  int tile_incl = wave_incl_scan(ntiles);
  int active = 0;
  float th = __builtin_huge_valf();
  if (a.mode == ECHO_THETA_EMA) {
    th = in ? a.theta[l] : th;
    active = !(isinf(th) && th > 0);
  } else if (a.mode == ECHO_THETA_NEG_INF) {
    th = -__builtin_huge_valf();
    active = 1;
  }
  int use_guard = 0;
  uint32_t guard_key = 0xFFFFFFFFu;
  if (in && a.guard && ctx > a.K) {
    const float g = a.guard[l];
    if (!isinf(g) && !isnan(g)) {
      const uint32_t key = topk_key(g);
      guard_key = key > 0xFFFFFFFFu - kGuardUlps ? 0xFFFFFFFFu : key + kGuardUlps;
      use_guard = 1;
    }
  }
  if (in) {
    ReqInfo r;
    r.use_guard = use_guard;
    r.guard_key = guard_key;
    r.ctx = ctx;
    r.base = base;
    r.cap = cap;
    r.off = cap_incl - cap;
    r.tile0 = tile_incl - ntiles;
    r.ntiles = ntiles;
    r.active = active && ctx > 0;
    r.theta = th;
    a.sc.req[l] = r;
  }
  if (l == kWave - 1) {
    a.sc.misc[M_TOTAL_TILES] = tile_incl;
    a.sc.misc[M_RESERVE] = cap_incl;
    a.sc.misc[M_TICKET_SCORE] = 0;
    a.sc.misc[M_TICKET_ALLOC] = 0;
  }
}

// Stage one request's query for the scoring kernel: per head j a power-of-two
// scale 2^e puts max |q_j| in [128, 256); q_hi = e4m3(q*2^e),
// q_lo = e4m3(q*2^e - q_hi), stored [64][128] zero-padded, and the weight
// w_j * 2^-e (zero for padded heads).  Block of 256 threads, thread =
// (head, quarter of the dims).
__device__ static void stage_query(const StepArgs &a, int b) {
  const int tid = threadIdx.x;
  const int j = tid >> 2, part = tid & 3;
  const int t = a.ctl[ECHO_CTL_STEP];
  const int slot = (int)((unsigned)t % (unsigned)a.q_ring);
  const uint16_t *src = a.q + ((int64_t)slot * a.B + b) * a.H * a.D;
  float x[32];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int d = part * 32 + i;
    float v = 0.0f;
    if (j < a.H && d < a.D) v = __uint_as_float((uint32_t)src[j * a.D + d] << 16);
    x[i] = v;
    amax = fmaxf(amax, fabsf(v));
  }
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  int e = 0;
  if (amax > 0.0f) {
    int E;
    frexpf(amax, &E);  // amax = m * 2^E, m in [0.5, 1)
    e = min(64, max(-64, 8 - E));
  }
  uint32_t whi[8], wlo[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) whi[i] = wlo[i] = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float xs = ldexpf(x[i], e);
    const uint8_t h8 = e4m3_encode(xs);
    const uint8_t l8 = e4m3_encode(xs - e4m3_decode(h8));
    whi[i >> 2] |= (uint32_t)h8 << (8 * (i & 3));
    wlo[i >> 2] |= (uint32_t)l8 << (8 * (i & 3));
  }
  uint4 *hv = (uint4 *)(a.sc.qhi + ((int64_t)b * kHeadsPad + j) * kDimPad + part * 32);
  uint4 *lv = (uint4 *)(a.sc.qlo + ((int64_t)b * kHeadsPad + j) * kDimPad + part * 32);
  hv[0] = make_uint4(whi[0], whi[1], whi[2], whi[3]);
  hv[1] = make_uint4(whi[4], whi[5], whi[6], whi[7]);
  lv[0] = make_uint4(wlo[0], wlo[1], wlo[2], wlo[3]);
  lv[1] = make_uint4(wlo[4], wlo[5], wlo[6], wlo[7]);
  if (part == 0)
    a.sc.wsc[(int64_t)b * kHeadsPad + j] = j < a.H ? ldexpf(a.w[(int64_t)b * a.H + j], -e) : 0.0f;
}

__device__ static void fill_u32(uint32_t *p, int64_t n, uint32_t v, int64_t i0, int64_t step) {
  for (int64_t i = i0; i < n; i += step) p[i] = v;
}

constexpr int kBeginClearBlocks = 32;

__global__ __launch_bounds__(256) void k_begin(StepArgs a, int roles) {
  if (failed(a.ws.status)) return;
  int blk = blockIdx.x;
  if (blk == 0) {
    if (roles & BEGIN_REQ) build_request_table(a, roles);
    // small per-request arrays
    const int tid = threadIdx.x;
    if ((roles & BEGIN_CLR_INDEX) && tid < a.max_batch) {
      a.ws.n_pf[tid] = 0;
      a.ws.n_cand[tid] = 0;
      a.sc.rq_next[tid] = 0;
    }
    if ((roles & BEGIN_CLR_INDEX) && tid == 0) a.ws.counters[ECHO_CNT_PREFETCH] = 0;
    if ((roles & BEGIN_CLR_TOPK) && tid == 0) a.ws.counters[ECHO_CNT_SHORTCUT] = 0;
    if ((roles & BEGIN_CLR_TOPK) && tid < a.max_batch) {
      a.sc.kmin[tid] = 0xFFFFFFFFu;
      a.sc.kmax[tid] = 0u;
      a.sc.tcand_n[tid] = 0;
      a.sc.gcand_n[tid] = 0;
      a.sc.gcand_ovf[tid] = 0;
    }
    if ((roles & BEGIN_CLR_MANAGE) && tid < 16) {
      if (tid < 4) a.sc.ecnt[tid] = 0;
      if (tid != ECHO_CNT_PREFETCH && tid != ECHO_CNT_SHORTCUT) a.ws.counters[tid] = 0;
    }
    return;
  }
  blk -= 1;
  if (roles & BEGIN_Q) {
    if (blk < a.B) {
      stage_query(a, blk);
      return;
    }
    blk -= a.B;
  }
  if (blk >= kBeginClearBlocks) return;
  const int64_t i0 = (int64_t)blk * blockDim.x + threadIdx.x;
  const int64_t step = (int64_t)kBeginClearBlocks * blockDim.x;
  if (roles & BEGIN_CLR_INDEX) fill_u32((uint32_t *)a.sc.tstate, 2LL * a.sc.max_tiles, 0u, i0, step);
  if (roles & BEGIN_CLR_TOPK) fill_u32(a.sc.thist, (int64_t)a.B * kBins, 0u, i0, step);
  if (roles & BEGIN_CLR_MANAGE) {
    fill_u32(a.sc.ehist, kBins, 0u, i0, step);
    fill_u32((uint32_t *)a.sc.astate, 2LL * a.sc.atiles, 0u, i0, step);
  }
}

hipError_t launch_begin(const StepArgs &a, int roles, hipStream_t s) {
  const int grid = 1 + ((roles & BEGIN_Q) ? a.B : 0) + kBeginClearBlocks;
  hipLaunchKernelGGL(k_begin, dim3(grid), dim3(256), 0, s, a, roles);
  return hipGetLastError();
}

// ------------------------------------------------------------------ score

constexpr int kChunks = kScoreTile / 64;  // 64-token chunks per work item

// K rows of one 64-token chunk for this lane: 4 MFMA sub-tiles of 16 tokens,
// 32 bytes each (dims chunk .. chunk+31 of token s0 + 16u + row).  The loads are
// branch-free -- out-of-range tokens and dims read a clamped in-bounds address
// and are zeroed by a select -- so the compiler can count them exactly and keep
// the next chunk in flight (a branch around a load makes it wait for all).
__device__ inline void load_k_chunk(const StepArgs &a, const ReqInfo &r, int s0, int row,
                                    int chunk, v8i (&kb)[4]) {
  const int cl = chunk < a.D ? chunk : a.D - 32;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int s = s0 + u * 16 + row;
    const bool ok = s < r.ctx && chunk < a.D;
    const int sc = s < r.ctx ? s : r.ctx - 1;
    const v4i *p = (const v4i *)(a.kidx + ((int64_t)r.base + sc) * a.D + cl);
    const v4i x0 = __builtin_nontemporal_load(p);
    const v4i x1 = __builtin_nontemporal_load(p + 1);
    v8i x;
    x[0] = ok ? x0[0] : 0; x[1] = ok ? x0[1] : 0; x[2] = ok ? x0[2] : 0; x[3] = ok ? x0[3] : 0;
    x[4] = ok ? x1[0] : 0; x[5] = ok ? x1[1] : 0; x[6] = ok ? x1[2] : 0; x[7] = ok ? x1[3] : 0;
    kb[u] = x;
  }
}

// Scores of one 64-token chunk: returns, in lane l, the score of token s0 + l.
// qa[hg][0] / qa[hg][1]: this lane's 32 bytes of q_hi / q_lo for head group hg.
template <int HG>
__device__ inline float score_chunk(const v8i (&kb)[4], const v8i (&qa)[HG][2],
                                    const float (&wr)[HG][4], int lane) {
  float sc4[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    float v = 0.0f;
#pragma unroll
    for (int hg = 0; hg < HG; ++hg) {
      v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[hg][0], kb[u], acc, 0, 0, 0, 0,
                                                             0, 0);
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[hg][1], kb[u], acc, 0, 0, 0, 0,
                                                             0, 0);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) v += wr[hg][rr] * fmaxf(acc[rr], 0.0f);
    }
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    sc4[u] = v;  // every lane with (lane & 15) == i holds the score of token 16u + i
  }
  const int sel = lane >> 4;
  return sel == 0 ? sc4[0] : sel == 1 ? sc4[1] : sel == 2 ? sc4[2] : sc4[3];
}

// LDS ring between the scoring waves (producers) and the copy wave (consumer).
// Entry p lives at p % kRing and is valid once seq == p + 1.
struct Ring {
  int32_t h[kRing], g[kRing], seq[kRing];
  int32_t tail;  // next position to reserve
  int32_t head;  // next position the copy wave will take
  int32_t done;  // scoring waves that have finished
};

__device__ inline int lds_load(const int32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ inline void lds_store(int32_t *p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// The copy wave: host rows -> GPU pool slots, up to 8 rows (8 x 72 chunks of
// 16 bytes, 9 per lane) in flight per round.
__device__ static void copy_wave(const StepArgs &a, Ring &ring) {
  const int lane = lane_id();
  const int cpr = a.latent * 2 / 16;
  const uint4 *src = (const uint4 *)a.host_kv;
  uint4 *dst = (uint4 *)a.gpu_kv;
  int head = 0;
  uint64_t t0 = wall_clock64();
  while (true) {
    const int pos = head + lane;
    const bool ready = lane < 8 && lds_load(&ring.seq[pos % kRing]) == pos + 1;
    const uint64_t rm = __ballot(ready);
    const int n = rm == 0 ? 0 : __ffsll((unsigned long long)~rm) - 1;  // leading ready run
    if (n == 0) {
      if (lds_load(&ring.done) == kScoreWaves && head == lds_load(&ring.tail)) break;
      __builtin_amdgcn_s_sleep(2);
      if ((long long)(wall_clock64() - t0) > kSpinLimit) {
        if (lane == 0) fail(a.ws.status, ECHO_ETIMEOUT);
        break;
      }
      continue;
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    const int my_h = lane < n ? lds_load(&ring.h[pos % kRing]) : 0;
    const int my_g = lane < n ? lds_load(&ring.g[pos % kRing]) : 0;
    const int nchunks = n * cpr;
    for (int c0 = lane; c0 < nchunks; c0 += 3 * 64) {  // three 16-byte loads in flight
      const int ca = c0, cb = min(c0 + 64, nchunks - 1), cc = min(c0 + 128, nchunks - 1);
      const int ea = ca / cpr, eb = cb / cpr, ec = cc / cpr;
      const int ha = __shfl(my_h, ea), hb = __shfl(my_h, eb), hc = __shfl(my_h, ec);
      const int ga = __shfl(my_g, ea), gb = __shfl(my_g, eb), gc = __shfl(my_g, ec);
      const uint4 va = src[(int64_t)ha * cpr + (ca - ea * cpr)];
      const uint4 vb = src[(int64_t)hb * cpr + (cb - eb * cpr)];
      const uint4 vc = src[(int64_t)hc * cpr + (cc - ec * cpr)];
      dst[(int64_t)ga * cpr + (ca - ea * cpr)] = va;
      if (c0 + 64 < nchunks) dst[(int64_t)gb * cpr + (cb - eb * cpr)] = vb;
      if (c0 + 128 < nchunks) dst[(int64_t)gc * cpr + (cc - ec * cpr)] = vc;
    }
    head += n;
    if (lane == 0) lds_store(&ring.head, head);
    t0 = wall_clock64();
  }
}

// Work items: 256-token tiles of one request, handed out in token order by a
// per-request counter.  A wave starts on its "home" request and stays there, so
// it loads that request's query once; when the request runs dry it moves to the
// request with the most tiles left.  Returns (request, tile) or request -1.
struct Tile {
  int b, i;
};

__device__ inline Tile take_tile(const StepArgs &a, const ReqInfo *s_req, int b) {
  const int lane = lane_id();
  while (true) {
    if (b >= 0) {
      int i = 0;
      if (lane == 0) i = atomicAdd(&a.sc.rq_next[b], 1);
      i = __builtin_amdgcn_readfirstlane(i);
      if (i < s_req[b].ntiles) return Tile{b, i};
    }
    // this request is done: find the one with the most tiles left
    int left = 0;
    if (lane < a.B)
      left = s_req[lane].ntiles -
             __hip_atomic_load(&a.sc.rq_next[lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int best = left > 0 ? (left << 6) | lane : -1;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) best = max(best, __shfl_xor(best, o));
    best = __builtin_amdgcn_readfirstlane(best);
    if (best < 0) return Tile{-1, 0};
    b = best & 63;
  }
}

template <int HG>
__device__ static void score_wave(const StepArgs &a, const ReqInfo *s_req, Ring &ring,
                                  int wave) {
  int32_t *status = a.ws.status;
  const int lane = lane_id();
  // Operand layout: lane l feeds row (l & 15) of A (a head) and column (l & 15)
  // of B (a token) with the 32 bytes at dims chunk .. chunk+31,
  // chunk = 32*(l >> 4).  A and B use the same dims for the same lane, so the
  // MFMA sums q . k over all 128 dims whatever order it adds them in.
  const int row = lane & 15, chunk = (lane >> 4) * 32;
  const int t = a.ctl[ECHO_CTL_STEP];
  const int nfree = a.ctl[ECHO_CTL_NFREE];
  if (a.B == 0) return;

  v8i qa[HG][2];
  float wr[HG][4];
  auto load_query = [&](int b) {
    const uint8_t *qh = a.sc.qhi + (int64_t)b * kHeadsPad * kDimPad;
    const uint8_t *ql = a.sc.qlo + (int64_t)b * kHeadsPad * kDimPad;
#pragma unroll
    for (int hg = 0; hg < HG; ++hg) {
      qa[hg][0] = *(const v8i *)(qh + (hg * 16 + row) * kDimPad + chunk);
      qa[hg][1] = *(const v8i *)(ql + (hg * 16 + row) * kDimPad + chunk);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        wr[hg][rr] = a.sc.wsc[(int64_t)b * kHeadsPad + hg * 16 + (lane >> 4) * 4 + rr];
    }
  };

  Tile cur = take_tile(a, s_req, wave % a.B);
  if (cur.b < 0) return;
  load_query(cur.b);
  // Two K buffers: chunk c of a tile lives in kb[c & 1]; the next chunk (the
  // next tile's first one at the end of a tile) is in flight while c computes.
  // Everything read between two chunks -- the tile claim, the request record --
  // is either a scalar load or issued before the stream loads, because vector
  // loads retire in order and waiting for a late one would drain the stream.
  v8i kb[2][4];
  load_k_chunk(a, s_req[cur.b], cur.i * kScoreTile, row, chunk, kb[0]);

  while (true) {
    const int b = __builtin_amdgcn_readfirstlane(cur.b);
    const ReqInfo r = s_req[b];  // LDS: does not queue behind the K stream
    const int tau = r.tile0 + cur.i;
    const int s_wave = cur.i * kScoreTile;
    int raw = 0;
    if (lane == 0) raw = atomicAdd(&a.sc.rq_next[b], 1);  // claim the next tile
    Tile nxt{-1, 0};
    float *out = a.ws.scores + (int64_t)b * a.max_ctx;
    uint64_t above[kChunks], gsel[kChunks];
    uint32_t keys[kChunks];
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      if (c + 1 < kChunks) {
        load_k_chunk(a, r, s_wave + (c + 1) * 64, row, chunk, kb[(c + 1) & 1]);
      } else {
        const int ni = __builtin_amdgcn_readfirstlane(raw);
        nxt = ni < r.ntiles ? Tile{b, ni} : take_tile(a, s_req, -1);
        if (nxt.b >= 0) {
          const ReqInfo rn = s_req[nxt.b];
          load_k_chunk(a, rn, nxt.i * kScoreTile, row, chunk, kb[(c + 1) & 1]);
        }
      }
      const float score = score_chunk<HG>(kb[c & 1], qa, wr, lane);
      const int s = s_wave + c * 64 + lane;
      const bool valid = s < r.ctx;
      if (valid) out[s] = score;
      keys[c] = topk_key(score);
      above[c] = __ballot(r.active && valid && score > r.theta);
      gsel[c] = __ballot(r.use_guard && valid && keys[c] <= r.guard_key);
    }

    // ---- top-k candidates above the selection guard: fixed slots of this tile
    if (r.use_guard) {
      int ng = 0;
#pragma unroll
      for (int c = 0; c < kChunks; ++c) {
        if ((gsel[c] >> lane) & 1ull) {
          const int p = ng + __popcll(gsel[c] & lanemask_lt());
          if (p < kGuardSlots) {
            a.sc.gcand_key[(int64_t)tau * kGuardSlots + p] = keys[c];
            a.sc.gcand_idx[(int64_t)tau * kGuardSlots + p] = s_wave + c * 64 + lane;
          }
        }
        ng += __popcll(gsel[c]);
      }
      if (lane == 0) {
        a.sc.gcand_cnt[tau] = ng;
        if (ng) atomicAdd(&a.sc.gcand_n[b], ng);  // result unused: no wait
        if (ng > kGuardSlots) atomicOr(&a.sc.gcand_ovf[b], 1);
      }
    }

    // ---- prefetch: above the threshold and not resident, first cap in token order
    if (r.active) {
      int g_of[kChunks];
#pragma unroll
      for (int c = 0; c < kChunks; ++c) {  // one batch of map lookups per work item
        g_of[c] = 0;
        if ((above[c] >> lane) & 1ull) g_of[c] = a.h2g[(int64_t)r.base + s_wave + c * 64 + lane];
      }
      uint64_t cand[kChunks];
      int c_all = 0;
#pragma unroll
      for (int c = 0; c < kChunks; ++c) {
        cand[c] = __ballot(((above[c] >> lane) & 1ull) && g_of[c] == -1);
        c_all += __popcll(cand[c]);
      }
      int base = lookback(a.sc.tstate, tau, r.tile0, c_all, status);
      uint64_t emit[kChunks];
      int slot[kChunks];
      int ne = 0;
#pragma unroll
      for (int c = 0; c < kChunks; ++c) {
        const uint64_t m = cand[c];
        slot[c] = -1;
        if ((m >> lane) & 1ull) {
          const int rank = base + __popcll(m & lanemask_lt());
          if (rank < r.cap) {
            const int j = r.off + rank;
            const int g = (j < nfree && j < a.n_gpu) ? a.idxbuf[j] : -1;
            if (g >= 0 && g < a.n_gpu) {
              const int s = s_wave + c * 64 + lane;
              const int64_t h = (int64_t)r.base + s;
              a.h2g[h] = g;
              a.g2h[g] = (int32_t)h;
              a.freef[g] = 0;
              a.prio[g] = t;
              a.ws.pf_tok[(int64_t)b * a.K + rank] = s;
              a.ws.pf_slot[(int64_t)b * a.K + rank] = g;
              slot[c] = g;
            }
          }
        }
        emit[c] = __ballot(slot[c] >= 0);
        ne += __popcll(emit[c]);
        base += __popcll(m);
      }
      if (ne) {  // hand the rows to the copy wave
        int pos = 0;
        if (lane == 0) pos = atomicAdd(&ring.tail, ne);
        pos = __shfl(pos, 0);
        const uint64_t tw = wall_clock64();
        while (pos + ne - lds_load(&ring.head) > kRing) {  // wait for room
          __builtin_amdgcn_s_sleep(1);
          if (__any((long long)(wall_clock64() - tw) > kSpinLimit)) {
            if (lane == 0) fail(status, ECHO_ETIMEOUT);
            break;
          }
        }
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
          if (slot[c] >= 0) {
            const int p = (pos + __popcll(emit[c] & lanemask_lt())) % kRing;
            ring.h[p] = (int32_t)((int64_t)r.base + s_wave + c * 64 + lane);
            ring.g[p] = slot[c];
          }
          pos += __popcll(emit[c]);
        }
        __threadfence_block();
        pos -= ne;
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
          if (slot[c] >= 0) {
            const int p = pos + __popcll(emit[c] & lanemask_lt());
            lds_store(&ring.seq[p % kRing], p + 1);
          }
          pos += __popcll(emit[c]);
        }
        if (lane == 0) {
          atomicAdd(&a.ws.n_pf[b], ne);
          atomicAdd(&a.ws.counters[ECHO_CNT_PREFETCH], ne);
        }
      }
      if (lane == 0 && c_all > 0) atomicAdd(&a.ws.n_cand[b], c_all);
    }
    if (nxt.b < 0) break;
    if (nxt.b != b) load_query(nxt.b);
    cur = nxt;
  }
}

template <int HG>
__global__ __launch_bounds__(512) void k_score(StepArgs a) {
  __shared__ ReqInfo s_req[kMaxBatch];
  __shared__ Ring ring;
  if (failed(a.ws.status)) return;
  const int tid = threadIdx.x;
  for (int i = tid; i < a.B; i += blockDim.x) s_req[i] = a.sc.req[i];
  for (int i = tid; i < kRing; i += blockDim.x) ring.seq[i] = 0;
  if (tid == 0) {
    ring.tail = 0;
    ring.head = 0;
    ring.done = 0;
  }
  __syncthreads();
  const int wid = tid / kWave;
  if (wid == kScoreWaves) {
    copy_wave(a, ring);
    return;
  }
  score_wave<HG>(a, s_req, ring, blockIdx.x * kScoreWaves + wid);
  __threadfence_block();
  if (lane_id() == 0) atomicAdd(&ring.done, 1);
}

hipError_t launch_score(const StepArgs &a, hipStream_t s) {
  const int hg = (a.H + 15) / 16;
  // persistent grid: one workgroup (7 scoring waves + 1 copy wave) per CU
  const int waves_needed = (a.sc.max_tiles + kScoreWaves - 1) / kScoreWaves;
  int grid = waves_needed < 256 ? waves_needed : 256;
  if (grid < 1) grid = 1;
  switch (hg) {
    case 1: hipLaunchKernelGGL(k_score<1>, dim3(grid), dim3(512), 0, s, a); break;
    case 2: hipLaunchKernelGGL(k_score<2>, dim3(grid), dim3(512), 0, s, a); break;
    case 3: hipLaunchKernelGGL(k_score<3>, dim3(grid), dim3(512), 0, s, a); break;
    default: hipLaunchKernelGGL(k_score<4>, dim3(grid), dim3(512), 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace echo
