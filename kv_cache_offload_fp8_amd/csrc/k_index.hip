// Step prologue, the indexer-K layout kernel and the fused lightning-indexer +
// prefetch kernel.
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
//
// K is stored in the MFMA operand order (echo_kindex_pack): for each group of 16
// tokens, one 16-byte load per lane reads 1 KB of contiguous memory holding
// exactly the operand bytes of the 64 lanes, so every load instruction covers
// whole cache lines (the row-major order needs two instructions per line and
// streams about 15% slower).  Each wave owns 64 tokens at a time: it loads their
// K straight into MFMA operand registers (no LDS staging: every K byte is used by
// exactly one lane), keeps the next 64 tokens' loads in flight while it computes,
// applies ReLU and the head weights in registers and reduces the 64 heads with
// two cross-lane adds.  Scores (and selection-guard candidates) collect in the
// wave's LDS and are written out at the end of its job, so no global store sits
// between its K loads.
//
// Work assignment.  Most workgroups score (eight waves each); a few only copy.
// Request b gets wb scoring waves (chosen so that no wave takes more 256-token
// work items than any other); its k-th wave scores items k, k + wb, k + 2wb, ...
// in order.  A wave therefore loads its request's query once, takes no ticket
// and touches no shared counter (device-scope atomics on one address serialize:
// a ticket counter per request doubled the scoring time), and the items of one
// request are scored in step by neighbouring waves.  The prefetch epilogue of an
// item (residency check, decoupled look-back, map installs) runs during the
// wave's next item: the item's candidate count is published at that item's first
// chunk and its rank resolved two chunks later, when the items before it have
// published theirs, so the look-back rarely waits and its lookups never drain
// the K stream.  Only a job's first item is resolved at once: the items before it
// are the other waves' first items, finished at about the same time, and its rows
// then reach the copy about 7 us sooner (1.2% on the capacity layer step).
// Installed rows are published by rank as self-validating 64-bit entries; the
// copy workgroups read them from mapped host memory into the GPU pool while
// scoring continues -- the MI355X form of the pages' dedicated prefetch role
// inside the indexer pipeline.  The copy runs on
// workgroups of its own because host reads issued from a compute unit hold up
// that unit's HBM stream (measured: scoring slowed from about 100 us to 190 us
// when each workgroup also read its rows from the host).  Scoring waves also
// keep the tokens whose score clears a guard just below the previous step's k-th
// score in fixed per-item slots; when at least k are found, the exact top-k needs
// only those candidates.
#include "copy.h"

namespace echo {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ begin

// Whether two requests' contiguous host ranges overlap, by the four waves of the
// calling workgroup: lane l holds request l, and wave w compares it with requests
// w, w + 4, ... (read from their lanes with scalar lane reads).  One wave walking
// all 32 requests took about 3 us of the prologue.  Block-uniform result.
__device__ static bool ranges_overlap(const StepArgs &a) {
  __shared__ int s_ovl;
  const int tid = threadIdx.x, l = tid & (kWave - 1), w = tid / kWave;
  const bool in = l < a.B;
  const int ctx = in ? a.ctx_len[l] : 0;
  const int base = in ? a.host_base[l] : 0;
  if (tid == 0) s_ovl = 0;
  bool bad = false;
  for (int o = w; o < a.B; o += 4) {
    const int c2 = __builtin_amdgcn_readlane(ctx, o), b2 = __builtin_amdgcn_readlane(base, o);
    if (in && o != l && ctx > 0 && c2 > 0 && base < b2 + c2 && b2 < base + ctx) bad = true;
  }
  __syncthreads();
  if (__any(bad) && l == 0) s_ovl = 1;
  __syncthreads();
  return s_ovl != 0;
}

__device__ static void build_request_table(const StepArgs &a, int32_t st0, bool overlap) {
  // one wave: lane b handles request b.  Every input is read before the status
  // (st0, loaded by the caller) is looked at, so the reads take one round trip.
  const int l = threadIdx.x;
  if (l >= kWave) return;
  const bool in = l < a.B;
  int ctx = in ? a.ctx_len[l] : 0;
  int base = in && !a.pages ? a.host_base[l] : 0;
  const float th_in = in && a.mode == ECHO_THETA_EMA ? a.theta[l] : __builtin_huge_valf();
  const float g_in = in && a.guard ? a.guard[l] : __builtin_huge_valf();
  if (st0 != 0) return;
  bool bad;
  if (a.pages) {
    // page table: the context fits the row (the pages themselves are checked by the
    // clear workgroups of this kernel; distinct pages are the admission's check)
    bad = in && (ctx < 0 || ctx > a.max_ctx || (ctx + 15) / 16 > a.page_stride);
  } else {
    bad = in && (ctx < 0 || ctx > a.max_ctx || base < 0 || (base & 15) != 0 ||
                 (int64_t)base + (int64_t)ctx > a.n_host);
    bad = bad || overlap;  // disjoint host ranges
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
    th = th_in;
    active = !(isinf(th) && th > 0);
  } else if (a.mode == ECHO_THETA_NEG_INF) {
    th = -__builtin_huge_valf();
    active = 1;
  }
  int use_guard = 0;
  uint32_t guard_key = 0xFFFFFFFFu;
  if (in && a.guard && ctx > a.K) {
    const float g = g_in;
    if (!isinf(g) && !isnan(g)) {
      const uint32_t key = topk_key(g);
      guard_key = key > 0xFFFFFFFFu - kGuardUlps ? 0xFFFFFFFFu : key + kGuardUlps;
      use_guard = 1;
    }
  }
  // Scoring jobs: the smallest R with sum_b ceil(n_b / R) <= W items per wave,
  // then wb = ceil(n_b / R) waves for request b.  With at least as many active
  // requests as waves, every request gets one wave and waves take several jobs.
  const int W = a.score_waves;
  const int N = wave_sum(ntiles);
  const int nact = wave_sum(ntiles > 0 ? 1 : 0);
  int nmax = ntiles;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) nmax = max(nmax, __shfl_xor(nmax, o));
  int R = nmax > 0 ? nmax : 1;
  if (N > 0 && nact < W) {
    // sum_b ceil(n_b / R) <= N / R + nact, so R = ceil(N / (W - nact)) always fits;
    // scan up from the lower bound ceil(N / W) (usually one or two candidates)
    const int hi = min(nmax, (N + (W - nact) - 1) / (W - nact));
    R = max(1, (N + W - 1) / W);
    while (R < hi && wave_sum((ntiles + R - 1) / R) > W) ++R;
  }
  const int wb = ntiles > 0 ? (ntiles + R - 1) / R : 0;
  const int slot_incl = wave_incl_scan(wb);
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
    r.wb = wb;
    r.slot0 = slot_incl - wb;
    a.sc.req[l] = r;
  }
  if (l == kWave - 1) {
    a.sc.misc[M_TOTAL_TILES] = tile_incl;
    a.sc.misc[M_RESERVE] = cap_incl;
    a.sc.misc[M_SLOTS] = slot_incl;
  }
}

// Stage a quarter of one request's query (16 heads) for the scoring kernel: per
// head j a power-of-two scale 2^e puts max |q_j| in [128, 256); q_hi = e4m3(q*2^e),
// q_lo = e4m3(q*2^e - q_hi), stored [64][128] zero-padded, and the weight
// w_j * 2^-e (zero for padded heads).  Block of 256 threads: thread = (head of
// the quarter, 8 dims); the 16 threads of a head are 16 neighbouring lanes.
__device__ static void stage_query(const StepArgs &a, int b, int quarter, int32_t st0) {
  const int tid = threadIdx.x;
  const int j = quarter * 16 + (tid >> 4), d0 = (tid & 15) * 8;
  const int t = a.ctl[ECHO_CTL_STEP];
  const int slot = (int)((unsigned)t % (unsigned)a.q_ring);
  const uint16_t *src = a.q + ((int64_t)slot * a.B + b) * a.H * a.D;
  // 8 bf16 = one 16-byte load (D is a multiple of 32: a group is all in or all out)
  const bool in = j < a.H && d0 < a.D;
  const uint4 w4 = in ? *(const uint4 *)(src + j * a.D + d0) : make_uint4(0, 0, 0, 0);
  const float wj = d0 == 0 && j < a.H ? a.w[(int64_t)b * a.H + j] : 0.0f;
  if (st0 != 0) return;
  const uint32_t wd[4] = {w4.x, w4.y, w4.z, w4.w};
  float x[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    x[2 * k] = __uint_as_float(wd[k] << 16);
    x[2 * k + 1] = __uint_as_float(wd[k] & 0xFFFF0000u);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  int e = 0;
  if (amax > 0.0f) {
    int E;
    frexpf(amax, &E);  // amax = m * 2^E, m in [0.5, 1)
    e = min(64, max(-64, 8 - E));
  }
  // the hardware conversion: round to nearest even, OCP E4M3FN (no value
  // reaches the saturation range)
  const float sc = ldexpf(1.0f, e);  // exact: |e| <= 64
  uint32_t whi[2], wlo[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const float x0 = x[4 * k] * sc, x1 = x[4 * k + 1] * sc;
    const float x2 = x[4 * k + 2] * sc, x3 = x[4 * k + 3] * sc;
    int h = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
    h = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, h, true);
    int l = __builtin_amdgcn_cvt_pk_fp8_f32(x0 - __builtin_amdgcn_cvt_f32_fp8(h, 0),
                                            x1 - __builtin_amdgcn_cvt_f32_fp8(h, 1), 0, false);
    l = __builtin_amdgcn_cvt_pk_fp8_f32(x2 - __builtin_amdgcn_cvt_f32_fp8(h, 2),
                                        x3 - __builtin_amdgcn_cvt_f32_fp8(h, 3), l, true);
    whi[k] = (uint32_t)h;
    wlo[k] = (uint32_t)l;
  }
  const int64_t o = ((int64_t)b * kHeadsPad + j) * kDimPad + d0;
  *(uint2 *)(a.sc.qhi + o) = make_uint2(whi[0], whi[1]);
  *(uint2 *)(a.sc.qlo + o) = make_uint2(wlo[0], wlo[1]);
  if (d0 == 0)
    a.sc.wsc[(int64_t)b * kHeadsPad + j] = j < a.H ? ldexpf(wj, -e) : 0.0f;
}

__device__ static void fill_u32(uint32_t *p, int64_t n, uint32_t v, int64_t i0, int64_t step) {
  for (int64_t i = i0; i < n; i += step) p[i] = v;
}

constexpr int kBeginClearBlocks = 32;

// With a page table: every page a request's tokens use lies in the pool
// (out-of-range contexts are the request table's error).  kPageBlocks workgroups,
// kPageBlocks / B per request, each taking every (kPageBlocks / B)-th run of 256
// entries of its request's row (no division per entry).
constexpr int kPageBlocks = 256;

__device__ static void check_pages(const StepArgs &a, int blk) {
  const int bpr = kPageBlocks / a.B;  // B <= kMaxBatch = 64, so at least 4
  const int b = blk / bpr, part = blk - b * bpr;
  if (b >= a.B) return;
  const int c = a.ctx_len[b];
  if (c <= 0 || c > a.max_ctx) return;
  const int np = (c + 15) / 16 < a.page_stride ? (c + 15) / 16 : a.page_stride;
  const int32_t *row = a.pages + (int64_t)b * a.page_stride;
  bool bad = false;
  for (int j = part * 256 + (int)threadIdx.x; j < np; j += bpr * 256)
    bad |= !page_in_pool(a, row[j]);
  if (bad) fail(a.ws.status, ECHO_EDEVARG);
}

__global__ __launch_bounds__(256) void k_begin(StepArgs a, int roles) {
  // the status is read here and looked at only after each role has issued its
  // own reads (a kernel that follows an error changes nothing)
  const int32_t st0 = __hip_atomic_load(a.ws.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  int blk = blockIdx.x;
  if (blk == 0) {
    if (roles & BEGIN_REQ) {
      const bool overlap = !a.pages && a.B > 1 && ranges_overlap(a);
      build_request_table(a, st0, overlap);
    }
    if (st0 != 0) return;
    // small per-request arrays and counters
    const int tid = threadIdx.x;
    if ((roles & BEGIN_CLR_INDEX) && tid < a.max_batch) {
      a.ws.n_pf[tid] = 0;
      a.ws.n_cand[tid] = 0;
    }
    if ((roles & BEGIN_CLR_INDEX) && tid == 0) a.ws.counters[ECHO_CNT_PREFETCH] = 0;
    if ((roles & BEGIN_CLR_INDEX) && (tid == M_SCORE_DONE || tid == M_TOPK_DONE))
      a.sc.misc[tid] = 0;
    if ((roles & BEGIN_CLR_TOPK) && tid == 0) a.ws.counters[ECHO_CNT_SHORTCUT] = 0;
    if (roles & BEGIN_CLR_MANAGE) {
      if (tid < 4) a.sc.ecnt[tid] = 0;
      if (tid >= M_BAR0 && tid <= M_TOPK_DONE) a.sc.misc[tid] = 0;
      if (tid < ECHO_NCOUNTERS && tid != ECHO_CNT_PREFETCH && tid != ECHO_CNT_SHORTCUT)
        a.ws.counters[tid] = 0;
    }
    return;
  }
  blk -= 1;
  if (roles & BEGIN_Q) {
    if (blk < 4 * a.B) {
      stage_query(a, blk >> 2, blk & 3, st0);
      return;
    }
    blk -= 4 * a.B;
  }
  if (blk >= kBeginClearBlocks) {
    blk -= kBeginClearBlocks;
    if ((roles & BEGIN_REQ) && a.pages && st0 == 0 && a.B > 0) check_pages(a, blk);
    return;
  }
  if (st0 != 0) return;
  const int64_t i0 = (int64_t)blk * blockDim.x + threadIdx.x;
  const int64_t step = (int64_t)kBeginClearBlocks * blockDim.x;
  if (roles & BEGIN_CLR_INDEX) {
    fill_u32((uint32_t *)a.sc.tstate, 2LL * a.sc.max_tiles, 0u, i0, step);
    fill_u32((uint32_t *)a.sc.pfn, 2LL * a.max_batch, 0u, i0, step);
    fill_u32((uint32_t *)a.sc.cstate, 2LL * kCopyBlocks * kScoreWaves, 0u, i0, step);
  }
  if (roles & BEGIN_CLR_MANAGE) {
    fill_u32(a.sc.ehist, kBins, 0u, i0, step);
    fill_u32((uint32_t *)a.sc.estate, 2LL * a.sc.atiles, 0u, i0, step);
    fill_u32((uint32_t *)a.sc.astate, 2LL * a.sc.atiles, 0u, i0, step);
  }
}

hipError_t launch_begin(const StepArgs &a, int roles, hipStream_t s) {
  const int grid = 1 + ((roles & BEGIN_Q) ? 4 * a.B : 0) + kBeginClearBlocks +
                   ((roles & BEGIN_REQ) && a.pages ? kPageBlocks : 0);
  hipLaunchKernelGGL(k_begin, dim3(grid), dim3(256), 0, s, a, roles);
  return hipGetLastError();
}

// ----------------------------------------------------------- indexer K layout

// Row-major [n_rows][D] -> tiled, one thread per 16-byte piece: piece q of group
// g is load j = q / (D/2) of lane l = q % (D/2) = 16c + r, i.e. dims
// 32c + 16j .. +15 of row 16g + r.
__global__ __launch_bounds__(256) void k_kindex_pack(const uint8_t *rows, uint8_t *tiled,
                                                     int64_t n_rows, int D) {
  const int64_t pieces = n_rows * D / 16;
  const int half = D / 2;
  for (int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x; p < pieces;
       p += (int64_t)gridDim.x * 256) {
    const int64_t g = p / D;
    const int q = (int)(p - g * D);
    const int j = q / half, l = q - j * half;
    const int c = l >> 4, r = l & 15;
    const uint4 v = *(const uint4 *)(rows + (g * 16 + r) * D + 32 * c + 16 * j);
    *(uint4 *)(tiled + p * 16) = v;
  }
}

hipError_t launch_kindex_pack(const uint8_t *rows, uint8_t *tiled, int64_t n_rows, int D,
                              hipStream_t s) {
  const int64_t pieces = n_rows * D / 16;
  if (pieces == 0) return hipSuccess;
  int64_t grid = (pieces + 255) / 256;
  if (grid > 8192) grid = 8192;
  hipLaunchKernelGGL(k_kindex_pack, dim3((unsigned)grid), dim3(256), 0, s, rows, tiled, n_rows,
                     D);
  return hipGetLastError();
}

// ------------------------------------------------------------------ score

constexpr int kChunks = kScoreTile / 64;  // 64-token chunks per work item

// The page table through the constant address space: no kernel writes it, and
// saying so lets the compiler read its wave-uniform entries with scalar loads.
// Through a generic pointer, in the kernels that also store (the prefetch
// installs), the entries became vector loads, and waiting for one -- it feeds the
// next chunk's K addresses -- also waited for every K load issued before it (the
// in-step scoring kernel took 132 us instead of 105).
typedef const int32_t __attribute__((address_space(4))) const_i32;
__device__ inline const const_i32 *page_table(const StepArgs &a) {
  return (const const_i32 *)a.pages;
}

// Tiled-K groups (host id / 16, wave-uniform) of the four 16-token sub-tiles of
// the chunk that starts at token s0 (a multiple of 64) of request b: from the page
// table (PAGED, one page per group: scalar loads, issued a chunk before the K loads
// that use them), or from the request's contiguous range.  Sub-tiles past the
// context take the request's last group (in bounds; their scores are dropped).
template <bool PAGED>
__device__ inline void chunk_groups(const StepArgs &a, const ReqInfo &r, int b, int s0,
                                    int32_t (&grp)[4]) {
  const int glast = (r.ctx - 1) & ~15;
  const int s0u = __builtin_amdgcn_readfirstlane(s0);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int st = s0u + 16 * u;
    const int sg = st < r.ctx ? st : glast;
    const int32_t g =
        PAGED ? page_table(a)[(int64_t)b * a.page_stride + (sg >> 4)] : (r.base + sg) >> 4;
    grp[u] = __builtin_amdgcn_readfirstlane(g);
  }
}

// K operands of one 64-token chunk for this lane (tokens s0 .. s0+63 of request
// r, s0 a multiple of 64, in the groups `grp`): sub-tile u holds tokens s0 + 16u .. +15; this lane
// feeds token s0 + 16u + (lane & 15) with dims 32c .. 32c+31, c = lane >> 4, read
// as two 16-byte pieces at 16*lane and 8*D + 16*lane inside the token's 16-row
// group.  The loads go straight into the operand registers, with no select
// after them, so the compiler waits for them only where the MFMA reads them and
// the next chunk stays in flight while this one computes.  Tokens past the
// context read the request's last group (in bounds; their scores are dropped),
// and lanes whose dims lie past D read the same token's first 32 dims, which
// meet the zero padding of q (an exact 0 for any finite e4m3 byte).
__device__ inline void load_k_chunk(const StepArgs &a, const int32_t (&grp)[4], int lane,
                                    v8i (&kb)[4], bool real = true) {
  const bool dim_ok = 32 * (lane >> 4) < a.D;
  const int lp = dim_ok ? lane : (lane & 15);
  // real = false (no next item): every lane reads the same 16 bytes, one cache
  // line per instruction, only to keep the load count the same on every path.
  // The choice is made on offsets, as products with a wave-uniform 0/1 that went
  // through readfirstlane: a select between two pointers lets the compiler turn
  // the load of a select into a select of two loads, which it lowers into two
  // exec-masked load paths joined by a wait for every load in flight (once per
  // work item, measured 3-4% of the scoring time).
  const uint32_t rl = (uint32_t)__builtin_amdgcn_readfirstlane(real ? 1 : 0);
  const uint32_t half = (uint32_t)(8 * a.D) * rl;
  // wave-uniform 64-bit group address + 32-bit lane offset: the loads use the
  // scalar-base addressing form and need no per-lane 64-bit arithmetic
  const uint32_t lo = (uint32_t)lp * 16u * rl;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const uint64_t go = (uint64_t)((int64_t)grp[u] * 16 * a.D) * rl;
    const uint32_t go_lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)go);
    const uint32_t go_hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(go >> 32));
    const uint8_t *g = a.kidx + (((uint64_t)go_hi << 32) | go_lo);
    const v4i x0 = __builtin_nontemporal_load((const v4i *)(g + lo));
    const v4i x1 = __builtin_nontemporal_load((const v4i *)(g + (lo + half)));
    kb[u] = __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
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
      // ReLU as an integer max on the bits: one instruction, where fmaxf also
      // quiets NaNs with a second one (an MFMA sum of finite products is finite)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        v += wr[hg][rr] * __int_as_float(max(__float_as_int(acc[rr]), 0));
    }
    v = sum_lane_groups16(v);
    sc4[u] = v;  // every lane with (lane & 15) == i holds the score of token 16u + i
  }
  const int sel = lane >> 4;
  return sel == 0 ? sc4[0] : sel == 1 ? sc4[1] : sel == 2 ? sc4[2] : sc4[3];
}

// Prefetch epilogue of work item pi of request r, in two parts.  Candidates are
// the tokens above the threshold (`above`) whose map entry (`gq`, read while
// scoring) is -1; pf_publish counts them and publishes the count for the
// look-back over the request's items.  pf_install, a few chunks later, gets
// their rank in token order from the look-back; ranks below the cap take
// free-list entries idxbuf[off + rank] (while the list lasts), are installed in
// the maps with priority t and published, by rank, to the copy waves.  The
// request's last item publishes n_cand, n_pf and the final count the copy waves
// stop at.
__device__ inline int pf_publish(const StepArgs &a, const ReqInfo &r, int pi,
                                 const uint64_t (&above)[kChunks], const int (&gq)[kChunks],
                                 uint64_t (&cand)[kChunks]) {
  const int lane = lane_id();
  int c_all = 0;
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    cand[c] = __ballot(((above[c] >> lane) & 1ull) && gq[c] == -1);
    c_all += __popcll(cand[c]);
  }
  lb_publish(a.sc.tstate, r.tile0 + pi, r.tile0, c_all);
  return c_all;
}

// Ranks of this lane's candidates in item pi (at most one per chunk), given the
// item's exclusive prefix E: bit c of `tk` says whether the chunk-c candidate
// takes a slot, and gi[c] is the free-list position it reads (0, a dummy read,
// where it takes none).  The caller issues the reads together, without branches,
// and pf_commit consumes them.
__device__ inline void pf_plan(const StepArgs &a, const ReqInfo &r, const uint64_t (&cand)[kChunks],
                               int E, int nfree, int (&rank)[kChunks], int &tk,
                               int (&gi)[kChunks]) {
  const int lane = lane_id();
  const int lim = nfree < a.n_gpu ? nfree : a.n_gpu;
  int rank0 = E;
  tk = 0;
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const uint64_t m = cand[c];
    rank[c] = rank0 + __popcll(m & lanemask_lt());
    if (((m >> lane) & 1ull) && rank[c] < r.cap && r.off + rank[c] < lim) tk |= 1 << c;
    rank0 += __popcll(m);
  }
#pragma unroll
  for (int c = 0; c < kChunks; ++c) gi[c] = ((tk >> c) & 1) ? r.off + rank[c] : 0;
}

// Installs the planned candidates of item pi (maps, priority t, the rank-ordered
// lists and the copy queue); the request's last item also publishes n_cand, n_pf
// and the final count the copy waves stop at.
template <bool PAGED>
__device__ inline void pf_commit(const StepArgs &a, const ReqInfo &r, int b, int pi, int c_all,
                                 int E, const int (&rank)[kChunks], int tk,
                                 const int (&gv)[kChunks], const int (&gp)[kChunks], int t,
                                 int nfree) {
  const int lane = lane_id();
  const int s_wave = pi * kScoreTile;
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const int g = gv[c];
    if (((tk >> c) & 1) && g >= 0 && g < a.n_gpu) {
      const int s = s_wave + c * 64 + lane;
      const int64_t h = PAGED ? 16LL * gp[c] + (s & 15) : (int64_t)r.base + s;
      a.h2g[h] = g;
      a.g2h[g] = (int32_t)h;
      a.freef[g] = 0;
      a.prio[g] = t;
      a.ws.pf_tok[(int64_t)b * a.K + rank[c]] = s;
      a.ws.pf_slot[(int64_t)b * a.K + rank[c]] = g;
      __hip_atomic_store(&a.sc.pfq[(int64_t)b * a.K + rank[c]],
                         (1ull << 63) | ((uint64_t)h << 31) | (uint64_t)g, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (pi == r.ntiles - 1 && lane == 0) {
    const int lim = nfree < a.n_gpu ? nfree : a.n_gpu;
    const int total = E + c_all;
    const int take = min(r.cap, total);
    const int npf = max(0, min(take, lim - r.off));
    a.ws.n_cand[b] = total;
    a.ws.n_pf[b] = npf;
    if (npf) atomicAdd(&a.ws.counters[ECHO_CNT_PREFETCH], npf);
    __hip_atomic_store(&a.sc.pfn[b], (1ull << 32) | (uint64_t)npf, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Whether item pi's epilogue has anything to do after its count is published:
// an item without candidates needs no rank (later items sum through its count),
// except the request's last item, which publishes the totals.
__device__ inline bool pf_needed(const ReqInfo &r, int pi, int c_all) {
  return c_all > 0 || pi == r.ntiles - 1;
}

// Page-table entries of the planned candidates of item pi (0 where a lane takes no
// slot: a dummy in-bounds read), issued with the free-list reads.
template <bool PAGED>
__device__ inline void pf_pages(const StepArgs &a, int b, int pi, int tk, int (&gp)[kChunks]) {
  const int lane = lane_id();
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    gp[c] = 0;
    if (PAGED) {
      const int s = pi * kScoreTile + c * 64 + lane;
      gp[c] = page_table(a)[(int64_t)b * a.page_stride + (((tk >> c) & 1) ? (s >> 4) : 0)];
    }
  }
}

// Blocking epilogue: resolve item pi's rank, then install.
template <bool PAGED>
__device__ static void pf_install(const StepArgs &a, const ReqInfo &r, int b, int pi,
                                  const uint64_t (&cand)[kChunks], int c_all, int t,
                                  int nfree) {
  const int E = lb_resolve(a.sc.tstate, r.tile0 + pi, r.tile0, c_all, a.ws.status);
  int rank[kChunks], tk = 0, gi[kChunks], gv[kChunks], gp[kChunks];
#pragma unroll
  for (int c = 0; c < kChunks; ++c) rank[c] = gi[c] = 0;
  if (c_all > 0) pf_plan(a, r, cand, E, nfree, rank, tk, gi);
#pragma unroll
  for (int c = 0; c < kChunks; ++c) gv[c] = a.idxbuf[gi[c]];
  pf_pages<PAGED>(a, b, pi, tk, gp);
  pf_commit<PAGED>(a, r, b, pi, c_all, E, rank, tk, gv, gp, t, nfree);
}

// Epilogues waiting for their rank, per wave, in a ring in LDS.  An item's count
// is published at the next item's chunk 0 and the item is queued; the oldest
// queued item's look-back states are read at chunk 1 and examined at chunk 2
// without waiting: if the items before it have all published, its free-list
// reads go out at chunk 2 and its installs at chunk 3, else it stays queued for
// the next item.  A wave that runs ahead of its neighbours therefore keeps
// scoring; it waits only when the ring is full or at the end of its job, always
// after publishing its own counts, so every wait ends.  (A short queue made the
// waves of a request move in lockstep with the slowest of them: with more waves
// per request the scoring time did not drop at all.)
constexpr int kPending = 8;

struct PendItem {
  int32_t pi, c;
  uint64_t cand[kChunks];
};

// A queued item's candidate masks as lane 0 wrote them.  Lane 0 alone writes an
// entry; the other lanes take its view through readfirstlane, since for them an
// LDS read of lane 0's write with no barrier between is a data race, which the
// compiler may resolve by reading before the write (a variant that installed an
// item right after queueing it got wrong masks and missing installs that way).
__device__ inline void pend_cand(const PendItem &e, uint64_t (&oc)[kChunks]) {
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const uint64_t v = e.cand[c];
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
    oc[c] = ((uint64_t)hi << 32) | lo;
  }
}

// Scores a wave holds in LDS before it writes them out (items of 256 tokens).
constexpr int kDeferItems = 8;

// A scoring wave's LDS: the scores and selection-guard candidates of its
// buffered items.
struct WaveBuf {
  float score[kDeferItems * kScoreTile];
  uint32_t gkey[kDeferItems * kGuardSlots];
  int32_t gidx[kDeferItems * kGuardSlots];
  int32_t gcnt[kDeferItems];
};

// Job k of request r: its items k, k + wb, ...  Scores and selection-guard
// candidates are written to LDS (`wbuf`, kDeferItems items of this wave) and go
// out to HBM only when that buffer is full or the job ends.  Score stores interleaved with the K stream
// cost more than their bytes: on 2.8M tokens, leaving them out shortened the
// launch by 5-8 us of about 70, and gathering them at the end of each wave's
// job shortened it by 4-5 us.
template <int HG, bool PF, bool PAGED>
__device__ static void score_job(const StepArgs &a, const ReqInfo &r, int b, int k, int t,
                                 int nfree, PendItem *pq, WaveBuf *wbuf) {
  const int lane = lane_id();
  // Operand layout: lane l feeds row (l & 15) of A (a head) and column (l & 15)
  // of B (a token) with the 32 bytes at dims chunk .. chunk+31,
  // chunk = 32*(l >> 4).  A and B use the same dims for the same lane, so the
  // MFMA sums q . k over all 128 dims whatever order it adds them in.
  const int row = lane & 15, chunk = (lane >> 4) * 32;
  v8i qa[HG][2];
  float wr[HG][4];
  {
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
  }
  float *out = a.ws.scores + (int64_t)b * a.max_ctx;
  // buffered items: i0, i0 + wb, ... (nbuf of them).  Each lane writes out the
  // scores it put in LDS itself; guard candidates were put there by other lanes
  // of the wave, whose LDS writes the fence orders before these reads.
  int nbuf = 0, i0 = k;
  auto flush = [&]() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    for (int j = 0; j < nbuf; ++j) {
      const int it = i0 + j * r.wb;
#pragma unroll
      for (int c = 0; c < kChunks; ++c) {
        const int s = it * kScoreTile + c * 64 + lane;
        const float v = wbuf->score[(j * kChunks + c) * 64 + lane];
        if (s < r.ctx) out[s] = v;
      }
      if (r.use_guard) {
        const int64_t tau = r.tile0 + it;
        const int n = __builtin_amdgcn_readfirstlane(wbuf->gcnt[j]);  // lane 0 wrote it
        if (lane < kGuardSlots && lane < n) {
          a.sc.gcand_key[tau * kGuardSlots + lane] = wbuf->gkey[j * kGuardSlots + lane];
          a.sc.gcand_idx[tau * kGuardSlots + lane] = wbuf->gidx[j * kGuardSlots + lane];
        }
        if (lane == 0) a.sc.gcand_cnt[tau] = n;
      }
    }
  };
  // Two K buffers: chunk c of an item lives in kb[c & 1]; the next chunk (the
  // next item's first one at the end of an item) is in flight while c computes.
  v8i kb[2][4];
  int i = k;
  // groups of the chunk being scored (gcur) and of the chunk whose loads go out next
  // (gnext); each chunk's groups are read one chunk before its loads are issued
  int32_t gcur[4], gnext[4];
  chunk_groups<PAGED>(a, r, b, i * kScoreTile, gcur);
  load_k_chunk(a, gcur, lane, kb[0]);
  chunk_groups<PAGED>(a, r, b, i * kScoreTile + 64, gnext);
  // the previous item's threshold bits and map entries (its epilogue's inputs)
  bool have_prev = false;
  int p_i = 0;
  uint64_t p_above[kChunks];
  int p_g[kChunks];
  // queued epilogues: ring pq[qh .. qh + qn) (see kPending), and the progress of
  // the oldest one
  int qh = 0, qn = 0;
  uint64_t sv = 0;
  bool planned = false;
  int o_i = 0, o_c = 0;  // the oldest queued item and its count
  int E0 = 0, tk = 0, rk[kChunks], gv[kChunks], gp[kChunks];
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    p_above[c] = 0;
    p_g[c] = 0;
    rk[c] = gv[c] = gp[c] = 0;
  }
  auto read_oldest = [&]() {
    o_i = __builtin_amdgcn_readfirstlane(pq[qh].pi);
    o_c = __builtin_amdgcn_readfirstlane(pq[qh].c);
  };
  auto install_oldest = [&]() {  // blocking
    uint64_t oc[kChunks];
    pend_cand(pq[qh], oc);
    read_oldest();
    pf_install<PAGED>(a, r, b, o_i, oc, o_c, t, nfree);
    qh = qh + 1 == kPending ? 0 : qh + 1;
    --qn;
  };
  // publish the previous item's count and queue its epilogue (finishing the
  // oldest queued one first if the ring is full)
  auto publish_prev = [&]() {
    uint64_t xc[kChunks];
    const int xcall = pf_publish(a, r, p_i, p_above, p_g, xc);
    if (!pf_needed(r, p_i, xcall)) return;
    if (qn == kPending) install_oldest();
    int slot = qh + qn;
    slot = slot >= kPending ? slot - kPending : slot;
    if (lane == 0) {
      pq[slot].pi = p_i;
      pq[slot].c = xcall;
#pragma unroll
      for (int c = 0; c < kChunks; ++c) pq[slot].cand[c] = xc[c];
    }
    ++qn;
  };
  while (true) {
    const int s_wave = i * kScoreTile;
    const int ni = i + r.wb;
    uint64_t above[kChunks], gsel[kChunks];
    uint32_t keys[kChunks];
    int gq[kChunks];
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int s = s_wave + c * 64 + lane;
      const bool valid = s < r.ctx;
      // the chunk's map entries go out before the next chunk's K loads: they are
      // consumed an item later, and a load issued after those K loads could not
      // be waited for without waiting for them too
      gq[c] = 0;
      if (PF) {
        // this lane's token (or the request's last one past the context), in the
        // group of its sub-tile
        const int ts = valid ? s : r.ctx - 1;
        const int u = lane >> 4;
        const int32_t g = u == 0 ? gcur[0] : u == 1 ? gcur[1] : u == 2 ? gcur[2] : gcur[3];
        gq[c] = a.h2g[16LL * g + (ts & 15)];
      }
      if (c + 1 < kChunks) {
        load_k_chunk(a, gnext, lane, kb[(c + 1) & 1]);
      } else {
        // unconditional (after the last item, a one-line dummy read): a load under
        // a branch would make the compiler drain every load before the join
        load_k_chunk(a, gnext, lane, kb[0], ni < r.ntiles);
      }
      {  // the groups of the chunk after the one just issued
        int32_t gafter[4];
        const int s_after = c + 2 < kChunks ? s_wave + (c + 2) * 64
                            : (ni < r.ntiles ? ni * kScoreTile + (c + 2 - kChunks) * 64 : s_wave);
        chunk_groups<PAGED>(a, r, b, s_after, gafter);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          gcur[u] = gnext[u];
          gnext[u] = gafter[u];
        }
      }
      const float score = score_chunk<HG>(kb[c & 1], qa, wr, lane);
      wbuf->score[(nbuf * kChunks + c) * 64 + lane] = score;
      keys[c] = topk_key(score);
      gsel[c] = __ballot(r.use_guard && valid && keys[c] <= r.guard_key);
      above[c] = 0;
      if (PF) {
        above[c] = __ballot(valid && score > r.theta);
        if (c == 0 && have_prev) publish_prev();
        // The look-back state loads (chunk 1) and the free-list reads (chunk 2) go
        // out on every item, dummy ones when nothing is queued or planned: loads
        // issued on some paths only would leave the compiler unable to count the
        // loads in flight where their results are used, and it would wait for all.
        if (c == 1) {
          if (qn > 0) read_oldest();
          sv = lb_try_load(a.sc.tstate, r.tile0 + (qn > 0 ? o_i : 0), r.tile0);
        }
        if (c == 2) {
          int gi[kChunks];
#pragma unroll
          for (int cc = 0; cc < kChunks; ++cc) gi[cc] = 0;
          tk = 0;
          if (qn > 0 &&
              lb_try_finish(a.sc.tstate, r.tile0 + o_i, r.tile0, o_c, sv, a.ws.status, E0)) {
            if (o_c > 0) {
              uint64_t oc[kChunks];
              pend_cand(pq[qh], oc);
              pf_plan(a, r, oc, E0, nfree, rk, tk, gi);
            }
            planned = true;
          }
#pragma unroll
          for (int cc = 0; cc < kChunks; ++cc) gv[cc] = a.idxbuf[gi[cc]];
          pf_pages<PAGED>(a, b, qn > 0 ? o_i : 0, tk, gp);
        }
        if (c == 3 && planned) {
          pf_commit<PAGED>(a, r, b, o_i, o_c, E0, rk, tk, gv, gp, t, nfree);
          planned = false;
          qh = qh + 1 == kPending ? 0 : qh + 1;
          --qn;
        }
      }
    }

    // ---- top-k candidates above the selection guard: fixed slots of this item
    // (buffered in LDS with the scores and written to item r.tile0 + i at the flush)
    if (r.use_guard) {
      int ng = 0;
#pragma unroll
      for (int c = 0; c < kChunks; ++c) {
        if ((gsel[c] >> lane) & 1ull) {
          const int p = ng + __popcll(gsel[c] & lanemask_lt());
          if (p < kGuardSlots) {
            wbuf->gkey[nbuf * kGuardSlots + p] = keys[c];
            wbuf->gidx[nbuf * kGuardSlots + p] = s_wave + c * 64 + lane;
          }
        }
        ng += __popcll(gsel[c]);
      }
      if (lane == 0) wbuf->gcnt[nbuf] = ng;
    }
    if (PF) {
      p_i = i;
#pragma unroll
      for (int c = 0; c < kChunks; ++c) {
        p_above[c] = above[c];
        p_g[c] = gq[c];
      }
      have_prev = true;
      if (i == k && ni < r.ntiles) {
        // the job's first item: its rank now, so that its rows reach the copy
        // waves early (the items before it are the other waves' first items,
        // finished at about the same time)
        publish_prev();
        while (qn > 0) install_oldest();
        have_prev = false;
      }
    }
    if (++nbuf == kDeferItems) {
      flush();
      nbuf = 0;
      i0 = ni;
    }
    if (ni >= r.ntiles) break;
    i = ni;
  }
  if (nbuf) flush();
  if (PF && have_prev) {
    publish_prev();
    while (qn > 0) install_oldest();
  }
}

// The request's fields in scalar registers: read from LDS they would sit in
// vector registers, and every address derived from them would take per-lane
// 64-bit arithmetic.
__device__ inline ReqInfo wave_uniform(const ReqInfo &x) {
  ReqInfo r;
  static_assert(sizeof(ReqInfo) % 4 == 0, "ReqInfo is made of 32-bit fields");
  const int32_t *src = (const int32_t *)&x;
  int32_t *dst = (int32_t *)&r;
#pragma unroll
  for (int i = 0; i < (int)(sizeof(ReqInfo) / 4); ++i)
    dst[i] = __builtin_amdgcn_readfirstlane(src[i]);
  return r;
}

// A scoring wave takes jobs w, w + W, ... (W = scoring waves of the launch); job
// slots are numbered request by request, so a wave meets its requests in
// increasing order and every look-back wait is on an item that a resident wave
// reaches without waiting on a later one.
template <int HG, bool ANY_PF, bool PAGED>
__device__ static void score_wave(const StepArgs &a, const ReqInfo *s_req, int w, PendItem *pq,
                                  WaveBuf *wbuf) {
  const int lane = lane_id();
  const int S = a.sc.misc[M_SLOTS];
  const int W = a.score_waves;
  const int t = a.ctl[ECHO_CTL_STEP];
  const int nfree = a.ctl[ECHO_CTL_NFREE];
  const int send = lane < a.B ? s_req[lane].slot0 + s_req[lane].wb : 0;
  for (int slot = w; slot < S; slot += W) {
    const int b = __popcll(__ballot(lane < a.B && send <= slot));
    const ReqInfo r = wave_uniform(s_req[b]);
    const int k = slot - r.slot0;
    if (ANY_PF && r.active)
      score_job<HG, true, PAGED>(a, r, b, k, t, nfree, pq, wbuf);
    else
      score_job<HG, false, PAGED>(a, r, b, k, t, nfree, pq, wbuf);
  }
}

// The first score_blocks workgroups score, the rest copy prefetched rows (until
// scoring ends, when the copy continues in the step's next kernels, else to the
// end).  ANY_PF = false (threshold +inf) compiles the prefetch path out.
template <int HG, bool ANY_PF, bool PAGED>
__global__ __launch_bounds__(512) void k_score(StepArgs a) {
  __shared__ ReqInfo s_req[kMaxBatch];
  __shared__ PendItem s_pend[ANY_PF ? kScoreWaves : 1][ANY_PF ? kPending : 1];
  __shared__ WaveBuf s_wbuf[kScoreWaves];  // 81 KB
  __shared__ int s_left, s_dead;
  const int tid = threadIdx.x;
  // the status and the request table in one round trip; the block decides as one
  for (int i = tid; i < a.B; i += blockDim.x) s_req[i] = a.sc.req[i];
  if (tid == 0) {
    s_left = kScoreWaves;
    s_dead = failed(a.ws.status);
  }
  __syncthreads();
  if (s_dead) return;
  const int wid = tid / kWave;
  int role_idx;
  const bool copy = xcd_copy_role((int)blockIdx.x, (int)gridDim.x, a.copy_waves / kScoreWaves,
                                  &role_idx);
  if (!copy) {
    // the wave index through readfirstlane: every job index derived from it is
    // then known to be wave-uniform and lives in scalar registers
    score_wave<HG, ANY_PF, PAGED>(a, s_req,
                           __builtin_amdgcn_readfirstlane(role_idx * kScoreWaves + wid),
                           &s_pend[ANY_PF ? wid : 0][0], &s_wbuf[wid]);
    if (lane_id() == 0 && atomicSub(&s_left, 1) == 1)
      __hip_atomic_fetch_add(&a.sc.misc[M_SCORE_DONE], 1, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
  } else if (ANY_PF) {
    copy_worker(a, s_req, role_idx * kScoreWaves + wid, 0, 1,
                a.copy_handoff ? &a.sc.misc[M_SCORE_DONE] : nullptr, a.score_blocks);
  }
}

template <bool ANY_PF, bool PAGED>
static void launch_score_hg(const StepArgs &a, int grid, hipStream_t s) {
  switch ((a.H + 15) / 16) {
    case 1: hipLaunchKernelGGL((k_score<1, ANY_PF, PAGED>), dim3(grid), dim3(512), 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_score<2, ANY_PF, PAGED>), dim3(grid), dim3(512), 0, s, a); break;
    case 3: hipLaunchKernelGGL((k_score<3, ANY_PF, PAGED>), dim3(grid), dim3(512), 0, s, a); break;
    default: hipLaunchKernelGGL((k_score<4, ANY_PF, PAGED>), dim3(grid), dim3(512), 0, s, a); break;
  }
}

// Compute units of the current device (cached per device).
int device_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n < 1)
      n = 1;
    cache[dev] = n;
  }
  return cache[dev];
}

int score_resident_per_cu() {
  static int cache[64] = {0};  // per device: 0 not asked yet, -1 none fits, else the count
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cache[dev] == 0) {
    const void *fns[] = {
        reinterpret_cast<const void *>(&k_score<1, false, false>),
        reinterpret_cast<const void *>(&k_score<2, false, false>),
        reinterpret_cast<const void *>(&k_score<3, false, false>),
        reinterpret_cast<const void *>(&k_score<4, false, false>),
        reinterpret_cast<const void *>(&k_score<1, true, false>),
        reinterpret_cast<const void *>(&k_score<2, true, false>),
        reinterpret_cast<const void *>(&k_score<3, true, false>),
        reinterpret_cast<const void *>(&k_score<4, true, false>),
        reinterpret_cast<const void *>(&k_score<1, false, true>),
        reinterpret_cast<const void *>(&k_score<2, false, true>),
        reinterpret_cast<const void *>(&k_score<3, false, true>),
        reinterpret_cast<const void *>(&k_score<4, false, true>),
        reinterpret_cast<const void *>(&k_score<1, true, true>),
        reinterpret_cast<const void *>(&k_score<2, true, true>),
        reinterpret_cast<const void *>(&k_score<3, true, true>),
        reinterpret_cast<const void *>(&k_score<4, true, true>)};
    int m = 1 << 30;
    for (const void *f : fns) {
      int n = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, f, 512, 0) != hipSuccess) n = 0;
      m = n < m ? n : m;
    }
    cache[dev] = m > 0 ? m : -1;
  }
  return cache[dev] > 0 ? cache[dev] : 0;
}

void index_grid(const echo_dims_t &d, bool with_copy, int *score_blocks, int *copy_blocks) {
  const int cus = device_cus();
  int gc = cus / 8 < kCopyBlocks ? cus / 8 : kCopyBlocks;
  if (gc < 1) gc = 1;
  if (!with_copy) gc = 0;  // prefetch off: every workgroup scores
  const int64_t max_tiles =
      (int64_t)d.max_batch * (((int64_t)d.max_ctx + kScoreTile - 1) / kScoreTile);
  int64_t gs = (max_tiles + kScoreWaves - 1) / kScoreWaves;
  if (gs > cus - gc) gs = cus - gc;
  if (gs < 1) gs = 1;
  *score_blocks = (int)gs;
  *copy_blocks = gc;
}

hipError_t launch_score(const StepArgs &a, hipStream_t s) {
  const int grid = a.score_blocks + a.copy_waves / kScoreWaves;
  const bool pf = a.mode != ECHO_THETA_POS_INF;
  if (a.pages) {
    if (pf) launch_score_hg<true, true>(a, grid, s);
    else launch_score_hg<false, true>(a, grid, s);
  } else {
    if (pf) launch_score_hg<true, false>(a, grid, s);
    else launch_score_hg<false, false>(a, grid, s);
  }
  return hipGetLastError();
}

}  // namespace echo
