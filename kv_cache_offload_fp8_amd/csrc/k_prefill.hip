// Chunked-prefill selection.
//
// The ECHO review ("Core method / prefill") splits a prefill into query chunks.
// While chunk i+1 is scored, the KV of the candidates already identified for
// chunk i moves over the host link.  The candidates come from a 256-bucket coarse
// histogram instead of a full top-k: the buckets strictly above the one holding
// the k-th score are certain members, and the boundary bucket waits for the exact
// selection.  Subtracting a predicted k-th score first makes the buckets fine near
// the boundary, so more tokens are certain; the exact fetch afterwards covers the
// rest.  "Core method / prefetch inside the indexer pipeline" splits the
// indexer's prefill work by query chunk.
//
// One request's history of N tokens (host ids hb .. hb+N-1, K resident in HBM in
// the tiled layout) is scored against the chunk's C queries.  Kernels per chunk:
//   k_pf_stage    q split into fp8 hi/lo with a per-head power-of-two scale
//   k_pf_score    scores [C][N] on the fp8 MFMA (the heads x tokens contraction
//                 for every query; each wave keeps two queries' operands in
//                 registers and streams 64-token K chunks; about one workgroup
//                 per compute unit, placed so that the workgroups of one XCD
//                 share one token range through its L2), and each query's
//                 histogram of the coarse buckets of fp16(score - pred),
//                 counted in LDS as the scores are made
//   k_pf_coarse   per query: the boundary bucket from that histogram, and the
//                 candidate flags above it (one pass over the row)
//   k_pf_flags_*  the union of flags as an ascending token list
//   k_pf_inst_*   install a list in order: resident tokens get priority t, the
//                 others take the next ascending free slots (idxbuf)
//   k_pf_exact    per query: exact top-k by (score desc, token asc), written in
//                 ascending token order, and its k-th score
//   k_pf_copy     host rows of an install list into the GPU pool
//   k_pf_shift_*  the unused rest of the free list moved to its front, the step
//                 counter
// The early install and its copy run right after the coarse pass, so the copy
// (on its own stream) overlaps the exact selection and the next chunk's scoring.
#include "prefill.h"
#include "select.h"

namespace echo {

typedef int v8i_pf __attribute__((ext_vector_type(8)));
typedef float v4f_pf __attribute__((ext_vector_type(4)));
typedef int v4i_pf __attribute__((ext_vector_type(4)));

constexpr int kPfCopyBlocks = 32;
// Word 3 of a raw buffer resource on gfx9: 32-bit data format (a zero format would
// make every access out of range), no swizzle, no stride.
constexpr int kRawBufWord3 = 0x00020000;  // a small grid keeps about 256 KB of host reads in flight

// The status as one workgroup sees it: read once and shared, so that all of its
// waves take the same branch before the block barriers that follow.
__device__ inline bool block_failed(const int32_t *status) {
  __shared__ int s_failed;
  if (threadIdx.x == 0) s_failed = failed(status) ? 1 : 0;
  __syncthreads();
  const bool f = s_failed != 0;
  __syncthreads();
  return f;
}

// ------------------------------------------------------------------ stage
// Query i, heads quarter*16 .. +15: thread = (head, 8 dims).  q' = q * 2^e with
// max |q'| in [128, 256); q_hi = e4m3(q'), q_lo = e4m3(q' - q_hi); the head weight
// takes 2^-e (ReLU is positively homogeneous).  Zero for padded heads and dims.
__global__ __launch_bounds__(256) void k_pf_stage(StepArgs a, PrefillArgs p) {
  if (failed(p.status)) return;
  const int i = blockIdx.x >> 2, quarter = blockIdx.x & 3;
  const int tid = threadIdx.x;
  const int j = quarter * 16 + (tid >> 4), d0 = (tid & 15) * 8;
  const uint16_t *src = p.q + (int64_t)i * a.H * a.D;
  const bool in = j < a.H && d0 < a.D;
  const uint4 w4 = in ? *(const uint4 *)(src + j * a.D + d0) : make_uint4(0, 0, 0, 0);
  const float wj = d0 == 0 && j < a.H ? p.w[(int64_t)i * a.H + j] : 0.0f;
  const uint32_t wd[4] = {w4.x, w4.y, w4.z, w4.w};
  float x[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    x[2 * k] = __uint_as_float(wd[k] << 16);
    x[2 * k + 1] = __uint_as_float(wd[k] & 0xFFFF0000u);
  }
  float amax = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(x[k]));
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  int e = 0;
  if (amax > 0.0f) {
    int E;
    frexpf(amax, &E);
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
  const int64_t o = ((int64_t)i * kHeadsPad + j) * kDimPad + d0;
  *(uint2 *)(p.qhi + o) = make_uint2(whi[0], whi[1]);
  *(uint2 *)(p.qlo + o) = make_uint2(wlo[0], wlo[1]);
  if (d0 == 0) p.wsc[(int64_t)i * kHeadsPad + j] = j < a.H ? ldexpf(wj, -e) : 0.0f;
  if (tid < 64) p.hist[(int64_t)i * 256 + quarter * 64 + tid] = 0;  // this chunk's histogram
}

// ------------------------------------------------------------------ score
// K operands of history tokens s0 .. s0+63 (s0 a multiple of 64): sub-tile u holds
// tokens s0 + 16u .. +15; lane l feeds token s0 + 16u + (l & 15) with dims
// 32(l >> 4) .. +31, two 16-byte pieces at 16 l and 8 D + 16 l inside the token's
// group of 16 (hb is a multiple of 16).  Tokens past the history read its last
// group (their scores are dropped); lanes whose dims lie past D read the first 32
// dims, which meet q's zero padding.
__device__ inline v8i_pf pf_load_k1(const StepArgs &a, const PrefillArgs &p, int s0, int u,
                                    int lane) {
  const int lp = 32 * (lane >> 4) < a.D ? lane : (lane & 15);
  const int glast = (p.N - 1) & ~15;
  const uint32_t lo = (uint32_t)lp * 16u, hi = lo + 8u * (uint32_t)a.D;
  const int st = __builtin_amdgcn_readfirstlane(s0) + 16 * u;
  const int sg = st < p.N ? st : glast;
  const uint8_t *g = a.kidx + ((int64_t)p.hb + sg) * a.D;
  const v4i_pf x0 = *(const v4i_pf *)(g + lo);
  const v4i_pf x1 = *(const v4i_pf *)(g + hi);
  return __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ inline void pf_load_k(const StepArgs &a, const PrefillArgs &p, int s0, int lane,
                                 v8i_pf (&kb)[4]) {
#pragma unroll
  for (int u = 0; u < 4; ++u) kb[u] = pf_load_k1(a, p, s0, u, lane);
}

// Bucket of a score shifted by the predicted k-th score: the difference in fp32,
// rounded to half precision (nearest even), then the top byte of an order key of
// the half bits (larger value, larger key; -0 counts as +0).
__device__ inline int pf_bucket(float score, float pred) {
  const _Float16 h = (_Float16)(score - pred);
  uint16_t u = __builtin_bit_cast(uint16_t, h);
  if (u == 0x8000) u = 0;
  const uint16_t key = (u & 0x8000) ? (uint16_t)~u : (uint16_t)(u | 0x8000);
  return key >> 8;
}

// Workgroup b: XCD x = b % 8 (the hardware's round-robin placement) takes token
// splits x * tsplits/8 .. , all query blocks of one split before the next, so the
// workgroups resident on one XCD read the same K range through its L2.
__global__ __launch_bounds__(kPfWaves * kWave) void k_pf_score(StepArgs a, PrefillArgs p) {
  // per-query histograms of this workgroup's coarse buckets, flushed at the end
  __shared__ uint32_t s_hist[kPfQBlock][256];
  for (int i = threadIdx.x; i < kPfQBlock * 256; i += kPfWaves * kWave) (&s_hist[0][0])[i] = 0;
  __syncthreads();
  const bool dead = failed(p.status);
  const int lane = lane_id(), wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int b = blockIdx.x, xcd = b & 7, jj = b >> 3;
  const int ts = xcd * (p.tsplits >> 3) + jj / p.qblocks, qb = jj % p.qblocks;
  const int q0 = qb * kPfQBlock + wave * kPfQ;
  const int nch = (p.N + 63) >> 6;
  const int per = (nch + p.tsplits - 1) / p.tsplits;
  const int c0 = ts * per, c1 = min(nch, c0 + per);
  // a wave with no query or no tokens does no work but still meets the barriers
  if (!dead && q0 < p.C && c0 < c1) {
    const int row = lane & 15, chunk = (lane >> 4) * 32;
    v8i_pf qa[kPfQ][4][2];
    float wr[kPfQ][4][4];
    float pr[kPfQ];
#pragma unroll
    for (int u = 0; u < kPfQ; ++u) {
      const int qi = min(q0 + u, p.C - 1);  // a missing second query repeats the first
      pr[u] = p.pred ? p.pred[qi] : 0.0f;
      const uint8_t *qh = p.qhi + (int64_t)qi * kHeadsPad * kDimPad;
      const uint8_t *ql = p.qlo + (int64_t)qi * kHeadsPad * kDimPad;
#pragma unroll
      for (int hg = 0; hg < 4; ++hg) {
        qa[u][hg][0] = *(const v8i_pf *)(qh + (hg * 16 + row) * kDimPad + chunk);
        qa[u][hg][1] = *(const v8i_pf *)(ql + (hg * 16 + row) * kDimPad + chunk);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          wr[u][hg][rr] = p.wsc[(int64_t)qi * kHeadsPad + hg * 16 + (lane >> 4) * 4 + rr];
      }
    }
    // Per chunk, lane l makes the score of token c*64 + l for each query: for each
    // sub-tile, head group and query, the q_hi and q_lo MFMAs, then ReLU (an integer
    // max on the float bits) and the weighted sum over the lane's four heads; the
    // four lane groups that share a token are summed last.  Sub-tile by sub-tile,
    // both queries' four head-group pairs run in sequence, and each pair's ReLU and
    // weighted sum are issued around the next pair's two MFMAs, so that the vector
    // work runs while the matrix core works.
    // One K register set: sub-tile u of chunk c + 1 loads as soon as the last MFMA
    // of chunk c that reads sub-tile u has issued (clamped to the split's last
    // chunk: at most one extra chunk read per wave, from L2).  A single set keeps
    // the wave near 210 registers, which leaves room on the compute unit for the
    // copy kernel's waves beside a scoring workgroup.
    // The scores go out through a raw buffer resource per query row: the hardware
    // drops stores at offsets past the resource's range (tokens past the history,
    // rows of missing queries, whose range is 0), so the chunk has no branch and
    // the compiler can count the loads in flight across it.
    v8i_pf kb[4];
    pf_load_k(a, p, c0 * 64, lane, kb);
    // Everything loaded so far is waited for here, so that the wait at the loop
    // head only covers what the previous chunk issued.  The immediate is gfx9's
    // s_waitcnt encoding of vmcnt(0) with the other counters left at their maxima.
    __builtin_amdgcn_s_waitcnt(0x0f70);
    const int sel = lane >> 4;
    __amdgpu_buffer_rsrc_t srow[kPfQ];
#pragma unroll
    for (int u = 0; u < kPfQ; ++u)
      srow[u] = __builtin_amdgcn_make_buffer_rsrc(p.scores + (int64_t)min(q0 + u, p.C - 1) * p.N,
                                                  0, q0 + u < p.C ? p.N * 4 : 0, kRawBufWord3);
    for (int c = c0; c < c1; ++c) {
      const int cn = min(c + 1, c1 - 1);
      float vs[kPfQ], vo[kPfQ];
      v4f_pf prev = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int j = 0; j <= 16 * kPfQ; ++j) {
        const bool mm = j < 16 * kPfQ, ep = j > 0;
        const int u = j / (4 * kPfQ), q = (j >> 2) % kPfQ, hg = j & 3;
        const int jp = j - 1, up = jp / (4 * kPfQ), qp = (jp >> 2) % kPfQ, hp = jp & 3;
        v4f_pf cur = {0.0f, 0.0f, 0.0f, 0.0f};
        float v = 0.0f;
        if (ep && hp != 0) v = vs[qp];
        if (mm)
          cur = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[q][hg][0], kb[u], cur, 0, 0,
                                                                 0, 0, 0, 0);
        if (ep) {
          v += wr[qp][hp][0] * __int_as_float(max(__float_as_int(prev[0]), 0));
          v += wr[qp][hp][1] * __int_as_float(max(__float_as_int(prev[1]), 0));
        }
        if (mm)
          cur = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[q][hg][1], kb[u], cur, 0, 0,
                                                                 0, 0, 0, 0);
        if (ep) {
          v += wr[qp][hp][2] * __int_as_float(max(__float_as_int(prev[2]), 0));
          v += wr[qp][hp][3] * __int_as_float(max(__float_as_int(prev[3]), 0));
          vs[qp] = v;
          if (hp == 3) {
            const float t = sum_lane_groups16(v);
            vo[qp] = (up == 0 || sel == up) ? t : vo[qp];
          }
        }
        if (mm && j % (4 * kPfQ) == 4 * kPfQ - 1) kb[u] = pf_load_k1(a, p, cn * 64, u, lane);
        // the order within the step: MFMA (q_hi), four vector instructions, MFMA
        // (q_lo), the rest; nothing crosses into the next step
        if (mm) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        prev = cur;
      }
      const int s = c * 64 + lane;
#pragma unroll
      for (int u = 0; u < kPfQ; ++u) {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(vo[u]), srow[u], s * 4, 0, 0);
        atomicAdd(&s_hist[wave * kPfQ + u][pf_bucket(vo[u], pr[u])],
                  (q0 + u < p.C && s < p.N) ? 1u : 0u);
      }
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kPfQBlock * 256; i += kPfWaves * kWave) {
    const int qq = qb * kPfQBlock + i / 256;
    const uint32_t v = (&s_hist[0][0])[i];
    if (v && qq < p.C) atomicAdd(&p.hist[(int64_t)qq * 256 + (i & 255)], v);
  }
}

// ------------------------------------------------------------------ coarse
__global__ __launch_bounds__(kSelThreads) void k_pf_coarse(StepArgs a, PrefillArgs p) {
  __shared__ int sh[kSelThreads / kWave + 1];
  __shared__ int s_beta;
  if (block_failed(p.status)) return;
  const int i = blockIdx.x, tid = threadIdx.x;
  const float pr = p.pred ? p.pred[i] : 0.0f;
  int beta = -1;
  if (p.N > a.K) {
    if (tid == 0) s_beta = 0;
    // the row's histogram, built by the scoring kernel; thread t < 256 holds bucket
    // 255 - t: the boundary is the first one, from the top, at which the running
    // count reaches k
    const int c = tid < 256 ? (int)p.hist[(int64_t)i * 256 + 255 - tid] : 0;
    int tot;
    const int excl = block_excl_scan<kSelThreads>(c, sh, &tot);
    if (tid < 256 && excl < a.K && excl + c >= a.K) s_beta = 255 - tid;
    __syncthreads();
    beta = s_beta;
  }
  // The row is read in 16-byte pieces of the score buffer (256-byte aligned, each
  // region padded to whole 256-byte lines): piece j holds the buffer's floats
  // 4j .. 4j+3, of which those outside the row are skipped.  Each thread loads
  // four pieces before it flags any token (the byte-wide flag stores may alias the
  // scores as far as the compiler knows), so four loads are in flight per thread.
  constexpr int U = 4;
  const int64_t f0 = (int64_t)i * p.N, f1 = f0 + p.N;
  const int64_t j0 = f0 >> 2, j1 = (f1 + 3) >> 2;
  const float4 *pc = reinterpret_cast<const float4 *>(p.scores);
  int cnt = 0;
  for (int64_t jb = j0 + tid; jb < j1; jb += (int64_t)U * kSelThreads) {
    float4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = jb + (int64_t)u * kSelThreads;
      v[u] = pc[j < j1 ? j : j0];  // a piece past the row rereads the row's first
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = jb + (int64_t)u * kSelThreads;
      const float e[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int64_t f = 4 * j + k;
        if (j < j1 && f >= f0 && f < f1 && (beta < 0 || pf_bucket(e[k], pr) > beta)) {
          p.cflag[f - f0] = 1;
          ++cnt;
        }
      }
    }
  }
  int tot;
  block_excl_scan<kSelThreads>(cnt, sh, &tot);
  if (tid == 0) {
    p.beta[i] = beta;
    p.n_qcand[i] = tot;
  }
}

// ------------------------------------------------------------------ lists
// Ordered passes over segments of kPfSeg entries, 4 per thread: a count per
// segment, then each segment's prefix from the counts before it and a block scan.
__device__ inline int pf_seg_before(const int32_t *seg, int blk, int nseg, int *total, int *sh) {
  const int tid = threadIdx.x;
  const int v = tid < nseg ? seg[tid] : 0;
  int tot;
  const int excl = block_excl_scan<kSelThreads>(v, sh, &tot);
  __shared__ int s_before;
  if (tid == blk) s_before = excl;
  __syncthreads();
  *total = tot;
  const int r = s_before;
  __syncthreads();
  return r;
}

// flags -> count per segment
__global__ __launch_bounds__(kSelThreads) void k_pf_flags_count(PrefillArgs p, const uint8_t *flag) {
  __shared__ int sh[kSelThreads / kWave + 1];
  if (block_failed(p.status)) return;
  const int s = blockIdx.x * kPfSeg + threadIdx.x * 4;
  const uint32_t f = *(const uint32_t *)(flag + s);  // padded to whole segments, zero past N
  int tot;
  block_excl_scan<kSelThreads>(__popc(f & 0x01010101u), sh, &tot);
  if (threadIdx.x == 0) p.seg[blockIdx.x] = tot;
}

// flags -> ascending list (and the flags cleared for the next chunk)
__global__ __launch_bounds__(kSelThreads) void k_pf_flags_list(PrefillArgs p, uint8_t *flag,
                                                               int32_t *list, int which) {
  __shared__ int sh[kSelThreads / kWave + 1];
  if (block_failed(p.status)) return;
  const int nseg = gridDim.x;
  int total;
  const int before = pf_seg_before(p.seg, blockIdx.x, nseg, &total, sh);
  const int s = blockIdx.x * kPfSeg + threadIdx.x * 4;
  uint32_t f = *(const uint32_t *)(flag + s) & 0x01010101u;
  int tot;
  int r = before + block_excl_scan<kSelThreads>(__popc(f), sh, &tot);
  if (f) {
#pragma unroll
    for (int v = 0; v < 4; ++v)
      if ((f >> (8 * v)) & 1) list[r++] = s + v;
    *(uint32_t *)(flag + s) = 0;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) p.counts[which] = total;
}

// install pass 1: tokens of the list without a slot, per segment
__global__ __launch_bounds__(kSelThreads) void k_pf_inst_count(StepArgs a, PrefillArgs p,
                                                               const int32_t *list, int which) {
  __shared__ int sh[kSelThreads / kWave + 1];
  if (block_failed(p.status)) return;
  const int n = p.counts[which];
  int cnt = 0;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int j = blockIdx.x * kPfSeg + threadIdx.x * 4 + v;
    if (j < n && a.h2g[(int64_t)p.hb + list[j]] == -1) ++cnt;
  }
  int tot;
  block_excl_scan<kSelThreads>(cnt, sh, &tot);
  if (threadIdx.x == 0) p.seg[blockIdx.x] = tot;
}

// install pass 2: in list order, a resident token gets priority t; the r-th one
// without a slot takes free slot idxbuf[cursor + r].  Every workgroup checks the
// total against the free slots first, so none writes if they do not suffice.
__global__ __launch_bounds__(kSelThreads) void k_pf_inst_write(StepArgs a, PrefillArgs p,
                                                               const int32_t *list, int which,
                                                               int late, int32_t *out_h,
                                                               int32_t *out_g) {
  __shared__ int sh[kSelThreads / kWave + 1];
  if (block_failed(p.status)) return;
  const int n = p.counts[which];
  const int t = a.ctl[ECHO_CTL_STEP];
  const int nfree = a.ctl[ECHO_CTL_NFREE];
  const int cursor = late ? p.counts[ECHO_PF_CNT_EARLY] : 0;
  int total;
  const int before = pf_seg_before(p.seg, blockIdx.x, gridDim.x, &total, sh);
  if (cursor + total > nfree) {
    if (blockIdx.x == 0 && threadIdx.x == 0) fail(p.status, ECHO_ECAPACITY);
    return;
  }
  int64_t h[4];
  int32_t g[4];
  int cnt = 0;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int j = blockIdx.x * kPfSeg + threadIdx.x * 4 + v;
    h[v] = j < n ? (int64_t)p.hb + list[j] : -1;
    g[v] = j < n ? a.h2g[h[v]] : 0;
    if (j < n && g[v] == -1) ++cnt;
  }
  int tot;
  int r = before + block_excl_scan<kSelThreads>(cnt, sh, &tot);
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    if (h[v] < 0) continue;
    if (g[v] >= 0) {
      a.prio[g[v]] = t;
    } else {
      const int32_t gs = a.idxbuf[cursor + r];
      a.h2g[h[v]] = gs;
      a.g2h[gs] = (int32_t)h[v];
      a.freef[gs] = 0;
      a.prio[gs] = t;
      out_h[r] = (int32_t)h[v];
      out_g[r] = gs;
      ++r;
    }
  }
  if (blockIdx.x == 0 && threadIdx.x == 0)
    p.counts[late ? ECHO_PF_CNT_LATE : ECHO_PF_CNT_EARLY] = total;
}

// ------------------------------------------------------------------ exact
// Query i's top-k: the tokens above the boundary bucket (n_qcand[i] < k of them,
// all certain) and the k - n_qcand[i] best of the boundary bucket by (score desc,
// token asc) -- the bucket of a rounded difference never decreases as the score
// grows, so the order of the whole row is bucket by bucket.  The boundary
// bucket's (key, token) composites are gathered in LDS (one atomic per wave and
// round of four 16-byte pieces per thread) and selected there; a bucket too large
// for LDS falls back to the radix select over the whole row.  pred[i] is read
// before kth[i] is written (the caller may pass this workspace's kth as pred).
constexpr int kPfBoundaryCap = 6144;

__global__ __launch_bounds__(kSelThreads) void k_pf_exact(StepArgs a, PrefillArgs p) {
  __shared__ int sh[kSelThreads / kWave + 1];
  __shared__ uint64_t shu[kSelThreads / kWave];
  __shared__ uint64_t s_list[kPfBoundaryCap];
  __shared__ int s_n;
  __shared__ SelectLds s_sel_lds;
  if (block_failed(p.status)) return;
  const int i = blockIdx.x, tid = threadIdx.x, lane = lane_id();
  const float *row = p.scores + (int64_t)i * p.N;
  const float pr = p.pred ? p.pred[i] : 0.0f;
  const int beta = p.beta[i];
  const int above = p.n_qcand[i];
  // The row in 16-byte pieces of the score buffer, as the coarse pass reads it:
  // piece j holds the buffer's floats 4j .. 4j+3, those outside the row skipped.
  const int64_t f0 = (int64_t)i * p.N, f1 = f0 + p.N;
  const int64_t j0 = f0 >> 2, j1 = (f1 + 3) >> 2;
  const float4 *pc = reinterpret_cast<const float4 *>(p.scores);
  uint64_t P = ~0ull;
  int pos = 0;
  bool in_lds = false;
  if (beta >= 0) {
    if (tid == 0) s_n = 0;
    __syncthreads();
    // The boundary bucket's composites: four pieces per thread and round, every
    // thread through every round (whole waves meet at the scan), one LDS atomic
    // per wave and round.
    constexpr int U = 4;
    const int rounds = (int)((j1 - j0 + U * kSelThreads - 1) / (U * kSelThreads));
    for (int rd = 0; rd < rounds; ++rd) {
      const int64_t jb = j0 + (int64_t)rd * U * kSelThreads + tid;
      float4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t j = jb + (int64_t)u * kSelThreads;
        v[u] = pc[j < j1 ? j : j0];
      }
      uint32_t m = 0;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t j = jb + (int64_t)u * kSelThreads;
        const float e[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int64_t f = 4 * j + k;
          const bool hit = j < j1 && f >= f0 && f < f1 && pf_bucket(e[k], pr) == beta;
          m |= (hit ? 1u : 0u) << (4 * u + k);
        }
      }
      const int cnt = __popc(m);
      const int incl = wave_incl_scan(cnt);
      const int wtot = __shfl(incl, kWave - 1);
      int b0 = 0;
      if (lane == 0 && wtot) b0 = atomicAdd(&s_n, wtot);
      int idx = __shfl(b0, 0) + incl - cnt;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t j = jb + (int64_t)u * kSelThreads;
        const float e[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if ((m >> (4 * u + k)) & 1u) {
            if (idx < kPfBoundaryCap)
              s_list[idx] = ((uint64_t)topk_key(e[k]) << 32) | (uint32_t)(4 * j + k - f0);
            ++idx;
          }
        }
      }
    }
    __syncthreads();
    const int n = s_n;
    in_lds = n <= kPfBoundaryCap;
    if (in_lds)
      block_select_by<kSelThreads>([&](int j) { return s_list[j]; }, n, a.K - above, &P, &pos,
                                   s_sel_lds);
    else
      block_select_by<kSelThreads>(
          [=](int s) { return ((uint64_t)topk_key(row[s]) << 32) | (uint32_t)s; }, p.N, a.K, &P,
          &pos, s_sel_lds);
  }
  // The selection in ascending token order, 1024 pieces per step (thread t takes
  // piece t), one block scan per step.
  int32_t *out = p.sel + (int64_t)i * a.K;
  int written = 0;
  uint64_t worst = 0;  // the largest selected composite: the k-th in selection order
  for (int64_t jb0 = j0; jb0 < j1; jb0 += kSelThreads) {
    const int64_t j = jb0 + tid;
    const float4 v = pc[j < j1 ? j : j0];
    const float e[4] = {v.x, v.y, v.z, v.w};
    uint32_t keys[4];
    uint32_t m = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t f = 4 * j + k;
      const int s = (int)(f - f0);
      keys[k] = topk_key(e[k]);
      bool sel = j < j1 && f >= f0 && f < f1;
      if (sel && beta >= 0) {
        if (in_lds) {
          const int b = pf_bucket(e[k], pr);
          sel = b > beta || (b == beta && composite_selected(keys[k], s, P, pos));
        } else {
          sel = composite_selected(keys[k], s, P, pos);
        }
      }
      m |= (sel ? 1u : 0u) << k;
    }
    int tot;
    int r = written + block_excl_scan<kSelThreads>(__popc(m), sh, &tot);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if ((m >> k) & 1u) {
        const int s = (int)(4 * j + k - f0);
        out[r++] = s;
        p.uflag[s] = 1;
        const uint64_t x = ((uint64_t)keys[k] << 32) | (uint32_t)s;
        worst = x > worst ? x : worst;
      }
    }
    written += tot;
  }
  worst = block_max_u64<kSelThreads>(worst, shu);
  if (tid == 0) {
    p.n_sel[i] = written;
    p.kth[i] = score_of_key((uint32_t)(worst >> 32));
  }
}

// ------------------------------------------------------------------ copy
__global__ __launch_bounds__(256) void k_pf_copy(StepArgs a, PrefillArgs p, const int32_t *hl,
                                                 const int32_t *gl, int which) {
  if (failed(p.status)) return;
  const int n = p.counts[which];
  if (n <= 0) return;
  const int cpr = a.latent * 2 / 16;
  const int64_t total = (int64_t)n * cpr;
  const v4i_pf *src = (const v4i_pf *)a.host_kv;
  v4i_pf *dst = (v4i_pf *)a.gpu_kv;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i0 = (int64_t)blockIdx.x * 256 + threadIdx.x; i0 < total; i0 += 4 * stride) {
    v4i_pf v[4];
    int64_t d[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {  // past the end: the last piece again (no branch)
      const int64_t x = i0 + u * stride < total ? i0 + u * stride : total - 1;
      const int r = (int)(x / cpr);
      const int c = (int)(x - (int64_t)r * cpr);
      d[u] = (int64_t)gl[r] * cpr + c;
      v[u] = src[(int64_t)hl[r] * cpr + c];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) dst[d[u]] = v[u];
  }
}

// ------------------------------------------------------------------ finish
// The installs took idxbuf[0 .. used) in order, so the free slots left are the
// rest of the list, still ascending: move it to the front (through a buffer, in
// two launches, so that no workgroup reads what another has overwritten), then
// the free-list length and the step counter.
constexpr int kPfShiftBlocks = 256;

__global__ __launch_bounds__(256) void k_pf_shift_out(StepArgs a, PrefillArgs p) {
  if (failed(p.status)) return;
  const int used = p.counts[ECHO_PF_CNT_EARLY] + p.counts[ECHO_PF_CNT_LATE];
  const int left = a.ctl[ECHO_CTL_NFREE] - used;
  for (int j = blockIdx.x * 256 + threadIdx.x; j < left; j += kPfShiftBlocks * 256)
    p.tmp[j] = a.idxbuf[used + j];
  if (blockIdx.x == 0 && threadIdx.x == 0) p.counts[ECHO_PF_CNT_LEFT] = left;
}

__global__ __launch_bounds__(256) void k_pf_shift_in(StepArgs a, PrefillArgs p) {
  if (failed(p.status)) return;
  const int left = p.counts[ECHO_PF_CNT_LEFT];
  for (int j = blockIdx.x * 256 + threadIdx.x; j < left; j += kPfShiftBlocks * 256)
    a.idxbuf[j] = p.tmp[j];
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    a.ctl[ECHO_CTL_NFREE] = left;
    a.ctl[ECHO_CTL_STEP] += 1;
  }
}

// ------------------------------------------------------------------ launchers
hipError_t launch_prefill_score(const StepArgs &a, const PrefillArgs &p, hipStream_t s) {
  const int nseg = (p.N + kPfSeg - 1) / kPfSeg;
  hipLaunchKernelGGL(k_pf_stage, dim3(p.C * 4), dim3(256), 0, s, a, p);
  hipLaunchKernelGGL(k_pf_score, dim3(p.qblocks * p.tsplits), dim3(kPfWaves * kWave), 0, s, a,
                     p);
  hipLaunchKernelGGL(k_pf_coarse, dim3(p.C), dim3(kSelThreads), 0, s, a, p);
  hipLaunchKernelGGL(k_pf_flags_count, dim3(nseg), dim3(kSelThreads), 0, s, p,
                     (const uint8_t *)p.cflag);
  hipLaunchKernelGGL(k_pf_flags_list, dim3(nseg), dim3(kSelThreads), 0, s, p, p.cflag, p.cand,
                     (int)ECHO_PF_CNT_CAND);
  return hipGetLastError();
}

hipError_t launch_prefill_early(const StepArgs &a, const PrefillArgs &p, hipStream_t s) {
  const int nseg = (p.N + kPfSeg - 1) / kPfSeg;
  hipLaunchKernelGGL(k_pf_inst_count, dim3(nseg), dim3(kSelThreads), 0, s, a, p,
                     (const int32_t *)p.cand, (int)ECHO_PF_CNT_CAND);
  hipLaunchKernelGGL(k_pf_inst_write, dim3(nseg), dim3(kSelThreads), 0, s, a, p,
                     (const int32_t *)p.cand, (int)ECHO_PF_CNT_CAND, 0, p.pf_h, p.pf_g);
  return hipGetLastError();
}

hipError_t launch_prefill_exact(const StepArgs &a, const PrefillArgs &p, hipStream_t s) {
  const int nseg = (p.N + kPfSeg - 1) / kPfSeg;
  hipLaunchKernelGGL(k_pf_exact, dim3(p.C), dim3(kSelThreads), 0, s, a, p);
  hipLaunchKernelGGL(k_pf_flags_count, dim3(nseg), dim3(kSelThreads), 0, s, p,
                     (const uint8_t *)p.uflag);
  hipLaunchKernelGGL(k_pf_flags_list, dim3(nseg), dim3(kSelThreads), 0, s, p, p.uflag, p.uni,
                     (int)ECHO_PF_CNT_UNION);
  hipLaunchKernelGGL(k_pf_inst_count, dim3(nseg), dim3(kSelThreads), 0, s, a, p,
                     (const int32_t *)p.uni, (int)ECHO_PF_CNT_UNION);
  hipLaunchKernelGGL(k_pf_inst_write, dim3(nseg), dim3(kSelThreads), 0, s, a, p,
                     (const int32_t *)p.uni, (int)ECHO_PF_CNT_UNION, 1, p.miss_h, p.miss_g);
  hipLaunchKernelGGL(k_pf_shift_out, dim3(kPfShiftBlocks), dim3(256), 0, s, a, p);
  hipLaunchKernelGGL(k_pf_shift_in, dim3(kPfShiftBlocks), dim3(256), 0, s, a, p);
  return hipGetLastError();
}

hipError_t launch_prefill_copy(const StepArgs &a, const PrefillArgs &p, int list, hipStream_t s) {
  if (list == 0)
    hipLaunchKernelGGL(k_pf_copy, dim3(kPfCopyBlocks), dim3(256), 0, s, a, p,
                       (const int32_t *)p.pf_h, (const int32_t *)p.pf_g, (int)ECHO_PF_CNT_EARLY);
  else
    hipLaunchKernelGGL(k_pf_copy, dim3(kPfCopyBlocks), dim3(256), 0, s, a, p,
                       (const int32_t *)p.miss_h, (const int32_t *)p.miss_g,
                       (int)ECHO_PF_CNT_LATE);
  return hipGetLastError();
}

}  // namespace echo
