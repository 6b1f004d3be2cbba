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
// MI355X mapping.  The heads x tokens contraction runs on the gfx950 bf16 MFMA
// (v_mfma_f32_16x16x32_bf16).  Every fp8 E4M3 value is exactly representable in
// bf16, so K is widened in registers (v_cvt_scalef32_pk_bf16_fp8, scale 1);
// q is used as it arrives, in bf16.  Products of a 4-bit and an 8-bit
// significand are exact in fp32 and the bf16 MFMA accumulates in fp32, so the
// scores carry only fp32 rounding.  (The fp8 MFMAs of gfx950 sum neighbouring
// products in a narrower internal window: measured on this chip, a cancelling
// 448 - 448 + 2^-6 returns 0, so they are not used here; the bf16 path has the
// same MFMA time, half the flops at half the rate.)  Each wave owns 64 tokens: it
// streams their K rows straight from HBM into registers (no LDS staging: every K
// byte is used by exactly one lane), runs 4*HG MFMAs per 16 tokens, applies ReLU
// and the head weights in registers, and reduces the 64 heads with two
// cross-lane adds.  Work items of 256 tokens are handed out by an atomic ticket;
// the prefetch ranks in token order come from a decoupled look-back over the
// work items of each request, and each workgroup copies its own emitted rows
// from mapped host memory while the other workgroups on the CU keep scoring.
#include "kernels.h"

namespace echo {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

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
  if (in) {
    ReqInfo r;
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

// Stage one request's query for the scoring kernel: bf16 [64][128], zero-padded
// heads and dims, and its weights [64] (zero for padded heads).  Block of 256
// threads, thread = (head, quarter of the dims).
__device__ static void stage_query(const StepArgs &a, int b) {
  const int tid = threadIdx.x;
  const int j = tid >> 2, part = tid & 3;
  const int t = a.ctl[ECHO_CTL_STEP];
  const int slot = (int)((unsigned)t % (unsigned)a.q_ring);
  const uint16_t *src = a.q + ((int64_t)slot * a.B + b) * a.H * a.D;
  uint32_t wv[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int d = part * 32 + 2 * i;
    uint32_t lo = 0, hi = 0;
    if (j < a.H && d < a.D) {
      lo = src[j * a.D + d];
      hi = src[j * a.D + d + 1];
    }
    wv[i] = lo | (hi << 16);
  }
  uint4 *dst = (uint4 *)(a.sc.qbf + ((int64_t)b * kHeadsPad + j) * kDimPad + part * 32);
#pragma unroll
  for (int i = 0; i < 4; ++i) dst[i] = make_uint4(wv[4 * i], wv[4 * i + 1], wv[4 * i + 2], wv[4 * i + 3]);
  if (part == 0)
    a.sc.wsc[(int64_t)b * kHeadsPad + j] = j < a.H ? a.w[(int64_t)b * a.H + j] : 0.0f;
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
    }
    if ((roles & BEGIN_CLR_INDEX) && tid == 0) a.ws.counters[ECHO_CNT_PREFETCH] = 0;
    if ((roles & BEGIN_CLR_TOPK) && tid < a.max_batch) {
      a.sc.kmin[tid] = 0xFFFFFFFFu;
      a.sc.kmax[tid] = 0u;
      a.sc.tcand_n[tid] = 0;
    }
    if ((roles & BEGIN_CLR_MANAGE) && tid < 16) {
      if (tid < 4) a.sc.ecnt[tid] = 0;
      if (tid != ECHO_CNT_PREFETCH) a.ws.counters[tid] = 0;
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

constexpr int kChunks = kScoreTile / 256;  // 64-token chunks per wave per work item

// K rows of one 64-token chunk for this lane: 4 MFMA sub-tiles of 16 tokens,
// 32 bytes each (dims chunk .. chunk+31 of token s0 + 16u + row).
__device__ inline void load_k_chunk(const StepArgs &a, const ReqInfo &r, int s0, int row,
                                    int chunk, v8i (&kb)[4]) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int s = s0 + u * 16 + row;
    v8i x = {0, 0, 0, 0, 0, 0, 0, 0};
    if (s < r.ctx && chunk < a.D) {
      const v4i *p = (const v4i *)(a.kidx + ((int64_t)r.base + s) * a.D + chunk);
      const v4i x0 = __builtin_nontemporal_load(p);
      const v4i x1 = __builtin_nontemporal_load(p + 1);
      x[0] = x0[0]; x[1] = x0[1]; x[2] = x0[2]; x[3] = x0[3];
      x[4] = x1[0]; x[5] = x1[1]; x[6] = x1[2]; x[7] = x1[3];
    }
    kb[u] = x;
  }
}

// Scores of one 64-token chunk: returns, in lane l, the score of token s0 + l.
template <int HG>
__device__ inline float score_chunk(const v8i (&kb)[4], const v8bf (&qa)[HG][4],
                                    const float (&wr)[HG][4], int lane) {
  float sc4[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    v8bf kf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int w0 = kb[u][2 * ks], w1 = kb[u][2 * ks + 1];
      const v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
      const v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
      const v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
      const v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
      kf[ks] = (v8bf){p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
    }
    float v = 0.0f;
#pragma unroll
    for (int hg = 0; hg < HG; ++hg) {
      v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[hg][ks], kf[ks], acc, 0, 0, 0);
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

template <int HG>
__global__ __launch_bounds__(256) void k_score(StepArgs a) {
  __shared__ __align__(16) uint16_t s_q[HG * 16][kDimPad];
  __shared__ ReqInfo s_req[kMaxBatch];
  __shared__ int s_next, s_E, s_nemit;
  __shared__ int s_wcnt[4];
  __shared__ uint32_t s_kmin[4], s_kmax[4];
  __shared__ int32_t s_emit_h[kScoreTile], s_emit_g[kScoreTile];

  int32_t *status = a.ws.status;
  if (failed(status)) return;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  // Operand layout: lane l feeds row (l & 15) of A (a head) and column (l & 15)
  // of B (a token), and for k-step ks the 8 elements at dims
  // chunk + 8*ks .. +7 with chunk = 32*(l >> 4); A and B use the same dims for
  // the same (lane, k-step), so the MFMA sums q . k over all 128 dims.
  const int row = lane & 15, chunk = (lane >> 4) * 32;
  const int total = a.sc.misc[M_TOTAL_TILES];
  const int t = a.ctl[ECHO_CTL_STEP];
  const int nfree = a.ctl[ECHO_CTL_NFREE];
  const int cpr = a.latent * 2 / 16;  // 16-byte chunks per latent row

  for (int i = tid; i < a.B; i += 256) s_req[i] = a.sc.req[i];
  if (tid == 0) s_next = atomicAdd(&a.sc.misc[M_TICKET_SCORE], 1);
  __syncthreads();

  int cur_b = -1;
  v8bf qa[HG][4];
  float wr[HG][4];

  for (;;) {
    const int tau = s_next;
    if (tau >= total) break;  // uniform
    __syncthreads();          // every thread has read s_next
    // fetch the next work item now; its latency hides behind this one
    if (tid == 0) s_next = atomicAdd(&a.sc.misc[M_TICKET_SCORE], 1);
    int b = 0;
    for (int i = 0; i < a.B; ++i)
      if (s_req[i].tile0 <= tau && tau < s_req[i].tile0 + s_req[i].ntiles) b = i;
    const ReqInfo r = s_req[b];

    if (b != cur_b) {  // stage this request's query, then keep it in registers
      const uint4 *src = (const uint4 *)(a.sc.qbf + (int64_t)b * kHeadsPad * kDimPad);
      uint4 *dst = (uint4 *)&s_q[0][0];
      for (int i = tid; i < HG * 16 * kDimPad * 2 / 16; i += 256) dst[i] = src[i];
      __syncthreads();
#pragma unroll
      for (int hg = 0; hg < HG; ++hg) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          qa[hg][ks] = *(const v8bf *)&s_q[hg * 16 + row][chunk + 8 * ks];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          wr[hg][rr] = a.sc.wsc[(int64_t)b * kHeadsPad + hg * 16 + (lane >> 4) * 4 + rr];
      }
      cur_b = b;
    }

    // ---- stream this wave's kChunks x 64 tokens, next chunk's loads in flight
    const int s_wave = (tau - r.tile0) * kScoreTile + wid * (kScoreTile / 4);
    float *out = a.ws.scores + (int64_t)b * a.max_ctx;
    v8i kb[2][4];
    load_k_chunk(a, r, s_wave, row, chunk, kb[0]);
    uint64_t above[kChunks];
    uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      if (c + 1 < kChunks) load_k_chunk(a, r, s_wave + (c + 1) * 64, row, chunk, kb[(c + 1) & 1]);
      const float score = score_chunk<HG>(kb[c & 1], qa, wr, lane);
      const int s = s_wave + c * 64 + lane;
      const bool valid = s < r.ctx;
      if (valid) out[s] = score;
      const uint32_t key = topk_key(score);
      kmn = valid ? min(kmn, key) : kmn;
      kmx = valid ? max(kmx, key) : kmx;
      above[c] = __ballot(r.active && valid && score > r.theta);
    }
    kmn = wave_min_u32(kmn);
    kmx = wave_max_u32(kmx);

    // ---- prefetch candidates: above the threshold and not resident
    int wc = 0;
    uint64_t cand[kChunks];
    if (r.active) {
      int g_of[kChunks];
#pragma unroll
      for (int c = 0; c < kChunks; ++c) {  // one batch of map lookups per work item
        g_of[c] = 0;
        if ((above[c] >> lane) & 1ull)
          g_of[c] = a.h2g[(int64_t)r.base + s_wave + c * 64 + lane];
      }
#pragma unroll
      for (int c = 0; c < kChunks; ++c) {
        cand[c] = __ballot(((above[c] >> lane) & 1ull) && g_of[c] == -1);
        wc += __popcll(cand[c]);
      }
    }
    if (lane == 0) {
      s_kmin[wid] = kmn;
      s_kmax[wid] = kmx;
      s_wcnt[wid] = wc;
    }
    if (tid == 0) s_nemit = 0;
    __syncthreads();
    if (tid == 0) {
      atomicMin(&a.sc.kmin[b], min(min(s_kmin[0], s_kmin[1]), min(s_kmin[2], s_kmin[3])));
      atomicMax(&a.sc.kmax[b], max(max(s_kmax[0], s_kmax[1]), max(s_kmax[2], s_kmax[3])));
    }

    if (r.active) {  // uniform over the block
      const int c_all = s_wcnt[0] + s_wcnt[1] + s_wcnt[2] + s_wcnt[3];
      int base = 0;
      for (int i = 0; i < wid; ++i) base += s_wcnt[i];
      if (wid == 0) {
        const int E = lookback(a.sc.tstate, tau, r.tile0, c_all, status);
        if (lane == 0) s_E = E;
      }
      __syncthreads();
      base += s_E;
#pragma unroll
      for (int c = 0; c < kChunks; ++c) {
        const uint64_t m = cand[c];
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
              const int e = atomicAdd(&s_nemit, 1);
              s_emit_h[e] = (int32_t)h;
              s_emit_g[e] = g;
            }
          }
        }
        base += __popcll(m);
      }
      __syncthreads();
      const int ne = s_nemit;
      if (ne > 0) {
        // copy the emitted latent rows host -> GPU pool, four loads in flight per thread
        const uint4 *src = (const uint4 *)a.host_kv;
        uint4 *dst = (uint4 *)a.gpu_kv;
        const int nchunks = ne * cpr;
        for (int i0 = tid; i0 < nchunks; i0 += 4 * 256) {
          uint4 v0, v1, v2, v3;
          int e0 = i0 / cpr, e1 = 0, e2 = 0, e3 = 0;
          const int i1 = i0 + 256, i2 = i0 + 512, i3 = i0 + 768;
          v0 = src[(int64_t)s_emit_h[e0] * cpr + (i0 - e0 * cpr)];
          if (i1 < nchunks) { e1 = i1 / cpr; v1 = src[(int64_t)s_emit_h[e1] * cpr + (i1 - e1 * cpr)]; }
          if (i2 < nchunks) { e2 = i2 / cpr; v2 = src[(int64_t)s_emit_h[e2] * cpr + (i2 - e2 * cpr)]; }
          if (i3 < nchunks) { e3 = i3 / cpr; v3 = src[(int64_t)s_emit_h[e3] * cpr + (i3 - e3 * cpr)]; }
          dst[(int64_t)s_emit_g[e0] * cpr + (i0 - e0 * cpr)] = v0;
          if (i1 < nchunks) dst[(int64_t)s_emit_g[e1] * cpr + (i1 - e1 * cpr)] = v1;
          if (i2 < nchunks) dst[(int64_t)s_emit_g[e2] * cpr + (i2 - e2 * cpr)] = v2;
          if (i3 < nchunks) dst[(int64_t)s_emit_g[e3] * cpr + (i3 - e3 * cpr)] = v3;
        }
        if (tid == 0) {
          atomicAdd(&a.ws.n_pf[b], ne);
          atomicAdd(&a.ws.counters[ECHO_CNT_PREFETCH], ne);
        }
      }
      if (tid == 0 && c_all > 0) atomicAdd(&a.ws.n_cand[b], c_all);
    }
    __syncthreads();  // s_next is written; LDS may be reused
  }
}

hipError_t launch_score(const StepArgs &a, hipStream_t s) {
  const int hg = (a.H + 15) / 16;
  // persistent grid: two workgroups per CU, work items handed out by ticket
  int grid = a.sc.max_tiles < 512 ? a.sc.max_tiles : 512;
  if (grid < 1) grid = 1;
  switch (hg) {
    case 1: hipLaunchKernelGGL(k_score<1>, dim3(grid), dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL(k_score<2>, dim3(grid), dim3(256), 0, s, a); break;
    case 3: hipLaunchKernelGGL(k_score<3>, dim3(grid), dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL(k_score<4>, dim3(grid), dim3(256), 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace echo
