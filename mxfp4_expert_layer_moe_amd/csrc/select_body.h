// Per-token expert selection shared by the routing kernels and the dense decode GEMM launch:
// exact float64 re-scoring, the small-batch selection (at most 32 tokens and 32 experts) and the
// grouping of its assignments.  The router, the top-k and the gates follow "gpt-oss architecture
// walk-through", section "Mixture of Experts" (a small network scores the experts; several are
// kept and weighted; gpt-oss keeps 4).
#pragma once
#include "moe_internal.h"

namespace moe {

constexpr double kBandRel = 36.0 * 5.9604644775390625e-8;     // 36 eps32

constexpr int kSmallKW = 16;

__device__ inline double wave_sum_f64(double v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
  return v;
}

// Exact float64 score of expert row wre for token row xr (bf16): 8-wide chunks per lane, the
// loads of kScoreBatch chunks issued together (all of a 3072-wide row), summed in chunk order.
constexpr int kScoreBatch = 6;
__device__ inline double score_f64(const uint16_t* __restrict__ xr, const float* __restrict__ wre, double bias, int D,
                            int lane) {
  double acc = 0.0;
  const int nc = D / 8;
  for (int c0 = lane; c0 < nc; c0 += 64 * kScoreBatch) {
    uint4 xv[kScoreBatch];
    float4 w0[kScoreBatch], w1[kScoreBatch];
#pragma unroll
    for (int b = 0; b < kScoreBatch; ++b) {
      const int c = c0 + 64 * b;
      if (c < nc) {
        xv[b] = *reinterpret_cast<const uint4*>(xr + 8 * c);
        w0[b] = *reinterpret_cast<const float4*>(wre + 8 * c);
        w1[b] = *reinterpret_cast<const float4*>(wre + 8 * c + 4);
      }
    }
#pragma unroll
    for (int b = 0; b < kScoreBatch; ++b) {
      if (c0 + 64 * b >= nc) break;
      const uint32_t xw[4] = {xv[b].x, xv[b].y, xv[b].z, xv[b].w};
      const float wf[8] = {w0[b].x, w0[b].y, w0[b].z, w0[b].w, w1[b].x, w1[b].y, w1[b].z, w1[b].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc += (double)__uint_as_float(xw[i] << 16) * (double)wf[2 * i];
        acc += (double)__uint_as_float(xw[i] & 0xFFFF0000u) * (double)wf[2 * i + 1];
      }
    }
  }
  return wave_sum_f64(acc) + bias;
}

// Inclusive prefix sum over each half (32 lanes) of the wavefront: shifts by 1, 2, 4, 8 inside
// rows of 16 lanes (DPP row_shr, zero shifted in), then lane 15 of rows 0 and 2 added into
// rows 1 and 3 (DPP row_bcast:15).
__device__ __forceinline__ int half_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);
  return v;
}

// The selection of up to 32 tokens by one workgroup of THREADS threads, one thread per (token t,
// expert e) pair: t = p * (THREADS / 32) + thread / 32 in pass p, e = thread % 32, so a wavefront
// holds two tokens, one per half.  1024 threads take all 32 tokens in one pass, 768 in two.
// Partial tiles -> scores in LDS; each pair's rank among its token's live experts (higher score
// first, lower id first on equal scores) selects the top k; the same band test, exact re-scoring
// and gate arithmetic as select_token.  With perm given it then groups the assignments by expert
// straight from the per-token selection masks: the position of (t, e) in expert e's segment is the
// number of earlier tokens that chose e.  Used by route_select_small_kernel (1024 threads) and by
// the first workgroup of the dense decode path's gate/up launch (gemm_dense.hip, 768 threads); the
// arithmetic of every pair is the same in both.
// The selection's LDS, provided by the caller (the dense decode launch lends it its staging buffer).
struct SelectSmem {
  double lt[32][34];          // [token][expert] scores (bias included); rows 16-byte aligned
  double kth[32], top[32];    // k-th and largest selected score per token
  float xn2[32], wn2[32];
  float ex_l[32][33];         // gate numerators
  uint32_t smask[32];         // selected experts per token (bit e)
  uint32_t fmask[32];         // candidates of the flagged tokens (0: not flagged)
};

template <int THREADS>
__device__ __forceinline__ void select_small(
    SelectSmem& S, int T, int D, int E, int k, const uint16_t* __restrict__ x, const float* __restrict__ wr,
    const float* __restrict__ br, const double* __restrict__ logit, const float* __restrict__ xsq,
    const float* __restrict__ wsq, int32_t* __restrict__ out_idx, float* __restrict__ out_w,
    float* __restrict__ out_logits, int bm, int slots, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv,
    int32_t* __restrict__ tiles) {
  constexpr int NT = 32;                      // tokens
  constexpr int TPP = THREADS / 32;           // tokens per pass
  constexpr int NP = (NT + TPP - 1) / TPP;    // passes
  constexpr int kWaves = THREADS / 64;
  static_assert(THREADS % 64 == 0 && THREADS >= 64, "whole wavefronts, the norms need 64 threads");
  auto& lt = S.lt;
  auto& xn2 = S.xn2;
  auto& wn2 = S.wn2;
  auto& kth = S.kth;
  auto& top = S.top;
  auto& ex_l = S.ex_l;
  auto& smask = S.smask;
  auto& fmask = S.fmask;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int e = tid & 31;
  const int hshift = lane & 32;               // this token's half of the wavefront ballots
  int tk[NP];
  bool live[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    tk[p] = p * TPP + (tid >> 5);
    live[p] = tk[p] < NT && tk[p] < T && e < E;
  }
  // the kSmallKW partials in order, then the bias; every load is issued before the sums
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    if (live[p]) {
      const int t = tk[p];
      double q16[kSmallKW];
#pragma unroll
      for (int q = 0; q < kSmallKW; ++q) q16[q] = logit[((size_t)q * T + t) * 32 + e];
      const float b = br[e];
      double s = 0.0;
#pragma unroll
      for (int q = 0; q < kSmallKW; ++q) s += q16[q];
      const double v = s + (double)b;
      lt[t][e] = v;
      if (out_logits) out_logits[(size_t)t * E + e] = (float)v;
    }
  }
  if (tid < 64) {
    // threads 0..31: squared norms of the expert rows; 32..63: of the token rows
    const int r = tid & 31;
    const bool in = tid < 32 ? r < E : r < T;
    float q16[kSmallKW];
#pragma unroll
    for (int q = 0; q < kSmallKW; ++q)
      q16[q] = !in ? 0.0f : (tid < 32 ? wsq[(size_t)q * 32 + r] : xsq[(size_t)q * T + r]);
    float v = 0.0f;
#pragma unroll
    for (int q = 0; q < kSmallKW; ++q) v += q16[q];
    (tid < 32 ? wn2 : xn2)[r] = v;
  }
  __syncthreads();
  // rank among the live experts of the token
  double v0[NP], v[NP];
  int rank[NP];
  bool sel[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int t = tk[p];
    v0[p] = live[p] ? lt[t][e] : 0.0;
    rank[p] = 0;
    const double2* row = reinterpret_cast<const double2*>(&lt[t < T && t < NT ? t : 0][0]);
#pragma unroll
    for (int j2 = 0; j2 < 16; ++j2) {
      const double2 w = row[j2];                          // one 16-byte read per two experts
      const int j = 2 * j2;
      rank[p] += (j < E && (w.x > v0[p] || (w.x == v0[p] && j < e))) ? 1 : 0;
      rank[p] += (j + 1 < E && (w.y > v0[p] || (w.y == v0[p] && j + 1 < e))) ? 1 : 0;
    }
    sel[p] = live[p] && rank[p] < k;
    if (sel[p] && rank[p] == k - 1) kth[t] = v0[p];
  }
  __syncthreads();
  // band test: any other live expert within the band of the k-th score flags the token
  float wmax2 = 0.0f;
#pragma unroll
  for (int j = 0; j < 32; ++j) wmax2 = fmaxf(wmax2, wn2[j]);             // zero past E
  bool cand[NP], flagged[NP];
  uint32_t cm[NP];
  bool any_flagged = false;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    cand[p] = false;
    if (live[p]) {
      const double band = kBandRel * sqrt((double)xn2[tk[p]] * (double)wmax2);
      cand[p] = sel[p] || v0[p] >= kth[tk[p]] - band;
    }
    cm[p] = (uint32_t)(__ballot(cand[p]) >> hshift);
    flagged[p] = live[p] && __popc(cm[p]) > k;
    any_flagged = any_flagged || flagged[p];
    v[p] = v0[p];
  }
  // flagged tokens: re-score every (token, candidate) pair exactly, the pairs dealt to the
  // workgroup's wavefronts in token-then-expert order (one wavefront per score), then rank again
  // among the candidates.  The whole section is skipped when no token is flagged.
  if (__syncthreads_or(any_flagged)) {
#pragma unroll
    for (int p = 0; p < NP; ++p)
      if (e == 0 && tk[p] < NT) fmask[tk[p]] = flagged[p] ? cm[p] : 0u;
    __syncthreads();
    const int wave = tid >> 6;
    int i = 0;
    for (int tt = 0; tt < NT && tt < T; ++tt) {
      uint32_t m = fmask[tt];                            // uniform
      while (m) {
        const int j = __ffs(m) - 1;
        m &= m - 1;
        if (i % kWaves == wave) {
          const double sc = score_f64(x + (size_t)tt * D, wr + (size_t)j * D, (double)br[j], D, lane);
          if (lane == 0) lt[tt][j] = sc;
        }
        ++i;
      }
    }
    __syncthreads();
  }
  uint32_t sm[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int t = tk[p];
    if (flagged[p]) {
      v[p] = cand[p] ? lt[t][e] : -INFINITY;
      int r = 0;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const double w = lt[t][j];
        r += (((cm[p] >> j) & 1u) && (w > v[p] || (w == v[p] && j < e))) ? 1 : 0;
      }
      rank[p] = r;
      sel[p] = cand[p] && r < k;
    }
    if (sel[p] && rank[p] == 0) top[t] = v[p];
    sm[p] = (uint32_t)(__ballot(sel[p]) >> hshift);
    if (live[p] && e == 0) smask[t] = sm[p];
  }
  __syncthreads();
  // gates: softmax over the selected scores, exponentials of the gaps in fp32, summed in
  // ascending expert id; slots in ascending expert id
  float g[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    g[p] = 0.0f;
    if (sel[p]) {
      g[p] = expf((float)(v[p] - top[tk[p]]));
      ex_l[tk[p]][e] = g[p];
    }
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    if (sel[p]) {
      const int t = tk[p];
      float sum = 0.0f;
      for (uint32_t m = sm[p]; m; m &= m - 1) sum += ex_l[t][__ffs(m) - 1];
      const int slot = __popc(sm[p] & ((1u << e) - 1u));
      out_idx[(size_t)t * k + slot] = e;
      out_w[(size_t)t * k + slot] = g[p] / sum;
    }
  }
  if (!perm) return;
  // grouping: the total per expert (the same in every pass: it depends on e only) and, per pass,
  // the tokens before t that chose e
  int total = 0;
#pragma unroll
  for (int j = 0; j < 32; ++j) total += j < T ? (int)((smask[j] >> e) & 1u) : 0;
  // exclusive scans over the 32 experts of this half-wavefront: segment offsets, first tiles
  const int ntl = (total + bm - 1) / bm;
  const int inc = half_scan(total), tinc = half_scan(ntl);
  const int off = inc - total, tst = tinc - ntl;
  const int used = __shfl(tinc, 31, 32);                 // tiles in use
  const int n = T * k;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int t = tk[p];
    int before = 0;
#pragma unroll
    for (int j = 0; j < 32; ++j) before += j < T && j < t ? (int)((smask[j] >> e) & 1u) : 0;
    if (sel[p] && off + before < n && tst + before / bm < slots) {   // always true; keeps stores in bounds
      const int slot = __popc(sm[p] & ((1u << e) - 1u));
      const int a = t * k + slot, pos = off + before;
      perm[pos] = a;
      inv[a] = pos;
      tiles[(size_t)(tst + before / bm) * tile_ints(bm) + 4 + before % bm] = a;
    }
  }
  // totals, offsets and the headers of expert e's tiles from the first half-wavefront; the
  // headers of the empty slots past the last tile from everyone
  if (tid < 32 && e < E) {
    counts[e] = total;
    offsets[e] = off;
    if (e == E - 1) offsets[E] = n;
    for (int i = 0; i < ntl && tst + i < slots; ++i)
      *reinterpret_cast<int4*>(tiles + (size_t)(tst + i) * tile_ints(bm)) =
          make_int4(e, off + i * bm, min(bm, total - i * bm), used);
  }
  for (int sl = used + tid; sl < slots; sl += THREADS)
    *reinterpret_cast<int4*>(tiles + (size_t)sl * tile_ints(bm)) = make_int4(-1, 0, 0, used);
}

}  // namespace moe
