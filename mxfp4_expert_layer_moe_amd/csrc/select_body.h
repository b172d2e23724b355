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

// One thread per (token t, expert e) pair of NT consecutive tokens from token0: local token
// tl = thread / 32, e = thread % 32, so a wavefront holds two tokens, one per half.  Partial tiles
// -> scores in LDS; each pair's rank among its token's live experts (higher score first, lower id
// first on equal scores) selects the top k; the same band test, exact re-scoring and gate
// arithmetic as select_token.  With perm given it then groups the assignments by expert straight
// from the per-token selection masks: the position of (t, e) in expert e's segment is the number
// of earlier tokens that chose e.  Used by route_select_small_kernel and by the first workgroup of
// the dense decode path's gate/up launch (gemm_dense.hip), both with NT = 32.
// The selection's LDS, provided by the caller (the dense decode launch lends it its staging buffer).
template <int NT>
struct SelectSmem {
  double lt[NT][34];          // [token][expert] scores (bias included); rows 16-byte aligned
  double kth[NT], top[NT];    // k-th and largest selected score per token
  float xn2[NT], wn2[32];
  float ex_l[NT][33];         // gate numerators
  uint32_t smask[NT];         // selected experts per token (bit e)
  uint32_t fmask[NT];         // candidates of the flagged tokens (0: not flagged)
};

template <int NT>
__device__ __forceinline__ void select_small(
    SelectSmem<NT>& S, int token0, int T, int D, int E, int k, const uint16_t* __restrict__ x, const float* __restrict__ wr,
    const float* __restrict__ br, const double* __restrict__ logit, const float* __restrict__ xsq,
    const float* __restrict__ wsq, int32_t* __restrict__ out_idx, float* __restrict__ out_w,
    float* __restrict__ out_logits, int bm, int slots, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv,
    int32_t* __restrict__ tiles) {
  constexpr int kThreads = NT * 32;
  constexpr int kWaves = kThreads / 64;
  static_assert(NT == 32, "one workgroup of 32 tokens (the grouping reads every token's selection)");
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
  const int tl = tid >> 5, e = tid & 31;
  const int t = token0 + tl;
  const int hshift = lane & 32;               // this token's half of the wavefront ballots
  const bool live = t < T && e < E;
  {
    // the kSmallKW partials in order, then the bias; every load is issued before the sums
    if (live) {
      double p[kSmallKW];
#pragma unroll
      for (int q = 0; q < kSmallKW; ++q) p[q] = logit[((size_t)q * T + t) * 32 + e];
      const float b = br[e];
      double s = 0.0;
#pragma unroll
      for (int q = 0; q < kSmallKW; ++q) s += p[q];
      const double v = s + (double)b;
      lt[tl][e] = v;
      if (out_logits) out_logits[(size_t)t * E + e] = (float)v;
    }
    if (tid < 32 + NT) {
      // threads 0..31: squared norms of the expert rows; 32..32+NT-1: of the token rows
      const int r = tid < 32 ? tid : tid - 32;
      const bool in = tid < 32 ? r < E : token0 + r < T;
      float p[kSmallKW];
#pragma unroll
      for (int q = 0; q < kSmallKW; ++q)
        p[q] = !in ? 0.0f : (tid < 32 ? wsq[(size_t)q * 32 + r] : xsq[(size_t)q * T + token0 + r]);
      float v = 0.0f;
#pragma unroll
      for (int q = 0; q < kSmallKW; ++q) v += p[q];
      (tid < 32 ? wn2 : xn2)[r] = v;
    }
  }
  __syncthreads();
  // rank among the live experts of the token
  const double v0 = live ? lt[tl][e] : 0.0;
  int rank = 0;
  {
    const double2* row = reinterpret_cast<const double2*>(&lt[t < T ? tl : 0][0]);
#pragma unroll
    for (int j2 = 0; j2 < 16; ++j2) {
      const double2 w = row[j2];                          // one 16-byte read per two experts
      const int j = 2 * j2;
      rank += (j < E && (w.x > v0 || (w.x == v0 && j < e))) ? 1 : 0;
      rank += (j + 1 < E && (w.y > v0 || (w.y == v0 && j + 1 < e))) ? 1 : 0;
    }
  }
  bool sel = live && rank < k;
  if (sel && rank == k - 1) kth[tl] = v0;
  __syncthreads();
  // band test: any other live expert within the band of the k-th score flags the token
  float wmax2 = 0.0f;
#pragma unroll
  for (int j = 0; j < 32; ++j) wmax2 = fmaxf(wmax2, wn2[j]);             // zero past E
  bool cand = false;
  if (live) {
    const double band = kBandRel * sqrt((double)xn2[tl] * (double)wmax2);
    cand = sel || v0 >= kth[tl] - band;
  }
  const uint32_t cm = (uint32_t)(__ballot(cand) >> hshift);
  const bool flagged = live && __popc(cm) > k;
  // flagged tokens: re-score every (token, candidate) pair exactly, the pairs dealt to the
  // workgroup's wavefronts in token-then-expert order (one wavefront per score), then rank again
  // among the candidates.  The whole section is skipped when no token is flagged.
  double v = v0;
  if (__syncthreads_or(flagged)) {
    if (e == 0) fmask[tl] = flagged ? cm : 0u;
    __syncthreads();
    const int wave = tid >> 6;
    int i = 0;
    for (int ttl = 0; ttl < NT && token0 + ttl < T; ++ttl) {
      uint32_t m = fmask[ttl];                           // uniform
      while (m) {
        const int j = __ffs(m) - 1;
        m &= m - 1;
        if (i % kWaves == wave) {
          const double sc = score_f64(x + (size_t)(token0 + ttl) * D, wr + (size_t)j * D, (double)br[j], D, lane);
          if (lane == 0) lt[ttl][j] = sc;
        }
        ++i;
      }
    }
    __syncthreads();
  }
  if (flagged) {
    v = cand ? lt[tl][e] : -INFINITY;
    rank = 0;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const double w = lt[tl][j];
      rank += (((cm >> j) & 1u) && (w > v || (w == v && j < e))) ? 1 : 0;
    }
    sel = cand && rank < k;
  }
  if (sel && rank == 0) top[tl] = v;
  const uint32_t sm = (uint32_t)(__ballot(sel) >> hshift);
  if (live && e == 0) smask[tl] = sm;
  __syncthreads();
  // gates: softmax over the selected scores, exponentials of the gaps in fp32, summed in
  // ascending expert id; slots in ascending expert id
  float g = 0.0f;
  if (sel) {
    g = expf((float)(v - top[tl]));
    ex_l[tl][e] = g;
  }
  __syncthreads();
  if (sel) {
    float sum = 0.0f;
    for (uint32_t m = sm; m; m &= m - 1) sum += ex_l[tl][__ffs(m) - 1];
    const int slot = __popc(sm & ((1u << e) - 1u));
    out_idx[(size_t)t * k + slot] = e;
    out_w[(size_t)t * k + slot] = g / sum;
  }
  if constexpr (NT == 32) {
    if (!perm) return;
    // grouping: tokens before t that chose e, and the total per expert
    int before = 0, total = 0;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const int bit = j < T ? (int)((smask[j] >> e) & 1u) : 0;
      total += bit;
      before += j < t ? bit : 0;
    }
    // exclusive scans over the 32 experts of this half-wavefront: segment offsets, first tiles
    const int ntl = (total + bm - 1) / bm;
    const int inc = half_scan(total), tinc = half_scan(ntl);
    const int off = inc - total, tst = tinc - ntl;
    const int used = __shfl(tinc, 31, 32);                 // tiles in use
    const int n = T * k;
    if (sel && off + before < n && tst + before / bm < slots) {   // always true; keeps stores in bounds
      const int slot = __popc(sm & ((1u << e) - 1u));
      const int a = t * k + slot, pos = off + before;
      perm[pos] = a;
      inv[a] = pos;
      tiles[(size_t)(tst + before / bm) * tile_ints(bm) + 4 + before % bm] = a;
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
    for (int sl = used + tid; sl < slots; sl += kThreads)
      *reinterpret_cast<int4*>(tiles + (size_t)sl * tile_ints(bm)) = make_int4(-1, 0, 0, used);
  }
}

}  // namespace moe
