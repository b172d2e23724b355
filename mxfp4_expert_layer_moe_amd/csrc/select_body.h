// Per-token expert selection shared by the routing kernels and the dense decode GEMM launch:
// exact float64 re-scoring, the small-batch selection (at most 32 tokens and 32 experts) and the
// grouping of its assignments.  The router, the top-k and the gates follow "gpt-oss architecture
// walk-through", section "Mixture of Experts" (a small network scores the experts; several are
// kept and weighted; gpt-oss keeps 4).
#pragma once
#include "mfma_ops.h"

namespace moe {

constexpr double kBandRel = 36.0 * 5.9604644775390625e-8;     // 36 eps32

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

// ---- router scores of at most 32 tokens and 32 experts in one workgroup ------------------------
//
// The router is a linear map with bias over the expert rows.  Scores run on the bf16 matrix cores:
// x is bf16 and the fp32 router weight is split exactly into three bf16 terms (truncation:
// hi + mid + lo == w), so every product is exact.  A k-step (16 K values) is three MFMAs from
// zero, an fp32 (32-token, 32-expert) tile whose only roundings are those of 16-term partial sums.
// The k-steps go in groups of kGroupSteps, each group's tiles added in float64 in a fixed tree
// (score_group_wave), and the groups' sums are added in group order from 0.0; the bias comes
// last.  The squared norms of the x rows and w rows (for the band test) are fp32 sums in the same
// order.  The arithmetic does not depend on how the work is dealt to wavefronts or workgroups.
constexpr int kGroupSteps = 16;     // k-steps per group
constexpr int kScoreRing = 1;       // pairs of k-steps whose loads a wavefront keeps in flight

__device__ inline uint32_t trunc_bf16_bits(float v) { return __float_as_uint(v) & 0xFFFF0000u; }

// operands of one k-step for lane l: token row / expert row l % 32, K half l / 32
struct ScoreStep {
  uint4 x;
  float4 w0, w1;
};

__device__ __forceinline__ ScoreStep score_step_load(int T, int D, int E, const uint16_t* __restrict__ x,
                                                     const float* __restrict__ wr, int s, int s_end, int lane) {
  ScoreStep L;
  L.x = make_uint4(0, 0, 0, 0);
  L.w0 = make_float4(0.f, 0.f, 0.f, 0.f);
  L.w1 = L.w0;
  const int row = lane & 31, half = lane >> 5;
  if (s < s_end) {
    if (row < T) L.x = *reinterpret_cast<const uint4*>(x + (size_t)row * D + 16 * s + 8 * half);
    if (row < E) {
      const float* wb = wr + (size_t)row * D + 16 * s + 8 * half;
      L.w0 = *reinterpret_cast<const float4*>(wb);
      L.w1 = *reinterpret_cast<const float4*>(wb + 4);
    }
  }
  return L;
}

// The k-step's fp32 tile (MFMA layout: lane l holds expert l % 32, tokens 8(r/4) + 4(l/32) + r%4)
// and the lane's squared-norm terms of its 8 x values (xs) and 8 w values (ws), in element order.
__device__ __forceinline__ v16f score_step_tile(const ScoreStep& L, float& xs, float& ws) {
  const uint32_t uw[4] = {L.x.x, L.x.y, L.x.z, L.x.w};
  xs = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = __uint_as_float(uw[i] << 16), hi = __uint_as_float(uw[i] & 0xFFFF0000u);
    xs = __fadd_rn(xs, __fmul_rn(lo, lo));
    xs = __fadd_rn(xs, __fmul_rn(hi, hi));
  }
  const float wv[8] = {L.w0.x, L.w0.y, L.w0.z, L.w0.w, L.w1.x, L.w1.y, L.w1.z, L.w1.w};
  ws = 0.0f;
  uint32_t hb[8], mb[8], lb[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    ws = __fadd_rn(ws, __fmul_rn(wv[i], wv[i]));
    const uint32_t h = trunc_bf16_bits(wv[i]);
    const float r1 = wv[i] - __uint_as_float(h);            // exact
    const uint32_t m = trunc_bf16_bits(r1);
    const float r2 = r1 - __uint_as_float(m);                // exact, <= 8 significant bits
    hb[i] = h >> 16; mb[i] = m >> 16; lb[i] = __float_as_uint(r2) >> 16;
  }
  const uint4 hu = make_uint4(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16), hb[4] | (hb[5] << 16), hb[6] | (hb[7] << 16));
  const uint4 mu = make_uint4(mb[0] | (mb[1] << 16), mb[2] | (mb[3] << 16), mb[4] | (mb[5] << 16), mb[6] | (mb[7] << 16));
  const uint4 lu = make_uint4(lb[0] | (lb[1] << 16), lb[2] | (lb[3] << 16), lb[4] | (lb[5] << 16), lb[6] | (lb[7] << 16));
  const v8bf a = __builtin_bit_cast(v8bf, L.x);
  v16f t = {};
  t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(v8bf, lu), t, 0, 0, 0);
  t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(v8bf, mu), t, 0, 0, 0);
  t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(v8bf, hu), t, 0, 0, 0);
  return t;
}

// The selection's LDS, provided by the caller (the dense decode launch lends it its staging buffer).
struct SelectSmem {
  double lt[32][34];          // [token][expert] scores (bias included); rows 16-byte aligned
  double kth[32], top[32];    // k-th and largest selected score per token
  float xn2[32], wn2[32];
  float ex_l[32][33];         // gate numerators
  uint32_t smask[32];         // selected experts per token (bit e)
  uint32_t fmask[32];         // candidates of the flagged tokens (0: not flagged)
};

// the group sums of one round (one group per wavefront)
template <int W>
struct ScoreSmem {
  double part[W][32][33];     // [group][token][expert]
  float xn[W][32], wn[W][32];
};

// float64 tile of one k-step, 0.0 + (double) of its fp32 tile (zero past the last k-step), and
// the lane's norm terms with the two K halves added (xs for token lane % 32, ws for expert
// lane % 32; a sum of two, the same in both halves)
__device__ __forceinline__ void score_step_f64(const ScoreStep& L, bool valid, double (&p)[16], float& xs, float& ws) {
  float xsi = 0.0f, wsi = 0.0f;
  v16f t = {};
  if (valid) t = score_step_tile(L, xsi, wsi);
#pragma unroll
  for (int r = 0; r < 16; ++r) p[r] = 0.0 + (double)t[r];
  xs = __fadd_rn(xsi, __shfl_xor(xsi, 32));
  ws = __fadd_rn(wsi, __shfl_xor(wsi, 32));
}

// Group g covers k-steps 16g + j, j = 0..15 (p_j their float64 tiles, zero past the last k-step):
// its sum is (p_0 + p_8) + (p_1 + p_9) + ... + (p_7 + p_15), added left to right; the norm terms
// the same way in fp32.  route_groups_kernel spreads a group over 16 wavefronts, one k-step each;
// score_group_wave is the same arithmetic by one wavefront (RING pairs of k-steps in flight).
template <int RING>
__device__ __forceinline__ void score_group_wave(int T, int D, int E, const uint16_t* __restrict__ x,
                                                 const float* __restrict__ wr, int grp, double (&acc)[16],
                                                 float& xs, float& ws) {
  const int lane = threadIdx.x & 63;
  const int nsteps = D / 16;
  const int s0 = grp * kGroupSteps;
  ScoreStep ra[RING], rb[RING];
#pragma unroll
  for (int i = 0; i < RING; ++i) {
    ra[i] = score_step_load(T, D, E, x, wr, s0 + i, nsteps, lane);
    rb[i] = score_step_load(T, D, E, x, wr, s0 + i + 8, nsteps, lane);
  }
  for (int j0 = 0; j0 < 8; j0 += RING) {
#pragma unroll
    for (int i = 0; i < RING; ++i) {
      const int j = j0 + i;
      if (j < 8) {
        const ScoreStep a = ra[i], b = rb[i];
        if (j + RING < 8) {
          ra[i] = score_step_load(T, D, E, x, wr, s0 + j + RING, nsteps, lane);
          rb[i] = score_step_load(T, D, E, x, wr, s0 + j + RING + 8, nsteps, lane);
        }
        double pr[16];                                  // p_j, then p_j + p_(j+8)
        float xa, wa, xb, wb;
        score_step_f64(a, s0 + j < nsteps, pr, xa, wa);
        {
          double pb[16];
          score_step_f64(b, s0 + j + 8 < nsteps, pb, xb, wb);
#pragma unroll
          for (int r = 0; r < 16; ++r) pr[r] += pb[r];
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = j == 0 ? pr[r] : acc[r] + pr[r];
        xs = j == 0 ? __fadd_rn(xa, xb) : __fadd_rn(xs, __fadd_rn(xa, xb));
        ws = j == 0 ? __fadd_rn(wa, wb) : __fadd_rn(ws, __fadd_rn(wa, wb));
      }
    }
  }
}

// element (token i, expert j) of a [32][32] tile held by lane l in MFMA register r
__device__ __forceinline__ int score_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// Scores of the up-to-32 tokens x (bf16 rows) against the up-to-32 expert rows wr (fp32) with
// bias br, into S.lt (and out_logits as fp32 when given), with the squared norms into S.xn2 and
// S.wn2 (zero past T and E): the group sums added in group order from 0.0, then the bias.  The
// group sums come from gpart / gnorm (route_groups_kernel: [group][32][32] float64, [group][2][32]
// fp32 with x norms first), or with IN_WG the workgroup computes them, one group per wavefront
// (score_group_wave), through G.  Every thread of the workgroup calls it; ends with a
// barrier.
template <int THREADS, bool IN_WG>
__device__ __forceinline__ void small_scores(SelectSmem& S, ScoreSmem<THREADS / 64>* G, int T, int D, int E,
                                             const uint16_t* __restrict__ x, const float* __restrict__ wr,
                                             const float* __restrict__ br, float* __restrict__ out_logits,
                                             const double* __restrict__ gpart, const float* __restrict__ gnorm) {
  constexpr int W = THREADS / 64;
  constexpr int OWN = (1024 + THREADS - 1) / THREADS;   // tile elements per thread
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int ngroups = (D / 16 + kGroupSteps - 1) / kGroupSteps;
  double acc[OWN];
#pragma unroll
  for (int o = 0; o < OWN; ++o) acc[o] = 0.0;
  float nacc = 0.0f;                                    // threads 0..31: ||w_e||^2, 32..63: ||x_t||^2
  if constexpr (!IN_WG) {
    for (int g = 0; g < ngroups; ++g) {
#pragma unroll
      for (int o = 0; o < OWN; ++o) {
        const int el = tid + o * THREADS;
        if (el < 1024) acc[o] += gpart[(size_t)g * 1024 + el];
      }
      if (tid < 64) nacc = __fadd_rn(nacc, gnorm[(size_t)g * 64 + (tid < 32 ? 32 + tid : tid - 32)]);
    }
  } else {
    for (int g0 = 0; g0 < ngroups; g0 += W) {
      if (g0 + wave < ngroups) {                        // uniform per wavefront
        double accd[16];
        float xs, ws;
        score_group_wave<kScoreRing>(T, D, E, x, wr, g0 + wave, accd, xs, ws);
#pragma unroll
        for (int r = 0; r < 16; ++r) G->part[wave][score_row(r, lane)][lane & 31] = accd[r];
        if (lane < 32) {
          G->xn[wave][lane] = xs;
          G->wn[wave][lane] = ws;
        }
      }
      __syncthreads();
      for (int w = 0; w < W && g0 + w < ngroups; ++w) {
#pragma unroll
        for (int o = 0; o < OWN; ++o) {
          const int el = tid + o * THREADS;
          if (el < 1024) acc[o] += G->part[w][el >> 5][el & 31];
        }
        if (tid < 64) nacc = __fadd_rn(nacc, tid < 32 ? G->wn[w][tid] : G->xn[w][tid - 32]);
      }
      __syncthreads();
    }
  }
#pragma unroll
  for (int o = 0; o < OWN; ++o) {
    const int el = tid + o * THREADS;
    const int t = el >> 5, e = el & 31;
    if (el < 1024 && t < T && e < E) {
      const double v = acc[o] + (double)br[e];
      S.lt[t][e] = v;
      if (out_logits) out_logits[(size_t)t * E + e] = (float)v;
    }
  }
  if (tid < 32) S.wn2[tid] = tid < E ? nacc : 0.0f;
  else if (tid < 64) S.xn2[tid - 32] = tid - 32 < T ? nacc : 0.0f;
  __syncthreads();
}

// The selection of up to 32 tokens by one workgroup of THREADS threads, one thread per (token t,
// expert e) pair: t = p * (THREADS / 32) + thread / 32 in pass p, e = thread % 32, so a wavefront
// holds two tokens, one per half.  1024 threads take all 32 tokens in one pass, 768 in two.
// Scores (small_scores: the group sums gpart / gnorm, or computed here with IN_WG) -> each pair's rank among its token's live experts (higher score first,
// lower id first on equal scores) selects the top k; the same band test, exact re-scoring and gate
// arithmetic as select_token.  With perm given it then groups the assignments by expert straight
// from the per-token selection masks: the position of (t, e) in expert e's segment is the number of
// earlier tokens that chose e.  Used by route_select_small_kernel (1024 threads) and by the first
// workgroup of the dense decode path's gate/up launch (gemm_dense.hip, 768 threads); the arithmetic
// of every pair is the same in both.
template <int THREADS, bool IN_WG>
__device__ __forceinline__ void select_small(
    SelectSmem& S, ScoreSmem<THREADS / 64>* G, const double* __restrict__ gpart, const float* __restrict__ gnorm,
    int T, int D, int E, int k, const uint16_t* __restrict__ x,
    const float* __restrict__ wr, const float* __restrict__ br, int32_t* __restrict__ out_idx,
    float* __restrict__ out_w, float* __restrict__ out_logits, int bm, int slots, int32_t* __restrict__ counts,
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
  small_scores<THREADS, IN_WG>(S, G, T, D, E, x, wr, br, out_logits, gpart, gnorm);
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
