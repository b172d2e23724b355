// Router, top-k and softmax gating.
//
// The router is a linear map with bias scoring every expert for every token;
// each token keeps its top_k experts and weights them by a softmax over the
// kept scores ("gpt-oss architecture walk-through", section "Mixture of
// Experts": the router picks several experts and weights them, e.g.
// A = 0.7 NN2 + 0.3 NN4; gpt-oss keeps 4 of 32 / 128).
//
// Kernels:
//  route_groups (at most 32 tokens and 32 experts, i.e. decode): the scores of every (token,
//     expert) pair on the bf16 matrix cores (x and the exact three-term bf16 split of the fp32
//     router weight, k-step tiles added in float64) in groups of 16 k-steps, one workgroup per
//     group, one k-step per wavefront, so a decode step spreads over about a dozen compute units;
//     with the activation split of x for the gate/up GEMM in the same launch.
//  route_select_small (the same batches): one workgroup adds the groups, ranks each pair among its
//     token's scores, applies the band test, exact re-scoring and gate arithmetic below, and for
//     the layer forward groups the assignments by expert.  The dense decode path runs the same code
//     in the first workgroup of its gate/up launch, computing the groups itself (same arithmetic).
//  front_pack (the dense decode path): one workgroup per token row splits the row into the packed
//     activation format, normalising it first when the RMSNorm in front of the layer is folded in.
//  route_logits_wide (larger batches): per k-step the arithmetic of small_scores, one workgroup of
//     8 wavefronts per (64-token block, 32-expert tile, K slice); the router chunk of each 64-wide
//     round is split once into an LDS ring shared by both 32-token tiles.
//  route_select: one wavefront per token.  Sums the KW partial tiles in a
//     fixed order (deterministic), adds the bias, takes the top-k by
//     wave-wide arg-max (larger logit first, lower id on ties).  If any other
//     expert lies within a band of the k-th largest, every expert in the band
//     is re-scored exactly in float64 and the top-k is re-taken over those
//     scores.  The band, 36 eps32 ||x_t|| max_e ||w_e||, is twice a worst-case
//     bound of the logit error (at most 18 fp32 roundings per k-step, each at
//     most eps32 times that k-step's sum of |x_d w_d|, and sum_d |x_d w_d| <=
//     ||x_t|| ||w_e|| by Cauchy-Schwarz), so the result is the float64
//     selection at any input scale.  Gates are the softmax of the selected
//     float64 scores, with the exponentials of their gaps taken in fp32.
#include "mfma_ops.h"
#include "norm_body.h"
#include "select_body.h"

namespace moe {

static bool route_small(int T, int E) { return T <= 32 && E <= 32; }

// ---- work split and workspace layout (shared by the ABI layer) --------------------
// Larger batches: route_logits_wide_kernel, one workgroup per (64-token block, 32-expert tile)
// and K slice.
constexpr int kWideWaves = 8;                  // 2 token tiles x 4 k-step lanes
constexpr int kWideTokens = 64;

static int route_kw(int T, int E) {
  const int blocks = ((T + kWideTokens - 1) / kWideTokens) * ((E + 31) / 32);
  return blocks <= 128 ? 4 : (blocks <= 256 ? 2 : 1);     // about two workgroups per compute unit
}

struct RouteWs {
  size_t logit, xsq, wsq, total;
};

__host__ __device__ inline int score_groups(int D) { return (D / 16 + kGroupSteps - 1) / kGroupSteps; }

// The larger batches: the K-partials of the scores.  The small batches: the group sums of
// route_groups ([group][32][32] float64 in logit, [group][2][32] fp32 norms in xsq).
static RouteWs route_ws_layout(int T, int D, int E) {
  RouteWs L = {0, 0, 0, 0};
  if (route_small(T, E)) {
    const size_t G = (size_t)score_groups(D);
    L.xsq = G * 1024 * 8;
    L.total = L.xsq + (G * 64 * 4 + 255) / 256 * 256;
    L.wsq = L.total;
    return L;
  }
  const int KW = route_kw(T, E);
  const size_t epad = (size_t)((E + 31) / 32) * 32;
  L.xsq = ((size_t)KW * T * epad * 8 + 255) / 256 * 256;
  L.wsq = L.xsq + ((size_t)KW * T * 4 + 255) / 256 * 256;
  L.total = L.wsq + ((size_t)KW * epad * 4 + 255) / 256 * 256;
  return L;
}

size_t route_workspace_bytes(int T, int D, int E) { return T > 0 ? route_ws_layout(T, D, E).total : 0; }

// Exact split of n fp32 router weights into three bf16 terms by truncation (hi + mid + lo == w),
// as in score_step_tile, packed two per dword in element order.
template <int N>
__device__ __forceinline__ void split_terms(const float (&wv)[N], uint32_t (&hu)[N / 2], uint32_t (&mu)[N / 2],
                                            uint32_t (&lu)[N / 2]) {
#pragma unroll
  for (int i = 0; i < N; i += 2) {
    uint32_t hb[2], mb[2], lb[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t h = trunc_bf16_bits(wv[i + j]);
      const float r1 = wv[i + j] - __uint_as_float(h);        // exact
      const uint32_t m = trunc_bf16_bits(r1);
      const float r2 = r1 - __uint_as_float(m);               // exact, <= 8 significant bits
      hb[j] = h >> 16; mb[j] = m >> 16; lb[j] = __float_as_uint(r2) >> 16;
    }
    hu[i / 2] = hb[0] | (hb[1] << 16);
    mu[i / 2] = mb[0] | (mb[1] << 16);
    lu[i / 2] = lb[0] | (lb[1] << 16);
  }
}

// ---- the small batches' launches before the selection ---------------------------------
// route_groups: workgroup g < ngroups (16 wavefronts) takes score group g of small_scores,
// wavefront j the k-step 16g + j, and adds its tiles in the group's tree through LDS: p_j + p_(j+8)
// in place, then the eight sums left to right; the norm terms the same way.  Writes the group sums
// to gpart / gnorm.  Workgroups past the groups (when xpack is given) split x into the packed
// activation format, one 32-value block per lane.
__global__ __launch_bounds__(1024) void route_groups_kernel(int T, int D, int E, const uint16_t* __restrict__ x,
                                                            const float* __restrict__ wr, int ngroups,
                                                            double* __restrict__ gpart, float* __restrict__ gnorm,
                                                            uint8_t* __restrict__ xpack, int af) {
  __shared__ double red[8][32][33];
  __shared__ float rn[8][2][32];
  const int tid = threadIdx.x;
  if ((int)blockIdx.x >= ngroups) {                   // activation split (no barriers)
    const long long blk = (long long)(blockIdx.x - ngroups) * 1024 + tid;
    pack_block_lane(x, D, (long long)T * (D / kBlock), blk, xpack, af);
    return;
  }
  const int lane = tid & 63;
  const int j = tid >> 6;
  const int s = blockIdx.x * kGroupSteps + j;
  const int nsteps = D / 16;
  const ScoreStep L = score_step_load(T, D, E, x, wr, s, nsteps, lane);
  double p[16];
  float xs, ws;
  score_step_f64(L, s < nsteps, p, xs, ws);
  const int col = lane & 31;
  if (j < 8) {
#pragma unroll
    for (int r = 0; r < 16; ++r) red[j][score_row(r, lane)][col] = p[r];
    if (lane < 32) {
      rn[j][0][lane] = xs;
      rn[j][1][lane] = ws;
    }
  }
  __syncthreads();
  if (j >= 8) {
#pragma unroll
    for (int r = 0; r < 16; ++r) red[j - 8][score_row(r, lane)][col] += p[r];
    if (lane < 32) {
      rn[j - 8][0][lane] = __fadd_rn(rn[j - 8][0][lane], xs);
      rn[j - 8][1][lane] = __fadd_rn(rn[j - 8][1][lane], ws);
    }
  }
  __syncthreads();
  const int i = tid >> 5, c = tid & 31;               // one element of the 32 x 32 tile per thread
  double v = red[0][i][c];
#pragma unroll
  for (int q = 1; q < 8; ++q) v += red[q][i][c];
  gpart[(size_t)blockIdx.x * 1024 + tid] = v;
  if (tid < 64) {
    const int which = tid >> 5;                        // 0: x norms, 1: w norms
    float n = rn[0][which][c];
#pragma unroll
    for (int q = 1; q < 8; ++q) n = __fadd_rn(n, rn[q][which][c]);
    gnorm[(size_t)blockIdx.x * 64 + tid] = n;
  }
}

// front_pack (the dense decode path): one workgroup of kNormThreads per token row.  With gamma (the
// RMSNorm in front of the layer folded in): r_t (row_rms_inv, the standalone RMSNorm's order), each
// thread's normalised 8-value chunk to xn and to an LDS copy of the row, then thread i packs block
// i of the normalised row (all of its 32 values in one lane); without, thread i packs block i of x.
constexpr int kFrontMaxD = 8192;               // the LDS row copy (rows wider go without it)
__global__ __launch_bounds__(kNormThreads) void front_pack_kernel(int D, const uint16_t* __restrict__ x,
                                                                  const float* __restrict__ gamma, double eps,
                                                                  uint16_t* __restrict__ xn,
                                                                  uint8_t* __restrict__ xpack, int af) {
  __shared__ double part[kNormThreads / 64];
  __shared__ __align__(16) uint4 srow[kFrontMaxD / 8];
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int nb = D / kBlock, nc = D / 8;
  auto pack = [&](int b, const uint4* src) {
    float v[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 q = src[i];
      const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * i + 2 * j] = __uint_as_float(w[j] << 16);
        v[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
      }
    }
    pack_block_values(v, D, row, b, xpack, af);
  };
  const uint16_t* xr = x + (size_t)row * D;
  const uint4* x4 = reinterpret_cast<const uint4*>(xr);
  if (!gamma) {
    for (int b = tid; b < nb; b += kNormThreads) {
      uint4 q[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) q[c] = x4[4 * b + c];
      pack(b, q);
    }
    return;
  }
  const float4* g4 = reinterpret_cast<const float4*>(gamma);
  const float4 ga = tid < nc ? g4[2 * tid] : make_float4(0.f, 0.f, 0.f, 0.f);
  const float4 gb = tid < nc ? g4[2 * tid + 1] : ga;
  uint4 held;
  const double r = row_rms_inv(xr, D, eps, part, held);
  uint4* o4 = reinterpret_cast<uint4*>(xn + (size_t)row * D);
  const bool staged = D <= kFrontMaxD;           // uniform
  for (int c = tid; c < nc; c += kNormThreads) {
    const uint4 q = c == tid ? chunk_rmsnorm(held, r, ga, gb) : chunk_rmsnorm(x4[c], r, gamma, c);
    o4[c] = q;
    if (staged) srow[c] = q;
  }
  if (staged) {
    __syncthreads();
    for (int b = tid; b < nb; b += kNormThreads) pack(b, srow + 4 * b);
  } else {
    __threadfence_block();                        // this workgroup's own xn stores, read back below
    __syncthreads();
    for (int b = tid; b < nb; b += kNormThreads) {
      uint4 q[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) q[c] = o4[4 * b + c];
      pack(b, q);
    }
  }
}

// Router logits for larger batches.  A workgroup of 8 wavefronts takes 64 tokens (two 32-token
// tiles) x one 32-expert tile x a contiguous slice of K (KW slices).  K goes in rounds of 64:
// every thread loads one float4 of the round's 32 x 64 router chunk, splits it into the three
// bf16 terms and stores them in an LDS ring of two rounds, so each router weight is split once
// per 64 tokens and read from LDS by both token tiles; wavefront (tile q, lane group j) takes
// k-step j of every round for tile q.  The arithmetic per k-step is that of logit_compute: three
// bf16 MFMAs from zero, their fp32 result added into float64.  The four k-step lanes' partial
// tiles are summed in LDS in a fixed order.  Loads run two rounds ahead.
constexpr int kWideRowBytes = 128 + 16;        // one expert row of a round in bf16, padded
constexpr int kWidePlane = 32 * kWideRowBytes; // one term of a round
constexpr int kWideBuf = 3 * kWidePlane;

template <int TQ>
__global__ __launch_bounds__(TQ * 256) void route_logits_wide_kernel(
    int T, int D, int E, int KW, const uint16_t* __restrict__ x, const float* __restrict__ wr,
    double* __restrict__ logit, float* __restrict__ xsq, float* __restrict__ wsq, int logit_wgs,
    uint8_t* __restrict__ xpack, int af) {
  constexpr int kThreads = TQ * 256;                             // TQ token tiles x 4 k-step lanes
  constexpr int kTokens = TQ * 32;
  constexpr int kPer = 2048 / kThreads;                          // router values per thread and round
  constexpr int kRowThreads = 64 / kPer;                         // threads per expert row of a round
  constexpr int kRedBytes = 4 * TQ * 32 * 33 * 8;                // [k-step lane][tile][token][expert]
  static_assert(2 * kWideBuf <= kRedBytes, "the ring fits the reduction area");
  __shared__ __align__(16) uint8_t smem[kRedBytes];
  __shared__ float rsx[4][TQ][32];                               // partial ||x_t||^2
  if ((int)blockIdx.x >= logit_wgs) {                           // activation split, one block per lane
    const long long blk = (long long)(blockIdx.x - logit_wgs) * kThreads + threadIdx.x;
    pack_block_lane(x, D, (long long)T * (D / kBlock), blk, xpack, af);
    return;
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int tq = wave % TQ, kq = wave / TQ;
  const int nte = (E + 31) / 32;
  const int kw = blockIdx.x % KW;
  const int nt = (blockIdx.x / KW) % nte;
  const int tb = blockIdx.x / (KW * nte);
  const int epad = nte * 32;
  const int row = lane & 31, half = lane >> 5;
  const int tok = tb * kTokens + tq * 32 + row;
  const int rounds = D / 64;
  const int r0 = rounds * kw / KW, r1 = rounds * (kw + 1) / KW;
  // the token norms are stored by the first expert tile's workgroups only (the 64-token form
  // computes them everywhere: the branch costs it more than the arithmetic)
  const bool norms = TQ == 2 || nt == 0;
  // this thread's kPer values of every router chunk, and its x row (clamped; masked at the end)
  const int wrow = tid / kRowThreads, wc = tid % kRowThreads;
  const bool wlive = nt * 32 + wrow < E;
  const float* wsrc = wr + (size_t)min(nt * 32 + wrow, E - 1) * D + kPer * wc;
  const uint16_t* xa = x + (size_t)min(tok, T - 1) * D + 16 * kq + 8 * half;
  typedef float vw __attribute__((ext_vector_type(kPer)));
  auto load_w = [&](const int r) {
    vw v = {};
    if (wlive && r < r1) v = *reinterpret_cast<const vw*>(wsrc + 64 * r);
    return v;
  };
  auto load_x = [&](const int r) {
    return r < r1 ? *reinterpret_cast<const uint4*>(xa + 64 * r) : make_uint4(0, 0, 0, 0);
  };
  vw wq[2] = {load_w(r0), load_w(r0 + 1)};
  uint4 xq[2] = {load_x(r0), load_x(r0 + 1)};
  double accd[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) accd[i] = 0.0;
  float xs = 0.0f, sq = 0.0f;
  auto round = [&](const int r, const int slot) __attribute__((always_inline)) {
    uint8_t* buf = smem + slot * kWideBuf;
    {
      float wv[kPer];
#pragma unroll
      for (int i = 0; i < kPer; ++i) wv[i] = wq[slot][i];
      uint32_t hu[kPer / 2], mu[kPer / 2], lu[kPer / 2];
      split_terms<kPer>(wv, hu, mu, lu);
#pragma unroll
      for (int i = 0; i < kPer; ++i) sq += wv[i] * wv[i];
      uint8_t* dst = buf + wrow * kWideRowBytes + wc * (2 * kPer);
      if constexpr (kPer == 4) {
        *reinterpret_cast<uint2*>(dst) = make_uint2(hu[0], hu[1]);
        *reinterpret_cast<uint2*>(dst + kWidePlane) = make_uint2(mu[0], mu[1]);
        *reinterpret_cast<uint2*>(dst + 2 * kWidePlane) = make_uint2(lu[0], lu[1]);
      } else {
        *reinterpret_cast<uint32_t*>(dst) = hu[0];
        *reinterpret_cast<uint32_t*>(dst + kWidePlane) = mu[0];
        *reinterpret_cast<uint32_t*>(dst + 2 * kWidePlane) = lu[0];
      }
    }
    const uint4 xu = xq[slot];
    wq[slot] = load_w(r + 2);
    xq[slot] = load_x(r + 2);
    __syncthreads();                                            // the round's terms are in LDS
    const uint8_t* bb = buf + row * kWideRowBytes + 32 * kq + 16 * half;
    const uint4 hb = *reinterpret_cast<const uint4*>(bb);
    const uint4 mb = *reinterpret_cast<const uint4*>(bb + kWidePlane);
    const uint4 lb = *reinterpret_cast<const uint4*>(bb + 2 * kWidePlane);
    if (norms) {
      const uint32_t uw[4] = {xu.x, xu.y, xu.z, xu.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float lo = __uint_as_float(uw[i] << 16), hi = __uint_as_float(uw[i] & 0xFFFF0000u);
        xs += lo * lo + hi * hi;
      }
    }
    const v8bf a = __builtin_bit_cast(v8bf, xu);
    v16f t = {};
    t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(v8bf, lb), t, 0, 0, 0);
    t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(v8bf, mb), t, 0, 0, 0);
    t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(v8bf, hb), t, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) accd[i] += (double)t[i];
  };
  // The ring slot of round r is (r - r0) & 1: a slot is rewritten two rounds after its reads, and
  // every wavefront has passed the barrier of the round in between.
  int r = r0;
  for (; r + 1 < r1; r += 2) {
    round(r, 0);
    round(r + 1, 1);
  }
  if (r < r1) round(r, 0);
  __syncthreads();                                              // the ring is free
  double (*red)[TQ][32][33] = reinterpret_cast<double (*)[TQ][32][33]>(smem);
#pragma unroll
  for (int i = 0; i < 16; ++i) red[kq][tq][8 * (i >> 2) + 4 * half + (i & 3)][row] = accd[i];
  if (norms) {
    xs += __shfl_xor(xs, 32);
    if (half == 0) rsx[kq][tq][row] = xs;
  }
  // the router rows' squared norms over this K slice: kRowThreads threads per row, summed in a
  // fixed order
#pragma unroll
  for (int d = kRowThreads / 2; d >= 1; d >>= 1) sq += __shfl_xor(sq, d);
  if (tb == 0 && wc == 0) wsq[(size_t)kw * epad + nt * 32 + wrow] = sq;
  __syncthreads();
  for (int j = tid; j < TQ * 32 * 32; j += kThreads) {
    const int q = j >> 10, m = (j >> 5) & 31, c = j & 31;
    const double v = ((red[0][q][m][c] + red[1][q][m][c]) + red[2][q][m][c]) + red[3][q][m][c];
    const int tj = tb * kTokens + q * 32 + m;
    if (tj < T) logit[((size_t)kw * T + tj) * epad + nt * 32 + c] = v;
  }
  if (nt == 0 && tid < TQ * 32) {
    const int q = tid >> 5, m = tid & 31;
    const float v = ((rsx[0][q][m] + rsx[1][q][m]) + rsx[2][q][m]) + rsx[3][q][m];
    const int tj = tb * kTokens + q * 32 + m;
    if (tj < T) xsq[(size_t)kw * T + tj] = v;
  }
}

__device__ __forceinline__ double readlane_f64(double v, int l) {
  const uint64_t u = __double_as_longlong(v);
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)u, l);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(u >> 32), l);
  return __longlong_as_double(((uint64_t)hi << 32) | lo);
}

// Lane-to-lane move inside rows of 16 lanes (DPP), applied to both halves of a double.
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = __double_as_longlong(v);
  const uint32_t lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xF, 0xF, false);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double(((uint64_t)hi << 32) | lo);
}

// Maximum over the 64 lanes, returned in every lane: quad swaps and row rotations by 4 and 8
// leave each row of 16 holding its maximum, then the four row maxima are read out.
__device__ __forceinline__ double wave_max_f64(double v) {
  v = fmax(v, dpp_f64<0xB1>(v));     // quad_perm [1,0,3,2]
  v = fmax(v, dpp_f64<0x4E>(v));     // quad_perm [2,3,0,1]
  v = fmax(v, dpp_f64<0x124>(v));    // row_ror:4
  v = fmax(v, dpp_f64<0x128>(v));    // row_ror:8
  return fmax(fmax(readlane_f64(v, 0), readlane_f64(v, 16)), fmax(readlane_f64(v, 32), readlane_f64(v, 48)));
}

// The k best live experts of the wavefront's token, in order of score (higher first, lower
// expert id first on equal scores): k rounds of a wave-wide maximum, each taking the lowest id
// that reaches it.  Lane l holds experts l + 64c.  Marks the winners in taken[]; returns the
// first and the k-th winning score.
__device__ __forceinline__ void top_k(const double* v, const bool* live, int k, int lane, bool* taken,
                                      double& first, double& kth) {
#pragma unroll
  for (int c = 0; c < 4; ++c) taken[c] = false;
  first = kth = -INFINITY;
  for (int r = 0; r < k; ++r) {
    double best = -INFINITY;
#pragma unroll
    for (int c = 0; c < 4; ++c) best = live[c] && !taken[c] ? fmax(best, v[c]) : best;
    const double mx = wave_max_f64(best);
    int win = -1;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint64_t m = __ballot(live[c] && !taken[c] && v[c] == mx);
      if (win < 0 && m) win = 64 * c + __ffsll((long long)m) - 1;
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) taken[c] = taken[c] || lane + 64 * c == win;
    if (r == 0) first = mx;
    kth = mx;
  }
}

// Selection and gates of token t by one wavefront (all 64 lanes).  wmax2 = max_e ||w_e||^2.
__device__ __forceinline__ void select_token(int t, int T, int D, int E, int k, int KW, float wmax2,
                                             const uint16_t* __restrict__ x, const float* __restrict__ wr,
                                             const float* __restrict__ br, const double* __restrict__ logit,
                                             const float* __restrict__ xsq, int32_t* __restrict__ out_idx,
                                             float* __restrict__ out_w, float* __restrict__ out_logits) {
  const int lane = threadIdx.x & 63;
  const int epad = ((E + 31) / 32) * 32;
  // the KW partial tiles are summed in a fixed order (KW <= 4)
  // loads are unconditional (indices clamped into range) so they issue together; the partials
  // past KW and experts past E are masked afterwards
  float xp[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) xp[q] = xsq[(size_t)min(q, KW - 1) * T + t];
  float xn2 = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) xn2 += q < KW ? xp[q] : 0.0f;
  double lp[4][4];
  float bias[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int ec = min(lane + 64 * c, E - 1);
    bias[c] = br[ec];
#pragma unroll
    for (int q = 0; q < 4; ++q) lp[c][q] = logit[((size_t)min(q, KW - 1) * T + t) * epad + ec];
  }
  double v[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int e = lane + 64 * c;
    double s = 0.0;
#pragma unroll
    for (int q = 0; q < 4; ++q) s += q < KW ? lp[c][q] : 0.0;
    v[c] = e < E ? s + (double)bias[c] : -INFINITY;
    if (out_logits && e < E) out_logits[(size_t)t * E + e] = (float)v[c];
  }
  bool live[4], taken[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) live[c] = lane + 64 * c < E;
  double mx, kth;
  top_k(v, live, k, lane, taken, mx, kth);
  const double band = kBandRel * sqrt((double)xn2 * (double)wmax2);
  bool cand[4];
  int n = 0;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    cand[c] = live[c] && (taken[c] || v[c] >= kth - band);
    n += __popcll(__ballot(cand[c]));
  }
  if (n > k) {
    // near the boundary: re-score every candidate exactly, then select again among the candidates
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint64_t m = __ballot(cand[c]);
      while (m) {                                        // uniform loop over the candidate set
        const int src = __ffsll((long long)m) - 1;
        m &= m - 1;
        const int e = src + 64 * c;
        const double s = score_f64(x + (size_t)t * D, wr + (size_t)e * D, (double)br[e], D, lane);
        if (lane == src) v[c] = s;
      }
    }
    top_k(v, cand, k, lane, taken, mx, kth);
  }
  // gates: softmax over the selected scores (mx is the largest), summed in ascending expert id
  // exponentials of the score gaps in fp32 (the gaps are exact differences of float64 scores);
  // the gates are then within a few fp32 ulps of the float64 softmax
  float ex[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) ex[c] = taken[c] ? expf((float)(v[c] - mx)) : 0.0f;
  float sum = 0.0f;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    uint64_t m = __ballot(taken[c]);
    while (m) {
      const int l = __ffsll((long long)m) - 1;
      m &= m - 1;
      sum += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ex[c]), l));
    }
  }
  int before = 0;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint64_t m = __ballot(taken[c]);
    const int slot = before + __popcll(m & ((1ull << lane) - 1ull));
    if (taken[c]) {
      out_idx[(size_t)t * k + slot] = lane + 64 * c;
      out_w[(size_t)t * k + slot] = ex[c] / sum;
    }
    before += __popcll(m);
  }
}

// max_e ||w_e||^2 over the KW partial sums (fixed order); one value per wavefront
__device__ __forceinline__ float max_wnorm2(int E, int KW, const float* __restrict__ wsq) {
  const int lane = threadIdx.x & 63;
  const int epad = ((E + 31) / 32) * 32;
  float wmax2 = 0.0f;
  for (int c = 0; 64 * c < E; ++c) {
    const int e = lane + 64 * c;
    float wp[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) wp[q] = wsq[(size_t)min(q, KW - 1) * epad + min(e, E - 1)];
    float s = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) s += q < KW ? wp[q] : 0.0f;
    wmax2 = fmaxf(wmax2, e < E ? s : 0.0f);
  }
  wmax2 = (float)wave_max_f64((double)wmax2);
  return wmax2;
}

__global__ __launch_bounds__(256) void route_select_kernel(int T, int D, int E, int k, int KW,
                                                           const uint16_t* __restrict__ x,
                                                           const float* __restrict__ wr,
                                                           const float* __restrict__ br,
                                                           const double* __restrict__ logit,
                                                           const float* __restrict__ xsq,
                                                           const float* __restrict__ wsq,
                                                           int32_t* __restrict__ out_idx, float* __restrict__ out_w,
                                                           float* __restrict__ out_logits) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;                                     // no barriers in this kernel
  select_token(t, T, D, E, k, KW, max_wnorm2(E, KW, wsq), x, wr, br, logit, xsq, out_idx, out_w, out_logits);
}

// ---- batches of at most 32 tokens and 32 experts --------------------------------------

// At most 32 tokens and 32 experts: one workgroup adds the score groups of route_groups, selects
// for every token and (perm given) groups the assignments.
__global__ __launch_bounds__(1024) void route_select_small_kernel(
    int T, int D, int E, int k, const uint16_t* __restrict__ x, const float* __restrict__ wr,
    const float* __restrict__ br, int32_t* __restrict__ out_idx, float* __restrict__ out_w,
    float* __restrict__ out_logits, int bm, int slots, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv,
    int32_t* __restrict__ tiles, const double* __restrict__ gpart, const float* __restrict__ gnorm) {
  __shared__ __align__(16) SelectSmem smem;
  select_small<1024, false>(smem, nullptr, gpart, gnorm, T, D, E, k, x, wr, br, out_idx, out_w, out_logits, bm, slots,
                     counts, offsets, perm, inv, tiles);
}



hipError_t launch_front_pack(int T, int D, const uint16_t* x, uint8_t* xpack, int af, hipStream_t s,
                             const FrontNorm* fn) {
  if (T == 0) return hipSuccess;
  front_pack_kernel<<<dim3((unsigned)T), dim3(kNormThreads), 0, s>>>(
      D, fn ? fn->raw : x, fn ? fn->gamma : nullptr, fn ? fn->eps : 0.0, fn ? const_cast<uint16_t*>(x) : nullptr,
      xpack, af);
  return hipGetLastError();
}

// Small batches: the score groups (and the packed rows when xpack is given) in one launch.
static hipError_t launch_groups(int T, int D, int E, const uint16_t* x, const float* wr, void* ws, uint8_t* xpack,
                                int af, hipStream_t s, const double** gpart, const float** gnorm) {
  const RouteWs L = route_ws_layout(T, D, E);
  uint8_t* base = reinterpret_cast<uint8_t*>(ws);
  double* gp = reinterpret_cast<double*>(base + L.logit);
  float* gn = reinterpret_cast<float*>(base + L.xsq);
  const int ngroups = score_groups(D);
  const long long pack_wgs = xpack ? ((long long)T * (D / kBlock) + 1023) / 1024 : 0;
  route_groups_kernel<<<dim3((unsigned)(ngroups + pack_wgs)), dim3(1024), 0, s>>>(T, D, E, x, wr, ngroups, gp, gn,
                                                                                  xpack, af);
  *gpart = gp;
  *gnorm = gn;
  return hipGetLastError();
}

// Larger batches: the K-partial score tiles, with the activation split of x into xpack (when
// given) in the same launch.
static hipError_t launch_logits_wide(int T, int D, int E, const uint16_t* x, const float* wr, void* ws,
                                     uint8_t* xpack, int af, hipStream_t s, double** logit, float** xsq,
                                     float** wsq, int* KW) {
  *KW = route_kw(T, E);
  const RouteWs L = route_ws_layout(T, D, E);
  uint8_t* base = reinterpret_cast<uint8_t*>(ws);
  *logit = reinterpret_cast<double*>(base + L.logit);
  *xsq = reinterpret_cast<float*>(base + L.xsq);
  *wsq = reinterpret_cast<float*>(base + L.wsq);
  const long long pack_blocks = xpack ? (long long)T * (D / kBlock) : 0;
  const int nte = (E + 31) / 32;
  // 128-token workgroups (16 wavefronts, one per compute unit) once they fill the chip, so each
  // router weight is split once per 128 tokens; 64-token workgroups of 8 wavefronts before that.
  // Not with the activation split in the same launch: its workgroups would take the 137 KB of LDS
  // too, one per compute unit, and wait behind the logit workgroups.
  if (!xpack && *KW == 1 && ((T + 127) / 128) * nte >= 256) {
    const int logit_wgs = ((T + 127) / 128) * nte;
    const long long pack_wgs = (pack_blocks + 1023) / 1024;
    route_logits_wide_kernel<4><<<dim3((unsigned)(logit_wgs + pack_wgs)), dim3(1024), 0, s>>>(
        T, D, E, 1, x, wr, *logit, *xsq, *wsq, logit_wgs, xpack, af);
    return hipGetLastError();
  }
  const int logit_wgs = ((T + kWideTokens - 1) / kWideTokens) * nte * *KW;
  const long long pack_wgs = (pack_blocks + kWideWaves * 64 - 1) / (kWideWaves * 64);
  route_logits_wide_kernel<2><<<dim3((unsigned)(logit_wgs + pack_wgs)), dim3(kWideWaves * 64), 0, s>>>(
      T, D, E, *KW, x, wr, *logit, *xsq, *wsq, logit_wgs, xpack, af);
  return hipGetLastError();
}

hipError_t launch_route(int T, int D, int E, int k, const uint16_t* x, const float* wr, const float* br,
                        int32_t* idx, float* w, float* logits, void* ws, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (route_small(T, E)) {
    const double* gp;
    const float* gn;
    hipError_t err = launch_groups(T, D, E, x, wr, ws, nullptr, kActSplit6, s, &gp, &gn);
    if (err != hipSuccess) return err;
    route_select_small_kernel<<<dim3(1), dim3(1024), 0, s>>>(T, D, E, k, x, wr, br, idx, w, logits, 0, 0, nullptr,
                                                             nullptr, nullptr, nullptr, nullptr, gp, gn);
    return hipGetLastError();
  }
  double* logit;
  float *xsq, *wsq;
  int KW;
  hipError_t err = launch_logits_wide(T, D, E, x, wr, ws, nullptr, kActSplit6, s, &logit, &xsq, &wsq, &KW);
  if (err != hipSuccess) return err;
  route_select_kernel<<<dim3((T + 3) / 4), dim3(256), 0, s>>>(T, D, E, k, KW, x, wr, br, logit, xsq, wsq, idx, w,
                                                              logits);
  return hipGetLastError();
}

hipError_t launch_route_front(int T, int D, int E, int k, const uint16_t* x, const float* wr, const float* br,
                              int32_t* idx, float* w, void* ws, uint8_t* xpack, int32_t* counts,
                              int32_t* offsets, int32_t* perm, int32_t* inv, int32_t* tiles, hipStream_t s,
                              int af, const FrontNorm* fn) {
  if (T == 0) return hipSuccess;
  hipError_t err;
  if (fn) return hipErrorInvalidValue;             // the caller normalises first
  if (route_small(T, E)) {
    const double* gp;
    const float* gn;
    if ((err = launch_groups(T, D, E, x, wr, ws, xpack, af, s, &gp, &gn)) != hipSuccess) return err;
    const long long n = (long long)T * k;
    route_select_small_kernel<<<dim3(1), dim3(1024), 0, s>>>(T, D, E, k, x, wr, br, idx, w, nullptr,
                                                             tile_rows(n, E), (int)tile_slots(n, E), counts, offsets,
                                                             perm, inv, tiles, gp, gn);
    return hipGetLastError();
  }
  double* logit;
  float *xsq, *wsq;
  int KW;
  if ((err = launch_logits_wide(T, D, E, x, wr, ws, xpack, af, s, &logit, &xsq, &wsq, &KW)) != hipSuccess) return err;
  route_select_kernel<<<dim3((T + 3) / 4), dim3(256), 0, s>>>(T, D, E, k, KW, x, wr, br, logit, xsq, wsq, idx, w,
                                                              nullptr);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  return launch_permute(T, E, k, idx, counts, offsets, perm, inv, tiles, s);
}

}  // namespace moe
