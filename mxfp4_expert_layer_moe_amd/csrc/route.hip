// Router, top-k and softmax gating.
//
// The router is a linear map with bias scoring every expert for every token;
// each token keeps its top_k experts and weights them by a softmax over the
// kept scores ("gpt-oss architecture walk-through", section "Mixture of
// Experts": the router picks several experts and weights them, e.g.
// A = 0.7 NN2 + 0.3 NN4; gpt-oss keeps 4 of 32 / 128).
//
// Kernels:
//  route_logits (at most 32 tokens and 32 experts, i.e. decode): 16 workgroups of 16 wavefronts
//     split the K loop of the (32-token, 32-expert) tile sixteen ways, so a decode step spreads
//     over sixteen compute units; each wavefront issues the loads of four k-steps before their
//     matrix instructions.  Logits run on the bf16 matrix cores: x is bf16 and the fp32 router
//     weight is split exactly into three bf16 terms (truncation: hi + mid + lo == w), so every
//     product is exact.  Each 16-wide k-step's three MFMAs start from zero and their small fp32
//     result is added into a float64 accumulator, so the only fp32 roundings are those of
//     16-term partial sums.  The 16 K-partials of a workgroup are summed in LDS in a fixed
//     order and its float64 tile is written to the workspace, with the squared norms of the x
//     rows and w rows.
//  route_logits_wide (larger batches): the same arithmetic per k-step, one workgroup of 8
//     wavefronts per (64-token block, 32-expert tile, K slice); the router chunk of each 64-wide
//     round is split once into an LDS ring shared by both 32-token tiles.
//  route_select_small (with route_logits): one workgroup, one thread per (token, expert) pair;
//     sums the partial tiles into an LDS logit table, ranks each pair among its token's scores,
//     applies the same rules and arithmetic as route_select, and for the layer forward groups
//     the assignments by expert in the same workgroup.
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
#include "select_body.h"

namespace moe {

constexpr int kRouteTokens = 32;

__device__ inline uint32_t trunc_bf16_bits(float v) { return __float_as_uint(v) & 0xFFFF0000u; }

// ---- work split and workspace layout (shared by the ABI layer) --------------------
constexpr int kLogitWaves = 16;
constexpr int kLogitBatch = 4;                 // k-steps whose loads are issued together

static bool route_small(int T, int E) { return T <= 32 && E <= 32; }

// Larger batches: route_logits_wide_kernel, one workgroup per (64-token block, 32-expert tile)
// and K slice.
constexpr int kWideWaves = 8;                  // 2 token tiles x 4 k-step lanes
constexpr int kWideTokens = 64;

static int route_kw(int T, int E) {
  if (route_small(T, E)) return kSmallKW;
  const int blocks = ((T + kWideTokens - 1) / kWideTokens) * ((E + 31) / 32);
  return blocks <= 128 ? 4 : (blocks <= 256 ? 2 : 1);     // about two workgroups per compute unit
}

struct RouteWs {
  size_t logit, xsq, wsq, total;
};

static RouteWs route_ws_layout(int T, int E) {
  const int KW = route_kw(T, E);
  const size_t epad = (size_t)((E + 31) / 32) * 32;
  RouteWs L;
  L.logit = 0;
  L.xsq = ((size_t)KW * T * epad * 8 + 255) / 256 * 256;
  L.wsq = L.xsq + ((size_t)KW * T * 4 + 255) / 256 * 256;
  L.total = L.wsq + ((size_t)KW * epad * 4 + 255) / 256 * 256;
  return L;
}

size_t route_workspace_bytes(int T, int D, int E) {
  (void)D;
  return T > 0 ? route_ws_layout(T, E).total : 0;
}

// One wavefront's share of a (32-token, 32-expert) logit tile: the k-steps s_first, s_first +
// s_stride, ... (16 K values each), BATCH of them loaded before their matrix instructions.
// Lane l: token row / expert row l % 32, K half l / 32.  Returns the float64 tile partial in the
// MFMA layout and the lane's partial squared norms of its x row (xs) and w row (sq).
template <int BATCH>
__device__ __forceinline__ void logit_steps(int T, int D, int E, const uint16_t* __restrict__ x,
                                            const float* __restrict__ wr, int tok, int e, int half, int s_first,
                                            int s_stride, double (&accd)[16], float& sq, float& xs) {
  const int nsteps = D / 16;
  const uint16_t* xa = x + (size_t)tok * D + 8 * half;
  const float* wb = wr + (size_t)e * D + 8 * half;
#pragma unroll
  for (int r = 0; r < 16; ++r) accd[r] = 0.0;
  sq = 0.0f;
  xs = 0.0f;
  for (int s0 = s_first; s0 < nsteps; s0 += BATCH * s_stride) {
    uint4 xu[BATCH];
    float4 wa[BATCH], wc[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const int s = s0 + b * s_stride;
      xu[b] = make_uint4(0, 0, 0, 0);
      wa[b] = make_float4(0.f, 0.f, 0.f, 0.f);
      wc[b] = wa[b];
      if (s < nsteps) {
        if (tok < T) xu[b] = *reinterpret_cast<const uint4*>(xa + 16 * s);
        if (e < E) {
          wa[b] = *reinterpret_cast<const float4*>(wb + 16 * s);
          wc[b] = *reinterpret_cast<const float4*>(wb + 16 * s + 4);
        }
      }
    }
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      if (s0 + b * s_stride >= nsteps) break;             // uniform
      const uint32_t uw[4] = {xu[b].x, xu[b].y, xu[b].z, xu[b].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float lo = __uint_as_float(uw[i] << 16), hi = __uint_as_float(uw[i] & 0xFFFF0000u);
        xs += lo * lo + hi * hi;
      }
      const v8bf a = __builtin_bit_cast(v8bf, xu[b]);
      const float wv[8] = {wa[b].x, wa[b].y, wa[b].z, wa[b].w, wc[b].x, wc[b].y, wc[b].z, wc[b].w};
      uint32_t hb[8], mb[8], lb[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        sq += wv[i] * wv[i];
        const uint32_t h = trunc_bf16_bits(wv[i]);
        const float r1 = wv[i] - __uint_as_float(h);            // exact
        const uint32_t m = trunc_bf16_bits(r1);
        const float r2 = r1 - __uint_as_float(m);                // exact, <= 8 significant bits
        hb[i] = h >> 16; mb[i] = m >> 16; lb[i] = __float_as_uint(r2) >> 16;
      }
      const uint4 hu = make_uint4(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16), hb[4] | (hb[5] << 16), hb[6] | (hb[7] << 16));
      const uint4 mu = make_uint4(mb[0] | (mb[1] << 16), mb[2] | (mb[3] << 16), mb[4] | (mb[5] << 16), mb[6] | (mb[7] << 16));
      const uint4 lu = make_uint4(lb[0] | (lb[1] << 16), lb[2] | (lb[3] << 16), lb[4] | (lb[5] << 16), lb[6] | (lb[7] << 16));
      v16f t = {};
      t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(v8bf, lu), t, 0, 0, 0);
      t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(v8bf, mu), t, 0, 0, 0);
      t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(v8bf, hu), t, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 16; ++r) accd[r] += (double)t[r];
    }
  }
}

// Exact split of n fp32 router weights into three bf16 terms by truncation (hi + mid + lo == w),
// as in logit_steps, packed two per dword in element order.
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

// Fixed-order sum of the 16 wavefronts' partial tiles: slot s = p_s + p_(s+8) is left in
// red[s] (the caller adds slots 0..7 in order); the squared-norm partials go to rsq.
__device__ __forceinline__ void reduce_partials(const double (&accd)[16], float sq, float xs,
                                                double (&red)[8][32][33], float (&rsq)[kLogitWaves][2][32],
                                                int wave, int half, int row) {
  sq += __shfl_xor(sq, 32);
  xs += __shfl_xor(xs, 32);
  if (half == 0) {
    rsq[wave][0][row] = xs;
    rsq[wave][1][row] = sq;
  }
  if (wave < 8) {
#pragma unroll
    for (int r = 0; r < 16; ++r) red[wave][8 * (r >> 2) + 4 * half + (r & 3)][row] = accd[r];
  }
  __syncthreads();
  if (wave >= 8) {
#pragma unroll
    for (int r = 0; r < 16; ++r) red[wave - 8][8 * (r >> 2) + 4 * half + (r & 3)][row] += accd[r];
  }
  __syncthreads();
}

// Workgroups past the logit tiles (when xpack is given) split x into the packed activation
// format for the gate/up GEMM instead: one 32-value block per lane.
__global__ __launch_bounds__(kLogitWaves * 64) void route_logits_kernel(int T, int D, int E, int KW,
                                                                         const uint16_t* __restrict__ x,
                                                                         const float* __restrict__ wr,
                                                                         double* __restrict__ logit,
                                                                         float* __restrict__ xsq,
                                                                         float* __restrict__ wsq,
                                                                         int logit_wgs,
                                                                         uint8_t* __restrict__ xpack, int af) {
  __shared__ double red[8][32][33];          // K-partials: waves 0..7, then 8..15 added in place
  __shared__ float rsq[kLogitWaves][2][32];  // partial ||x_t||^2 (0) and ||w_e||^2 (1)
  if ((int)blockIdx.x >= logit_wgs) {        // activation split, one block per lane (no barriers)
    const long long blk = (long long)(blockIdx.x - logit_wgs) * (kLogitWaves * 64) + threadIdx.x;
    pack_block_lane(x, D, (long long)T * (D / kBlock), blk, xpack, af);
    return;
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nte = (E + 31) / 32;
  const int kw = blockIdx.x % KW;
  const int nt = (blockIdx.x / KW) % nte;
  const int tt = blockIdx.x / (KW * nte);
  const int epad = nte * 32;
  const int kstride = kLogitWaves * KW;
  const int row = lane & 31;
  const int half = lane >> 5;
  const int e = nt * 32 + row;
  const int tok = tt * kRouteTokens + row;
  double accd[16];
  float sq, xs;
  logit_steps<kLogitBatch>(T, D, E, x, wr, tok, e, half, kw * kLogitWaves + wave, kstride, accd, sq, xs);
  reduce_partials(accd, sq, xs, red, rsq, wave, half, row);
  double* lt = logit + ((size_t)kw * T + (size_t)tt * kRouteTokens) * epad + nt * 32;
  for (int j = tid; j < 32 * 32; j += kLogitWaves * 64) {
    const int m = j >> 5, c = j & 31;
    double v = red[0][m][c];
#pragma unroll
    for (int s = 1; s < 8; ++s) v += red[s][m][c];
    if (tt * kRouteTokens + m < T) lt[(size_t)m * epad + c] = v;
  }
  if (tid < 64) {
    const int which = tid >> 5, r = tid & 31;
    float v = 0.0f;
    for (int w = 0; w < kLogitWaves; ++w) v += rsq[w][which][r];
    if (which == 0 && nt == 0 && tt * kRouteTokens + r < T) xsq[(size_t)kw * T + tt * kRouteTokens + r] = v;
    if (which == 1 && tt == 0) wsq[(size_t)kw * epad + nt * 32 + r] = v;
  }
}

// Router logits for larger batches.  A workgroup of 8 wavefronts takes 64 tokens (two 32-token
// tiles) x one 32-expert tile x a contiguous slice of K (KW slices).  K goes in rounds of 64:
// every thread loads one float4 of the round's 32 x 64 router chunk, splits it into the three
// bf16 terms and stores them in an LDS ring of two rounds, so each router weight is split once
// per 64 tokens and read from LDS by both token tiles; wavefront (tile q, lane group j) takes
// k-step j of every round for tile q.  The arithmetic per k-step is that of logit_steps: three
// bf16 MFMAs from zero, their fp32 result added into float64.  The four k-step lanes' partial
// tiles are summed in LDS in a fixed order.  Loads run two rounds ahead.
constexpr int kWideRowBytes = 128 + 16;        // one expert row of a round in bf16, padded
constexpr int kWidePlane = 32 * kWideRowBytes; // one term of a round
constexpr int kWideBuf = 3 * kWidePlane;

__global__ __launch_bounds__(kWideWaves * 64) void route_logits_wide_kernel(
    int T, int D, int E, int KW, const uint16_t* __restrict__ x, const float* __restrict__ wr,
    double* __restrict__ logit, float* __restrict__ xsq, float* __restrict__ wsq, int logit_wgs,
    uint8_t* __restrict__ xpack, int af) {
  constexpr int kRedBytes = 4 * 2 * 32 * 33 * 8;                 // [k-step lane][tile][token][expert]
  static_assert(2 * kWideBuf <= kRedBytes, "the ring fits the reduction area");
  __shared__ __align__(16) uint8_t smem[kRedBytes];
  __shared__ float rsx[4][2][32];                               // partial ||x_t||^2
  if ((int)blockIdx.x >= logit_wgs) {                           // activation split, one block per lane
    const long long blk = (long long)(blockIdx.x - logit_wgs) * (kWideWaves * 64) + threadIdx.x;
    pack_block_lane(x, D, (long long)T * (D / kBlock), blk, xpack, af);
    return;
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int tq = wave & 1, kq = wave >> 1;
  const int nte = (E + 31) / 32;
  const int kw = blockIdx.x % KW;
  const int nt = (blockIdx.x / KW) % nte;
  const int tb = blockIdx.x / (KW * nte);
  const int epad = nte * 32;
  const int row = lane & 31, half = lane >> 5;
  const int tok = tb * kWideTokens + tq * 32 + row;
  const int rounds = D / 64;
  const int r0 = rounds * kw / KW, r1 = rounds * (kw + 1) / KW;
  // this thread's float4 of every router chunk, and its x row (clamped; masked at the end)
  const int wrow = tid >> 4, wc4 = tid & 15;
  const bool wlive = nt * 32 + wrow < E;
  const float* wsrc = wr + (size_t)min(nt * 32 + wrow, E - 1) * D + 4 * wc4;
  const uint16_t* xa = x + (size_t)min(tok, T - 1) * D + 16 * kq + 8 * half;
  auto load_w = [&](const int r) {
    return wlive && r < r1 ? *reinterpret_cast<const float4*>(wsrc + 64 * r) : make_float4(0.f, 0.f, 0.f, 0.f);
  };
  auto load_x = [&](const int r) {
    return r < r1 ? *reinterpret_cast<const uint4*>(xa + 64 * r) : make_uint4(0, 0, 0, 0);
  };
  float4 wq[2] = {load_w(r0), load_w(r0 + 1)};
  uint4 xq[2] = {load_x(r0), load_x(r0 + 1)};
  double accd[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) accd[i] = 0.0;
  float xs = 0.0f, sq = 0.0f;
  auto round = [&](const int r, const int slot) __attribute__((always_inline)) {
    uint8_t* buf = smem + slot * kWideBuf;
    {
      const float wv[4] = {wq[slot].x, wq[slot].y, wq[slot].z, wq[slot].w};
      uint32_t hu[2], mu[2], lu[2];
      split_terms<4>(wv, hu, mu, lu);
#pragma unroll
      for (int i = 0; i < 4; ++i) sq += wv[i] * wv[i];
      uint8_t* dst = buf + wrow * kWideRowBytes + wc4 * 8;
      *reinterpret_cast<uint2*>(dst) = make_uint2(hu[0], hu[1]);
      *reinterpret_cast<uint2*>(dst + kWidePlane) = make_uint2(mu[0], mu[1]);
      *reinterpret_cast<uint2*>(dst + 2 * kWidePlane) = make_uint2(lu[0], lu[1]);
    }
    const uint4 xu = xq[slot];
    wq[slot] = load_w(r + 2);
    xq[slot] = load_x(r + 2);
    __syncthreads();                                            // the round's terms are in LDS
    const uint8_t* bb = buf + row * kWideRowBytes + 32 * kq + 16 * half;
    const uint4 hb = *reinterpret_cast<const uint4*>(bb);
    const uint4 mb = *reinterpret_cast<const uint4*>(bb + kWidePlane);
    const uint4 lb = *reinterpret_cast<const uint4*>(bb + 2 * kWidePlane);
    const uint32_t uw[4] = {xu.x, xu.y, xu.z, xu.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = __uint_as_float(uw[i] << 16), hi = __uint_as_float(uw[i] & 0xFFFF0000u);
      xs += lo * lo + hi * hi;
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
  double (*red)[2][32][33] = reinterpret_cast<double (*)[2][32][33]>(smem);
#pragma unroll
  for (int i = 0; i < 16; ++i) red[kq][tq][8 * (i >> 2) + 4 * half + (i & 3)][row] = accd[i];
  xs += __shfl_xor(xs, 32);
  if (half == 0) rsx[kq][tq][row] = xs;
  // the router rows' squared norms over this K slice: 16 threads per row, summed in a fixed order
#pragma unroll
  for (int d = 8; d >= 1; d >>= 1) sq += __shfl_xor(sq, d);
  if (tb == 0 && wc4 == 0) wsq[(size_t)kw * epad + nt * 32 + wrow] = sq;
  __syncthreads();
  for (int j = tid; j < 2 * 32 * 32; j += kWideWaves * 64) {
    const int q = j >> 10, m = (j >> 5) & 31, c = j & 31;
    const double v = ((red[0][q][m][c] + red[1][q][m][c]) + red[2][q][m][c]) + red[3][q][m][c];
    const int tj = tb * kWideTokens + q * 32 + m;
    if (tj < T) logit[((size_t)kw * T + tj) * epad + nt * 32 + c] = v;
  }
  if (nt == 0 && tid < 64) {
    const int q = tid >> 5, m = tid & 31;
    const float v = ((rsx[0][q][m] + rsx[1][q][m]) + rsx[2][q][m]) + rsx[3][q][m];
    const int tj = tb * kWideTokens + q * 32 + m;
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

// At most 32 tokens and 32 experts: one workgroup selects for every token and (perm given)
// groups the assignments.
__global__ __launch_bounds__(1024) void route_select_small_kernel(
    int T, int D, int E, int k, const uint16_t* __restrict__ x, const float* __restrict__ wr,
    const float* __restrict__ br, const double* __restrict__ logit, const float* __restrict__ xsq,
    const float* __restrict__ wsq, int32_t* __restrict__ out_idx, float* __restrict__ out_w,
    float* __restrict__ out_logits, int bm, int slots, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv,
    int32_t* __restrict__ tiles) {
  __shared__ __align__(16) SelectSmem smem;
  select_small<1024>(smem, T, D, E, k, x, wr, br, logit, xsq, wsq, out_idx, out_w, out_logits, bm, slots, counts,
                     offsets, perm, inv, tiles);
}

static hipError_t launch_logits(int T, int D, int E, const uint16_t* x, const float* wr, void* ws, uint8_t* xpack,
                                int af,
                                hipStream_t s, double** logit, float** xsq, float** wsq, int* KW) {
  *KW = route_kw(T, E);
  const RouteWs L = route_ws_layout(T, E);
  uint8_t* base = reinterpret_cast<uint8_t*>(ws);
  *logit = reinterpret_cast<double*>(base + L.logit);
  *xsq = reinterpret_cast<float*>(base + L.xsq);
  *wsq = reinterpret_cast<float*>(base + L.wsq);
  const long long pack_blocks = xpack ? (long long)T * (D / kBlock) : 0;
  const int nte = (E + 31) / 32;
  if (route_small(T, E)) {
    const int logit_wgs = ((T + kRouteTokens - 1) / kRouteTokens) * nte * *KW;
    const long long pack_wgs = (pack_blocks + kLogitWaves * 64 - 1) / (kLogitWaves * 64);
    route_logits_kernel<<<dim3((unsigned)(logit_wgs + pack_wgs)), dim3(kLogitWaves * 64), 0, s>>>(
        T, D, E, *KW, x, wr, *logit, *xsq, *wsq, logit_wgs, xpack, af);
  } else {
    const int logit_wgs = ((T + kWideTokens - 1) / kWideTokens) * nte * *KW;
    const long long pack_wgs = (pack_blocks + kWideWaves * 64 - 1) / (kWideWaves * 64);
    route_logits_wide_kernel<<<dim3((unsigned)(logit_wgs + pack_wgs)), dim3(kWideWaves * 64), 0, s>>>(
        T, D, E, *KW, x, wr, *logit, *xsq, *wsq, logit_wgs, xpack, af);
  }
  return hipGetLastError();
}

hipError_t launch_route_partials(int T, int D, int E, const uint16_t* x, const float* wr, void* ws, uint8_t* xpack,
                                 hipStream_t s, DenseSelection* sel) {
  double* logit;
  float *xsq, *wsq;
  int KW;
  const hipError_t err = launch_logits(T, D, E, x, wr, ws, xpack, kActSplit6, s, &logit, &xsq, &wsq, &KW);
  sel->logit = logit;
  sel->xsq = xsq;
  sel->wsq = wsq;
  return err;
}

hipError_t launch_route(int T, int D, int E, int k, const uint16_t* x, const float* wr, const float* br,
                        int32_t* idx, float* w, float* logits, void* ws, hipStream_t s) {
  if (T == 0) return hipSuccess;
  double* logit;
  float *xsq, *wsq;
  int KW;
  hipError_t err = launch_logits(T, D, E, x, wr, ws, nullptr, kActSplit6, s, &logit, &xsq, &wsq, &KW);
  if (err != hipSuccess) return err;
  if (route_small(T, E)) {
    route_select_small_kernel<<<dim3(1), dim3(1024), 0, s>>>(T, D, E, k, x, wr, br, logit, xsq, wsq, idx, w,
                                                             logits, 0, 0, nullptr, nullptr, nullptr, nullptr,
                                                             nullptr);
    return hipGetLastError();
  }
  route_select_kernel<<<dim3((T + 3) / 4), dim3(256), 0, s>>>(T, D, E, k, KW, x, wr, br, logit, xsq, wsq, idx, w,
                                                              logits);
  return hipGetLastError();
}

hipError_t launch_route_front(int T, int D, int E, int k, const uint16_t* x, const float* wr, const float* br,
                              int32_t* idx, float* w, void* ws, uint8_t* xpack, int32_t* counts,
                              int32_t* offsets, int32_t* perm, int32_t* inv, int32_t* tiles, hipStream_t s,
                              int af) {
  if (T == 0) return hipSuccess;
  double* logit;
  float *xsq, *wsq;
  int KW;
  hipError_t err = launch_logits(T, D, E, x, wr, ws, xpack, af, s, &logit, &xsq, &wsq, &KW);
  if (err != hipSuccess) return err;
  if (route_small(T, E)) {
    const long long n = (long long)T * k;
    route_select_small_kernel<<<dim3(1), dim3(1024), 0, s>>>(T, D, E, k, x, wr, br, logit, xsq, wsq, idx, w,
                                                             nullptr, tile_rows(n, E), (int)tile_slots(n, E),
                                                             counts, offsets, perm, inv, tiles);
    return hipGetLastError();
  }
  route_select_kernel<<<dim3((T + 3) / 4), dim3(256), 0, s>>>(T, D, E, k, KW, x, wr, br, logit, xsq, wsq, idx, w,
                                                              nullptr);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  return launch_permute(T, E, k, idx, counts, offsets, perm, inv, tiles, s);
}

}  // namespace moe
