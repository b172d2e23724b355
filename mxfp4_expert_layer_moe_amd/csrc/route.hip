// Router, top-k and softmax gating.
//
// The router is a linear map with bias scoring every expert for every token;
// each token keeps its top_k experts and weights them by a softmax over the
// kept scores ("gpt-oss architecture walk-through", section "Mixture of
// Experts": the router picks several experts and weights them, e.g.
// A = 0.7 NN2 + 0.3 NN4; gpt-oss keeps 4 of 32 / 128).
//
// Design (one workgroup of 8 wavefronts per 32 tokens):
//  1. Logits on the bf16 matrix cores.  x is bf16; the fp32 router weight is
//     split exactly into three bf16 terms (truncation: hi + mid + lo == w), so
//     every product is exact.  Each 16-wide k-step's three MFMAs start from
//     zero and their small fp32 result is added into a float64 accumulator, so
//     the only fp32 roundings are those of 16-term partial sums.  Work items
//     are (32-expert tile, K slice) pairs spread over the 8 waves; K slices are
//     summed in LDS in a fixed order (deterministic).
//  2. Per token (one wave per token): top-k by wave-wide arg-max over the
//     float64 logits (larger first, lower id on ties).
//  3. If any other expert lies within a band of the k-th largest, every expert
//     in the band is re-scored exactly in float64 and the top-k is re-taken
//     over those scores.  The band, 36 eps32 ||x_t|| max_e ||w_e||, is twice a
//     worst-case bound of the step-1 error (at most 18 fp32 roundings per
//     k-step, each at most eps32 times that k-step's sum of |x_d w_d|, and
//     sum_d |x_d w_d| <= ||x_t|| ||w_e|| by Cauchy-Schwarz), so the result is
//     the float64 selection at any input scale.  Gates are the softmax of the
//     selected float64 scores.
#include "moe_internal.h"

namespace moe {

constexpr int kRouteTokens = 32;
constexpr int kRouteWaves = 8;
constexpr double kBandRel = 36.0 * 5.9604644775390625e-8;     // 36 eps32

__device__ inline uint32_t trunc_bf16_bits(float v) { return __float_as_uint(v) & 0xFFFF0000u; }

__device__ inline double wave_sum_f64(double v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
  return v;
}

// Exact float64 score of expert row wre for token row xr (bf16): 8-wide chunks per lane.
__device__ double score_f64(const uint16_t* __restrict__ xr, const float* __restrict__ wre, double bias, int D,
                            int lane) {
  double acc = 0.0;
  for (int c = lane; c < D / 8; c += 64) {
    const uint4 xv = *reinterpret_cast<const uint4*>(xr + 8 * c);
    const float4 w0 = *reinterpret_cast<const float4*>(wre + 8 * c);
    const float4 w1 = *reinterpret_cast<const float4*>(wre + 8 * c + 4);
    const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
    const float wf[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc += (double)__uint_as_float(xw[i] << 16) * (double)wf[2 * i];
      acc += (double)__uint_as_float(xw[i] & 0xFFFF0000u) * (double)wf[2 * i + 1];
    }
  }
  return wave_sum_f64(acc) + bias;
}

__global__ __launch_bounds__(kRouteWaves * 64) void route_kernel(int T, int D, int E, int k,
                                                                 const uint16_t* __restrict__ x,
                                                                 const float* __restrict__ wr,
                                                                 const float* __restrict__ br,
                                                                 int32_t* __restrict__ out_idx,
                                                                 float* __restrict__ out_w,
                                                                 float* __restrict__ out_logits) {
  __shared__ double part[kRouteWaves][kRouteTokens][33];   // per work item: [token][expert in tile]
  __shared__ float wsq[kRouteWaves][32];                    // partial ||w_e||^2 per work item
  __shared__ float xsq[kRouteWaves][kRouteTokens];          // partial ||x_t||^2 per work item

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int t0 = blockIdx.x * kRouteTokens;
  const int nte = (E + 31) / 32;                   // <= 8
  const int KS = nte >= kRouteWaves ? 1 : kRouteWaves / nte;
  const int items = nte * KS;
  const int nsteps = D / 16;
  const int row = lane & 31;
  const int half = lane >> 5;

  // ---- 1. logits: work item (nt, ks) handles expert tile nt over k-steps ks, ks+KS, ... ----
  if (wave < items) {
    const int nt = wave / KS, ks = wave % KS;
    const int e = nt * 32 + row;
    const int tok = t0 + row;
    const uint16_t* xa = x + (size_t)tok * D + 8 * half;
    const float* wb = wr + (size_t)e * D + 8 * half;
    double accd[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) accd[r] = 0.0;
    float sq = 0.0f, xs = 0.0f;
#pragma unroll 2
    for (int s = ks; s < nsteps; s += KS) {
      v8bf a = {};
      if (tok < T) {
        const uint4 u = *reinterpret_cast<const uint4*>(xa + 16 * s);
        a = __builtin_bit_cast(v8bf, u);
        const uint32_t uw[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float lo = __uint_as_float(uw[i] << 16), hi = __uint_as_float(uw[i] & 0xFFFF0000u);
          xs += lo * lo + hi * hi;
        }
      }
      float wv[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (e < E) {
        const float4 w0 = *reinterpret_cast<const float4*>(wb + 16 * s);
        const float4 w1 = *reinterpret_cast<const float4*>(wb + 16 * s + 4);
        wv[0] = w0.x; wv[1] = w0.y; wv[2] = w0.z; wv[3] = w0.w;
        wv[4] = w1.x; wv[5] = w1.y; wv[6] = w1.z; wv[7] = w1.w;
      }
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
#pragma unroll
    for (int r = 0; r < 16; ++r) part[wave][8 * (r >> 2) + 4 * half + (r & 3)][row] = accd[r];
    sq += __shfl_xor(sq, 32);
    xs += __shfl_xor(xs, 32);
    if (half == 0) {
      wsq[wave][row] = sq;
      xsq[wave][row] = xs;
    }
  }
  __syncthreads();
  // fixed-order sum of the K slices, in place into slice 0 of each tile
  for (int j = tid; j < kRouteTokens * nte * 32; j += kRouteWaves * 64) {
    const int m = j / (nte * 32), ec = j % (nte * 32), nt = ec >> 5, c = ec & 31;
    double s = part[nt * KS][m][c];
    for (int ks = 1; ks < KS; ++ks) s += part[nt * KS + ks][m][c];
    part[nt * KS][m][c] = s;
  }
  __syncthreads();

  // ---- 2./3. per-token selection -------------------------------------------------------
  float wmax2 = 0.0f;
  for (int e = lane; e < E; e += 64) {
    float s = 0.0f;
    for (int ks = 0; ks < KS; ++ks) s += wsq[(e >> 5) * KS + ks][e & 31];
    wmax2 = fmaxf(wmax2, s);
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) wmax2 = fmaxf(wmax2, __shfl_xor(wmax2, d));

  for (int i = wave; i < kRouteTokens; i += kRouteWaves) {
    const int t = t0 + i;
    if (t >= T) break;                                   // uniform per wave
    float xn2 = 0.0f;
    for (int ks = 0; ks < KS; ++ks) xn2 += xsq[ks][i];
    double v[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int e = lane + 64 * c;
      v[c] = e < E ? part[(e >> 5) * KS][i][e & 31] + (double)br[e] : -INFINITY;
      if (out_logits && e < E) out_logits[(size_t)t * E + e] = (float)v[c];
    }
    // k rounds of arg-max; taken experts are excluded by a per-lane bit mask
    uint32_t taken = 0;
    double kth = 0.0;
    for (int j = 0; j < k; ++j) {
      double bv = -INFINITY;
      int be = 0x7fffffff;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int e = lane + 64 * c;
        if (e < E && !(taken & (1u << c)) && (v[c] > bv || (v[c] == bv && e < be))) { bv = v[c]; be = e; }
      }
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) {
        const double ov = __shfl_xor(bv, d);
        const int oe = __shfl_xor(be, d);
        if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
      }
      if ((be & 63) == lane) taken |= 1u << (be >> 6);
      kth = bv;
    }
    const double band = kBandRel * sqrt((double)xn2 * (double)wmax2);
    bool cand[4];
    int n = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int e = lane + 64 * c;
      cand[c] = e < E && ((taken & (1u << c)) || v[c] >= kth - band);
      n += __popcll(__ballot(cand[c]));
    }
    if (n > k) {
      // near the boundary: re-score every candidate exactly, then re-take the top-k
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint64_t m = __ballot(cand[c]);
        while (m) {                                      // uniform loop over the candidate set
          const int src = __ffsll((long long)m) - 1;
          m &= m - 1;
          const int e = src + 64 * c;
          const double s = score_f64(x + (size_t)t * D, wr + (size_t)e * D, (double)br[e], D, lane);
          if (lane == src) v[c] = s;
        }
        if (!cand[c]) v[c] = -INFINITY;
      }
      taken = 0;
      for (int j = 0; j < k; ++j) {
        double bv = -INFINITY;
        int be = 0x7fffffff;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int e = lane + 64 * c;
          if (cand[c] && !(taken & (1u << c)) && (v[c] > bv || (v[c] == bv && e < be))) { bv = v[c]; be = e; }
        }
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) {
          const double ov = __shfl_xor(bv, d);
          const int oe = __shfl_xor(be, d);
          if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
        }
        if ((be & 63) == lane) taken |= 1u << (be >> 6);
      }
    }
    // gates: softmax over the selected scores; slots in ascending expert id
    double mx = -INFINITY;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (taken & (1u << c)) mx = fmax(mx, v[c]);
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) mx = fmax(mx, __shfl_xor(mx, d));
    double ex[4], part_sum = 0.0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      ex[c] = (taken & (1u << c)) ? exp(v[c] - mx) : 0.0;
      part_sum += ex[c];
    }
    const double sum = wave_sum_f64(part_sum);
    int before = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint64_t m = __ballot((taken >> c) & 1u);
      const int slot = before + __popcll(m & ((1ull << lane) - 1ull));
      if (taken & (1u << c)) {
        out_idx[(size_t)t * k + slot] = lane + 64 * c;
        out_w[(size_t)t * k + slot] = (float)(ex[c] / sum);
      }
      before += __popcll(m);
    }
  }
}

hipError_t launch_route(int T, int D, int E, int k, const uint16_t* x, const float* wr, const float* br,
                        int32_t* idx, float* w, float* logits, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int blocks = (T + kRouteTokens - 1) / kRouteTokens;
  route_kernel<<<dim3(blocks), dim3(kRouteWaves * 64), 0, s>>>(T, D, E, k, x, wr, br, idx, w, logits);
  return hipGetLastError();
}

}  // namespace moe
