// Router, top-k and softmax gating.
//
// The router is a linear map with bias scoring every expert for every token;
// each token keeps its top_k experts and weights them by a softmax over the
// kept scores ("gpt-oss architecture walk-through", section "Mixture of
// Experts": the router picks several experts and weights them, e.g.
// A = 0.7 NN2 + 0.3 NN4; gpt-oss keeps 4 of 32 / 128).
//
// Design (one workgroup of 4 wavefronts per 32 tokens):
//  1. Logits on the bf16 matrix cores.  x is bf16; the fp32 router weight is
//     split exactly into three bf16 terms (truncation: hi + mid + lo == w), so
//     every product is exact and only the fp32 accumulation rounds.  The four
//     waves split K; their partial tiles are summed in LDS in a fixed order.
//  2. Per token (one wave per token, 8 tokens per wave): top-k by wave-wide
//     arg-max (larger logit first, lower id on ties).
//  3. Every expert whose fp32 logit is within a band of the k-th largest is
//     re-scored in float64 (exact products, fp64 sums), and the final top-k is
//     taken over those float64 scores, so the selection is the float64
//     selection whenever the fp32 error is below half the band.  The band is
//     kBandAbs + kBandRel * ||x_t|| * max_e ||w_e||: the fp32 summation error of
//     a dot product is a small multiple of eps32 * sum_d |x_d w_d|, which
//     Cauchy-Schwarz bounds by ||x_t|| ||w_e||, so the band keeps a margin of
//     about 16 eps32-multiples at any input scale.  The gates are the softmax of
//     the float64 scores of the selected experts.
#include "moe_internal.h"

namespace moe {

constexpr float kBandAbs = 1e-4f;
constexpr float kBandRel = 32.0f * 5.9604645e-8f;   // 32 eps32
constexpr int kRouteTokens = 32;

__device__ inline uint32_t trunc_bf16_bits(float v) { return __float_as_uint(v) & 0xFFFF0000u; }

__device__ inline double wave_sum_f64(double v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
  return v;
}

// float64 score of expert e for token row xr (bf16), exact products.
__device__ double score_f64(const uint16_t* __restrict__ xr, const float* __restrict__ wre, float bias, int D,
                            int lane) {
  double acc = 0.0;
  for (int d = lane; d < D; d += 64) acc += (double)bf16_bits_to_float(xr[d]) * (double)wre[d];
  return wave_sum_f64(acc) + (double)bias;
}

__global__ __launch_bounds__(256) void route_kernel(int T, int D, int E, int k, const uint16_t* __restrict__ x,
                                                    const float* __restrict__ wr, const float* __restrict__ br,
                                                    int32_t* __restrict__ out_idx, float* __restrict__ out_w,
                                                    float* __restrict__ out_logits) {
  __shared__ float lg[kRouteTokens][kMaxExperts];
  __shared__ float wsq[4][kMaxExperts];        // per-wave partial ||w_e||^2

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * kRouteTokens;
  const int nte = (E + 31) / 32;
  const int kq = D / 4;                // K range of this wave: [wave*kq, wave*kq + kq), kq % 16 == 0
  const int row = lane & 31;
  const int half = lane >> 5;
  const int tok = t0 + row;

  // ---- 1. logits tile [32 tokens][E] ----------------------------------------
  for (int nt = 0; nt < nte; ++nt) {
    const int e = nt * 32 + row;
    v16f acc = {}, acc_s = {};     // hi products / the two small terms (keeps the big sum's roundings few)
    float sq = 0.0f;
    const uint16_t* xa = x + (size_t)tok * D + wave * kq + 8 * half;
    const float* wb = wr + (size_t)e * D + wave * kq + 8 * half;
    for (int k0 = 0; k0 < kq; k0 += 16) {
      v8bf a = {};
      if (tok < T) {
        uint4 u = *reinterpret_cast<const uint4*>(xa + k0);
        a = __builtin_bit_cast(v8bf, u);
      }
      float wv[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (e < E) {
        float4 w0 = *reinterpret_cast<const float4*>(wb + k0);
        float4 w1 = *reinterpret_cast<const float4*>(wb + k0 + 4);
        wv[0] = w0.x; wv[1] = w0.y; wv[2] = w0.z; wv[3] = w0.w;
        wv[4] = w1.x; wv[5] = w1.y; wv[6] = w1.z; wv[7] = w1.w;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) sq += wv[i] * wv[i];
      uint32_t hb[8], mb[8], lb[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t h = trunc_bf16_bits(wv[i]);
        const float r1 = wv[i] - __uint_as_float(h);            // exact
        const uint32_t m = trunc_bf16_bits(r1);
        const float r2 = r1 - __uint_as_float(m);                // exact, <= 8 significant bits
        hb[i] = h >> 16; mb[i] = m >> 16; lb[i] = __float_as_uint(r2) >> 16;
      }
      uint4 hu = make_uint4(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16), hb[4] | (hb[5] << 16), hb[6] | (hb[7] << 16));
      uint4 mu = make_uint4(mb[0] | (mb[1] << 16), mb[2] | (mb[3] << 16), mb[4] | (mb[5] << 16), mb[6] | (mb[7] << 16));
      uint4 lu = make_uint4(lb[0] | (lb[1] << 16), lb[2] | (lb[3] << 16), lb[4] | (lb[5] << 16), lb[6] | (lb[7] << 16));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(v8bf, hu), acc, 0, 0, 0);
      acc_s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(v8bf, mu), acc_s, 0, 0, 0);
      acc_s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(v8bf, lu), acc_s, 0, 0, 0);
    }
    acc += acc_s;
    sq += __shfl_xor(sq, 32);
    if (half == 0) wsq[wave][nt * 32 + row] = sq;
    // fixed-order reduction of the four K-partials: wave 0 stores, waves 1..3 add in turn
    for (int wv = 0; wv < 4; ++wv) {
      if (wave == wv) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = 8 * (r >> 2) + 4 * half + (r & 3);
          const int col = nt * 32 + row;
          if (wv == 0) lg[m][col] = acc[r];
          else lg[m][col] += acc[r];
        }
      }
      __syncthreads();
    }
  }

  // ---- 2./3. per-token selection ---------------------------------------------
  // max_e ||w_e||^2 (the K-partials of the four waves are summed in a fixed order)
  float wmax2 = 0.0f;
  for (int e = lane; e < E; e += 64) wmax2 = fmaxf(wmax2, ((wsq[0][e] + wsq[1][e]) + wsq[2][e]) + wsq[3][e]);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) wmax2 = fmaxf(wmax2, __shfl_xor(wmax2, d));
  for (int i = wave * 8; i < wave * 8 + 8; ++i) {
    const int t = t0 + i;
    if (t >= T) break;                                   // uniform per wave
    float xsq = 0.0f;
    for (int d = lane; d < D; d += 64) {
      const float xv = bf16_bits_to_float(x[(size_t)t * D + d]);
      xsq += xv * xv;
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) xsq += __shfl_xor(xsq, d);
    float band = kBandAbs + kBandRel * sqrtf(xsq * wmax2);
    float v[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int e = lane + 64 * c;
      v[c] = e < E ? lg[i][e] + br[e] : -INFINITY;
      if (out_logits && e < E) out_logits[(size_t)t * E + e] = v[c];
    }
    // k rounds of arg-max; taken experts are excluded by a per-lane bit mask
    uint32_t taken = 0;
    float kth = 0.0f;
    for (int j = 0; j < k; ++j) {
      float bv = -INFINITY;
      int be = 0x7fffffff;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int e = lane + 64 * c;
        if (e < E && !(taken & (1u << c)) && (v[c] > bv || (v[c] == bv && e < be))) { bv = v[c]; be = e; }
      }
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) {
        const float ov = __shfl_xor(bv, d);
        const int oe = __shfl_xor(be, d);
        if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
      }
      if ((be & 63) == lane) taken |= 1u << (be >> 6);
      kth = bv;
    }
    band += 4.0f * 5.9604645e-8f * fabsf(kth);           // rounding of the logit itself (bias-sized logits)
    // candidates: every expert within the band of the k-th largest (includes the k picks),
    // enumerated in ascending id; candidate n lives in lane n % 64, slot n / 64.
    double cl[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    int ce[4] = {0x7fffffff, 0x7fffffff, 0x7fffffff, 0x7fffffff};
    int n = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int e = lane + 64 * c;
      const bool is_c = e < E && ((taken & (1u << c)) || v[c] >= kth - band);
      uint64_t m = __ballot(is_c);
      while (m) {                                        // uniform loop over the candidate set
        const int src = __ffsll((long long)m) - 1;
        m &= m - 1;
        const int cand = src + 64 * c;
        const double s = score_f64(x + (size_t)t * D, wr + (size_t)cand * D, br[cand], D, lane);
        if ((n & 63) == lane) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (q == (n >> 6)) { cl[q] = s; ce[q] = cand; }
        }
        ++n;
      }
    }
    // final top-k over the float64 scores (larger first, lower id on ties)
    uint32_t sel = 0;
    double mx = -INFINITY;
    for (int j = 0; j < k; ++j) {
      double bv = -INFINITY;
      int be = 0x7fffffff;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (ce[q] != 0x7fffffff && !(sel & (1u << q)) && (cl[q] > bv || (cl[q] == bv && ce[q] < be))) {
          bv = cl[q]; be = ce[q];
        }
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) {
        const double ov = __shfl_xor(bv, d);
        const int oe = __shfl_xor(be, d);
        if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (ce[q] == be) sel |= 1u << q;
      if (j == 0) mx = bv;                               // the first pick is the maximum
    }
    // gates: softmax over the selected float64 scores; slots in ascending id, which is
    // candidate order, so a slot is the number of selected candidates before it
    double ex[4];
    double part = 0.0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      ex[q] = (sel & (1u << q)) ? exp(cl[q] - mx) : 0.0;
      part += ex[q];
    }
    const double sum = wave_sum_f64(part);
    int before = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint64_t m = __ballot((sel >> q) & 1u);
      const int slot = before + __popcll(m & ((1ull << lane) - 1ull));
      if (sel & (1u << q)) {
        out_idx[(size_t)t * k + slot] = ce[q];
        out_w[(size_t)t * k + slot] = (float)(ex[q] / sum);
      }
      before += __popcll(m);
    }
  }
}

hipError_t launch_route(int T, int D, int E, int k, const uint16_t* x, const float* wr, const float* br,
                        int32_t* idx, float* w, float* logits, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int blocks = (T + kRouteTokens - 1) / kRouteTokens;
  route_kernel<<<dim3(blocks), dim3(256), 0, s>>>(T, D, E, k, x, wr, br, idx, w, logits);
  return hipGetLastError();
}

}  // namespace moe
