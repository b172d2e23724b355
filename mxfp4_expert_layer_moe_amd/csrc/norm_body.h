// RMSNorm arithmetic shared by the standalone kernel (norm.hip) and the routing front end that
// folds it in (route.hip): gpt-oss normalises the residual stream with RMSNorm before each
// sublayer, dividing by the root mean square and multiplying by a learned per-channel scale, with
// no mean subtraction and no bias ("From GPT-2 to gpt-oss", section 7, Figures 11 and 12;
// rms_norm_eps = 1e-5 in the model cards' config tables).
//
//   r_t      = 1 / sqrt(sum_d x[t,d]^2 / D + eps)
//   xn[t,d]  = bf16( (x[t,d] * r_t) * gamma[d] )
//
// Everything is float64 (the squares of bf16 values are exact); xn is rounded once to bf16, to
// nearest even, from float64.  The sum of a row is taken by one workgroup in a fixed order
// (row_rms_inv), so every kernel that computes r_t gets the same bits.
#pragma once
#include "moe_internal.h"

namespace moe {

// float64 -> bf16 bits, round to nearest, ties to even, with no branch.  With 2^e <= |v| < 2^(e+1),
// the bf16 spacing at v is 2^p, p = max(e, -126) - 7 (below 2^-126 the bf16 subnormals, 2^-133).
// Adding c = 1.5 * 2^(p+52) puts v + c in a binade whose float64 spacing is 2^p, so (v + c) - c is v
// rounded to a multiple of 2^p, ties to even (c / 2^p is even, so the tie goes the same way for
// either sign); the sign is copied back so that a value rounding to zero keeps it.  The result has
// at most 8 significant bits: its float32 conversion is exact (the launch preserves float32
// denormals), float32 overflow gives infinity as bf16 does, and the bf16 bits are the float32's
// upper half.  e is capped at 128: anything at or above 2^128 becomes infinity either way.
// Contraction is off: v must be the float64 value it is given, not a product fused into v + c.
__device__ inline uint32_t f64_to_bf16_rne(double v) {
#pragma clang fp contract(off)
  const int e = min(max(__builtin_amdgcn_frexp_exp(v) - 1, -126), 128);
  const double c = __builtin_amdgcn_ldexp(1.5, e + 45);
  const double r = __builtin_copysign((v + c) - c, v);
  return __float_as_uint((float)r) >> 16;
}

// sum of the squares of one 8-value bf16 chunk, in element order
__device__ inline double chunk_sum_sq(const uint4 q) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const double lo = (double)__uint_as_float(w[i] << 16), hi = (double)__uint_as_float(w[i] & 0xFFFF0000u);
    s += lo * lo;
    s += hi * hi;
  }
  return s;
}

// r_t of row xr (bf16, D % 8 == 0) by one workgroup of kNormThreads threads: thread i sums the
// 8-value chunks i, i + kNormThreads, ... of the row, each chunk's squares in element order; each
// wavefront adds its threads' sums by a butterfly, then the wavefront sums are added in order
// (part: kNormThreads / 64 doubles of LDS).  Every thread returns r_t.  The thread's first chunk is
// returned in held (zeros past the row); later chunks (rows over 8 * kNormThreads wide) are loaded
// as they are summed.  Contains a workgroup barrier: every thread of the workgroup calls it.
constexpr int kNormThreads = 512;
__device__ inline double row_rms_inv(const uint16_t* __restrict__ xr, int D, double eps, double* part, uint4& held) {
  const int tid = threadIdx.x;
  const int nc = D / 8;
  const uint4* x4 = reinterpret_cast<const uint4*>(xr);
  held = tid < nc ? x4[tid] : make_uint4(0, 0, 0, 0);
  double ss = tid < nc ? chunk_sum_sq(held) : 0.0;
  for (int c = tid + kNormThreads; c < nc; c += kNormThreads) ss += chunk_sum_sq(x4[c]);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) ss += __shfl_xor(ss, d);
  if ((tid & 63) == 0) part[tid >> 6] = ss;
  __syncthreads();
  ss = part[0];
#pragma unroll
  for (int w = 1; w < kNormThreads / 64; ++w) ss += part[w];
  return 1.0 / sqrt(ss / (double)D + eps);
}

// xn of one 8-value chunk of a row with its eight gamma values ga, gb: bf16((x * r) * gamma),
// packed as in the input
__device__ inline uint4 chunk_rmsnorm(const uint4 q, double r, const float4 ga, const float4 gb) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  const float g[8] = {ga.x, ga.y, ga.z, ga.w, gb.x, gb.y, gb.z, gb.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const double lo = (double)__uint_as_float(w[i] << 16), hi = (double)__uint_as_float(w[i] & 0xFFFF0000u);
    o[i] = f64_to_bf16_rne((lo * r) * (double)g[2 * i]) | (f64_to_bf16_rne((hi * r) * (double)g[2 * i + 1]) << 16);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// the same for chunk c of a row, gamma read from memory
__device__ inline uint4 chunk_rmsnorm(const uint4 q, double r, const float* __restrict__ gamma, int c) {
  const float4* g4 = reinterpret_cast<const float4*>(gamma);
  return chunk_rmsnorm(q, r, g4[2 * c], g4[2 * c + 1]);
}

}  // namespace moe
