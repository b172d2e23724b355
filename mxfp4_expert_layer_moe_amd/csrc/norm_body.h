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

// float64 -> bf16 bits, round to nearest, ties to even, directly from the float64 value.
__device__ inline uint32_t f64_to_bf16_rne(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t sign = (uint32_t)(u >> 48) & 0x8000u;
  const uint64_t a = u & 0x7FFFFFFFFFFFFFFFull;
  const int e = (int)(a >> 52) - 1023;                  // exponent before rounding
  if (e < -126) {
    // below the normal range: multiples of 2^-133 (bf16 subnormal spacing), rounded with rint
    const double q = rint(fabs(v) * 0x1p133);          // exact scaling, then nearest even integer
    return sign | (uint32_t)q;                          // q <= 128; 128 is the smallest normal
  }
  // keep 7 stored mantissa bits: the last kept bit is bit 45 of the float64 pattern
  const uint64_t r = (a + 0x00000FFFFFFFFFFFull + ((a >> 45) & 1u)) & ~0x00001FFFFFFFFFFFull;
  const int er = (int)(r >> 52) - 1023;                // a carry may raise the exponent
  if (er > 127) return sign | 0x7F80u;                  // overflow: infinity
  return sign | ((uint32_t)(er + 127) << 7) | (uint32_t)((r >> 45) & 0x7Fu);
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
