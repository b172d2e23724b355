// RMSNorm in front of the MoE layer.
//
// gpt-oss normalises the residual stream with RMSNorm before each sublayer:
// the activations are divided by their root mean square and multiplied by a
// learned per-channel scale, with no mean subtraction and no bias ("From GPT-2
// to gpt-oss", section 7, Figures 11 and 12; every transformer block holds two
// such normalisation blocks, "gpt-oss architecture walk-through", section
// "Transformer Blocks"; rms_norm_eps = 1e-5 in the model cards' config tables).
//
//   r_t      = 1 / sqrt(sum_d x[t,d]^2 / D + eps)
//   xn[t,d]  = bf16( (x[t,d] * r_t) * gamma[d] )
//
// Everything is float64 (the squares of bf16 values are exact, the sum is
// float64); the result is rounded once to bf16, to nearest even, straight from
// float64.  One workgroup of 256 threads per row: squares summed per thread,
// across each wavefront, then over the four wavefronts in a fixed order; the
// row stays in registers for the scaling.  Memory-bound: reads 2D + 4D bytes,
// writes 2D bytes per row.
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

__device__ inline double wave_sum_f64_xor(double v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
  return v;
}

constexpr int kNormThreads = 256;
constexpr int kNormHeld = 2;            // 8-value chunks a thread keeps in registers (D <= 4096)

// One workgroup per row; thread i handles the 8-value chunks i, i + 256, ...; the chunks of a row
// up to 4096 wide stay in registers between the sum and the scaling.
__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(int D, const uint16_t* __restrict__ x,
                                                               const float* __restrict__ gamma, double eps,
                                                               uint16_t* __restrict__ xn) {
  __shared__ double part[kNormThreads / 64];
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int nc = D / 8;
  const uint4* xr = reinterpret_cast<const uint4*>(x + (size_t)row * D);
  uint4 held[kNormHeld];
#pragma unroll
  for (int i = 0; i < kNormHeld; ++i) {
    const int c = tid + kNormThreads * i;
    held[i] = c < nc ? xr[c] : make_uint4(0, 0, 0, 0);
  }
  auto sum_sq = [](const uint4 q) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    double s = 0.0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const double lo = (double)__uint_as_float(w[i] << 16), hi = (double)__uint_as_float(w[i] & 0xFFFF0000u);
      s += lo * lo;
      s += hi * hi;
    }
    return s;
  };
  double ss = 0.0;
#pragma unroll
  for (int i = 0; i < kNormHeld; ++i) ss += sum_sq(held[i]);
  for (int c = tid + kNormThreads * kNormHeld; c < nc; c += kNormThreads) ss += sum_sq(xr[c]);
  ss = wave_sum_f64_xor(ss);
  if ((tid & 63) == 0) part[tid >> 6] = ss;
  __syncthreads();
  ss = part[0];
#pragma unroll
  for (int w = 1; w < kNormThreads / 64; ++w) ss += part[w];
  const double r = 1.0 / sqrt(ss / (double)D + eps);
  uint4* out = reinterpret_cast<uint4*>(xn + (size_t)row * D);
  const float4* g4 = reinterpret_cast<const float4*>(gamma);
  auto scale = [&](const int c, const uint4 q) {
    const float4 ga = g4[2 * c], gb = g4[2 * c + 1];
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    const float g[8] = {ga.x, ga.y, ga.z, ga.w, gb.x, gb.y, gb.z, gb.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const double lo = (double)__uint_as_float(w[i] << 16), hi = (double)__uint_as_float(w[i] & 0xFFFF0000u);
      o[i] = f64_to_bf16_rne((lo * r) * (double)g[2 * i]) | (f64_to_bf16_rne((hi * r) * (double)g[2 * i + 1]) << 16);
    }
    out[c] = make_uint4(o[0], o[1], o[2], o[3]);
  };
#pragma unroll
  for (int i = 0; i < kNormHeld; ++i) {
    const int c = tid + kNormThreads * i;
    if (c < nc) scale(c, held[i]);
  }
  for (int c = tid + kNormThreads * kNormHeld; c < nc; c += kNormThreads) scale(c, xr[c]);
}

hipError_t launch_rmsnorm(int T, int D, const uint16_t* x, const float* gamma, float eps, uint16_t* xn,
                          hipStream_t s) {
  if (T == 0) return hipSuccess;
  rmsnorm_kernel<<<dim3((unsigned)T), dim3(kNormThreads), 0, s>>>(D, x, gamma, (double)eps, xn);
  return hipGetLastError();
}

}  // namespace moe
