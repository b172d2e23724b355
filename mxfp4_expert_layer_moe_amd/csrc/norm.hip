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
// The arithmetic (float64 throughout, one bf16 rounding, and the order in which
// a row's squares are summed) lives in norm_body.h, shared with the routing
// front end that folds the normalisation into its own launch for small
// batches, so both give the same bits.  Here: one workgroup of 512 threads per
// row, one 8-value chunk per thread.  Memory-bound: reads 2D + 4D bytes, writes
// 2D bytes per row.
#include "norm_body.h"

namespace moe {

// One workgroup of kNormThreads per row: r_t (row_rms_inv), then every thread scales its chunks.
__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(int D, const uint16_t* __restrict__ x,
                                                               const float* __restrict__ gamma, double eps,
                                                               uint16_t* __restrict__ xn) {
  __shared__ double part[kNormThreads / 64];
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int nc = D / 8;
  const uint16_t* xr = x + (size_t)row * D;
  const float4* g4 = reinterpret_cast<const float4*>(gamma);
  // gamma of the first chunk, loaded beside the row
  const float4 ga = tid < nc ? g4[2 * tid] : make_float4(0.f, 0.f, 0.f, 0.f);
  const float4 gb = tid < nc ? g4[2 * tid + 1] : ga;
  uint4 held;
  const double r = row_rms_inv(xr, D, eps, part, held);
  const uint4* x4 = reinterpret_cast<const uint4*>(xr);
  uint4* out = reinterpret_cast<uint4*>(xn + (size_t)row * D);
  if (tid < nc) out[tid] = chunk_rmsnorm(held, r, ga, gb);
  for (int c = tid + kNormThreads; c < nc; c += kNormThreads) out[c] = chunk_rmsnorm(x4[c], r, gamma, c);
}

hipError_t launch_rmsnorm(int T, int D, const uint16_t* x, const float* gamma, float eps, uint16_t* xn,
                          hipStream_t s) {
  if (T == 0) return hipSuccess;
  rmsnorm_kernel<<<dim3((unsigned)T), dim3(kNormThreads), 0, s>>>(D, x, gamma, (double)eps, xn);
  return hipGetLastError();
}

}  // namespace moe
