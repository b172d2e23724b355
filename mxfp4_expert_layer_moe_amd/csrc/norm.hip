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
// batches, so both give the same bits.  Memory-bound: reads 2D + 4D bytes,
// writes 2D bytes per row.  Rows up to 4096 wide: one wavefront per row, four
// rows per workgroup, every chunk of the row in flight at once and no barrier;
// wider rows: one workgroup of 512 threads per row.
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

// One wavefront per row (D / 8 <= kNormRowChunks chunks), with row_rms_inv's sum, term for term.
// There, thread 64 w + l of the 512 sums the chunks 64 w + l, 64 w + l + 512, ... in order; each
// wavefront w adds its 64 sums by a butterfly; the eight wavefront sums are added in order w = 0..7.
// Here lane l keeps the eight sums of w = 0..7 side by side (with at most 512 chunks each holds one
// chunk or none: 0.0 + s = s exactly), runs the same butterfly on each and adds them in the same
// order, so r_t has the same bits.  The row's chunks stay in registers for the scaling pass.
constexpr int kNormRowChunks = 512;
constexpr int kNormRowHold = kNormRowChunks / 64;       // chunks per lane
__global__ __launch_bounds__(256) void rmsnorm_rows_kernel(int T, int D, const uint16_t* __restrict__ x,
                                                           const float* __restrict__ gamma, double eps,
                                                           uint16_t* __restrict__ xn) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= T) return;                                  // uniform per wavefront; no barrier follows
  const int nc = D / 8;
  const uint4* x4 = reinterpret_cast<const uint4*>(x + (size_t)row * D);
  uint4 held[kNormRowHold];
#pragma unroll
  for (int w = 0; w < kNormRowHold; ++w) {
    const int c = lane + 64 * w;
    held[w] = c < nc ? x4[c] : make_uint4(0, 0, 0, 0);
  }
  double part[kNormRowHold];
#pragma unroll
  for (int w = 0; w < kNormRowHold; ++w) part[w] = lane + 64 * w < nc ? chunk_sum_sq(held[w]) : 0.0;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1)
#pragma unroll
    for (int w = 0; w < kNormRowHold; ++w) part[w] += __shfl_xor(part[w], d);
  double ss = part[0];
#pragma unroll
  for (int w = 1; w < kNormRowHold; ++w) ss += part[w];
  const double r = 1.0 / sqrt(ss / (double)D + eps);
  uint4* out = reinterpret_cast<uint4*>(xn + (size_t)row * D);
#pragma unroll
  for (int w = 0; w < kNormRowHold; ++w) {
    const int c = lane + 64 * w;
    if (c < nc) out[c] = chunk_rmsnorm(held[w], r, gamma, c);
  }
}
static_assert(kNormRowChunks == kNormThreads, "the row kernel mirrors row_rms_inv's 512 partial sums");

hipError_t launch_rmsnorm(int T, int D, const uint16_t* x, const float* gamma, float eps, uint16_t* xn,
                          hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (D / 8 <= kNormRowChunks)
    rmsnorm_rows_kernel<<<dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s>>>(T, D, x, gamma, (double)eps, xn);
  else
    rmsnorm_kernel<<<dim3((unsigned)T), dim3(kNormThreads), 0, s>>>(D, x, gamma, (double)eps, xn);
  return hipGetLastError();
}

}  // namespace moe
