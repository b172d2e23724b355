// Weighted combine of the selected experts' outputs.
//
// The layer output of a token is the gate-weighted sum of its experts' outputs
// ("gpt-oss architecture walk-through", section "Mixture of Experts": A = 0.7
// NN2 + 0.3 NN4).  The gate is already applied by the down-projection epilogue,
// so this kernel gathers the k fp16 rows of each token (positions inv[t*k + j])
// and sums them in fp32 in slot order (ascending expert id): no atomics, the
// same bits on every run.  HBM-bound: reads k rows, writes one.  A thread owns 8
// columns of a token and issues the index and row loads of 4 slots at a time, so
// a token's gather costs two memory round trips per 4 slots.  When the down
// projection wrote the rows in assignment order (row t*k + j, the whole-layer
// path), the rows are read directly: one round trip.
//
// With a residual (the MoE half of a pre-norm transformer block, y = x + MoE(xn):
// the block's input and output are both [N x D], "gpt-oss architecture
// walk-through", section "Transformer Blocks"), the bf16 residual row is added
// to the slot-order sum with one more fp32 addition.
#include <type_traits>

#include "moe_internal.h"

namespace moe {

constexpr int kCombineCols = 8;        // columns per thread: one 16-byte fp16 load per row
constexpr int kCombineBatch = 4;       // slots whose index and row loads are issued together

template <bool BF16_OUT, bool RESIDUAL, bool DIRECT>
__global__ __launch_bounds__(256) void combine_kernel(int T, int D, int k, const _Float16* __restrict__ y_perm,
                                                      const int32_t* __restrict__ inv,
                                                      const uint16_t* __restrict__ residual, void* __restrict__ y) {
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  const int d8 = D / kCombineCols;
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long long)T * d8) return;
  const int t = (int)(gid / d8);
  const int c = (int)(gid - (long long)t * d8) * kCombineCols;
  float acc[kCombineCols];
#pragma unroll
  for (int i = 0; i < kCombineCols; ++i) acc[i] = 0.0f;
  for (int j0 = 0; j0 < k; j0 += kCombineBatch) {
    int p[kCombineBatch];
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u)
      p[u] = j0 + u >= k ? 0 : DIRECT ? t * k + j0 + u : inv[(size_t)t * k + j0 + u];
    h8 v[kCombineBatch];
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u)
      if (j0 + u < k && p[u] >= 0) v[u] = *reinterpret_cast<const h8*>(y_perm + (size_t)p[u] * D + c);
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u)                 // slot order; a slot with inv = -1 has no row
      if (j0 + u < k && p[u] >= 0) {
#pragma unroll
        for (int i = 0; i < kCombineCols; ++i) acc[i] += (float)v[u][i];
      }
  }
  if constexpr (RESIDUAL) {
    const uint4 r = *reinterpret_cast<const uint4*>(residual + (size_t)t * D + c);
    const uint32_t rw[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < kCombineCols / 2; ++i) {
      acc[2 * i] = __uint_as_float(rw[i] << 16) + acc[2 * i];
      acc[2 * i + 1] = __uint_as_float(rw[i] & 0xFFFF0000u) + acc[2 * i + 1];
    }
  }
  if (BF16_OUT) {
    uint32_t w[kCombineCols / 2];
#pragma unroll
    for (int i = 0; i < kCombineCols / 2; ++i)
      w[i] = (__float_as_uint(bf16_round(acc[2 * i])) >> 16) | (__float_as_uint(bf16_round(acc[2 * i + 1])) & 0xFFFF0000u);
    *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(y) + (size_t)t * D + c) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    float4* o = reinterpret_cast<float4*>(reinterpret_cast<float*>(y) + (size_t)t * D + c);
    o[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    o[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
}

hipError_t launch_combine(int T, int D, int k, const _Float16* y_perm, const int32_t* inv, const uint16_t* residual,
                          void* y, int y_bf16, hipStream_t s) {
  const long long n = (long long)T * (D / kCombineCols);
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 255) / 256)), block(256);
  auto go = [&](auto direct) {
    constexpr bool DIRECT = decltype(direct)::value;
    if (residual) {
      if (y_bf16) combine_kernel<true, true, DIRECT><<<grid, block, 0, s>>>(T, D, k, y_perm, inv, residual, y);
      else combine_kernel<false, true, DIRECT><<<grid, block, 0, s>>>(T, D, k, y_perm, inv, residual, y);
    } else {
      if (y_bf16) combine_kernel<true, false, DIRECT><<<grid, block, 0, s>>>(T, D, k, y_perm, inv, nullptr, y);
      else combine_kernel<false, false, DIRECT><<<grid, block, 0, s>>>(T, D, k, y_perm, inv, nullptr, y);
    }
  };
  if (inv) go(std::false_type{});
  else go(std::true_type{});
  return hipGetLastError();
}

}  // namespace moe
