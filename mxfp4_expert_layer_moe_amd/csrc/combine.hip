// Weighted combine of the selected experts' outputs.
//
// The layer output of a token is the gate-weighted sum of its experts' outputs
// ("gpt-oss architecture walk-through", section "Mixture of Experts": A = 0.7
// NN2 + 0.3 NN4).  The gate is already applied by the down-projection epilogue,
// so this kernel gathers the k fp16 rows of each token (positions inv[t*k + j])
// and sums them in fp32 in slot order (ascending expert id): no atomics, the
// same bits on every run.  HBM-bound: reads k rows, writes one.
#include "moe_internal.h"

namespace moe {

template <bool BF16_OUT>
__global__ __launch_bounds__(256) void combine_kernel(int T, int D, int k, const _Float16* __restrict__ y_perm,
                                                      const int32_t* __restrict__ inv, void* __restrict__ y) {
  const int d4 = D / 4;
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long long)T * d4) return;
  const int t = (int)(gid / d4);
  const int c = (int)(gid - (long long)t * d4) * 4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const int p = inv[(size_t)t * k + j];
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
    const h4 v = *reinterpret_cast<const h4*>(y_perm + (size_t)p * D + c);
    acc.x += (float)v.x; acc.y += (float)v.y; acc.z += (float)v.z; acc.w += (float)v.w;
  }
  if (BF16_OUT) {
    const uint32_t b0 = __float_as_uint(bf16_round(acc.x)) >> 16, b1 = __float_as_uint(bf16_round(acc.y)) >> 16;
    const uint32_t b2 = __float_as_uint(bf16_round(acc.z)) >> 16, b3 = __float_as_uint(bf16_round(acc.w)) >> 16;
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(y) + (size_t)t * D + c) =
        make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
  } else {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(y) + (size_t)t * D + c) = acc;
  }
}

hipError_t launch_combine(int T, int D, int k, const _Float16* y_perm, const int32_t* inv, void* y, int y_bf16,
                          hipStream_t s) {
  const long long n = (long long)T * (D / 4);
  if (n == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((n + 255) / 256);
  if (y_bf16)
    combine_kernel<true><<<dim3(blocks), dim3(256), 0, s>>>(T, D, k, y_perm, inv, y);
  else
    combine_kernel<false><<<dim3(blocks), dim3(256), 0, s>>>(T, D, k, y_perm, inv, y);
  return hipGetLastError();
}

}  // namespace moe
