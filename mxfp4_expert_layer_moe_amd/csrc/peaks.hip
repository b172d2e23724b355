// Probes of the MI355X ceilings the layer's roofline fractions are quoted against: the issue rate
// of the matrix instruction for one operand-format pair, and a streaming read.  Declared in
// include/moe_peaks.h; built into its own library.  No code is shared with the layer.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_peaks.h"

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kChains = 4;        // independent accumulators per wavefront

// FA / FB: the instruction's format codes (0 FP8 E4M3, 2 FP6 E2M3, 4 FP4 E2M1).  Operand bits and
// scales come from the thread id: the values do not matter to the rate, only that they are finite.
template <int FA, int FB>
__global__ __launch_bounds__(256) void mfma_scaled_probe(int iters, float* __restrict__ sink) {
  const int tid = threadIdx.x;
  const uint32_t seed = 0x9E3779B9u * (blockIdx.x * 256u + tid + 1u);
  v8i a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (int)((seed * (2u * i + 1u)) & 0x33333333u);     // small codes of every format
    b[i] = (int)((seed * (2u * i + 3u)) & 0x33333333u);
  }
  const uint32_t sa = 120u, sb = 121u;
  v16f acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = v16f{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[c], FA, FB, 0, sa, 0, sb);
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  sink[blockIdx.x * 256 + tid] = s;
}

__global__ __launch_bounds__(256) void mfma_bf16_probe(int iters, float* __restrict__ sink) {
  const int tid = threadIdx.x;
  v8bf a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)((tid + i) & 7));
    b[i] = (__bf16)(0.002f * (float)((tid * 3 + i) & 7));
  }
  v16f acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = v16f{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  sink[blockIdx.x * 256 + tid] = s;
}

// Grid-stride streaming read: thread g reads the 16-byte pieces g, g + G, g + 2G, ... (G = all
// threads), eight loads in flight per round, and XORs them into one word per thread.
template <int NT>
__global__ __launch_bounds__(256) void stream_read_probe(const uint8_t* __restrict__ buf, uint32_t pieces_lo,
                                                         uint32_t pieces_hi, uint32_t* __restrict__ sink) {
  const uint64_t pieces = ((uint64_t)pieces_hi << 32) | pieces_lo;
  const uint64_t G = (uint64_t)gridDim.x * 256u;
  uint64_t i = (uint64_t)blockIdx.x * 256u + threadIdx.x;
  uint32_t x = 0;
  constexpr int kBatch = 8;
  for (; i + (kBatch - 1) * G < pieces; i += kBatch * G) {
    v4i v[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const v4i* p = reinterpret_cast<const v4i*>(buf) + i + b * G;
      v[b] = NT ? __builtin_nontemporal_load(p) : *p;
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) x ^= (uint32_t)(v[b].x ^ v[b].y ^ v[b].z ^ v[b].w);
  }
  for (; i < pieces; i += G) {
    const v4i v = reinterpret_cast<const v4i*>(buf)[i];
    x ^= (uint32_t)(v.x ^ v.y ^ v.z ^ v.w);
  }
  sink[blockIdx.x * 256 + threadIdx.x] = x;
}

}  // namespace

extern "C" {

double moe_peak_mfma_flops(moe_peak_format format, int32_t workgroups, int32_t iters) {
  const double per = format == MOE_PEAK_BF16 ? 2.0 * 32 * 32 * 16 : 2.0 * 32 * 32 * 64;
  return (double)workgroups * 4 * (double)iters * kChains * per;
}

moe_peak_status moe_peak_mfma(moe_peak_format format, int32_t workgroups, int32_t iters, float* sink,
                              hipStream_t stream) {
  if (workgroups <= 0 || iters <= 0 || !sink) return MOE_PEAK_EINVAL;
  const dim3 grid((unsigned)workgroups), block(256);
  switch (format) {
    case MOE_PEAK_FP6_FP4: mfma_scaled_probe<2, 4><<<grid, block, 0, stream>>>(iters, sink); break;
    case MOE_PEAK_FP4_FP4: mfma_scaled_probe<4, 4><<<grid, block, 0, stream>>>(iters, sink); break;
    case MOE_PEAK_FP8_FP4: mfma_scaled_probe<0, 4><<<grid, block, 0, stream>>>(iters, sink); break;
    case MOE_PEAK_BF16: mfma_bf16_probe<<<grid, block, 0, stream>>>(iters, sink); break;
    default: return MOE_PEAK_EINVAL;
  }
  return hipGetLastError() == hipSuccess ? MOE_PEAK_OK : MOE_PEAK_EHIP;
}

moe_peak_status moe_peak_stream_read(const void* buf, size_t bytes, int32_t nontemporal, int32_t workgroups,
                                     uint32_t* sink, hipStream_t stream) {
  if (!buf || !sink || workgroups <= 0 || bytes % 16 || ((uintptr_t)buf % 16)) return MOE_PEAK_EINVAL;
  const uint64_t pieces = bytes / 16;
  const dim3 grid((unsigned)workgroups), block(256);
  if (nontemporal)
    stream_read_probe<1><<<grid, block, 0, stream>>>((const uint8_t*)buf, (uint32_t)pieces,
                                                     (uint32_t)(pieces >> 32), sink);
  else
    stream_read_probe<0><<<grid, block, 0, stream>>>((const uint8_t*)buf, (uint32_t)pieces,
                                                     (uint32_t)(pieces >> 32), sink);
  return hipGetLastError() == hipSuccess ? MOE_PEAK_OK : MOE_PEAK_EHIP;
}

}  // extern "C"
