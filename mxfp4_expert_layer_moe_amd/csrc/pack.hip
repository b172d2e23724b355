// Activation split: bf16 rows -> packed hi/lo FP6 E2M3 terms with E8M0 block scales.
//
// The gfx950 scaled matrix-core instruction takes its operands in FP8/FP6/FP4
// with one E8M0 scale per 32 values along K; it has no bf16 input.  A bf16
// activation row is therefore written as the sum of two MX terms: hi is the
// row's 32-blocks rounded to E2M3 under the OCP shared-exponent rule, lo the
// same encoding of what hi left over.  Both terms run at the FP4 x FP6 issue
// rate, so the expert GEMMs run two MFMAs per weight tile instead of one.
#include "moe_internal.h"

namespace moe {

// One thread per 32-value block.  Thread (row, b) reads 64 bytes of bf16,
// writes 24 B of hi codes, 24 B of lo codes and one scale byte for each term.
__global__ __launch_bounds__(256) void pack_act_kernel(int K, int rows, const uint16_t* __restrict__ a,
                                                       uint8_t* __restrict__ packed) {
  const int nblk = K / kBlock;
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long long)rows * nblk) return;
  const int row = (int)(gid / nblk);
  const int b = (int)(gid - (long long)row * nblk);

  const uint4* src = reinterpret_cast<const uint4*>(a + (size_t)row * K + (size_t)b * kBlock);
  float v[32];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint4 u = src[q];
    uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[q * 8 + 2 * i] = __uint_as_float(w4[i] << 16);
      v[q * 8 + 2 * i + 1] = __uint_as_float(w4[i] & 0xFFFF0000u);
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const uint32_t s_hi = e2m3_scale_byte(amax);
  const float inv_hi = e8m0_to_inv(s_hi), sc_hi = e8m0_to_float(s_hi);
  uint32_t hi[6] = {0, 0, 0, 0, 0, 0};
  float amax_r = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    float d;
    uint32_t c = e2m3_encode(v[i], inv_hi, sc_hi, &d);
    v[i] -= d;                                    // residual for the lo term
    amax_r = fmaxf(amax_r, fabsf(v[i]));
    const int bit = 6 * i, w = bit >> 5, sh = bit & 31;
    hi[w] |= c << sh;
    if (sh > 26) hi[w + 1] |= c >> (32 - sh);
  }
  const uint32_t s_lo = e2m3_scale_byte(amax_r);
  const float inv_lo = e8m0_to_inv(s_lo), sc_lo = e8m0_to_float(s_lo);
  uint32_t lo[6] = {0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    float d;
    uint32_t c = e2m3_encode(v[i], inv_lo, sc_lo, &d);
    const int bit = 6 * i, w = bit >> 5, sh = bit & 31;
    lo[w] |= c << sh;
    if (sh > 26) lo[w + 1] |= c >> (32 - sh);
  }
  uint8_t* dst = packed + (size_t)row * act_row_bytes(K);
  uint2* ph = reinterpret_cast<uint2*>(dst + (size_t)b * 24);
  uint2* pl = reinterpret_cast<uint2*>(dst + act_lo_codes_off(K) + (size_t)b * 24);
  ph[0] = make_uint2(hi[0], hi[1]); ph[1] = make_uint2(hi[2], hi[3]); ph[2] = make_uint2(hi[4], hi[5]);
  pl[0] = make_uint2(lo[0], lo[1]); pl[1] = make_uint2(lo[2], lo[3]); pl[2] = make_uint2(lo[4], lo[5]);
  const int ktp = act_ktp(K);
  dst[act_hi_scales_off(K) + (b & 1) * ktp + (b >> 1)] = (uint8_t)s_hi;
  dst[act_lo_scales_off(K) + (b & 1) * ktp + (b >> 1)] = (uint8_t)s_lo;
}

hipError_t launch_pack(int K, int rows, const uint16_t* a, uint8_t* packed, hipStream_t s) {
  const long long n = (long long)rows * (K / kBlock);
  if (n == 0) return hipSuccess;
  const int threads = 256;
  const long long blocks = (n + threads - 1) / threads;
  pack_act_kernel<<<dim3((unsigned)blocks), dim3(threads), 0, s>>>(K, rows, a, packed);
  return hipGetLastError();
}

}  // namespace moe
