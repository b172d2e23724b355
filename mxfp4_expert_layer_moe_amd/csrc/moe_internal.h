// Internal definitions shared by the library's kernels and its C ABI layer.
// gfx950 (CDNA4) only: wave64, scaled FP4/FP6 matrix-core instructions.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kBlock = 32;          // MX block: one E8M0 scale per 32 values along K
constexpr int kKTile = 64;          // K per scaled MFMA 32x32x64
constexpr int kMTile = 32;          // rows per MFMA tile
constexpr int kNTile = 32;          // output columns per MFMA tile
constexpr int kMaxExperts = 256;

// ---------------------------------------------------------------------------
// Packed activation rows ("split MX6"): hi and lo FP6 E2M3 terms per 32-block.
//   [hi codes K/32 x 24 B][lo codes K/32 x 24 B][hi scales 2 x KTp][lo scales 2 x KTp]
// ---------------------------------------------------------------------------
__host__ __device__ inline int act_ktiles(int K) { return K / kKTile; }
__host__ __device__ inline int act_ktp(int K) { return (act_ktiles(K) + 3) & ~3; }
__host__ __device__ inline size_t act_row_bytes(int K) {
  return (size_t)(K / kBlock) * 48 + 4 * (size_t)act_ktp(K);
}
__host__ __device__ inline size_t act_lo_codes_off(int K) { return (size_t)(K / kBlock) * 24; }
__host__ __device__ inline size_t act_hi_scales_off(int K) { return (size_t)(K / kBlock) * 48; }
__host__ __device__ inline size_t act_lo_scales_off(int K) {
  return (size_t)(K / kBlock) * 48 + 2 * (size_t)act_ktp(K);
}

// ---------------------------------------------------------------------------
// Prepacked weights: for each expert, for each output tile q of 32 rows, for
// each k-tile kt of 64: 64 lanes x 16 B of codes (lane l = row l%32 of the
// tile, K block l/32 of the k-tile).  Scales: for each (q, group of 4 k-tiles)
// 64 lanes x 4 B, byte j = scale of k-tile 4g+j for that lane.
// Gate/up tiles interleave: q = 2j is gate rows 32j.., q = 2j+1 is up rows I+32j..
// ---------------------------------------------------------------------------
__host__ __device__ inline int w_kgroups(int K) { return (K / kKTile + 3) / 4; }
__host__ __device__ inline size_t w_codes_per_expert(int N, int K) { return (size_t)N * K / 2; }
__host__ __device__ inline size_t w_scales_per_expert(int N, int K) {
  return (size_t)(N / kNTile) * w_kgroups(K) * 256;
}

// ---------------------------------------------------------------------------
// FP6 E2M3 encoding of v / 2^e (round to nearest even, saturate at 7.5).
// Returns the 6-bit code; *dec receives the decoded value times 2^e.
// ---------------------------------------------------------------------------
__device__ inline uint32_t e2m3_encode(float v, float inv_scale, float scale, float* dec) {
  float a = fabsf(v) * inv_scale;        // exact: inv_scale is a power of two
  float c;
  if (a < 2.0f) {
    c = __builtin_rintf(a * 8.0f);                    // codes 0..16 (16 == 2.0)
  } else if (a < 4.0f) {
    c = 16.0f + __builtin_rintf((a - 2.0f) * 4.0f);   // codes 16..24
  } else {
    c = 24.0f + __builtin_rintf((fminf(a, 7.5f) - 4.0f) * 2.0f);   // codes 24..31
  }
  uint32_t code = (uint32_t)c;
  float mag = code < 16 ? (float)code * 0.125f
                        : (code < 24 ? 2.0f + (float)(code - 16) * 0.25f : 4.0f + (float)(code - 24) * 0.5f);
  float val = mag * scale;
  bool neg = v < 0.0f;
  *dec = neg ? -val : val;
  return code | (neg && code ? 32u : 0u);
}

// Shared exponent of a block whose largest magnitude is amax: floor(log2 amax) - 2,
// returned as the E8M0 byte (clamped to [1, 254]); amax == 0 gives 127.
__device__ inline uint32_t e2m3_scale_byte(float amax) {
  if (!(amax > 0.0f)) return 127u;
  int e = (int)((__float_as_uint(amax) >> 23) & 0xFF) - 127 - 2;
  int b = e + 127;
  return (uint32_t)(b < 1 ? 1 : (b > 254 ? 254 : b));
}

__device__ inline float e8m0_to_float(uint32_t b) { return __uint_as_float(b << 23); }
__device__ inline float e8m0_to_inv(uint32_t b) { return __uint_as_float((254u - b) << 23); }

__device__ inline float bf16_round(float v) {
  uint32_t u = __float_as_uint(v);
  u = (u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u;
  return __uint_as_float(u);
}

__device__ inline float bf16_bits_to_float(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// ---------------------------------------------------------------------------
// Host-side launchers (one translation unit each); return the launch status.
// ---------------------------------------------------------------------------
hipError_t launch_route(int T, int D, int E, int k, const uint16_t* x, const float* wr, const float* br,
                        int32_t* idx, float* w, float* logits, hipStream_t s);
hipError_t launch_permute(int T, int E, int k, const int32_t* idx, int32_t* counts, int32_t* offsets,
                          int32_t* perm, int32_t* inv, hipStream_t s);
hipError_t launch_pack(int K, int rows, const uint16_t* a, uint8_t* packed, hipStream_t s);
hipError_t launch_gemm(int stage, int T, int D, int I, int E, int k, float limit, const uint8_t* a_packed,
                       const int32_t* perm, const int32_t* offsets, const uint8_t* codes,
                       const uint8_t* scales, const float* topk_w, void* out, hipStream_t s);
hipError_t launch_combine(int T, int D, int k, const float* y_perm, const int32_t* inv, void* y,
                          int y_bf16, hipStream_t s);

}  // namespace moe
