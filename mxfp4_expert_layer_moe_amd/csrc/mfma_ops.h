// gfx950 operand helpers shared by the expert GEMM kernels.
//
// V_MFMA_SCALE_F32_32X32X64_F8F6F4 computes a 32x32 fp32 tile from a 32x64
// A block and a 64x32 B block, each in an FP8/FP6/FP4 format with one E8M0
// scale per 32 K values.  Here B is always the MXFP4 weight (E2M1 codes and
// E8M0 scales as stored, "gpt-oss architecture walk-through", section
// "Quantization") and A one FP6 E2M3 term of the activation.
// Lane l holds row l%32 (A) / column l%32 (B) and the 32 K values of block
// l/32; its scale is byte `opsel` of the lane's scale dword.  Result: lane l,
// register r holds row 8(r/4) + 4(l/32) + r%4, column l%32.
#pragma once
#include "moe_internal.h"

namespace moe {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v6i __attribute__((ext_vector_type(6)));
typedef float v32f __attribute__((ext_vector_type(32)));

// FP4 operand: 16 bytes per lane (32 E2M1 codes) in the low four dwords
__device__ inline v8i b_operand(const v4i b) {
  v8i v = {b.x, b.y, b.z, b.w, 0, 0, 0, 0};
  return v;
}

// Raw buffer resource over [base, base + bytes): loads take a 32-bit lane offset in a vector
// register and a scalar offset, and any read past `bytes` returns zero.
__device__ inline __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// Cache-policy field of a buffer load: bit 1 is the non-temporal (streaming) hint.  Weights that a
// launch reads once go through it: a plain 265 MB streaming read takes about 44 us with the hint
// against 48 us without it on the MI355X.
constexpr int kLoadStream = 2;

// scaled MFMA, A = FP6 E2M3 (scale byte 0 of sa), B = FP4 E2M1 (scale byte OB of sb)
template <int OB>
__device__ inline v16f mma_fp6_fp4(v8i a, v8i b, v16f c, uint32_t sa, uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 2, 4, 0, sa, OB, sb);
}

// scaled MFMA whose A scale is byte OA of sa (the per-lane scale register holds several bytes)
template <int OA, int OB>
__device__ inline v16f mma_fp6_fp4_sel(v8i a, v8i b, v16f c, uint32_t sa, uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 2, 4, OA, sa, OB, sb);
}

template <int OA>
__device__ inline v16f mma_sel_a(int ob, v8i a, v8i b, v16f c, uint32_t sa, uint32_t sb) {
  switch (ob) {
    case 0: return mma_fp6_fp4_sel<OA, 0>(a, b, c, sa, sb);
    case 1: return mma_fp6_fp4_sel<OA, 1>(a, b, c, sa, sb);
    case 2: return mma_fp6_fp4_sel<OA, 2>(a, b, c, sa, sb);
    default: return mma_fp6_fp4_sel<OA, 3>(a, b, c, sa, sb);
  }
}

// scaled MFMA with both operands FP4 E2M1 (A scale byte 0 of sa, B scale byte OB of sb)
template <int OB>
__device__ inline v16f mma_fp4_fp4(v8i a, v8i b, v16f c, uint32_t sa, uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, 0, sa, OB, sb);
}

__device__ inline v16f mma4_sel(int ob, v8i a, v8i b, v16f c, uint32_t sa, uint32_t sb) {
  switch (ob) {
    case 0: return mma_fp4_fp4<0>(a, b, c, sa, sb);
    case 1: return mma_fp4_fp4<1>(a, b, c, sa, sb);
    case 2: return mma_fp4_fp4<2>(a, b, c, sa, sb);
    default: return mma_fp4_fp4<3>(a, b, c, sa, sb);
  }
}

// ob is a compile-time constant after unrolling, so the switch folds away
__device__ inline v16f mma_sel(int ob, v8i a, v8i b, v16f c, uint32_t sa, uint32_t sb) {
  switch (ob) {
    case 0: return mma_fp6_fp4<0>(a, b, c, sa, sb);
    case 1: return mma_fp6_fp4<1>(a, b, c, sa, sb);
    case 2: return mma_fp6_fp4<2>(a, b, c, sa, sb);
    default: return mma_fp6_fp4<3>(a, b, c, sa, sb);
  }
}

// ---------------------------------------------------------------------------
// gfx950 packed FP6 conversions.  cvt_fp6x32: 32 fp32 values -> 32 E2M3 codes
// of v / 2^e (e = the exponent of `scale`), rounded to nearest even and
// saturated at 7.5; the two 16-value halves are interleaved, so passing the
// even and the odd elements puts element i at bits 6i.  dequant_fp6x32 is the
// inverse (code value times 2^e).  Written as inline asm with an early-clobber
// output: the 6- and 32-register results must not overlap the sources, which
// the instructions still read while writing.
// ---------------------------------------------------------------------------
__device__ inline v6i cvt_fp6x32(const v16f even, const v16f odd, float scale) {
  v6i c;
  asm("v_cvt_scalef32_2xpk16_fp6_f32 %0, %1, %2, %3" : "=&v"(c) : "v"(even), "v"(odd), "v"(scale));
  return c;
}

__device__ inline v32f dequant_fp6x32(const v6i c, float scale) {
  v32f d;
  asm("v_cvt_scalef32_pk32_f32_fp6 %0, %1, %2" : "=&v"(d) : "v"(c), "v"(scale));
  return d;
}

// hi/lo MX6 split of one 32-value block held by one lane: hi = E2M3(v) with the block scale
// 2^(floor(log2 amax) - 2), lo = the same of v - hi.  Codes element i at bits 6i.
struct Fp6Split {
  v6i hi, lo;
  uint32_t s_hi, s_lo;
};

__device__ __forceinline__ Fp6Split split_fp6x32(const float (&v)[32]) {
  Fp6Split r;
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  r.s_hi = e2m3_scale_byte(amax);
  const float sh = e8m0_to_float(r.s_hi);
  v16f ev, od;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    ev[j] = v[2 * j];
    od[j] = v[2 * j + 1];
  }
  r.hi = cvt_fp6x32(ev, od, sh);
  const v32f d = dequant_fp6x32(r.hi, sh);
  float amax2 = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    ev[j] = v[2 * j] - d[2 * j];
    od[j] = v[2 * j + 1] - d[2 * j + 1];
    amax2 = fmaxf(amax2, fmaxf(fabsf(ev[j]), fabsf(od[j])));
  }
  r.s_lo = e2m3_scale_byte(amax2);
  r.lo = cvt_fp6x32(ev, od, e8m0_to_float(r.s_lo));
  return r;
}

// Store the split block b of a packed activation row (format in moe_mxfp4.h): the chunk of k-tile
// b / 2 holds hi codes at 24 * (b % 2), lo codes at 48 + 24 * (b % 2), scale bytes at 96 + b % 2
// (hi) and 98 + b % 2 (lo).  Rows are 8-byte aligned, so the 24-byte code groups go out as
// three 8-byte stores.
__device__ __forceinline__ void store_fp6_block(uint8_t* row, int b, const Fp6Split& sp) {
  uint8_t* chunk = row + (size_t)(b >> 1) * kActChunk;
  const int half = b & 1;
  uint2* ph = reinterpret_cast<uint2*>(chunk + 24 * half);
  uint2* pl = reinterpret_cast<uint2*>(chunk + 48 + 24 * half);
  ph[0] = make_uint2(sp.hi[0], sp.hi[1]);
  ph[1] = make_uint2(sp.hi[2], sp.hi[3]);
  ph[2] = make_uint2(sp.hi[4], sp.hi[5]);
  pl[0] = make_uint2(sp.lo[0], sp.lo[1]);
  pl[1] = make_uint2(sp.lo[2], sp.lo[3]);
  pl[2] = make_uint2(sp.lo[4], sp.lo[5]);
  chunk[96 + half] = (uint8_t)sp.s_hi;
  chunk[98 + half] = (uint8_t)sp.s_lo;
}

// ---------------------------------------------------------------------------
// MXFP4 quantization of one 32-value block held by one lane (OCP MX v1.0 conversion): shared
// exponent E = floor(log2 amax) - 2 (the E2M1 emax), clamped to the E8M0 range, byte E + 127;
// each element v / 2^E rounded to the nearest E2M1 value (ties to the even code), magnitudes
// past 6 saturate; an all-zero block gets scale byte 0 and zero codes.  Codes: element i in
// nibble i of the 16 bytes (low nibble first), bit 3 the sign.
// ---------------------------------------------------------------------------
struct Fp4Block {
  uint4 codes;
  uint32_t scale;
};

__device__ __forceinline__ uint32_t e2m1_code(float v, float inv) {
  const float q = fabsf(v) * inv;
  float c;
  if (q < 2.0f) c = rintf(q * 2.0f);                         // 0, 0.5, ..., 2 -> codes 0..4
  else if (q < 4.0f) c = 4.0f + rintf(q - 2.0f);              // 2, 3, 4 -> codes 4..6
  else c = 6.0f + rintf(fminf(q, 6.0f) * 0.5f - 2.0f);         // 4, 6 -> codes 6, 7
  return (uint32_t)c | (v < 0.0f ? 8u : 0u);
}

__device__ __forceinline__ Fp4Block quant_fp4x32(const float (&v)[32]) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  Fp4Block r;
  if (amax == 0.0f) {
    r.codes = make_uint4(0, 0, 0, 0);
    r.scale = 0;
    return r;
  }
  int E = (int)((__float_as_uint(amax) >> 23) & 0xFFu) - 127 - 2;
  E = E < -127 ? -127 : (E > 127 ? 127 : E);
  r.scale = (uint32_t)(E + 127);
  uint32_t w[4];
  if (E > -126) {
    // the packed conversion divides by the scale and rounds exactly as above (checked against
    // e2m1_code over ties, saturation and signs at scales 2^-20 .. 2^10); two values per call
    const float sc = ldexpf(1.0f, E);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t x = 0;
      x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, v[8 * d + 0], v[8 * d + 1], sc, 0);
      x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, v[8 * d + 2], v[8 * d + 3], sc, 1);
      x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, v[8 * d + 4], v[8 * d + 5], sc, 2);
      x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, v[8 * d + 6], v[8 * d + 7], sc, 3);
      w[d] = x;
    }
  } else {
    // scales below the fp32 normal range: element by element
    const float inv = ldexpf(1.0f, -E);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t x = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) x |= e2m1_code(v[8 * d + j], inv) << (4 * j);
      w[d] = x;
    }
  }
  r.codes = make_uint4(w[0], w[1], w[2], w[3]);
  return r;
}

// Store quantized block b of an MXFP4-packed activation row (format in moe_internal.h).
__device__ __forceinline__ void store_fp4_block(uint8_t* row, int b, const Fp4Block& q) {
  uint8_t* chunk = row + (size_t)(b >> 1) * kAct4Chunk;
  *reinterpret_cast<uint4*>(chunk + 16 * (b & 1)) = q.codes;
  chunk[32 + (b & 1)] = (uint8_t)q.scale;
}

// Store block b (32 values, each already a bf16 value held in fp32) of a bf16 row: 64 bytes.
__device__ __forceinline__ void store_bf16_block(uint16_t* row, int b, const float (&v)[32]) {
  uint4* dst = reinterpret_cast<uint4*>(row + (size_t)b * kBlock);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = (__float_as_uint(v[8 * q + 2 * j]) >> 16) | (__float_as_uint(v[8 * q + 2 * j + 1]) & 0xFFFF0000u);
    dst[q] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Store the 32 values of block b of activation row `row` (bf16 values held in fp32) in the packed
// activation format: the hi/lo FP6 split (af = kActSplit6) or the MXFP4 quantization (af = kActFp4).
__device__ __forceinline__ void pack_block_values(const float (&v)[32], int K, long long row, int b,
                                                  uint8_t* __restrict__ packed, int af = kActSplit6) {
  if (af == kActFp4) store_fp4_block(packed + (size_t)row * act4_row_bytes(K), b, quant_fp4x32(v));
  else store_fp6_block(packed + (size_t)row * act_row_bytes(K), b, split_fp6x32(v));
}

// Pack block `blk` (= row * K/32 + b) of bf16 rows [rows][K] (16-byte aligned) in one lane:
// four 16-byte loads, then pack_block_values.  Lanes past the last block do nothing.
__device__ __forceinline__ void pack_block_lane(const uint16_t* __restrict__ a, int K, long long nblocks,
                                                long long blk, uint8_t* __restrict__ packed, int af = kActSplit6) {
  if (blk >= nblocks) return;
  const int nb = K / kBlock;
  const long long row = blk / nb;
  const int b = (int)(blk - row * nb);
  const uint4* src = reinterpret_cast<const uint4*>(a + (size_t)row * K + (size_t)b * kBlock);
  float v[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 u = src[i];
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[8 * i + 2 * k] = __uint_as_float(w[k] << 16);
      v[8 * i + 2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
    }
  }
  pack_block_values(v, K, row, b, packed, af);
}

}  // namespace moe
