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
// scratch of the entry point that allocates nothing (moe_forward_noalloc), per GPU
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;

// ---------------------------------------------------------------------------
// Packed activation rows ("split MX6"): hi and lo FP6 E2M3 terms per 32-block.
// A row of K values is K/64 chunks of 112 bytes, one per 64-wide k-tile kt:
//   [0,24) hi codes of block 2kt   [24,48) hi codes of block 2kt+1
//   [48,72) lo codes of block 2kt  [72,96) lo codes of block 2kt+1
//   [96] [97] hi scales of blocks 2kt, 2kt+1   [98] [99] lo scales   [100,112) unused
// so one 16-byte-aligned chunk holds everything a k-tile of the GEMM reads.
// ---------------------------------------------------------------------------
constexpr int kActChunk = 112;
__host__ __device__ inline int act_ktiles(int K) { return K / kKTile; }
__host__ __device__ inline size_t act_row_bytes(int K) { return (size_t)act_ktiles(K) * kActChunk; }

// ---------------------------------------------------------------------------
// Packed MXFP4 activation rows (the activation-quantized variant): per 64-wide
// k-tile kt a 48-byte chunk:
//   [0,16) E2M1 codes of block 2kt (element i in nibble i, low nibble first)
//   [16,32) codes of block 2kt+1   [32] [33] E8M0 scales of the two blocks   [34,48) unused
// ---------------------------------------------------------------------------
constexpr int kAct4Chunk = 48;
__host__ __device__ inline size_t act4_row_bytes(int K) { return (size_t)act_ktiles(K) * kAct4Chunk; }
// activation formats of the expert GEMMs
constexpr int kActSplit6 = 0;      // bf16 as hi + lo FP6 terms (the default)
constexpr int kActFp4 = 1;         // MXFP4 activations
__host__ __device__ inline int act_chunk(int af) { return af == kActFp4 ? kAct4Chunk : kActChunk; }
__host__ __device__ inline size_t act_row_bytes_af(int af, int K) {
  return af == kActFp4 ? act4_row_bytes(K) : act_row_bytes(K);
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
// Row-tile table (written by the permutation, read by the expert GEMMs): the
// grouped rows of every expert are cut into tiles of tile_rows() rows; slot s
// (tile_ints() int32 each) holds {expert (-1 = empty slot), first grouped
// position p0, rows, tiles in use} and then the assignment id perm[p0 + i] of
// each row i < rows.  Batches of at most 6 assignments per expert on average use
// 8-row tiles (the small-batch GEMM streams every weight tile once per 8 rows of
// an expert), larger ones 128-row tiles.  Measured at the 2880 shape: at 5 per
// expert the 8-row path is 5-17% faster, at 6 within 3% either way, at 7-8 the
// 128-row path is 3-17% faster (32 and 128 experts).
// ---------------------------------------------------------------------------
constexpr int kTileInts = 48;      // slot of an 8-row tile: 4 header ints + ids, padded to 192 bytes
constexpr int kPrefillRows = 128;  // rows per tile of large batches
constexpr int kSmallTileLimit = 6;  // average assignments per expert served by 8-row tiles
__host__ __device__ inline int tile_rows(long long n_assign, int E) {
  return n_assign <= (long long)kSmallTileLimit * E ? 8 : kPrefillRows;
}
__host__ __device__ inline int tile_ints(int bm) { return 4 + bm > kTileInts ? 4 + bm : kTileInts; }
__host__ __device__ inline long long tile_slots(long long n_assign, int E) {
  const int bm = tile_rows(n_assign, E);
  return (n_assign + bm - 1) / bm + (E < n_assign ? E : n_assign);
}
// The table buffer continues with the grouping's scratch: per-workgroup expert counts [G][E]
// (G = workgroups of 1024 assignments) and the first tile slot of every expert [E + 1].
constexpr int kPermChunk = 1024;   // assignments per grouping workgroup (one per thread)
__host__ __device__ inline long long perm_groups(long long n_assign) { return (n_assign + kPermChunk - 1) / kPermChunk; }
__host__ __device__ inline long long tile_table_ints(long long n_assign, int E) {
  return tile_slots(n_assign, E) * tile_ints(tile_rows(n_assign, E));
}
__host__ __device__ inline long long tile_buffer_ints(long long n_assign, int E) {
  return tile_table_ints(n_assign, E) + perm_groups(n_assign) * E + E + 1;
}

// Shared exponent of a block whose largest magnitude is amax: floor(log2 amax) - 2,
// returned as the E8M0 byte, clamped to [1, 253] so that both the scale and its
// inverse are normal fp32 numbers; amax == 0 gives 127.
__device__ inline uint32_t e2m3_scale_byte(float amax) {
  if (!(amax > 0.0f)) return 127u;
  int e = (int)((__float_as_uint(amax) >> 23) & 0xFF) - 127 - 2;
  int b = e + 127;
  return (uint32_t)(b < 1 ? 1 : (b > 253 ? 253 : b));
}

__device__ inline float e8m0_to_float(uint32_t b) { return __uint_as_float(b << 23); }

// fp32 -> bf16 -> fp32, round to nearest even: the hardware conversion (v_cvt_pk_bf16_f32), which
// gives the same bits as integer round-to-nearest-even for every non-NaN fp32 value (all 2^32
// patterns checked on the MI355X)
__device__ inline float bf16_round(float v) { return (float)(__bf16)v; }

// SwiGLU of one (gate, up) pair: h = bf16(silu(clamp(g)) * clamp(u)), both pre-activations
// clamped to [-limit, limit].  silu(g) = g / (1 + e^-g) uses the hardware exp2 and reciprocal
// (about 1 ulp each in fp32), far inside the bf16 rounding of h.
__device__ inline float swiglu_bf16(float g, float u, float limit) {
  const float gv = __builtin_amdgcn_fmed3f(g, -limit, limit);   // clamp to [-limit, limit]
  const float uv = __builtin_amdgcn_fmed3f(u, -limit, limit);
  const float e = __builtin_amdgcn_exp2f(gv * -1.4426950408889634f);
  return bf16_round(gv * __builtin_amdgcn_rcpf(1.0f + e) * uv);
}




// ---------------------------------------------------------------------------
// Host-side launchers (one translation unit each); return the launch status.
// ---------------------------------------------------------------------------
hipError_t launch_route(int T, int D, int E, int k, const uint16_t* x, const float* wr, const float* br,
                        int32_t* idx, float* w, float* logits, void* ws, hipStream_t s);
// The whole routing front end of a forward pass: logits (with the activation split of x
// into xpack done by extra workgroups), selection and grouping; small batches fuse the
// selection and the grouping into one workgroup.
// The RMSNorm in front of the layer, folded into the first launch of the dense decode path: the
// launch reads the raw rows, normalises them with the standalone RMSNorm's arithmetic and writes
// the normalised rows to its x argument.
struct FrontNorm {
  const uint16_t* raw;
  const float* gamma;
  double eps;
};

hipError_t launch_route_front(int T, int D, int E, int k, const uint16_t* x, const float* wr, const float* br,
                              int32_t* idx, float* w, void* ws, uint8_t* xpack, int32_t* counts,
                              int32_t* offsets, int32_t* perm, int32_t* inv, int32_t* tiles, hipStream_t s,
                              int af = kActSplit6, const FrontNorm* fn = nullptr);
size_t route_workspace_bytes(int T, int D, int E);
hipError_t launch_permute(int T, int E, int k, const int32_t* idx, int32_t* counts, int32_t* offsets,
                          int32_t* perm, int32_t* inv, int32_t* tiles, hipStream_t s);
// The row-tile table of a grouping given as offsets [E + 1] and perm (the grouped assignment ids),
// the same table launch_permute writes (without the grouping's scratch after it).
hipError_t launch_tiles_from_groups(int T, int E, int k, const int32_t* offsets, const int32_t* perm,
                                    int32_t* tiles, hipStream_t s);
hipError_t launch_pack(int K, int rows, const uint16_t* a, uint8_t* packed, hipStream_t s, int af = kActSplit6);
// out_assign (down stage only): row p of the output goes to the row of its assignment perm[p];
// h_bf16 (gate/up stage, split activations only): h written as bf16 rows of d_ff, not packed
// = t*k + j instead of row p, so the combine reads a token's rows without the inverse permutation.
// dense_rows (down stage only, 8-row tiles): the activation of tile row p is packed h row e*T + t
// (the dense decode path's gate/up output) instead of row p.
hipError_t launch_gemm(int stage, int T, int D, int I, int E, int k, float limit, const uint8_t* a_packed,
                       const int32_t* tiles, const uint8_t* codes, const uint8_t* scales, const float* topk_w,
                       void* out, hipStream_t s, int af = kActSplit6, int out_assign = 0, int dense_rows = 0,
                       int h_bf16 = 0);
hipError_t launch_gemm_prefill(int stage, int T, int D, int I, int E, int k, float limit,
                               const uint8_t* a_packed, const int32_t* tiles, const uint8_t* codes,
                               const uint8_t* scales, const float* topk_w, void* out, hipStream_t s,
                               int af = kActSplit6, int out_assign = 0, int h_bf16 = 0);
// inv null: the rows are in assignment order (row t*k + j), as the down stage writes with out_assign
hipError_t launch_combine(int T, int D, int k, const _Float16* y_perm, const int32_t* inv, const uint16_t* residual,
                          void* y, int y_bf16, hipStream_t s);

// ---------------------------------------------------------------------------
// The dense decode path of the whole-layer entry points (gemm_dense.hip): at most 32 tokens and
// 32 experts, d_model up to 2880, and so many assignments that an expert goes untouched with
// probability (1 - k/E)^T <= 0.15.  The gate/up projection then runs over every (expert, token) pair with the
// selection and grouping in the same launch; the down projection is the routed one.
// ---------------------------------------------------------------------------
constexpr int kDenseMaxKT = 45;              // the dense gate/up stages all of K in LDS: up to 2880
__host__ inline bool dense_decode(int T, int E, int k, int D) {
  if (T < 1 || T > 32 || E > 32 || (long long)T * k > (long long)kSmallTileLimit * E) return false;
  if (D / kKTile > kDenseMaxKT) return false;
  double untouched = 1.0;
  for (int t = 0; t < T; ++t) untouched *= 1.0 - (double)k / E;
  return untouched <= 0.15;
}
// the router inputs of a forward pass, which the dense launch scores and selects from, and where
// the selection and the grouping go
struct DenseSelection {
  const uint16_t* x;
  const float* wr;
  const float* br;
  int32_t* idx;
  float* w;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm;
  int32_t* inv;
  int32_t* tiles;
};
// The first launch of the dense decode path: x split into xpack, one workgroup per row; with fn,
// the normalised rows written to x and packed instead.
hipError_t launch_front_pack(int T, int D, const uint16_t* x, uint8_t* xpack, int af, hipStream_t s,
                             const FrontNorm* fn = nullptr);
// the dense gate/up projection: packed x (T rows) -> packed h rows e*T + t for every expert e,
// with the scores, the selection and the grouping of every token (sel) in the same launch
hipError_t launch_gemm_dense_gate_up(int T, int D, int I, int E, int k, float limit, const uint8_t* xpack,
                                     const uint8_t* codes, const uint8_t* scales, void* hpack,
                                     const DenseSelection* sel, hipStream_t s);
hipError_t launch_rmsnorm(int T, int D, const uint16_t* x, const float* gamma, float eps, uint16_t* xn,
                          hipStream_t s);

}  // namespace moe
