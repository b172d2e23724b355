// Grouped expert GEMM on MXFP4 weights with the gfx950 scaled matrix cores.
//
// Each expert is a SwiGLU feed-forward block: gate and up projections, then
// silu(gate) * up, then the down projection ("From GPT-2 to gpt-oss", section 3,
// Swish/SwiGLU, Fig. 6-7; Swish = x * sigmoid(x)).  gpt-oss clamps both
// pre-activations to +-swiglu_limit (= 7, model card raw config).  The expert
// weights are MXFP4: 4-bit E2M1 values with one 8-bit scale per 32 values
// ("gpt-oss architecture walk-through", section "Quantization").
//
// Matrix cores: V_MFMA_SCALE_F32_32X32X64_F8F6F4 with B = the FP4 weights
// (E8M0 block scales applied by the instruction) and A = one of the two FP6
// E2M3 terms of the activation (moe_pack_act / the gate-up epilogue), so each
// 32x32x64 weight tile costs two instructions, both at the FP4 issue rate.
// Operand layout (gfx950): lane l holds row l%32 and the 32 contiguous K values
// of block l/32; the scale of that (row, block) comes from the lane's scale
// dword, byte `opsel`.  Result: lane l, register r holds row 8(r/4)+4(l/32)+r%4,
// column l%32.
//
// The activation-quantized variant (AF = kActFp4) takes A as MXFP4 (one FP4 x FP4 instruction per
// weight tile, 48-byte chunks per k-tile) and quantizes h to MXFP4 in the gate/up epilogue.
//
// Work decomposition: grid.y walks the row tiles of every expert (the row-tile
// table written by the permutation; empty slots exit), and
// grid.x walks output units: a gate/up pair of 32-column tiles (stage 0) or
// one 32-column tile (stage 1), one unit per wavefront.  Weights stream from
// HBM once per (row tile, unit); a wavefront issues the loads of four k-tiles
// before their eight matrix instructions.
#include "mfma_ops.h"

namespace moe {

struct GemmArgs {
  int T, k, E, K, KT, KG, units, out_K;
  int out_assign;                                       // down: rows to their assignment index
  int dense_rows;                                       // down: packed h row e*T + t (dense decode path)
  int h_bf16;                                           // gate/up: h as bf16 rows instead of packed
  float limit;
  const uint8_t* a_packed;
  const int32_t* tiles;
  const uint8_t* codes;
  const uint8_t* scales;
  const float* topk_w;
  void* out;
  size_t codes_per_expert, scales_per_expert;
};

// LDS for staged activation rows: 8 rows of K = 2880 fit whole, and with the row ids the workgroup
// takes 40960 bytes, so four workgroups share a compute unit's 160 KB
constexpr int kAStageBytes = 40 * 1024 - 32;

__device__ inline v8i a_operand_lds(const uint8_t* p) {      // 24 bytes, 8-byte aligned
  const uint2* q = reinterpret_cast<const uint2*>(p);
  const uint2 a = q[0], b = q[1], c = q[2];
  v8i v = {(int)a.x, (int)a.y, (int)b.x, (int)b.y, (int)c.x, (int)c.y, 0, 0};
  return v;
}

// Staged rows in LDS: the packed row's chunks for k-tiles [c0, c0 + KC), row stride KC * 112 + 8
// bytes.  The 8-byte pad keeps the rows of one read on different banks (KC * 112 alone is a
// multiple of the 128-byte bank cycle for every even KC).
__host__ __device__ inline int stage_stride(int KC, int chunk = kActChunk) { return KC * chunk + 8; }

// KTC: the number of 64-wide k-tiles when known at compile time (K = 2880 gives 45), else 0.
// With KTC the whole K range is staged at once and the k-loop is fully unrolled, so the
// weight ring is never drained at a loop back-edge.
// ABUF: 2 reads the next k-tile's activations from LDS while the current one computes (costs
// registers), 1 reads them at the start of each k-tile.  SB: with KTC, a scheduling barrier
// after every SB k-tiles pins the refill loads in place.
// NB: 32-column weight tiles per wavefront (gate/up: the gate and up tiles of one SwiGLU pair).
template <int STAGE, int P, int BM, int KTC, int ABUF, int SB = 1, int NB = (STAGE == 0 ? 2 : 1),
          int AF = kActSplit6>
__global__ __launch_bounds__(256) void expert_gemm_kernel(GemmArgs g) {
  constexpr int CH = AF == kActFp4 ? kAct4Chunk : kActChunk;     // packed bytes per row and k-tile
  static_assert(STAGE == 1 || NB == 2, "a gate/up wavefront holds one gate/up tile pair");
  static_assert(P % 4 == 0, "prefetch depth must cover whole scale groups");
  static_assert(BM <= kMTile && BM * CH * P <= kAStageBytes, "a chunk of P k-tiles must fit for BM rows");
  __shared__ __attribute__((aligned(16))) uint8_t sA[kAStageBytes];
  __shared__ int srow[BM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int u = blockIdx.x * 4 + wave;                  // output unit of this wavefront
  const bool active = u < g.units;                      // inactive waves still join the barriers
  const int32_t* tile = g.tiles + (size_t)blockIdx.y * kTileInts;
  const int4 hdr = *reinterpret_cast<const int4*>(tile);
  const int e = __builtin_amdgcn_readfirstlane(hdr.x);
  if (e < 0) return;                                    // empty slot (uniform per workgroup)
  const int p0 = __builtin_amdgcn_readfirstlane(hdr.y);
  const int nrows = __builtin_amdgcn_readfirstlane(hdr.z);

  const int i = lane & 31;
  const int half = lane >> 5;
  const bool valid = i < nrows;
  // activation row of each tile row: gate/up the token's x row; down the grouped row of h, or on the
  // dense decode path (whose gate/up wrote h for every expert and token) row e*T + t
  if (tid < nrows)
    srow[tid] = STAGE == 0 ? tile[4 + tid] / g.k : (g.dense_rows ? e * g.T + tile[4 + tid] / g.k : p0 + tid);
  // down: each row's gate weight topk_w[perm[p]], fetched now so it is there for the epilogue
  float wl = 0.0f;
  int al = 0;
  if (STAGE == 1 && valid) {
    al = tile[4 + i];
    wl = g.topk_w[al];
  }

  // K chunk staged at once: everything if it fits, else a multiple of the prefetch depth
  int KC = KTC > 0 ? KTC : g.KT;
  if (KTC == 0 && nrows * stage_stride(KC, CH) > kAStageBytes) KC = ((kAStageBytes / nrows - 8) / CH) / P * P;
  const int rs = stage_stride(KC, CH);
  const size_t arb = act_row_bytes_af(AF, g.K);

  // this expert's weights as buffer resources; tile q starts at q*KT k-tiles (codes) / q*KG groups (scales)
  const __amdgpu_buffer_rsrc_t rsB = buffer_rsrc(g.codes + (size_t)e * g.codes_per_expert,
                                                 (uint32_t)g.codes_per_expert);
  const __amdgpu_buffer_rsrc_t rsS = buffer_rsrc(g.scales + (size_t)e * g.scales_per_expert,
                                                 (uint32_t)g.scales_per_expert);
  const int voffB = lane * 16, voffS = lane * 4;
  int sbase[NB], ssbase[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int q = NB * u + nb;
    sbase[nb] = q * g.KT * 1024;
    ssbase[nb] = q * g.KG * 256;
  }
  auto load_b = [&](const int nb, const int kt) {
    return __builtin_amdgcn_raw_buffer_load_b128(rsB, voffB, sbase[nb] + kt * 1024, kLoadStream);
  };
  auto load_s = [&](const int nb, const int grp) {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rsS, voffS, ssbase[nb] + grp * 256, kLoadStream);
  };

  // weight ring: slot j holds k-tile kt with kt % P == j; scale slot s holds group (kt / 4) with (kt/4) % (P/4) == s
  v4i bq[P][NB];
  uint32_t sbq[P / 4][NB];
  // With K known at compile time all of K is staged at once.  The staging loads (16-byte pieces,
  // up to kPieces per thread) are issued before the weight ring, so waiting for them does not
  // wait for the weights (loads complete in issue order).
  constexpr int kPieces = KTC > 0 ? (BM * KTC * (CH / 16) + 255) / 256 : 1;
  uint4 stg[kPieces];
  if constexpr (KTC > 0) {
    __syncthreads();                                    // srow visible
    const int n16 = KTC * (CH / 16);
#pragma unroll
    for (int q = 0; q < kPieces; ++q) {
      const int w = tid + 256 * q;
      if (w < nrows * n16) {
        const int r = w / n16, o = w - r * n16;
        stg[q] = *reinterpret_cast<const uint4*>(g.a_packed + (size_t)srow[r] * arb + (size_t)o * 16);
      }
    }
  }
  if (active) {
#pragma unroll
    for (int j = 0; j < P; ++j)
      if (j < g.KT) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) bq[j][nb] = load_b(nb, j);
      }
#pragma unroll
    for (int s = 0; s < P / 4; ++s)
      if (s < g.KG) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) sbq[s][nb] = load_s(nb, s);
      }
  }
  if constexpr (KTC > 0) {
    const int n16 = KTC * (CH / 16);
#pragma unroll
    for (int q = 0; q < kPieces; ++q) {
      const int w = tid + 256 * q;
      if (w < nrows * n16) {
        const int r = w / n16, o = w - r * n16;
        uint2* dst = reinterpret_cast<uint2*>(sA + r * rs + o * 16);     // rows are 8-byte aligned
        dst[0] = make_uint2(stg[q].x, stg[q].y);
        dst[1] = make_uint2(stg[q].z, stg[q].w);
      }
    }
  }

  v16f acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = v16f{};

  for (int c0 = 0; c0 < g.KT; c0 += KC) {
    const int kcn = min(KC, g.KT - c0);
    if constexpr (KTC == 0) {
      __syncthreads();                                  // previous chunk consumed; srow visible
      // stage rows [0, nrows) x k-tiles [c0, c0 + kcn): contiguous chunks, 8-byte words
      const int n8 = kcn * (CH / 8);
      for (int w = tid; w < nrows * n8; w += 256) {
        const int r = w / n8, o = w - r * n8;
        const uint8_t* src = g.a_packed + (size_t)srow[r] * arb + (size_t)c0 * CH + (size_t)o * 8;
        *reinterpret_cast<uint2*>(sA + r * rs + o * 8) = *reinterpret_cast<const uint2*>(src);
      }
    }
    __syncthreads();
    if (active) {
      const uint8_t* arow = sA + min(i, BM - 1) * rs;       // lanes past BM rows are masked below
      const int kend = c0 + kcn;
      // A operands of k-tile kt from LDS; rows past nrows read stale bytes and are masked to zero
      auto lds_a = [&](const int kt, v8i& hi, v8i& lo, uint32_t& sh, uint32_t& sl) {
        const uint8_t* chunk = arow + (kt - c0) * CH;
        if constexpr (AF == kActFp4) {
          // the lane's block: 16 bytes of E2M1 codes and its scale byte (lo is unused)
          const uint2* q = reinterpret_cast<const uint2*>(chunk + half * 16);
          const uint2 a = q[0], b = q[1];
          hi = v8i{(int)a.x, (int)a.y, (int)b.x, (int)b.y, 0, 0, 0, 0};
          lo = hi;
          sh = chunk[32 + half];
          sl = sh;
        } else {
          hi = a_operand_lds(chunk + half * 24);
          lo = a_operand_lds(chunk + 48 + half * 24);
          sh = chunk[96 + half];
          sl = chunk[98 + half];
        }
        const v8i z = {0, 0, 0, 0, 0, 0, 0, 0};
        hi = valid ? hi : z;
        lo = valid ? lo : z;
        sh = valid ? sh : 127u;
        sl = valid ? sl : 127u;
      };
      // one k-tile (slot j = kt % P): A from LDS, two MFMAs per weight tile, then refill slot j
      // with k-tile kt + P (address clamped to the last k-tile so there is no branch; a clamped
      // reload hits the cache).  The scheduling barrier keeps every refill where it is written,
      // so each wavefront keeps P k-tiles of weights in flight.
      v8i ah[ABUF], al[ABUF];
      uint32_t sh[ABUF], sl[ABUF];
      if constexpr (ABUF == 2) lds_a(c0, ah[0], al[0], sh[0], sl[0]);
      auto step = [&](const int j, const int kt) {
        const int cur = ABUF == 2 ? (j & 1) : 0;
        if constexpr (ABUF == 2)
          lds_a(min(kt + 1, kend - 1), ah[cur ^ 1], al[cur ^ 1], sh[cur ^ 1], sl[cur ^ 1]);
        else
          lds_a(kt, ah[0], al[0], sh[0], sl[0]);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const v8i bv = b_operand(bq[j][nb]);
          if constexpr (AF == kActFp4) {
            acc[nb] = mma4_sel(j & 3, ah[cur], bv, acc[nb], sh[cur], sbq[j >> 2][nb]);
          } else {
            acc[nb] = mma_sel(j & 3, ah[cur], bv, acc[nb], sh[cur], sbq[j >> 2][nb]);
            acc[nb] = mma_sel(j & 3, al[cur], bv, acc[nb], sl[cur], sbq[j >> 2][nb]);
          }
        }
        // the refill runs past the staged chunk into the next one (chunks start at multiples of
        // P, so slot j of the next chunk is k-tile kt + P); only the end of K clamps it
        const int kn = min(kt + P, g.KT - 1);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) bq[j][nb] = load_b(nb, kn);
        if ((j & 3) == 3) {
          const int grp = min((kt + P - 3) / 4, (g.KT - 1) / 4);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) sbq[j >> 2][nb] = load_s(nb, grp);
        }
        if constexpr (KTC > 0 && SB > 0) {
          if (kt % SB == SB - 1) __builtin_amdgcn_sched_barrier(0);
        }
      };
      if constexpr (KTC > 0) {
#pragma unroll
        for (int kt = 0; kt < KTC; ++kt) step(kt % P, kt);    // single chunk: c0 == 0, kcn == KTC
      } else {
        int kb = c0;
        for (; kb + P <= kend; kb += P) {
#pragma unroll
          for (int j = 0; j < P; ++j) step(j, kb + j);
        }
#pragma unroll
        for (int j = 0; j < P; ++j)
          if (kb + j < kend) step(j, kb + j);              // tail of the chunk (uniform)
      }
    }
  }
  if constexpr (STAGE == 0) {
    // SwiGLU epilogue: h = bf16(silu(clamp(g)) * clamp(u)), then a transpose through LDS (the
    // staged rows are free once every wavefront is past its k-loop) so that lane m holds the 32
    // values of row m's block and splits them into hi/lo FP6 with the packed conversions.
    __syncthreads();
    if (!active) return;
    constexpr int kEpStride = 36;                        // floats per row: 8 rows on 8 bank groups
    static_assert(4 * BM * kEpStride * 4 <= kAStageBytes, "transpose fits the staging buffer");
    float* ep = reinterpret_cast<float*>(sA) + wave * BM * kEpStride;
    const int I = g.out_K;
    const size_t orb = act_row_bytes_af(AF, I);
    uint8_t* out = reinterpret_cast<uint8_t*>(g.out);
    const int c = lane & 31;
    // register r holds rows 8(r/4) + 4(l/32) + r%4; tiles of BM rows only fill r < BM/2
#pragma unroll
    for (int r = 0; r < BM / 2; ++r) {
      const int m = 8 * (r >> 2) + 4 * half + (r & 3);
      ep[m * kEpStride + c] = swiglu_bf16(acc[0][r], acc[1][r], g.limit);
    }
    __builtin_amdgcn_wave_barrier();
    if (lane < BM && lane < nrows) {
      float v[32];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float4 f = *reinterpret_cast<const float4*>(ep + lane * kEpStride + 4 * q);
        v[4 * q] = f.x; v[4 * q + 1] = f.y; v[4 * q + 2] = f.z; v[4 * q + 3] = f.w;
      }
      if constexpr (AF == kActFp4) store_fp4_block(out + (size_t)(p0 + lane) * orb, u, quant_fp4x32(v));
      else if (g.h_bf16) store_bf16_block(reinterpret_cast<uint16_t*>(g.out) + (size_t)(p0 + lane) * I, u, v);
      else store_fp6_block(out + (size_t)(p0 + lane) * orb, u, split_fp6x32(v));
    }
  } else {
    // down epilogue: scale row p by its gate weight topk_w[perm[p]], store fp16
    if (!active) return;
    const int D = g.out_K;
    _Float16* out = reinterpret_cast<_Float16*>(g.out);
#pragma unroll
    for (int r = 0; r < BM / 2; ++r) {
      if (8 * (r >> 2) >= nrows) break;
      const int m = 8 * (r >> 2) + 4 * half + (r & 3);
      const float wm = __shfl(wl, m);
      const int orow = g.out_assign ? __shfl(al, m) : p0 + m;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        if (m < nrows) out[(size_t)orow * D + (size_t)(NB * u + nb) * kNTile + (lane & 31)] = (_Float16)(acc[nb][r] * wm);
    }
  }
}

constexpr int kGateUpP = 8;     // gate/up weight k-tiles in flight per wavefront
constexpr int kDownNB = 1;      // down-projection weight tiles per wavefront
constexpr int kDownP = 8;       // and k-tiles in flight

hipError_t launch_gemm(int stage, int T, int D, int I, int E, int k, float limit, const uint8_t* a_packed,
                       const int32_t* tiles, const uint8_t* codes, const uint8_t* scales, const float* topk_w,
                       void* out, hipStream_t s, int af, int out_assign, int dense_rows, int h_bf16) {
  if (T == 0) return hipSuccess;
  if (h_bf16 && (stage != 0 || af != kActSplit6)) return hipErrorInvalidValue;
  GemmArgs g;
  g.T = T; g.k = k; g.E = E; g.limit = limit;
  g.out_assign = stage == 1 && out_assign;
  g.dense_rows = stage == 1 && dense_rows;
  g.h_bf16 = h_bf16;
  g.a_packed = a_packed; g.tiles = tiles; g.codes = codes; g.scales = scales;
  g.topk_w = topk_w; g.out = out;
  const int N = stage == 0 ? 2 * I : D;
  g.K = stage == 0 ? D : I;
  g.KT = g.K / kKTile;
  g.KG = w_kgroups(g.K);
  g.units = stage == 0 ? I / kNTile : D / (kNTile * kDownNB);
  g.out_K = stage == 0 ? I : D;
  g.codes_per_expert = w_codes_per_expert(N, g.K);
  g.scales_per_expert = w_scales_per_expert(N, g.K);
  const long long n_assign = (long long)T * k;
  // batches with many rows per expert (128-row tiles) go to the prefill kernel
  if (tile_rows(n_assign, E) != 8) {
    if (g.dense_rows) return hipErrorInvalidValue;     // the dense decode path uses 8-row tiles only
    return launch_gemm_prefill(stage, T, D, I, E, k, limit, a_packed, tiles, codes, scales, topk_w, out, s, af,
                               out_assign, h_bf16);
  }
  // decode-sized batches (8-row tiles whose activations fit LDS whole)
  const dim3 grid((g.units + 3) / 4, (unsigned)tile_slots(n_assign, E));
  // the model's K = 2880 (45 k-tiles): fully unrolled k-loop
  const bool k45 = g.KT == 45 && 8 * stage_stride(45) <= kAStageBytes;   // 40384 <= 40928
  if (af == kActFp4) {
    if (stage == 0) {
      if (k45) expert_gemm_kernel<0, kGateUpP, 8, 45, 1, 1, 2, kActFp4><<<grid, dim3(256), 0, s>>>(g);
      else expert_gemm_kernel<0, 8, 8, 0, 1, 1, 2, kActFp4><<<grid, dim3(256), 0, s>>>(g);
    } else {
      if (k45) expert_gemm_kernel<1, kDownP, 8, 45, 2, 1, kDownNB, kActFp4><<<grid, dim3(256), 0, s>>>(g);
      else expert_gemm_kernel<1, kDownP, 8, 0, 1, 1, kDownNB, kActFp4><<<grid, dim3(256), 0, s>>>(g);
    }
    return hipGetLastError();
  }
  if (stage == 0) {
    if (k45) expert_gemm_kernel<0, kGateUpP, 8, 45, 1><<<grid, dim3(256), 0, s>>>(g);
    else expert_gemm_kernel<0, 8, 8, 0, 1><<<grid, dim3(256), 0, s>>>(g);
  } else {
    if (k45) expert_gemm_kernel<1, kDownP, 8, 45, 2, 1, kDownNB><<<grid, dim3(256), 0, s>>>(g);
    else expert_gemm_kernel<1, kDownP, 8, 0, 1, 1, kDownNB><<<grid, dim3(256), 0, s>>>(g);
  }
  return hipGetLastError();
}

}  // namespace moe
