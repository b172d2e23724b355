// Grouped expert GEMM for batches with many rows per expert (prefill).
//
// The same operation as the small-batch kernel in gemm.hip: the gate/up
// projection with the SwiGLU epilogue, or the down projection scaled by the
// gate ("From GPT-2 to gpt-oss", section 3, Swish/SwiGLU, with gpt-oss's clamp
// at swiglu_limit = 7 from the model card's raw config; MXFP4 weights as in the
// walk-through's "Quantization" section).  Here every expert has hundreds of
// rows, so the kernel is organised for the matrix cores, not for the weight
// stream:
//
//  - A workgroup computes a 128-row x 512-column output tile with 4
//    wavefronts. Each wavefront holds 4 row blocks x 4 column tiles of 32x32
//    fp32 accumulators (256 registers).
//  - Each 64-wide k-tile of the tile's 128 activation rows (hi/lo FP6 chunks)
//    is staged once in LDS and read by all four wavefronts. Each wavefront
//    streams its own four weight tiles through a 4-deep register ring.
//  - The LDS holds a ring of 4 staged k-tiles. k-tile kt+2 is written from
//    registers while kt is computed, and kt+4 is loading into registers.
//    There is one barrier per k-tile.
//  - Staged layout: the 128 rows' 112-byte chunks back to back.  The staging
//    loads give consecutive lanes consecutive 16-byte pieces of a row (each load
//    instruction reads about 9 whole gathered row chunks), and an operand read
//    by 8 consecutive rows hits 8 different 16-byte bank groups (7r mod 8).
//  - Work items (row tile, 512-column group) are dealt to the 8 XCDs in
//    contiguous blocks, so the workgroups sharing an expert's weights share
//    an L2.
//  - Gate/up epilogue: SwiGLU in registers, then a transpose of the h tile
//    through LDS. Each lane then holds one 32-value block of an h row and
//    splits it into hi/lo FP6 with the packed conversion instructions.
#include "mfma_ops.h"

namespace moe {

struct PrefillArgs {
  int k, KT, KG, nt, ngroups, out_K;
  float limit;
  const uint8_t* a_packed;
  uint32_t a_bytes, arb;
  const int32_t* tiles;
  const float* topk_w;
  const uint8_t* codes;
  const uint8_t* scales;
  void* out;
  size_t codes_per_expert, scales_per_expert;
};

constexpr int kPWaveTiles = 4;                         // 32-column weight tiles per wavefront
constexpr int kPGroupTiles = 4 * kPWaveTiles;          // per workgroup
constexpr int kPSlots = 4;                             // staged k-tiles in the LDS ring
constexpr int kPPieces = kActChunk / 16;               // 16-byte pieces per row chunk (7)
constexpr int kPBlockBytes = 32 * kActChunk;           // one 32-row block of a staged k-tile
constexpr int kPStagePieces = kPrefillRows * kPPieces; // 896 pieces per staged k-tile
constexpr int kPSlotBytes = 1024 * 16;                 // 896 pieces + 128 dummy (4 unconditional per thread)
constexpr int kPStageAhead = 2;                        // k-tile kt + 2 is written to LDS during k-tile kt
constexpr int kPEpiStride = 68;                        // floats per row of the transposed h block
static_assert(kPSlots * kPSlotBytes >= 4 * 32 * kPEpiStride * 4, "h transposition fits the ring");

// FP6 operand of one staged row chunk: lane half h takes bytes [base + 24h, base + 24h + 24)
// (base 0: hi term, 48: lo term), i.e. 16 bytes at base + 32h and 8 bytes at base + 16 + 8h.
__device__ __forceinline__ v8i staged_operand(const uint8_t* row, int h, int base) {
  const v4i q = *reinterpret_cast<const v4i*>(row + base + 32 * h);
  const uint2 t = *reinterpret_cast<const uint2*>(row + base + 16 + 8 * h);
  const bool up = h != 0;
  v8i v = {up ? (int)t.x : q.x, up ? (int)t.y : q.y, up ? q.x : q.z, up ? q.y : q.w,
           up ? q.z : (int)t.x, up ? q.w : (int)t.y, 0, 0};
  return v;
}

// NA: activation k-tiles in flight in registers (k-tile t is fetched NA k-tiles before it is
// written to LDS); P: weight k-tiles in flight per wavefront.  Both divide 8.
template <int STAGE, int KTC, int NA, int P>
__global__ __launch_bounds__(256) void expert_gemm_prefill_kernel(PrefillArgs g) {
  static_assert(8 % NA == 0 && 8 % P == 0 && P >= 4, "ring depths divide the 8-step unroll");
  __shared__ __attribute__((aligned(16))) uint8_t sA[kPSlots * kPSlotBytes];
  __shared__ int srow[kPrefillRows];
  __shared__ float sgate[kPrefillRows];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int KT = KTC > 0 ? KTC : g.KT;

  // ---- work item: XCD x (= blockIdx % 8) takes the x-th contiguous block of items -------------
  const int used = __builtin_amdgcn_readfirstlane(g.tiles[3]);
  const int total = used * g.ngroups;
  const int per = (total + 7) >> 3;
  const int local = blockIdx.x >> 3;
  const int item = (blockIdx.x & 7) * per + local;
  if (local >= per || item >= total) return;             // uniform per workgroup
  const int slot = item / g.ngroups;
  const int cgrp = item - slot * g.ngroups;
  const int32_t* tile = g.tiles + (size_t)slot * tile_ints(kPrefillRows);
  const int4 hdr = *reinterpret_cast<const int4*>(tile);
  const int e = __builtin_amdgcn_readfirstlane(hdr.x);
  const int p0 = __builtin_amdgcn_readfirstlane(hdr.y);
  const int nrows = __builtin_amdgcn_readfirstlane(hdr.z);

  if (tid < kPrefillRows) {
    const int r = min(tid, nrows - 1);                   // rows past the tile repeat its last row
    const int a = tile[4 + r];
    srow[tid] = STAGE == 0 ? a / g.k : p0 + r;
    if constexpr (STAGE == 1) sgate[tid] = g.topk_w[a];
  }
  __syncthreads();

  // ---- activation staging: thread tid moves pieces tid + 256 i (i < 4) of every k-tile ----------
  const __amdgpu_buffer_rsrc_t rsA = buffer_rsrc(g.a_packed, g.a_bytes);
  uint32_t aoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = min(tid + 256 * i, kPStagePieces - 1); // the dummy pieces re-read a real one
    const int row = q / kPPieces;
    aoff[i] = (uint32_t)srow[row] * g.arb + (uint32_t)(q - row * kPPieces) * 16u;
  }
  auto load_a = [&](const int kt, v4i (&buf)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) buf[i] = __builtin_amdgcn_raw_buffer_load_b128(rsA, aoff[i], kt * kActChunk, 0);
  };
  auto store_a = [&](const int s, const v4i (&buf)[4]) __attribute__((always_inline)) {
    uint8_t* dst = sA + s * kPSlotBytes + tid * 16;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<v4i*>(dst + i * 4096) = buf[i];
  };

  // ---- weights: this wavefront's four 32-column tiles of expert e -----------------------------
  const __amdgpu_buffer_rsrc_t rsB = buffer_rsrc(g.codes + (size_t)e * g.codes_per_expert,
                                                 (uint32_t)g.codes_per_expert);
  const __amdgpu_buffer_rsrc_t rsS = buffer_rsrc(g.scales + (size_t)e * g.scales_per_expert,
                                                 (uint32_t)g.scales_per_expert);
  int bbase[kPWaveTiles], sbase[kPWaveTiles];
#pragma unroll
  for (int cb = 0; cb < kPWaveTiles; ++cb) {
    const int q = min(cgrp * kPGroupTiles + wave * kPWaveTiles + cb, g.nt - 1);
    bbase[cb] = q * KT * 1024;
    sbase[cb] = q * g.KG * 256;
  }
  auto load_b = [&](const int cb, const int kt) __attribute__((always_inline)) {
    return __builtin_amdgcn_raw_buffer_load_b128(rsB, lane * 16, bbase[cb] + kt * 1024, 0);
  };
  auto load_s = [&](const int cb, const int grp) __attribute__((always_inline)) {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rsS, lane * 4, sbase[cb] + grp * 256, 0);
  };

  // ---- prologue: k-tiles 0, 1 staged; the next NA in registers; weight ring filled -------------
  // Every load index is clamped to the last k-tile, so no load or store depends on K: a k-tile
  // past the end is staged into a slot nobody reads.  Register set t % NA holds k-tile t.
  v4i abuf[NA][4];
  load_a(0, abuf[0 % NA]);
  store_a(0, abuf[0 % NA]);
  load_a(min(1, KT - 1), abuf[1 % NA]);
  store_a(1, abuf[1 % NA]);
#pragma unroll
  for (int t = kPStageAhead; t < kPStageAhead + NA; ++t) load_a(min(t, KT - 1), abuf[t % NA]);
  v4i bq[P][kPWaveTiles];
  uint32_t sq[2][kPWaveTiles];
#pragma unroll
  for (int j = 0; j < P; ++j)
#pragma unroll
    for (int cb = 0; cb < kPWaveTiles; ++cb) bq[j][cb] = load_b(cb, min(j, KT - 1));
#pragma unroll
  for (int cb = 0; cb < kPWaveTiles; ++cb) {
    sq[0][cb] = load_s(cb, 0);
    sq[1][cb] = load_s(cb, min(1, g.KG - 1));
  }
  __syncthreads();

  v16f acc[4][kPWaveTiles];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < kPWaveTiles; ++cb) acc[rb][cb] = v16f{};

  const int r32 = lane & 31;
  const int h = lane >> 5;
  // A operands of (k-tile kt, row block rb) from the staged slot kt % 4
  struct AOps {
    v8i hi, lo;
    uint32_t sh, sl;
  };
  auto read_ops = [&](const int kt, const int rb) __attribute__((always_inline)) {
    const uint8_t* row = sA + (kt & 3) * kPSlotBytes + rb * kPBlockBytes + r32 * kActChunk;
    AOps o;
    o.hi = staged_operand(row, h, 0);
    o.lo = staged_operand(row, h, 48);
    const uint32_t s4 = *reinterpret_cast<const uint32_t*>(row + 96);
    o.sh = s4 >> (8 * h);
    o.sl = s4 >> (16 + 8 * h);
    return o;
  };
  // Operands are read one row block ahead of the matrix instructions that use them; the first
  // block of k-tile kt + 1 is read before the barrier that ends k-tile kt (its slot was published
  // before the previous barrier), so no k-tile starts by waiting on LDS.
  AOps nxt = read_ops(0, 0);
  // k-tile kt, j = kt % 8 (compile-time: selects the register ring slots)
  auto step = [&](const int kt, const int j) __attribute__((always_inline)) {
    constexpr int D = kPStageAhead;
    store_a((kt + D) & 3, abuf[(j + D) % NA]);           // publish k-tile kt + D
    load_a(min(kt + D + NA, KT - 1), abuf[(j + D) % NA]);  // fetch k-tile kt + D + NA
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const AOps cur = nxt;
      nxt = rb < 3 ? read_ops(kt, rb + 1) : read_ops(min(kt + 1, KT - 1), 0);
#pragma unroll
      for (int cb = 0; cb < kPWaveTiles; ++cb) {
        const v8i bv = b_operand(bq[j % P][cb]);
        acc[rb][cb] = mma_sel(j & 3, cur.hi, bv, acc[rb][cb], cur.sh, sq[(j >> 2) & 1][cb]);
        acc[rb][cb] = mma_sel(j & 3, cur.lo, bv, acc[rb][cb], cur.sl, sq[(j >> 2) & 1][cb]);
      }
    }
#pragma unroll
    for (int cb = 0; cb < kPWaveTiles; ++cb) bq[j % P][cb] = load_b(cb, min(kt + P, KT - 1));
    if ((j & 3) == 3) {                                   // scale group kt/4 done: fetch group kt/4 + 2
#pragma unroll
      for (int cb = 0; cb < kPWaveTiles; ++cb) sq[(j >> 2) & 1][cb] = load_s(cb, min(kt / 4 + 2, g.KG - 1));
    }
    // Pin this k-tile's matrix instructions before the barrier: they have no memory side effects,
    // so instruction selection would otherwise gather all of them after the unrolled loop (and keep
    // every staged operand alive until then).
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int cb = 0; cb < kPWaveTiles; ++cb) asm volatile("" : "+a"(acc[rb][cb]));
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };
  if constexpr (KTC > 0) {
#pragma unroll
    for (int kt = 0; kt < KTC; ++kt) step(kt, kt & 7);
  } else {
    for (int kb = 0; kb < KT; kb += 8) {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj)
        if (kb + jj < KT) step(kb + jj, jj);             // uniform
    }
  }

  if constexpr (STAGE == 0) {
    // ---- SwiGLU, transpose through LDS, hi/lo FP6 split of each 32-value block of h ------------
    // (the ring is free: every wavefront passed the last k-tile's barrier)
    float* ep = reinterpret_cast<float*>(sA) + wave * 32 * kPEpiStride;
    const int I = g.out_K;
    const uint32_t orb = (uint32_t)act_row_bytes(I);
    uint8_t* out = reinterpret_cast<uint8_t*>(g.out);
    const int uu = lane >> 5;                            // after the transpose: block of this lane
    const int ublk = cgrp * (kPGroupTiles / 2) + wave * (kPWaveTiles / 2) + uu;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      if (rb * 32 >= nrows) break;                       // uniform
#pragma unroll
      for (int u2 = 0; u2 < kPWaveTiles / 2; ++u2) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = 8 * (r >> 2) + 4 * h + (r & 3);
          ep[m * kPEpiStride + u2 * 32 + r32] = swiglu_bf16(acc[rb][2 * u2][r], acc[rb][2 * u2 + 1][r], g.limit);
        }
      }
      __builtin_amdgcn_wave_barrier();
      float v[32];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float4 f = *reinterpret_cast<const float4*>(ep + r32 * kPEpiStride + uu * 32 + 4 * i);
        v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
      }
      __builtin_amdgcn_wave_barrier();
      const Fp6Split sp = split_fp6x32(v);
      const int m = rb * 32 + r32;
      if (m < nrows && 2 * ublk < g.nt) {
        uint8_t* chunk = out + (size_t)(p0 + m) * orb + (size_t)(ublk >> 1) * kActChunk;
        const int half = ublk & 1;
        uint2* ph = reinterpret_cast<uint2*>(chunk + 24 * half);
        uint2* pl = reinterpret_cast<uint2*>(chunk + 48 + 24 * half);
        ph[0] = make_uint2(sp.hi[0], sp.hi[1]); ph[1] = make_uint2(sp.hi[2], sp.hi[3]);
        ph[2] = make_uint2(sp.hi[4], sp.hi[5]);
        pl[0] = make_uint2(sp.lo[0], sp.lo[1]); pl[1] = make_uint2(sp.lo[2], sp.lo[3]);
        pl[2] = make_uint2(sp.lo[4], sp.lo[5]);
        chunk[96 + half] = (uint8_t)sp.s_hi;
        chunk[98 + half] = (uint8_t)sp.s_lo;
      }
    }
  } else {
    // ---- down: scale row p by its gate weight, store fp32 ---------------------------------------
    const int D = g.out_K;
    float* out = reinterpret_cast<float*>(g.out);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      if (rb * 32 >= nrows) break;                       // uniform
#pragma unroll
      for (int cb = 0; cb < kPWaveTiles; ++cb) {
        const int q = cgrp * kPGroupTiles + wave * kPWaveTiles + cb;
        if (q >= g.nt) break;                            // uniform
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = rb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          if (m < nrows) out[(size_t)(p0 + m) * D + q * 32 + r32] = acc[rb][cb][r] * sgate[m];
        }
      }
    }
  }
}

#ifndef MOE_PREFILL_NA
#define MOE_PREFILL_NA 2
#endif
#ifndef MOE_PREFILL_P
#define MOE_PREFILL_P 4
#endif
constexpr int kPNA = MOE_PREFILL_NA;
constexpr int kPP = MOE_PREFILL_P;

hipError_t launch_gemm_prefill(int stage, int T, int D, int I, int E, int k, float limit,
                               const uint8_t* a_packed, const int32_t* tiles, const uint8_t* codes,
                               const uint8_t* scales, const float* topk_w, void* out, hipStream_t s) {
  PrefillArgs g;
  const int K = stage == 0 ? D : I;
  const int N = stage == 0 ? 2 * I : D;
  g.k = k;
  g.KT = K / kKTile;
  g.KG = w_kgroups(K);
  g.nt = N / kNTile;
  g.ngroups = (g.nt + kPGroupTiles - 1) / kPGroupTiles;
  g.out_K = stage == 0 ? I : D;
  g.limit = limit;
  g.a_packed = a_packed;
  g.arb = (uint32_t)act_row_bytes(K);
  g.a_bytes = (uint32_t)((size_t)(stage == 0 ? T : (long long)T * k) * g.arb);
  g.tiles = tiles;
  g.topk_w = topk_w;
  g.codes = codes;
  g.scales = scales;
  g.out = out;
  g.codes_per_expert = w_codes_per_expert(N, K);
  g.scales_per_expert = w_scales_per_expert(N, K);
  const long long items = tile_slots((long long)T * k, E) * g.ngroups;
  const dim3 grid((unsigned)((items + 7) / 8 * 8));
#ifdef MOE_PREFILL_GENERIC_ONLY
  g.KT = g.KT + 0 * 45;
  if (stage == 0) expert_gemm_prefill_kernel<0, 0, kPNA, kPP><<<grid, dim3(256), 0, s>>>(g);
  else expert_gemm_prefill_kernel<1, 0, kPNA, kPP><<<grid, dim3(256), 0, s>>>(g);
  return hipGetLastError();
#endif
  if (stage == 0) {
    if (g.KT == 45) expert_gemm_prefill_kernel<0, 45, kPNA, kPP><<<grid, dim3(256), 0, s>>>(g);
    else expert_gemm_prefill_kernel<0, 0, kPNA, kPP><<<grid, dim3(256), 0, s>>>(g);
  } else {
    if (g.KT == 45) expert_gemm_prefill_kernel<1, 45, kPNA, kPP><<<grid, dim3(256), 0, s>>>(g);
    else expert_gemm_prefill_kernel<1, 0, kPNA, kPP><<<grid, dim3(256), 0, s>>>(g);
  }
  return hipGetLastError();
}

}  // namespace moe
