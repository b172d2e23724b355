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
//  - Staged layout, per 32-row block: the seven 16-byte pieces of every row's
//    112-byte chunk, piece-major (piece j of row r at (j*32 + r) * 16). A half
//    wavefront's operand read then covers 512 contiguous bytes.
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
constexpr int kPBlockBytes = kPPieces * 32 * 16;       // one 32-row block of a staged k-tile
constexpr int kPStagePieces = kPrefillRows * kPPieces; // 896 pieces per staged k-tile
constexpr int kPSlotBytes = 1024 * 16;                 // 896 pieces + 128 dummy (4 unconditional per thread)
constexpr int kPRing = 4;                              // weight k-tiles in flight per wavefront
constexpr int kPEpiStride = 68;                        // floats per row of the transposed h block
static_assert(kPSlots * kPSlotBytes >= 4 * 32 * kPEpiStride * 4, "h transposition fits the ring");

// FP6 operand from a piece-major staged block: this lane's 24 bytes are bytes [24h, 24h+24) of the
// hi (or lo) half of its row's chunk, i.e. the 16 bytes of piece p16 and 8 bytes of piece p8.
__device__ __forceinline__ v8i staged_operand(const uint8_t* blk, int r, int h, int p16, int p8) {
  const v4i q = *reinterpret_cast<const v4i*>(blk + (p16 * 32 + r) * 16);
  const uint2 t = *reinterpret_cast<const uint2*>(blk + (p8 * 32 + r) * 16 + 8 * h);
  const bool up = h != 0;
  v8i v = {up ? (int)t.x : q.x, up ? (int)t.y : q.y, up ? q.x : q.z, up ? q.y : q.w,
           up ? q.z : (int)t.x, up ? q.w : (int)t.y, 0, 0};
  return v;
}

template <int STAGE, int KTC>
__global__ __launch_bounds__(256) void expert_gemm_prefill_kernel(PrefillArgs g) {
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
    const int rb = q / (32 * kPPieces);
    const int rem = q - rb * 32 * kPPieces;
    aoff[i] = (uint32_t)srow[rb * 32 + (rem & 31)] * g.arb + (uint32_t)(rem >> 5) * 16u;
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

  // ---- prologue: k-tiles 0, 1 staged; 2, 3 in registers; weight ring filled ---------------------
  // Every load index is clamped to the last k-tile, so no load or store depends on K: a k-tile
  // past the end is staged into a slot nobody reads.
  v4i abuf[2][4];
  load_a(0, abuf[0]);
  load_a(min(1, KT - 1), abuf[1]);
  v4i bq[kPRing][kPWaveTiles];
  uint32_t sq[2][kPWaveTiles];
#pragma unroll
  for (int j = 0; j < kPRing; ++j)
#pragma unroll
    for (int cb = 0; cb < kPWaveTiles; ++cb) bq[j][cb] = load_b(cb, min(j, KT - 1));
#pragma unroll
  for (int cb = 0; cb < kPWaveTiles; ++cb) {
    sq[0][cb] = load_s(cb, 0);
    sq[1][cb] = load_s(cb, min(1, g.KG - 1));
  }
  store_a(0, abuf[0]);
  store_a(1, abuf[1]);
  load_a(min(2, KT - 1), abuf[0]);
  load_a(min(3, KT - 1), abuf[1]);
  __syncthreads();

  v16f acc[4][kPWaveTiles];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < kPWaveTiles; ++cb) acc[rb][cb] = v16f{};

  const int r32 = lane & 31;
  const int h = lane >> 5;
  // k-tile kt, j = kt % 8 (compile-time: selects the register ring slots)
  auto step = [&](const int kt, const int j) __attribute__((always_inline)) {
    store_a((kt + 2) & 3, abuf[j & 1]);                  // publish k-tile kt + 2
    load_a(min(kt + 4, KT - 1), abuf[j & 1]);            // fetch k-tile kt + 4
    const uint8_t* slotp = sA + (kt & 3) * kPSlotBytes;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const uint8_t* blk = slotp + rb * kPBlockBytes;
      const v8i ahi = staged_operand(blk, r32, h, h ? 2 : 0, 1);
      const v8i alo = staged_operand(blk, r32, h, h ? 5 : 3, 4);
      const uint32_t s4 = *reinterpret_cast<const uint32_t*>(blk + (6 * 32 + r32) * 16);
      const uint32_t sh = s4 >> (8 * h), sl = s4 >> (16 + 8 * h);
#pragma unroll
      for (int cb = 0; cb < kPWaveTiles; ++cb) {
        const v8i bv = b_operand(bq[j & 3][cb]);
        acc[rb][cb] = mma_sel(j & 3, ahi, bv, acc[rb][cb], sh, sq[(j >> 2) & 1][cb]);
        acc[rb][cb] = mma_sel(j & 3, alo, bv, acc[rb][cb], sl, sq[(j >> 2) & 1][cb]);
      }
    }
#pragma unroll
    for (int cb = 0; cb < kPWaveTiles; ++cb) bq[j & 3][cb] = load_b(cb, min(kt + kPRing, KT - 1));
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
          const float gv = fminf(fmaxf(acc[rb][2 * u2][r], -g.limit), g.limit);
          const float uv = fminf(fmaxf(acc[rb][2 * u2 + 1][r], -g.limit), g.limit);
          ep[m * kPEpiStride + u2 * 32 + r32] = bf16_round(gv / (1.0f + expf(-gv)) * uv);
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
  if (stage == 0) {
    if (g.KT == 45) expert_gemm_prefill_kernel<0, 45><<<grid, dim3(256), 0, s>>>(g);
    else expert_gemm_prefill_kernel<0, 0><<<grid, dim3(256), 0, s>>>(g);
  } else {
    if (g.KT == 45) expert_gemm_prefill_kernel<1, 45><<<grid, dim3(256), 0, s>>>(g);
    else expert_gemm_prefill_kernel<1, 0><<<grid, dim3(256), 0, s>>>(g);
  }
  return hipGetLastError();
}

}  // namespace moe
