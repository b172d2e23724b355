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
//  - The LDS holds a ring of staged k-tiles. In the gate/up stage (8 slots,
//    128 KB) k-tile kt+3 is written from registers while kt is computed and
//    kt+5 is loading into registers, and a barrier after every second k-tile
//    publishes the two staged since the previous one; the down stage (4
//    slots) writes kt+2 and has a barrier per k-tile.
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
//  - The activation-quantized variant (AF = kActFp4) stages 48-byte MXFP4
//    chunks and issues one FP4 x FP4 instruction per weight tile in the plain
//    operand layout (lanes 0-31 block 0, lanes 32-63 block 1, weights as
//    loaded); its gate/up epilogue quantizes h to MXFP4.
#include <type_traits>

#include "mfma_ops.h"

namespace moe {

struct PrefillArgs {
  int k, KT, KG, nt, ngroups, out_K;
  int out_assign;                                        // down: rows to their assignment index
  int h_bf16;                                            // gate/up: h as bf16 rows instead of packed
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
constexpr int kPSlots = 8;                             // LDS ring slots of the gate/up stage (slot = k-tile % 8)
constexpr int kPSlotBytes = 1024 * 16;                 // 896 pieces + 128 dummy (4 unconditional per thread)
// The gate/up stage stages k-tile kt + 3 during kt into an 8-slot ring and publishes with a barrier
// after every second k-tile; the down stage (fewer registers to spare) stages kt + 2 into 4 slots
// and has a barrier per k-tile.
template <int STAGE>
constexpr int stage_ahead() { return STAGE == 0 ? 3 : 2; }
template <int STAGE>
constexpr int barrier_every() { return STAGE == 0 ? 2 : 1; }
template <int STAGE>
constexpr int ring_slots() { return STAGE == 0 ? kPSlots : 4; }
constexpr int kPEpiStride = 68;                        // floats per row of the transposed h block
constexpr int kPOutStride = 136;                       // halves per row of the transposed y block
static_assert(kPSlots * kPSlotBytes >= 4 * 32 * kPEpiStride * 4, "h transposition fits the gate/up ring");
static_assert(4 * kPSlotBytes / 4 >= 32 * kPOutStride * 2, "y transposition fits a wavefront's quarter of the down ring");

// Matrix-instruction pairing.  Each 64-wide k-tile holds two 32-value blocks b = 0, 1 of the
// activation, each stored as hi + lo FP6 terms.  Two MFMAs per weight tile, one per term: lane half
// b supplies block b's hi term to the first and its lo term to the second, as the instruction's K
// halves, so the weight operand and its scales are used as loaded (lane half b: block b).  The
// lane's two 24-byte terms sit at 24b and 48 + 24b of the row chunk: read as twelve dwords, the hi
// operand is dwords 0-5 and the lo operand dwords 6-11 (register sub-ranges, no copies).
typedef int v16i __attribute__((ext_vector_type(16)));

// NA: activation k-tiles in flight in registers (k-tile t is fetched NA k-tiles before it is
// written to LDS); P: weight k-tiles in flight per wavefront.  Both divide 8.
template <int STAGE, int KTC, int NA, int P, int AF = kActSplit6>
__global__ __launch_bounds__(256) void expert_gemm_prefill_kernel(PrefillArgs g) {
  static_assert(8 % NA == 0 && 8 % P == 0 && P >= 4, "ring depths divide the 8-step unroll");
  constexpr bool F4 = AF == kActFp4;
  constexpr int CH = F4 ? kAct4Chunk : kActChunk;        // packed bytes per row and k-tile
  constexpr int NPC = F4 ? 2 : 4;                         // staged 16-byte pieces per thread per k-tile
  constexpr int kStagePieces = kPrefillRows * (CH / 16);  // 384 or 896 (the rest re-read a real one)
  constexpr int kBlockBytes = 32 * CH;                    // one 32-row block of a staged k-tile
  constexpr int kSlots = ring_slots<STAGE>();
  __shared__ __attribute__((aligned(16))) uint8_t sA[kSlots * kPSlotBytes];
  __shared__ int srow[kPrefillRows];
  __shared__ float sgate[kPrefillRows];
  __shared__ int sdst[kPrefillRows];                     // down: output row of each tile row

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
  // the header and the row ids in one round trip (a slot always holds 128 id entries)
  const int a_id = tile[4 + (tid & (kPrefillRows - 1))];
  const int4 hdr = *reinterpret_cast<const int4*>(tile);
  const int e = __builtin_amdgcn_readfirstlane(hdr.x);
  const int p0 = __builtin_amdgcn_readfirstlane(hdr.y);
  const int nrows = __builtin_amdgcn_readfirstlane(hdr.z);

  // With K known at compile time the rest of the kernel exists in four copies, one per number NRB
  // of 32-row blocks that hold rows of the tile: a partial tile's empty row blocks get neither
  // operand reads, staging nor matrix instructions.  Every other step is the same in all copies.
  auto body = [&](auto nrb_c) __attribute__((always_inline)) {
  constexpr int NRB = decltype(nrb_c)::value;

  // down: each row's gate weight, loaded now and waited for only in the epilogue
  float wrow = 0.0f;
  if (tid < nrows) {
    srow[tid] = STAGE == 0 ? a_id / g.k : p0 + tid;
    if constexpr (STAGE == 1) wrow = g.topk_w[a_id];
  }
  __syncthreads();

  // ---- activation staging: thread tid moves pieces tid + 256 i (i < 4) of every k-tile ----------
  const __amdgpu_buffer_rsrc_t rsA = buffer_rsrc(g.a_packed, g.a_bytes);
  uint32_t aoff[NPC];
#pragma unroll
  for (int i = 0; i < NPC; ++i) {
    const int q = min(tid + 256 * i, kStagePieces - 1);  // the dummy pieces re-read a real one
    const int row = q / (CH / 16);
    // rows past the tile repeat its last row
    aoff[i] = (uint32_t)srow[min(row, nrows - 1)] * g.arb + (uint32_t)(q - row * (CH / 16)) * 16u;
  }
  // piece sets i whose pieces all lie past the occupied row blocks are neither loaded nor staged
  constexpr int kLivePieces = NRB * 32 * (CH / 16);
  auto load_a = [&](const int kt, v4i (&buf)[NPC]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NPC; ++i)
      if (256 * i < kLivePieces) buf[i] = __builtin_amdgcn_raw_buffer_load_b128(rsA, aoff[i], kt * CH, 0);
  };
  auto store_a = [&](const int s, const v4i (&buf)[NPC]) __attribute__((always_inline)) {
    uint8_t* dst = sA + s * kPSlotBytes + tid * 16;
#pragma unroll
    for (int i = 0; i < NPC; ++i)
      if (256 * i < kLivePieces) *reinterpret_cast<v4i*>(dst + i * 4096) = buf[i];
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

  // ---- prologue: the first stage_ahead k-tiles staged; the next NA in registers; weight ring ----
  constexpr int kAhead = stage_ahead<STAGE>();
  // Every load index is clamped to the last k-tile, so no load or store depends on K: a k-tile
  // past the end is staged into a slot nobody reads.  Register set t % NA holds k-tile t.
  v4i abuf[NA][NPC];
#pragma unroll
  for (int t = 0; t < kAhead; ++t) {
    load_a(min(t, KT - 1), abuf[t % NA]);
    store_a(t, abuf[t % NA]);
  }
#pragma unroll
  for (int t = kAhead; t < kAhead + NA; ++t) load_a(min(t, KT - 1), abuf[t % NA]);
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
  // A operands of (k-tile kt, row block rb) from the staged ring slot
  // this lane half's block h has its hi term at bytes [24h, 24h + 24) of the row chunk and its lo
  // term at [48 + 24h, 72 + 24h); the scale bytes are [hi0, hi1, lo0, lo1] at 96, so the scale
  // dword shifted right by 8h holds the block's hi scale in byte 0 and its lo scale in byte 2
  // (chosen by the instruction's A-scale byte select).
  // Loads only: nothing waits for them until the operands are used a phase later.
  struct AOps {
    v16i q;
    uint32_t s;
  };
  auto read_ops = [&](const int kt, const int rb) __attribute__((always_inline)) {
    const uint8_t* row = sA + (kt & (kSlots - 1)) * kPSlotBytes + rb * kBlockBytes + r32 * CH;
    AOps o;
    if constexpr (F4) {                                   // the lane's block: 16 bytes and a scale byte
      const v4i q0 = *reinterpret_cast<const v4i*>(row + 16 * h);
      o.q = v16i{q0.x, q0.y, q0.z, q0.w, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
      o.s = row[32 + h];
      return o;
    }
    typedef int v2i __attribute__((ext_vector_type(2)));
    const uint8_t* hi = row + 24 * h;
    const v2i q0 = *reinterpret_cast<const v2i*>(hi);
    const v2i q1 = *reinterpret_cast<const v2i*>(hi + 8);
    const v2i q2 = *reinterpret_cast<const v2i*>(hi + 16);
    const v2i q3 = *reinterpret_cast<const v2i*>(hi + 48);
    const v2i q4 = *reinterpret_cast<const v2i*>(hi + 56);
    const v2i q5 = *reinterpret_cast<const v2i*>(hi + 64);
    o.q = v16i{q0.x, q0.y, q1.x, q1.y, q2.x, q2.y, q3.x, q3.y, q4.x, q4.y, q5.x, q5.y, 0, 0, 0, 0};
    o.s = *reinterpret_cast<const uint32_t*>(row + 96) >> (8 * h);
    return o;
  };
  // Software pipeline of one k-tile (kt, j = kt % 8, compile-time ring slots), in four phases of
  // eight matrix instructions (one row block each).  Other work rides in the phases' shadows:
  //  - operands are read one row block ahead; the next k-tile's first block is read at the end of
  //    this k-tile (its slot was published by an earlier barrier);
  //  - phase 0 stages k-tile kt + A, phase 1 fetches k-tile kt + A + NA (A = stage_ahead);
  //  - phase 3 refills the weight ring slot just consumed.
  // A scheduling barrier between phases keeps each phase's work next to its matrix instructions.
  AOps nxt = read_ops(0, 0);
  auto step = [&](const int kt, const int j) __attribute__((always_inline)) {
    constexpr int D = kAhead;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      AOps cur;
      if (rb < NRB) {                                     // resolved at compile time
        cur = nxt;
        nxt = rb + 1 < NRB ? read_ops(kt, rb + 1) : read_ops(min(kt + 1, KT - 1), 0);
      }
      if (rb >= NRB) {
      } else if constexpr (F4) {
        const v8i a = __builtin_shufflevector(cur.q, cur.q, 0, 1, 2, 3, 12, 13, 14, 15);
#pragma unroll
        for (int cb = 0; cb < kPWaveTiles; ++cb)
          acc[rb][cb] = mma4_sel(j & 3, a, b_operand(bq[j % P][cb]), acc[rb][cb], cur.s, sq[(j >> 2) & 1][cb]);
      } else {
        const v8i ahi = __builtin_shufflevector(cur.q, cur.q, 0, 1, 2, 3, 4, 5, 6, 7);
        const v8i alo = __builtin_shufflevector(cur.q, cur.q, 6, 7, 8, 9, 10, 11, 12, 13);
#pragma unroll
        for (int cb = 0; cb < kPWaveTiles; ++cb) {
          const v8i b = b_operand(bq[j % P][cb]);
          const uint32_t sb = sq[(j >> 2) & 1][cb];
          acc[rb][cb] = mma_sel_a<0>(j & 3, ahi, b, acc[rb][cb], cur.s, sb);
          acc[rb][cb] = mma_sel_a<2>(j & 3, alo, b, acc[rb][cb], cur.s, sb);
        }
      }
      if (rb == 0) store_a((kt + D) & (kSlots - 1), abuf[(j + D) % NA]);       // stage kt + D
      if (rb == 1) load_a(min(kt + D + NA, KT - 1), abuf[(j + D) % NA]);        // fetch kt + D + NA
      if (rb == 3) {
#pragma unroll
        for (int cb = 0; cb < kPWaveTiles; ++cb) bq[j % P][cb] = load_b(cb, min(kt + P, KT - 1));
        if ((j & 3) == 3) {                               // scale group kt/4 done: fetch group kt/4 + 2
#pragma unroll
          for (int cb = 0; cb < kPWaveTiles; ++cb) sq[(j >> 2) & 1][cb] = load_s(cb, min(kt / 4 + 2, g.KG - 1));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // Pin this k-tile's matrix instructions before the barrier: they have no memory side effects,
    // so instruction selection would otherwise gather all of them after the unrolled loop (and keep
    // every staged operand alive until then).
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int cb = 0; cb < kPWaveTiles; ++cb) asm volatile("" : "+a"(acc[rb][cb]));
    // A barrier after every B-th k-tile publishes the k-tiles staged since the last one (B =
    // barrier_every, staging A = stage_ahead >= B + 1 ahead into 8 >= A + B slots).  The first
    // operands of kt + 1, read at the end of kt, were staged during kt + 1 - A, and one of the B
    // k-tiles before kt ends with a barrier; the slot kt + A takes last held kt + A - 8, which
    // every wavefront finished before the last barrier.
    constexpr int B = barrier_every<STAGE>();
    static_assert(kAhead >= B + 1 && kSlots >= kAhead + B, "ring publishing order");
    if (j % B == B - 1) __syncthreads();
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

  __syncthreads();                                       // every wavefront is done with the ring
  if constexpr (STAGE == 0) {
    // ---- SwiGLU, transpose through LDS, hi/lo FP6 split of each 32-value block of h ------------
    float* ep = reinterpret_cast<float*>(sA) + wave * 32 * kPEpiStride;
    const int I = g.out_K;
    const uint32_t orb = (uint32_t)act_row_bytes_af(AF, I);
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
      const int m = rb * 32 + r32;
      if constexpr (F4) {
        const Fp4Block q4 = quant_fp4x32(v);
        if (m < nrows && 2 * ublk < g.nt) store_fp4_block(out + (size_t)(p0 + m) * orb, ublk, q4);
      } else {
        if (g.h_bf16) {
          if (m < nrows && 2 * ublk < g.nt) store_bf16_block(reinterpret_cast<uint16_t*>(g.out) + (size_t)(p0 + m) * I, ublk, v);
        } else {
          const Fp6Split sp = split_fp6x32(v);
          if (m < nrows && 2 * ublk < g.nt) store_fp6_block(out + (size_t)(p0 + m) * orb, ublk, sp);
        }
      }
    }
  } else {
    // ---- down: scale row p by its gate weight, fp16, transpose through LDS, 16-byte row stores --
    if (tid < kPrefillRows) {
      sgate[tid] = wrow;
      sdst[tid] = g.out_assign ? a_id : p0 + tid;
    }
    __syncthreads();
    const int D = g.out_K;
    uint8_t* out = reinterpret_cast<uint8_t*>(g.out);
    _Float16* ep = reinterpret_cast<_Float16*>(sA + wave * (kSlots * kPSlotBytes / 4));
    const int c0 = (cgrp * kPGroupTiles + wave * kPWaveTiles) * 32;   // first column of the wavefront
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      if (rb * 32 >= nrows) break;                       // uniform
#pragma unroll
      for (int cb = 0; cb < kPWaveTiles; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = 8 * (r >> 2) + 4 * h + (r & 3);
          ep[m * kPOutStride + cb * 32 + r32] = (_Float16)(acc[rb][cb][r] * sgate[rb * 32 + m]);
        }
      __builtin_amdgcn_wave_barrier();
      // 32 rows x 128 columns = 512 pieces of 8 values; piece = row * 16 + column / 8
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int pc = lane + 64 * i;
        const int row = pc >> 4, c8 = (pc & 15) * 8;
        const uint4 v = *reinterpret_cast<const uint4*>(ep + row * kPOutStride + c8);
        const int m = rb * 32 + row;
        if (m < nrows && c0 + c8 < D)
          *reinterpret_cast<uint4*>(out + ((size_t)sdst[m] * D + c0 + c8) * 2) = v;
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
  };
  // (the generic-K kernel keeps one copy: its k-loop is not unrolled and it serves odd shapes only)
  const int live_blocks = KTC > 0 ? (nrows + 31) >> 5 : 4;   // 1..4, uniform
  if (live_blocks >= 4) body(std::integral_constant<int, 4>{});
  else if (live_blocks == 3) body(std::integral_constant<int, 3>{});
  else if (live_blocks == 2) body(std::integral_constant<int, 2>{});
  else body(std::integral_constant<int, 1>{});
}

constexpr int kPNA = 2;         // activation k-tiles in flight in registers
constexpr int kPP = 4;          // weight k-tiles in flight per wavefront

hipError_t launch_gemm_prefill(int stage, int T, int D, int I, int E, int k, float limit,
                               const uint8_t* a_packed, const int32_t* tiles, const uint8_t* codes,
                               const uint8_t* scales, const float* topk_w, void* out, hipStream_t s, int af,
                               int out_assign, int h_bf16) {
  PrefillArgs g;
  g.out_assign = stage == 1 && out_assign;
  g.h_bf16 = stage == 0 && h_bf16;
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
  g.arb = (uint32_t)act_row_bytes_af(af, K);
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
  if (af == kActFp4) {
    if (stage == 0) {
      if (g.KT == 45) expert_gemm_prefill_kernel<0, 45, kPNA, kPP, kActFp4><<<grid, dim3(256), 0, s>>>(g);
      else expert_gemm_prefill_kernel<0, 0, kPNA, kPP, kActFp4><<<grid, dim3(256), 0, s>>>(g);
    } else {
      if (g.KT == 45) expert_gemm_prefill_kernel<1, 45, kPNA, kPP, kActFp4><<<grid, dim3(256), 0, s>>>(g);
      else expert_gemm_prefill_kernel<1, 0, kPNA, kPP, kActFp4><<<grid, dim3(256), 0, s>>>(g);
    }
    return hipGetLastError();
  }
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
