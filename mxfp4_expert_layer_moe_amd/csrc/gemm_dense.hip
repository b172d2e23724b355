// Dense gate/up projection of the whole-layer path at decode sizes: routing off the weight stream.
//
// At decode sizes (at most 32 tokens, and so many assignments per expert that nearly every expert
// is touched) the layer is bound by streaming the experts' MXFP4 weights ("gpt-oss architecture
// walk-through", section "Quantization": 4.25 bits per parameter) from HBM, and the selection of
// the top-k experts ("Mixture of Experts" section of the same page) would otherwise sit between the
// router and that stream.  Here the gate/up projection does not wait for the selection: it
// computes h = bf16(silu(clamp(g)) * clamp(u)) ("From GPT-2 to gpt-oss", section 3, Swish/SwiGLU;
// clamp at swiglu_limit) for every (expert, token) pair, each expert's T tokens filling the rows of
// one 32-row matrix tile, and writes packed h row e*T + t.  The first workgroup of the same launch
// scores the router and runs the selection of the top-k experts, their gates and the grouping by
// expert (select_small, the code of the routed path's selection kernel), which only the next launch
// needs: the routed
// small-batch down projection (gemm.hip), reading h row e*T + t for each row of its tiles.
//
// Each row goes through exactly the instruction sequence of the routed small-batch kernel: per
// 64-wide k-tile, for each 32-column weight tile, the scaled FP6 x FP4 matrix instruction on the hi
// term, then on the lo term, into one fp32 accumulator; the same SwiGLU, bf16 rounding and FP6 split
// in the epilogue.  Matrix rows are independent, so every routed row has the bits of the routed
// path; the rows of unselected pairs are computed and never read.
//
// Layout: the (expert, output unit) pairs (a unit is a gate/up pair of 32-column weight tiles) are
// dealt 12 to a workgroup of 12 wavefronts (three per SIMD), one pair per wavefront; the activation
// rows are the same x for every expert.  At d_ff = 2880 (90 units) 32 experts give 240 workgroups,
// which with the selection workgroup (dispatched first, 768 threads in two passes of 24 tokens) are
// all resident at once, one per compute unit (the staged rows take most of its LDS).  A workgroup stages the T token rows of all of K in
// LDS once (the
// packed rows' 112-byte chunks cut to their 104 used bytes: 32 x 45 x 104 = 146 KB at K = 2880; a
// row stride of an odd number of 8-byte words puts 16 consecutive rows of one 8-byte read on
// distinct banks), issuing those loads before the weight ring, and then runs a k-loop with no
// barrier, each wavefront streaming its weights through a P-deep register ring.
#include "mfma_ops.h"
#include "select_body.h"

namespace moe {

typedef int v2i __attribute__((ext_vector_type(2)));

struct DenseArgs {
  int T, k, E, K, KT, KG, units, out_K;
  float limit;
  const uint8_t* a;                 // packed x, T rows
  uint32_t a_bytes;
  const uint8_t* codes;
  const uint8_t* scales;
  size_t codes_per_expert, scales_per_expert;
  void* out;                        // packed h rows e*T + t
  // the selection workgroup (blockIdx.x == 0)
  int D;
  const uint16_t* x;
  const float* wr;
  const float* br;
  int32_t* sel_idx;
  float* sel_w;
  int bm, slots;                    // the grouping's tile height and slot count
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm;
  int32_t* inv;
  int32_t* tiles;
};

constexpr int kDenseTokens = 32;            // rows of the dense tile: every token of the batch
constexpr int kDenseWaves = 12;             // wavefronts per workgroup (three per SIMD), one (expert, unit) each
constexpr int kDenseThreads = kDenseWaves * 64;

constexpr int kDenseChunk = 104;            // staged bytes per row and k-tile (the used bytes, 8-aligned)
constexpr int kDenseStageBytes = kDenseTokens * kDenseMaxKT * kDenseChunk;   // 149760

template <int P, int KTC>
__global__ __launch_bounds__(kDenseThreads) void expert_gemm_dense_kernel(DenseArgs g) {
  constexpr int NB = 2;                     // a SwiGLU pair of 32-column tiles per wavefront
  static_assert(P % 4 == 0, "prefetch depth covers whole scale groups");
  __shared__ __attribute__((aligned(16))) uint8_t sA[kDenseStageBytes];
  using Scores = ScoreSmem<kDenseWaves>;
  constexpr size_t kScoresAt = (sizeof(SelectSmem) + 15) / 16 * 16;
  static_assert(kScoresAt + sizeof(Scores) <= kDenseStageBytes, "the selection borrows the staging buffer");
  if (blockIdx.x == 0) {
    // the scores, the selection and the grouping of all tokens, beside the dense gate/up projection
    select_small<kDenseThreads, true>(*reinterpret_cast<SelectSmem*>(sA), reinterpret_cast<Scores*>(sA + kScoresAt),
                                nullptr, nullptr, g.T, g.D, g.E, g.k, g.x, g.wr, g.br, g.sel_idx, g.sel_w, nullptr,
                                g.bm, g.slots, g.counts, g.offsets, g.perm, g.inv, g.tiles);
    return;
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = (blockIdx.x - 1) * kDenseWaves + wave;   // (expert, unit) pair of this wavefront
  const bool active = pair < g.E * g.units;             // inactive waves still join the barriers
  const int pc = active ? pair : g.E * g.units - 1;
  const int e = pc / g.units;
  const int u = pc - e * g.units;
  const int i = lane & 31;
  const int half = lane >> 5;
  const int T = g.T;
  const int KT = KTC > 0 ? KTC : g.KT;
  const int rs = KT * kDenseChunk;                       // row stride in LDS
  const size_t arb = act_row_bytes(g.K);

  const __amdgpu_buffer_rsrc_t rsB = buffer_rsrc(g.codes + (size_t)e * g.codes_per_expert,
                                                 (uint32_t)g.codes_per_expert);
  const __amdgpu_buffer_rsrc_t rsS = buffer_rsrc(g.scales + (size_t)e * g.scales_per_expert,
                                                 (uint32_t)g.scales_per_expert);
  const int voffB = lane * 16, voffS = lane * 4;
  int sbase[NB], ssbase[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int q = NB * u + nb;                           // inactive waves load nothing
    sbase[nb] = q * g.KT * 1024;
    ssbase[nb] = q * g.KG * 256;
  }
  auto load_b = [&](const int nb, const int kt) {
    return __builtin_amdgcn_raw_buffer_load_b128(rsB, voffB, sbase[nb] + kt * 1024, kLoadStream);
  };
  auto load_s = [&](const int nb, const int grp) {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rsS, voffS, ssbase[nb] + grp * 256, kLoadStream);
  };

  // ---- staging: 8-byte pieces w = (row, k-tile, piece of 13); the loads go out before the weight
  // ring (loads complete in issue order, so waiting for them does not wait for the weights) -------
  constexpr int kPieces = kDenseChunk / 8;               // 8-byte pieces per staged chunk
  const __amdgpu_buffer_rsrc_t rsA = buffer_rsrc(g.a, g.a_bytes);
  const int n8 = KT * kPieces;
  const int total = T * n8;
  constexpr int kPer = KTC > 0 ? (kDenseTokens * KTC * kPieces + kDenseThreads - 1) / kDenseThreads : 1;
  uint2 stg[kPer];
  auto piece_src = [&](const int w) {
    const int r = w / n8, o = w - r * n8;
    const int kt = o / kPieces, b = o - kt * kPieces;
    return (uint32_t)((size_t)r * arb + (size_t)kt * kActChunk + (size_t)b * 8);
  };
  auto piece_dst = [&](const int w) {
    const int r = w / n8, o = w - r * n8;
    return r * rs + o * 8;                               // o * 8 = kt * 104 + b * 8
  };
  if constexpr (KTC > 0) {
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int w = tid + kDenseThreads * q;
      if (w < total) {
        const v2i v = __builtin_amdgcn_raw_buffer_load_b64(rsA, piece_src(w), 0, 0);
        stg[q] = make_uint2((uint32_t)v.x, (uint32_t)v.y);
      }
    }
  }
  v4i bq[P][NB];
  uint32_t sbq[P / 4][NB];
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
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int w = tid + kDenseThreads * q;
      if (w < total) *reinterpret_cast<uint2*>(sA + piece_dst(w)) = stg[q];
    }
  } else {
    for (int w = tid; w < total; w += kDenseThreads) {
      const v2i v = __builtin_amdgcn_raw_buffer_load_b64(rsA, piece_src(w), 0, 0);
      *reinterpret_cast<uint2*>(sA + piece_dst(w)) = make_uint2((uint32_t)v.x, (uint32_t)v.y);
    }
  }
  __syncthreads();

  v16f acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = v16f{};
  if (active) {
    const bool valid = i < T;
    const uint8_t* arow = sA + i * rs;                   // rows past T read unused bytes, masked below
    // one k-tile (slot j = kt % P): A from LDS, two MFMAs per weight tile (hi, then lo), then the
    // refill of slot j with k-tile kt + P (clamped to the last k-tile: a repeated load hits cache)
    auto step = [&](const int j, const int kt) {
      const uint8_t* chunk = arow + kt * kDenseChunk;
      const uint2* ph = reinterpret_cast<const uint2*>(chunk + 24 * half);
      const uint2* pl = reinterpret_cast<const uint2*>(chunk + 48 + 24 * half);
      const uint2 h0 = ph[0], h1 = ph[1], h2 = ph[2], l0 = pl[0], l1 = pl[1], l2 = pl[2];
      const v8i z = {0, 0, 0, 0, 0, 0, 0, 0};
      v8i ah = {(int)h0.x, (int)h0.y, (int)h1.x, (int)h1.y, (int)h2.x, (int)h2.y, 0, 0};
      v8i al = {(int)l0.x, (int)l0.y, (int)l1.x, (int)l1.y, (int)l2.x, (int)l2.y, 0, 0};
      uint32_t sh = chunk[96 + half];
      uint32_t sl = chunk[98 + half];
      ah = valid ? ah : z;
      al = valid ? al : z;
      sh = valid ? sh : 127u;
      sl = valid ? sl : 127u;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const v8i bv = b_operand(bq[j][nb]);
        acc[nb] = mma_sel(j & 3, ah, bv, acc[nb], sh, sbq[j >> 2][nb]);
        acc[nb] = mma_sel(j & 3, al, bv, acc[nb], sl, sbq[j >> 2][nb]);
      }
      const int kn = min(kt + P, g.KT - 1);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) bq[j][nb] = load_b(nb, kn);
      if ((j & 3) == 3) {
        const int grp = min((kt + P - 3) / 4, (g.KT - 1) / 4);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) sbq[j >> 2][nb] = load_s(nb, grp);
      }
      if constexpr (KTC > 0) __builtin_amdgcn_sched_barrier(0);
    };
    if constexpr (KTC > 0) {
#pragma unroll
      for (int kt = 0; kt < KTC; ++kt) step(kt % P, kt);
    } else {
      int kb = 0;
      for (; kb + P <= KT; kb += P) {
#pragma unroll
        for (int j = 0; j < P; ++j) step(j, kb + j);
      }
#pragma unroll
      for (int j = 0; j < P; ++j)
        if (kb + j < KT) step(j, kb + j);               // the tail (uniform)
    }
  }
  // SwiGLU epilogue, then a transpose through LDS (the staged rows are free once every wavefront
  // is past its k-loop) so that lane m holds the 32 values of row m's block and splits them into
  // hi/lo FP6, as the routed kernel does
  __syncthreads();
  if (!active) return;
  constexpr int kEpStride = 36;                          // floats per row: 8 rows on 8 bank groups
  static_assert(kDenseWaves * kDenseTokens * kEpStride * 4 <= kDenseStageBytes, "transpose fits");
  float* ep = reinterpret_cast<float*>(sA) + wave * kDenseTokens * kEpStride;
  const size_t orb = act_row_bytes(g.out_K);
  uint8_t* out = reinterpret_cast<uint8_t*>(g.out);
  const int c = lane & 31;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int m = 8 * (r >> 2) + 4 * half + (r & 3);
    ep[m * kEpStride + c] = swiglu_bf16(acc[0][r], acc[1][r], g.limit);
  }
  __builtin_amdgcn_wave_barrier();
  if (lane < T) {
    float v[32];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float4 f = *reinterpret_cast<const float4*>(ep + lane * kEpStride + 4 * q);
      v[4 * q] = f.x; v[4 * q + 1] = f.y; v[4 * q + 2] = f.z; v[4 * q + 3] = f.w;
    }
    store_fp6_block(out + ((size_t)e * T + lane) * orb, u, split_fp6x32(v));
  }
}

constexpr int kDenseP = 8;        // weight k-tiles in flight per wavefront

hipError_t launch_gemm_dense_gate_up(int T, int D, int I, int E, int k, float limit, const uint8_t* xpack,
                                     const uint8_t* codes, const uint8_t* scales, void* hpack,
                                     const DenseSelection* sel, hipStream_t s) {
  if (T == 0) return hipSuccess;
  DenseArgs g = {};
  g.T = T; g.k = k; g.E = E; g.limit = limit;
  g.K = D;
  g.KT = D / kKTile;
  g.KG = w_kgroups(D);
  g.units = I / kNTile;
  g.out_K = I;
  g.a = xpack;
  g.a_bytes = (uint32_t)((size_t)T * act_row_bytes(D));
  g.codes = codes; g.scales = scales;
  g.codes_per_expert = w_codes_per_expert(2 * I, D);
  g.scales_per_expert = w_scales_per_expert(2 * I, D);
  g.out = hpack;
  g.D = D;
  g.x = sel->x; g.wr = sel->wr; g.br = sel->br;
  g.sel_idx = sel->idx; g.sel_w = sel->w;
  const long long n = (long long)T * k;
  g.bm = tile_rows(n, E);
  g.slots = (int)tile_slots(n, E);
  g.counts = sel->counts; g.offsets = sel->offsets; g.perm = sel->perm; g.inv = sel->inv; g.tiles = sel->tiles;
  // workgroup 0: the selection; then the (expert, unit) pairs, 12 per workgroup
  const dim3 grid(1 + (E * g.units + kDenseWaves - 1) / kDenseWaves);
  if (g.KT == kDenseMaxKT) expert_gemm_dense_kernel<kDenseP, kDenseMaxKT><<<grid, dim3(kDenseThreads), 0, s>>>(g);
  else expert_gemm_dense_kernel<kDenseP, 0><<<grid, dim3(kDenseThreads), 0, s>>>(g);
  return hipGetLastError();
}

}  // namespace moe
