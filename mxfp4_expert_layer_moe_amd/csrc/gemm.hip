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
// Work decomposition: grid.y walks the 32-row tiles of every expert's rows
// (located from `offsets` on the device; slots past the last tile exit), and
// grid.x walks output units: a gate/up pair of 32-column tiles (stage 0) or
// one 32-column tile (stage 1), one unit per wavefront.  Weights stream from
// HBM once per (row tile, unit); a wavefront issues the loads of four k-tiles
// before their eight matrix instructions.
#include "moe_internal.h"

namespace moe {

struct GemmArgs {
  int T, k, E, K, KT, KG, units, out_K;
  float limit;
  const uint8_t* a_packed;
  const int32_t* perm;
  const int32_t* offsets;
  const uint8_t* codes;
  const uint8_t* scales;
  const float* topk_w;
  void* out;
  size_t codes_per_expert, scales_per_expert;
};

// Locate row tile `mt` among all experts' 32-row tiles.  Every lane gets the
// expert, the first grouped position and the number of valid rows (<= 32).
__device__ bool find_row_tile(const int32_t* __restrict__ offsets, int E, int mt, int& e_out, int& p0,
                              int& nrows) {
  const int lane = threadIdx.x & 63;
  int before = 0;
  for (int c = 0; c < E; c += 64) {
    const int e = c + lane;
    int off = 0, cnt = 0;
    if (e < E) { off = offsets[e]; cnt = offsets[e + 1] - off; }
    const int tiles = (cnt + kMTile - 1) / kMTile;
    int incl = tiles;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d);
      if (lane >= d) incl += o;
    }
    const int excl = incl - tiles;
    const bool mine = e < E && mt >= before + excl && mt < before + incl;
    const uint64_t m = __ballot(mine);
    if (m) {
      const int src = __ffsll((long long)m) - 1;
      e_out = c + src;
      const int lt = mt - before - __shfl(excl, src);
      p0 = __shfl(off, src) + lt * kMTile;
      nrows = min(kMTile, __shfl(cnt, src) - lt * kMTile);
      return true;
    }
    before += __shfl(incl, 63);
  }
  return false;
}

__device__ inline v8i load_a24(const uint8_t* p) {
  const uint2* q = reinterpret_cast<const uint2*>(p);
  const uint2 a = q[0], b = q[1], c = q[2];
  v8i v = {(int)a.x, (int)a.y, (int)b.x, (int)b.y, (int)c.x, (int)c.y, 0, 0};
  return v;
}

__device__ inline v8i load_b16(const uint8_t* p) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  v8i v = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  return v;
}

template <int NB>
struct KStep {
  v8i ahi, alo;
  v8i b[NB];
};

template <int NB>
__device__ inline void load_step(KStep<NB>& s, bool valid, const uint8_t* arow, size_t lo_off, int blk,
                                 const uint8_t* const* bptr, int kt) {
  if (valid) {
    s.ahi = load_a24(arow + (size_t)blk * 24);
    s.alo = load_a24(arow + lo_off + (size_t)blk * 24);
  } else {
    s.ahi = v8i{0, 0, 0, 0, 0, 0, 0, 0};
    s.alo = s.ahi;
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) s.b[nb] = load_b16(bptr[nb] + (size_t)kt * 1024);
}

template <int J, int NB>
__device__ inline void mma_step(v16f* acc, const KStep<NB>& s, uint32_t sah, uint32_t sal, const uint32_t* sb) {
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    acc[nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(s.ahi, s.b[nb], acc[nb], 2, 4, J, sah, J, sb[nb]);
    acc[nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(s.alo, s.b[nb], acc[nb], 2, 4, J, sal, J, sb[nb]);
  }
}

__device__ inline float half_max(float v) {
#pragma unroll
  for (int d = 1; d < 32; d <<= 1) v = fmaxf(v, __shfl_xor(v, d));
  return v;
}

template <int STAGE>
__global__ __launch_bounds__(256) void expert_gemm_kernel(GemmArgs g) {
  constexpr int NB = STAGE == 0 ? 2 : 1;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int u = blockIdx.x * 4 + wave;                  // output unit of this wavefront
  if (u >= g.units) return;
  int e, p0, nrows;
  if (!find_row_tile(g.offsets, g.E, blockIdx.y, e, p0, nrows)) return;

  const int i = lane & 31;
  const int half = lane >> 5;
  const bool valid = i < nrows;
  const size_t arb = act_row_bytes(g.K);
  const uint8_t* arow = g.a_packed;
  if (valid) {
    const size_t src = STAGE == 0 ? (size_t)(g.perm[p0 + i] / g.k) : (size_t)(p0 + i);
    arow = g.a_packed + src * arb;
  }
  const size_t lo_off = act_lo_codes_off(g.K);
  const size_t hs_off = act_hi_scales_off(g.K) + (size_t)half * act_ktp(g.K);
  const size_t ls_off = act_lo_scales_off(g.K) + (size_t)half * act_ktp(g.K);

  const uint8_t* bptr[NB];
  const uint8_t* sptr[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int q = STAGE == 0 ? 2 * u + nb : u;
    bptr[nb] = g.codes + (size_t)e * g.codes_per_expert + (size_t)q * g.KT * 1024 + (size_t)lane * 16;
    sptr[nb] = g.scales + (size_t)e * g.scales_per_expert + (size_t)q * g.KG * 256 + (size_t)lane * 4;
  }

  v16f acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = v16f{};

  for (int kg = 0; kg < g.KG; ++kg) {
    uint32_t sah = 0x7f7f7f7fu, sal = 0x7f7f7f7fu;
    if (valid) {
      sah = *reinterpret_cast<const uint32_t*>(arow + hs_off + 4 * kg);
      sal = *reinterpret_cast<const uint32_t*>(arow + ls_off + 4 * kg);
    }
    uint32_t sb[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) sb[nb] = *reinterpret_cast<const uint32_t*>(sptr[nb] + (size_t)kg * 256);
    const int kt0 = 4 * kg;
    if (kt0 + 3 < g.KT) {
      KStep<NB> s0, s1, s2, s3;
      load_step<NB>(s0, valid, arow, lo_off, 2 * (kt0 + 0) + half, bptr, kt0 + 0);
      load_step<NB>(s1, valid, arow, lo_off, 2 * (kt0 + 1) + half, bptr, kt0 + 1);
      load_step<NB>(s2, valid, arow, lo_off, 2 * (kt0 + 2) + half, bptr, kt0 + 2);
      load_step<NB>(s3, valid, arow, lo_off, 2 * (kt0 + 3) + half, bptr, kt0 + 3);
      mma_step<0, NB>(acc, s0, sah, sal, sb);
      mma_step<1, NB>(acc, s1, sah, sal, sb);
      mma_step<2, NB>(acc, s2, sah, sal, sb);
      mma_step<3, NB>(acc, s3, sah, sal, sb);
    } else {
      KStep<NB> s;
      load_step<NB>(s, valid, arow, lo_off, 2 * kt0 + half, bptr, kt0);
      mma_step<0, NB>(acc, s, sah, sal, sb);
      if (kt0 + 1 < g.KT) {
        load_step<NB>(s, valid, arow, lo_off, 2 * (kt0 + 1) + half, bptr, kt0 + 1);
        mma_step<1, NB>(acc, s, sah, sal, sb);
      }
      if (kt0 + 2 < g.KT) {
        load_step<NB>(s, valid, arow, lo_off, 2 * (kt0 + 2) + half, bptr, kt0 + 2);
        mma_step<2, NB>(acc, s, sah, sal, sb);
      }
    }
  }

  if (STAGE == 0) {
    // SwiGLU epilogue: h = bf16(silu(clamp(g)) * clamp(u)), written as hi/lo MX6 block u of row p
    const int I = g.out_K;
    const size_t orb = act_row_bytes(I);
    const int ktp = act_ktp(I);
    uint8_t* out = reinterpret_cast<uint8_t*>(g.out);
    const int c = lane & 31;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = 8 * (r >> 2) + 4 * half + (r & 3);
      const float gv = fminf(fmaxf(acc[0][r], -g.limit), g.limit);
      const float uv = fminf(fmaxf(acc[1][r], -g.limit), g.limit);
      const float h = bf16_round(gv / (1.0f + expf(-gv)) * uv);
      const uint32_t s_hi = e2m3_scale_byte(half_max(fabsf(h)));
      float d;
      const uint32_t c_hi = e2m3_encode(h, e8m0_to_inv(s_hi), e8m0_to_float(s_hi), &d);
      const float res = h - d;
      const uint32_t s_lo = e2m3_scale_byte(half_max(fabsf(res)));
      const uint32_t c_lo = e2m3_encode(res, e8m0_to_inv(s_lo), e8m0_to_float(s_lo), &d);
      uint32_t vh = c_hi << (6 * (c & 3));
      uint32_t vl = c_lo << (6 * (c & 3));
      vh |= __shfl_xor(vh, 1);
      vl |= __shfl_xor(vl, 1);
      vh |= __shfl_xor(vh, 2);
      vl |= __shfl_xor(vl, 2);
      if (m < nrows) {
        uint8_t* row = out + (size_t)(p0 + m) * orb;
        if ((c & 3) == 0) {
          uint8_t* ph = row + (size_t)u * 24 + 3 * (c >> 2);
          uint8_t* pl = row + act_lo_codes_off(I) + (size_t)u * 24 + 3 * (c >> 2);
          ph[0] = (uint8_t)vh; ph[1] = (uint8_t)(vh >> 8); ph[2] = (uint8_t)(vh >> 16);
          pl[0] = (uint8_t)vl; pl[1] = (uint8_t)(vl >> 8); pl[2] = (uint8_t)(vl >> 16);
        }
        if (c == 0) {
          row[act_hi_scales_off(I) + (size_t)(u & 1) * ktp + (u >> 1)] = (uint8_t)s_hi;
          row[act_lo_scales_off(I) + (size_t)(u & 1) * ktp + (u >> 1)] = (uint8_t)s_lo;
        }
      }
    }
  } else {
    // down epilogue: scale row p by its gate weight topk_w[perm[p]], store fp32
    const int D = g.units * kNTile;
    float wl = 0.0f;
    if (valid) wl = g.topk_w[g.perm[p0 + i]];
    float* out = reinterpret_cast<float*>(g.out);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = 8 * (r >> 2) + 4 * half + (r & 3);
      const float wm = __shfl(wl, m);
      if (m < nrows) out[(size_t)(p0 + m) * D + (size_t)u * kNTile + (lane & 31)] = acc[0][r] * wm;
    }
  }
}

hipError_t launch_gemm(int stage, int T, int D, int I, int E, int k, float limit, const uint8_t* a_packed,
                       const int32_t* perm, const int32_t* offsets, const uint8_t* codes, const uint8_t* scales,
                       const float* topk_w, void* out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  GemmArgs g;
  g.T = T; g.k = k; g.E = E; g.limit = limit;
  g.a_packed = a_packed; g.perm = perm; g.offsets = offsets; g.codes = codes; g.scales = scales;
  g.topk_w = topk_w; g.out = out;
  const int N = stage == 0 ? 2 * I : D;
  g.K = stage == 0 ? D : I;
  g.KT = g.K / kKTile;
  g.KG = w_kgroups(g.K);
  g.units = stage == 0 ? I / kNTile : D / kNTile;
  g.out_K = stage == 0 ? I : D;
  g.codes_per_expert = w_codes_per_expert(N, g.K);
  g.scales_per_expert = w_scales_per_expert(N, g.K);
  const long long n_assign = (long long)T * k;
  const unsigned tiles_y = (unsigned)((n_assign + kMTile - 1) / kMTile + (E < n_assign ? E : n_assign));
  const dim3 grid((g.units + 3) / 4, tiles_y);
  if (stage == 0)
    expert_gemm_kernel<0><<<grid, dim3(256), 0, s>>>(g);
  else
    expert_gemm_kernel<1><<<grid, dim3(256), 0, s>>>(g);
  return hipGetLastError();
}

}  // namespace moe
