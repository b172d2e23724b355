// Grouping of the (token, expert) assignments by expert, executed by one
// workgroup of THREADS threads (see permute.hip for the method): the whole
// grouping of batches of up to 1024 assignments, in one launch.
#pragma once
#include "moe_internal.h"

namespace moe {

constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / 64;
constexpr int kPermRegs = 32;          // assignments held per thread per pass

template <int THREADS>
__device__ inline void permute_group(int n, int E, int bm, int slots,
                                     const int32_t* __restrict__ idx,
                                     int32_t* __restrict__ counts,
                                     int32_t* __restrict__ offsets,
                                     int32_t* __restrict__ perm,
                                     int32_t* __restrict__ inv,
                                     int32_t* __restrict__ tiles) {
  __shared__ int cnt[kMaxExperts];
  __shared__ int base[kMaxExperts];
  __shared__ int off0[kMaxExperts];
  __shared__ int tstart[kMaxExperts + 1];
  __shared__ int wcnt[(THREADS / 64)][kMaxExperts];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  const int ti = tile_ints(bm);

  for (int e = tid; e < E; e += THREADS) cnt[e] = 0;
  __syncthreads();

  // ---- histogram (integer LDS atomics: the totals do not depend on order) ----
  for (int a = tid; a < n; a += THREADS) {
    const int e = idx[a];
    if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();

  // ---- exclusive scan by wave 0 --------------------------------------------
  if (wave == 0) {
    int carry = 0;
    for (int c = 0; c < E; c += 64) {
      const int e = c + lane;
      const int v = e < E ? cnt[e] : 0;
      int incl = v;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(incl, d);
        if (lane >= d) incl += o;
      }
      if (e < E) {
        base[e] = carry + incl - v;
        off0[e] = carry + incl - v;
        counts[e] = v;
        offsets[e] = carry + incl - v;
      }
      carry += __shfl(incl, 63);
    }
    if (lane == 0) offsets[E] = carry;
    // first tile slot of every expert
    int tcarry = 0;
    for (int c = 0; c < E; c += 64) {
      const int e = c + lane;
      const int v = e < E ? (cnt[e] + bm - 1) / bm : 0;
      int incl = v;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(incl, d);
        if (lane >= d) incl += o;
      }
      if (e < E) tstart[e] = tcarry + incl - v;
      tcarry += __shfl(incl, 63);
    }
    if (lane == 0) tstart[E] = tcarry;
  }
  __syncthreads();
  // tile headers: slot s of expert e (binary search over tstart); slots past the last tile are
  // empty.  Every header's 4th field holds the number of tiles in use.
  for (int s = tid; s < slots; s += THREADS) {
    int4 h = make_int4(-1, 0, 0, tstart[E]);
    if (s < tstart[E]) {
      int lo = 0, hi = E - 1;                       // largest e with tstart[e] <= s
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (tstart[mid] <= s) lo = mid; else hi = mid - 1;
      }
      const int t = s - tstart[lo];
      h = make_int4(lo, off0[lo] + t * bm, min(bm, cnt[lo] - t * bm), tstart[E]);
    }
    *reinterpret_cast<int4*>(tiles + (size_t)s * ti) = h;
  }

  // ---- stable scatter, chunk by chunk --------------------------------------
  const int nchunks = (n + THREADS - 1) / THREADS;
  for (int c0 = 0; c0 < nchunks; c0 += kPermRegs) {
    int ev[kPermRegs];
#pragma unroll
    for (int r = 0; r < kPermRegs; ++r) {
      const int a = (c0 + r) * THREADS + tid;
      ev[r] = (c0 + r < nchunks && a < n) ? idx[a] : -1;
    }
#pragma unroll
    for (int r = 0; r < kPermRegs; ++r) {
      if (c0 + r >= nchunks) break;                      // uniform
      const int a = (c0 + r) * THREADS + tid;
      const int e = ev[r];
      const bool valid = (unsigned)e < (unsigned)E;
      // lanes holding the same expert: intersect ballots over the id bits
      uint64_t same = __ballot(valid);
#pragma unroll
      for (int bit = 0; bit < 8; ++bit) {
        const uint64_t b = __ballot(valid && ((e >> bit) & 1));
        same &= ((e >> bit) & 1) ? b : ~b;
      }
      const int rank = __popcll(same & lt_mask);
      for (int e2 = tid; e2 < (THREADS / 64) * kMaxExperts; e2 += THREADS) (&wcnt[0][0])[e2] = 0;
      __syncthreads();
      if (valid && rank == 0) wcnt[wave][e] = __popcll(same);
      __syncthreads();
      if (!valid && a < n) inv[a] = -1;                  // an id outside [0, E): no row
      if (valid) {
        int pos = base[e] + rank;
        for (int w = 0; w < wave; ++w) pos += wcnt[w][e];
        perm[pos] = a;
        inv[a] = pos;
        const int r = pos - off0[e];
        tiles[(size_t)(tstart[e] + r / bm) * ti + 4 + r % bm] = a;
      }
      __syncthreads();
      for (int e2 = tid; e2 < E; e2 += THREADS) {
        int s = 0;
        for (int w = 0; w < (THREADS / 64); ++w) s += wcnt[w][e2];
        base[e2] += s;
      }
      __syncthreads();
    }
  }
}

}  // namespace moe
