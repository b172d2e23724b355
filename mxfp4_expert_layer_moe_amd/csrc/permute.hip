// Grouping of the T*k (token, expert) assignments by expert.
//
// Only a subset of experts runs per token ("From GPT-2 to gpt-oss", section 4,
// Mixture of Experts: the MoE block is sparse), so the expert GEMMs work on the
// rows each expert received.  This builds that grouping:
//   counts[e], offsets = exclusive prefix sum, perm (assignment ids grouped by
//   expert, ascending token within an expert) and its inverse.
// The result is unique and deterministic: positions come from counts and
// in-order ranks, never from the order in which atomics land.
//
// It also writes the row-tile table the expert GEMMs start from (expert, first
// row, row count and the assignment id of every row of each tile), so a GEMM
// workgroup learns everything about its rows with one load.
//
// Batches of up to 1024 assignments: one workgroup does everything
// (permute_body.h; 256 threads up to 256 assignments, else 1024).  Larger batches: three kernels over workgroups of 1024
// consecutive assignments.
//   1. count: each workgroup's expert histogram (LDS atomics, order-free);
//   2. scan: one workgroup turns the histograms into each workgroup's first
//      position per expert (exclusive over workgroups), the expert offsets and
//      the tile headers;
//   3. scatter: each assignment's position = its workgroup's base for its
//      expert + its rank among the workgroup's assignments of that expert
//      (a ballot match inside a wavefront, per-wavefront counts across them).
// The per-workgroup counts and the expert tile starts live in the scratch tail
// of the tile buffer.
// An expert id outside [0, E) (a caller error) gets no row: it is left out of
// counts, perm and the tiles, and its inv entry is -1, which the combine skips.
#include "permute_body.h"

namespace moe {

template <int THREADS>
__global__ __launch_bounds__(THREADS) void permute_kernel(int n, int E, int bm, int slots,
                                                         const int32_t* __restrict__ idx,
                                                         int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ perm,
                                                         int32_t* __restrict__ inv,
                                                         int32_t* __restrict__ tiles) {
  permute_group<THREADS>(n, E, bm, slots, idx, counts, offsets, perm, inv, tiles);
}

__global__ __launch_bounds__(kPermThreads) void perm_count_kernel(int n, int E, const int32_t* __restrict__ idx,
                                                                  int32_t* __restrict__ hist) {
  __shared__ int cnt[kMaxExperts];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kPermThreads) cnt[e] = 0;
  __syncthreads();
  const long long a = (long long)blockIdx.x * kPermChunk + tid;
  if (a < n) {
    const int e = idx[a];
    if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  for (int e = tid; e < E; e += kPermThreads) hist[(size_t)blockIdx.x * E + e] = cnt[e];
}

// hist[g][e] -> exclusive prefix over g (per expert); totals -> counts, offsets, tile starts, headers
__global__ __launch_bounds__(kPermThreads) void perm_scan_kernel(int n, int E, int G, int bm, int slots,
                                                                 int32_t* __restrict__ hist,
                                                                 int32_t* __restrict__ tstart_out,
                                                                 int32_t* __restrict__ counts,
                                                                 int32_t* __restrict__ offsets,
                                                                 int32_t* __restrict__ tiles) {
  __shared__ int cnt[kMaxExperts];
  __shared__ int off0[kMaxExperts];
  __shared__ int tstart[kMaxExperts + 1];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  for (int e = tid; e < E; e += kPermThreads) {
    int run = 0;
    for (int g0 = 0; g0 < G; g0 += 8) {                 // eight independent loads per round trip
      int v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = g0 + i < G ? hist[(size_t)(g0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (g0 + i < G) hist[(size_t)(g0 + i) * E + e] = run;
        run += v[i];
      }
    }
    cnt[e] = run;
  }
  __syncthreads();
  if (wave == 0) {
    int carry = 0, tcarry = 0;
    for (int c = 0; c < E; c += 64) {
      const int e = c + lane;
      const int v = e < E ? cnt[e] : 0;
      const int tv = e < E ? (v + bm - 1) / bm : 0;
      int incl = v, tincl = tv;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(incl, d), to = __shfl_up(tincl, d);
        if (lane >= d) {
          incl += o;
          tincl += to;
        }
      }
      if (e < E) {
        off0[e] = carry + incl - v;
        counts[e] = v;
        offsets[e] = carry + incl - v;
        tstart[e] = tcarry + tincl - tv;
      }
      carry += __shfl(incl, 63);
      tcarry += __shfl(tincl, 63);
    }
    if (lane == 0) {
      offsets[E] = carry;
      tstart[E] = tcarry;
    }
  }
  __syncthreads();
  for (int e = tid; e <= E; e += kPermThreads) tstart_out[e] = tstart[e];
  const int ti = tile_ints(bm);
  for (int s = tid; s < slots; s += kPermThreads) {
    int4 h = make_int4(-1, 0, 0, tstart[E]);
    if (s < tstart[E]) {
      int lo = 0, hi = E - 1;                           // largest e with tstart[e] <= s
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (tstart[mid] <= s) lo = mid; else hi = mid - 1;
      }
      const int t = s - tstart[lo];
      h = make_int4(lo, off0[lo] + t * bm, min(bm, cnt[lo] - t * bm), tstart[E]);
    }
    *reinterpret_cast<int4*>(tiles + (size_t)s * ti) = h;
  }
}

__global__ __launch_bounds__(kPermThreads) void perm_scatter_kernel(int n, int E, int bm,
                                                                    const int32_t* __restrict__ idx,
                                                                    const int32_t* __restrict__ base,
                                                                    const int32_t* __restrict__ tstart,
                                                                    const int32_t* __restrict__ offsets,
                                                                    int32_t* __restrict__ perm,
                                                                    int32_t* __restrict__ inv,
                                                                    int32_t* __restrict__ tiles) {
  __shared__ int wcnt[kPermWaves][kMaxExperts];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  for (int i = tid; i < kPermWaves * E; i += kPermThreads) wcnt[i / E][i % E] = 0;
  const long long a = (long long)blockIdx.x * kPermChunk + tid;
  const int e = a < n ? idx[a] : -1;
  const bool valid = (unsigned)e < (unsigned)E;
  // lanes holding the same expert: intersect ballots over the id bits (E <= 256)
  uint64_t same = __ballot(valid);
#pragma unroll
  for (int bit = 0; bit < 8; ++bit) {
    const uint64_t b = __ballot(valid && ((e >> bit) & 1));
    same &= ((e >> bit) & 1) ? b : ~b;
  }
  const int rank = __popcll(same & ((1ull << lane) - 1ull));
  __syncthreads();
  if (valid && rank == 0) wcnt[wave][e] = __popcll(same);
  __syncthreads();
  if (!valid) {
    if (a < n) inv[a] = -1;                             // an id outside [0, E): no row
    return;
  }
  int pos = offsets[e] + base[(size_t)blockIdx.x * E + e] + rank;
  for (int w = 0; w < wave; ++w) pos += wcnt[w][e];
  perm[pos] = (int32_t)a;
  inv[a] = pos;
  const int r = pos - offsets[e];
  tiles[(size_t)(tstart[e] + r / bm) * tile_ints(bm) + 4 + r % bm] = (int32_t)a;
}

hipError_t launch_permute(int T, int E, int k, const int32_t* idx, int32_t* counts, int32_t* offsets,
                          int32_t* perm, int32_t* inv, int32_t* tiles, hipStream_t s) {
  const long long n = (long long)T * k;
  const int bm = tile_rows(n, E);
  const int slots = (int)tile_slots(n, E);
  if (n <= 256) {
    permute_kernel<256><<<dim3(1), dim3(256), 0, s>>>((int)n, E, bm, slots, idx, counts, offsets, perm, inv, tiles);
    return hipGetLastError();
  }
  if (n <= kPermChunk) {
    permute_kernel<kPermThreads><<<dim3(1), dim3(kPermThreads), 0, s>>>((int)n, E, bm, slots, idx, counts, offsets,
                                                                        perm, inv, tiles);
    return hipGetLastError();
  }
  const int G = (int)perm_groups(n);
  int32_t* hist = tiles + tile_table_ints(n, E);
  int32_t* tstart = hist + (size_t)G * E;
  perm_count_kernel<<<dim3(G), dim3(kPermThreads), 0, s>>>((int)n, E, idx, hist);
  perm_scan_kernel<<<dim3(1), dim3(kPermThreads), 0, s>>>((int)n, E, G, bm, slots, hist, tstart, counts, offsets,
                                                          tiles);
  perm_scatter_kernel<<<dim3(G), dim3(kPermThreads), 0, s>>>((int)n, E, bm, idx, hist, tstart, offsets, perm, inv,
                                                             tiles);
  return hipGetLastError();
}

// ---- the row-tile table from a grouping given as offsets and perm ----------------------------
// Every workgroup takes the tile counts per expert, ceil((offsets[e+1] - offsets[e]) / bm), and
// their exclusive scan (the first slot of each expert) in LDS; workgroup 0 writes the slot
// headers, and every workgroup writes the assignment ids of its share of the grouped positions
// (grouped position p of expert e is row (p - offsets[e]) % bm of tile (p - offsets[e]) / bm).
// The result equals the table launch_permute writes for the same grouping.
constexpr int kTileFromThreads = 256;              // one thread per expert (E <= 256)
__global__ __launch_bounds__(kTileFromThreads) void tiles_from_groups_kernel(int E, int bm, int slots,
                                                                             const int32_t* __restrict__ offsets,
                                                                             const int32_t* __restrict__ perm,
                                                                             int32_t* __restrict__ tiles) {
  __shared__ int soff[kTileFromThreads + 1];
  __shared__ int sfirst[kTileFromThreads];
  const int tid = threadIdx.x;
  for (int e = tid; e <= E; e += kTileFromThreads) soff[e] = offsets[e];
  __syncthreads();
  const int cnt = tid < E ? soff[tid + 1] - soff[tid] : 0;
  const int ntl = (cnt + bm - 1) / bm;
  // inclusive scan of ntl over the experts (Hillis-Steele in LDS)
  sfirst[tid] = ntl;
  __syncthreads();
  for (int d = 1; d < kTileFromThreads; d <<= 1) {
    const int v = tid >= d ? sfirst[tid - d] : 0;
    __syncthreads();
    sfirst[tid] += v;
    __syncthreads();
  }
  const int used = sfirst[kTileFromThreads - 1];
  const int first = sfirst[tid] - ntl;              // exclusive
  __syncthreads();
  sfirst[tid] = first;
  __syncthreads();
  const int ints = tile_ints(bm);
  if (blockIdx.x == 0) {
    for (int i = 0; i < ntl && first + i < slots; ++i)
      *reinterpret_cast<int4*>(tiles + (size_t)(first + i) * ints) =
          make_int4(tid, soff[tid] + i * bm, min(bm, cnt - i * bm), used);
    for (int sl = used + tid; sl < slots; sl += kTileFromThreads)
      *reinterpret_cast<int4*>(tiles + (size_t)sl * ints) = make_int4(-1, 0, 0, used);
  }
  const int n = soff[E];
  for (int p = blockIdx.x * kTileFromThreads + tid; p < n; p += gridDim.x * kTileFromThreads) {
    int lo = 0, hi = E;                               // the last e with soff[e] <= p
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (soff[mid] <= p) lo = mid;
      else hi = mid;
    }
    const int q = p - soff[lo];
    const int slot = sfirst[lo] + q / bm;
    if (slot < slots) tiles[(size_t)slot * ints + 4 + q % bm] = perm[p];
  }
}

hipError_t launch_tiles_from_groups(int T, int E, int k, const int32_t* offsets, const int32_t* perm,
                                    int32_t* tiles, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (E > kTileFromThreads) return hipErrorInvalidValue;
  const long long n = (long long)T * k;
  const int bm = tile_rows(n, E);
  const long long slots = tile_slots(n, E);
  const long long wgs = (n + kTileFromThreads - 1) / kTileFromThreads;
  tiles_from_groups_kernel<<<dim3((unsigned)(wgs < 1024 ? wgs : 1024)), dim3(kTileFromThreads), 0, s>>>(
      E, bm, (int)slots, offsets, perm, tiles);
  return hipGetLastError();
}

}  // namespace moe
