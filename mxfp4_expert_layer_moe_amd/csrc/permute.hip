// Grouping of the T*k (token, expert) assignments by expert.
//
// Only a subset of experts runs per token ("From GPT-2 to gpt-oss", section 4,
// Mixture of Experts: the MoE block is sparse), so the expert GEMMs work on the
// rows each expert received.  This kernel builds that grouping:
//   counts[e], offsets = exclusive prefix sum, perm (assignment ids grouped by
//   expert, ascending token within an expert) and its inverse.
// The result is unique and deterministic: positions come from counts and
// in-order ranks, never from the order in which atomics land.
//
// It also writes the row-tile table the expert GEMMs start from (expert, first
// row, row count and the assignment id of every row of each tile), so a GEMM
// workgroup learns everything about its rows with one load.
//
// One workgroup of 1024 threads walks the assignments in chunks of 1024 (each
// thread keeps its assignments in registers).  Within a wavefront, a thread's
// rank among equal experts comes from a ballot-based match (one ballot per
// expert-id bit); across wavefronts, per-(wave, expert) counts in LDS give the
// offsets.
#include "permute_body.h"

namespace moe {

__global__ __launch_bounds__(kPermThreads) void permute_kernel(int n, int E, int bm, int slots,
                                                               const int32_t* __restrict__ idx,
                                                               int32_t* __restrict__ counts,
                                                               int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ perm,
                                                               int32_t* __restrict__ inv,
                                                               int32_t* __restrict__ tiles) {
  permute_group(n, E, bm, slots, idx, counts, offsets, perm, inv, tiles);
}

hipError_t launch_permute(int T, int E, int k, const int32_t* idx, int32_t* counts, int32_t* offsets,
                          int32_t* perm, int32_t* inv, int32_t* tiles, hipStream_t s) {
  const int n = T * k;
  permute_kernel<<<dim3(1), dim3(kPermThreads), 0, s>>>(n, E, tile_rows(n, E), (int)tile_slots(n, E), idx, counts,
                                                        offsets, perm, inv, tiles);
  return hipGetLastError();
}

}  // namespace moe
