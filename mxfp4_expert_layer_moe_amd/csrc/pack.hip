// Activation split: bf16 rows -> packed hi/lo FP6 E2M3 terms with E8M0 block scales.
//
// The gfx950 scaled matrix-core instruction takes its operands in FP8/FP6/FP4
// with one E8M0 scale per 32 values along K; it has no bf16 input.  A bf16
// activation row is therefore written as the sum of two MX terms: hi is the
// row's 32-blocks rounded to E2M3 under the OCP shared-exponent rule, lo the
// same encoding of what hi left over.  Both terms run at the FP4 x FP6 issue
// rate, so the expert GEMMs run two MFMAs per weight tile instead of one.
//
// One lane per 32-value block: the lane loads its 64 bytes, finds the block
// maxima itself and encodes the 32 values of each term with one packed
// conversion instruction (split_fp6x32).
//
// The activation-quantized variant instead quantizes each block to MXFP4 with
// the OCP conversion (quant_fp4x32): one FP4 x FP4 instruction per weight tile.
#include "mfma_ops.h"

namespace moe {

__global__ __launch_bounds__(256) void pack_act_kernel(int K, long long nblocks, const uint16_t* __restrict__ a,
                                                       uint8_t* __restrict__ packed, int af) {
  pack_block_lane(a, K, nblocks, (long long)blockIdx.x * blockDim.x + threadIdx.x, packed, af);
}

hipError_t launch_pack(int K, int rows, const uint16_t* a, uint8_t* packed, hipStream_t s, int af) {
  const long long n = (long long)rows * (K / kBlock);          // blocks = threads
  if (n == 0) return hipSuccess;
  const int threads = 256;
  const long long blocks = (n + threads - 1) / threads;
  pack_act_kernel<<<dim3((unsigned)blocks), dim3(threads), 0, s>>>(K, n, a, packed, af);
  return hipGetLastError();
}

}  // namespace moe
