// C ABI of the MoE layer: argument validation, workspace layout, launch order,
// and the host-side MXFP4 quantizer and weight prepack.
#include <math.h>
#include <string.h>

#include <mutex>

#include "../../include/moe_mxfp4.h"
#include "moe_internal.h"

using namespace moe;

namespace {

constexpr size_t kAlignWs = 256;

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

moe_status check_dims(const moe_dims* d) {
  if (!d) return MOE_EINVAL;
  if (d->d_model <= 0 || d->d_ff <= 0 || d->n_experts <= 0 || d->top_k <= 0) return MOE_EINVAL;
  if (!(d->swiglu_limit > 0.0f) || !isfinite(d->swiglu_limit)) return MOE_EINVAL;
  if (d->d_model % kKTile || d->d_ff % kKTile) return MOE_EUNSUPPORTED;
  if (d->top_k > d->n_experts || d->n_experts > kMaxExperts) return MOE_EUNSUPPORTED;
  // one expert's weights are addressed with 32-bit buffer offsets
  if ((int64_t)d->d_model * d->d_ff >= (int64_t)1 << 32) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

moe_status check_T(const moe_dims* d, int32_t T) {
  if (T < 0) return MOE_EINVAL;
  if ((int64_t)T * d->top_k >= (1 << 24)) return MOE_EUNSUPPORTED;
  // packed activation rows (x and h) are addressed with 32-bit buffer offsets
  const int kmax = d->d_model > d->d_ff ? d->d_model : d->d_ff;
  if ((int64_t)T * d->top_k * (int64_t)act_row_bytes(kmax) >= (int64_t)1 << 32) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

struct WsLayout {
  size_t idx, w, counts, offsets, perm, inv, tiles, xpack, hpack, yperm, route, total;
};

size_t tile_table_bytes(const moe_dims* d, int32_t T) {
  const long long n = (long long)T * d->top_k;
  return (size_t)(tile_buffer_ints(n, d->n_experts) + 3) / 4 * 16;
}

WsLayout ws_layout(const moe_dims* d, int32_t T, int af = kActSplit6) {
  WsLayout L;
  const size_t n = (size_t)T * d->top_k;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = round_up(o + bytes, kAlignWs); return at; };
  L.idx = take(n * 4);
  L.w = take(n * 4);
  L.counts = take((size_t)d->n_experts * 4);
  L.offsets = take(((size_t)d->n_experts + 1) * 4);
  L.perm = take(n * 4);
  L.inv = take(n * 4);
  L.tiles = take(tile_table_bytes(d, T));
  L.xpack = take((size_t)T * act_row_bytes_af(af, d->d_model));
  // the dense decode path writes h for every (expert, token) pair
  const size_t hrows = af == kActSplit6 && dense_decode(T, d->n_experts, d->top_k, d->d_model)
                           ? (n > (size_t)T * d->n_experts ? n : (size_t)T * d->n_experts) : n;
  L.hpack = take(hrows * act_row_bytes_af(af, d->d_ff));
  L.yperm = take(n * (size_t)d->d_model * 2);
  L.route = take(route_workspace_bytes(T, d->d_model, d->n_experts));
  L.total = o;
  return L;
}

// the whole-layer arguments other than the workspace
moe_status check_layer_args(const moe_dims* d, int32_t T, const void* x_bf16, const float* w_router,
                            const float* b_router, const moe_weights* wts, const void* y, moe_dtype y_dtype) {
  moe_status st = check_dims(d);
  if (st != MOE_OK) return st;
  if ((st = check_T(d, T)) != MOE_OK) return st;
  if (y_dtype != MOE_BF16 && y_dtype != MOE_FP32) return MOE_EINVAL;
  if (!x_bf16 || !w_router || !b_router || !wts || !y) return MOE_EINVAL;
  if (!wts->gu_codes || !wts->gu_scales || !wts->dn_codes || !wts->dn_scales) return MOE_EINVAL;
  if (!aligned(x_bf16, 16) || !aligned(w_router, 16) || !aligned(b_router, 4) || !aligned(y, 16) ||
      !aligned(wts->gu_codes, 16) || !aligned(wts->dn_codes, 16) || !aligned(wts->gu_scales, 4) ||
      !aligned(wts->dn_scales, 4))
    return MOE_EINVAL;
  return MOE_OK;
}

moe_status check_forward(const moe_dims* d, int32_t T, const void* x_bf16, const float* w_router,
                         const float* b_router, const moe_weights* wts, const void* y, moe_dtype y_dtype,
                         const void* ws) {
  const moe_status st = check_layer_args(d, T, x_bf16, w_router, b_router, wts, y, y_dtype);
  if (st != MOE_OK) return st;
  if (!ws || !aligned(ws, kAlignWs)) return MOE_EINVAL;
  return MOE_OK;
}

// normalised rows of the block forward, at the start of its workspace
size_t block_xn_bytes(const moe_dims* d, int32_t T) {
  return round_up((size_t)T * d->d_model * 2, kAlignWs);
}

// The layer on activations x (already validated; ws holds ws_layout(d, T).total bytes); with a
// residual, the combine adds it to the output.
moe_status forward_impl(const moe_dims* d, int32_t T, const uint16_t* x, const uint16_t* residual,
                        const float* w_router, const float* b_router, const moe_weights* wts, void* y,
                        moe_dtype y_dtype, uint8_t* base, hipStream_t stream, int af = kActSplit6,
                        const FrontNorm* fn = nullptr) {
  const WsLayout L = ws_layout(d, T, af);
  int32_t* idx = (int32_t*)(base + L.idx);
  float* w = (float*)(base + L.w);
  int32_t* counts = (int32_t*)(base + L.counts);
  int32_t* offsets = (int32_t*)(base + L.offsets);
  int32_t* perm = (int32_t*)(base + L.perm);
  int32_t* inv = (int32_t*)(base + L.inv);
  int32_t* tiles = (int32_t*)(base + L.tiles);
  uint8_t* xpack = base + L.xpack;
  uint8_t* hpack = base + L.hpack;
  _Float16* yperm = (_Float16*)(base + L.yperm);
  const int D = d->d_model, I = d->d_ff, E = d->n_experts, k = d->top_k;
  if (fn && !(af == kActSplit6 && dense_decode(T, E, k, D))) {
    // the normalisation as a launch of its own, into x
    if (launch_rmsnorm(T, D, fn->raw, fn->gamma, (float)fn->eps, const_cast<uint16_t*>(x), stream)) return MOE_EHIP;
    fn = nullptr;
  }
  if (af == kActSplit6 && dense_decode(T, E, k, D)) {
    // routing off the weight stream: the packed rows, then the dense gate/up with the scores and
    // the selection beside it, then the down projection of each expert's selected tokens (rows at
    // t*k + j)
    DenseSelection sel = {x, w_router, b_router, idx, w, counts, offsets, perm, inv, tiles};
    if (launch_front_pack(T, D, x, xpack, kActSplit6, stream, fn)) return MOE_EHIP;
    if (launch_gemm_dense_gate_up(T, D, I, E, k, d->swiglu_limit, xpack, wts->gu_codes, wts->gu_scales, hpack, &sel,
                                  stream))
      return MOE_EHIP;
    // the routed down projection, reading packed h row e*T + t for each tile row
    if (launch_gemm(1, T, D, I, E, k, d->swiglu_limit, hpack, tiles, wts->dn_codes, wts->dn_scales, w, yperm, stream,
                    kActSplit6, /*out_assign=*/1, /*dense_rows=*/1))
      return MOE_EHIP;
    if (launch_combine(T, D, k, yperm, nullptr, residual, y, y_dtype == MOE_BF16, stream)) return MOE_EHIP;
    return MOE_OK;
  }
  if (launch_route_front(T, D, E, k, x, w_router, b_router, idx, w, base + L.route, xpack, counts, offsets, perm,
                         inv, tiles, stream, af, fn))
    return MOE_EHIP;
  if (launch_gemm(0, T, D, I, E, k, d->swiglu_limit, xpack, tiles, wts->gu_codes, wts->gu_scales, nullptr, hpack,
                  stream, af))
    return MOE_EHIP;
  // the down projection writes each row at its assignment index t*k + j, so the combine reads a
  // token's rows directly (same values and sums as the step-by-step entry points)
  if (launch_gemm(1, T, D, I, E, k, d->swiglu_limit, hpack, tiles, wts->dn_codes, wts->dn_scales, w, yperm, stream,
                  af, 1))
    return MOE_EHIP;
  if (launch_combine(T, D, k, yperm, nullptr, residual, y, y_dtype == MOE_BF16, stream)) return MOE_EHIP;
  return MOE_OK;
}

}  // namespace

// ---- the whole layer with no allocation ------------------------------------------------------
// For callers that cannot allocate (code under HIP graph capture, tight serving loops, harnesses
// that forbid it): moe_forward's scratch lives in this file-scope device array instead of a
// workspace argument.  Each GPU holds its own copy, at its own address, until the process ends.
// Host code never passes the array's name to a kernel (on the host it is only a stand-in for the
// symbol): the device address comes from hipGetSymbolAddress, looked up once per device with
// that device current, and kept in scratch_ptr.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];
static_assert(kNoAllocScratchBytes % 256 == 0, "scratch regions are 256-byte aligned");
static_assert(kNoAllocScratchBytes == MOE_FORWARD_NOALLOC_MAX_WORKSPACE, "the header states the limit");

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
uint8_t* scratch_ptr[kMaxDevices];

// The device address of the current device's scratch array (looked up on the first call per device).
moe_status scratch_of_current_device(hipStream_t stream, uint8_t** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_EHIP;
  if (stream) {                          // the stream must run on the current device
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return MOE_EHIP;
    if (sdev != dev) return MOE_EINVAL;
  }
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_EHIP;
    scratch_ptr[dev] = (uint8_t*)p;
  }
  *out = scratch_ptr[dev];
  return MOE_OK;
}
}  // namespace

extern "C" {

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_EINVAL: return "MOE_EINVAL: invalid argument";
    case MOE_EUNSUPPORTED: return "MOE_EUNSUPPORTED: unsupported shape";
    case MOE_EWORKSPACE: return "MOE_EWORKSPACE: workspace too small";
    case MOE_EHIP: return "MOE_EHIP: HIP launch or runtime error";
  }
  return "unknown moe_status";
}

size_t moe_act_pack_bytes(int32_t K, int32_t rows) {
  if (K <= 0 || K % kKTile || rows < 0) return 0;
  return (size_t)rows * act_row_bytes(K);
}

size_t moe_prepacked_codes_bytes(const moe_dims* d, moe_stage stage) {
  if (check_dims(d) != MOE_OK) return 0;
  const int N = stage == MOE_STAGE_GATE_UP ? 2 * d->d_ff : d->d_model;
  const int K = stage == MOE_STAGE_GATE_UP ? d->d_model : d->d_ff;
  return (size_t)d->n_experts * w_codes_per_expert(N, K);
}

size_t moe_prepacked_scales_bytes(const moe_dims* d, moe_stage stage) {
  if (check_dims(d) != MOE_OK) return 0;
  const int N = stage == MOE_STAGE_GATE_UP ? 2 * d->d_ff : d->d_model;
  const int K = stage == MOE_STAGE_GATE_UP ? d->d_model : d->d_ff;
  return (size_t)d->n_experts * w_scales_per_expert(N, K);
}

size_t moe_workspace_bytes(const moe_dims* d, int32_t T) {
  if (check_dims(d) != MOE_OK || check_T(d, T) != MOE_OK) return 0;
  return ws_layout(d, T).total;
}

size_t moe_route_workspace_bytes(const moe_dims* d, int32_t T) {
  if (check_dims(d) != MOE_OK || check_T(d, T) != MOE_OK) return 0;
  return route_workspace_bytes(T, d->d_model, d->n_experts);
}

moe_status moe_route(const moe_dims* d, int32_t T, const void* x_bf16, const float* w_router,
                     const float* b_router, int32_t* topk_idx, float* topk_w, float* logits, void* ws,
                     size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_dims(d);
  if (st != MOE_OK) return st;
  if ((st = check_T(d, T)) != MOE_OK) return st;
  const size_t need = route_workspace_bytes(T, d->d_model, d->n_experts);
  if (!x_bf16 || !w_router || !b_router || !topk_idx || !topk_w || (need > 0 && !ws)) return MOE_EINVAL;
  if (!aligned(x_bf16, 16) || !aligned(w_router, 16) || !aligned(b_router, 4) || !aligned(topk_idx, 4) ||
      !aligned(topk_w, 4) || (logits && !aligned(logits, 4)) || !aligned(ws, kAlignWs))
    return MOE_EINVAL;
  if (ws_bytes < need) return MOE_EWORKSPACE;
  if (T == 0) return MOE_OK;
  return hip_status(launch_route(T, d->d_model, d->n_experts, d->top_k, (const uint16_t*)x_bf16, w_router,
                                 b_router, topk_idx, topk_w, logits, ws, stream));
}

size_t moe_tile_table_bytes(const moe_dims* d, int32_t T) {
  if (check_dims(d) != MOE_OK || check_T(d, T) != MOE_OK) return 0;
  return tile_table_bytes(d, T);
}

moe_status moe_permute_tiles(const moe_dims* d, int32_t T, const int32_t* topk_idx, int32_t* counts,
                             int32_t* offsets, int32_t* perm, int32_t* inv, int32_t* tiles, hipStream_t stream) {
  moe_status st = check_dims(d);
  if (st != MOE_OK) return st;
  if ((st = check_T(d, T)) != MOE_OK) return st;
  if (!topk_idx || !counts || !offsets || !perm || !inv || !tiles) return MOE_EINVAL;
  if (!aligned(topk_idx, 4) || !aligned(counts, 4) || !aligned(offsets, 4) || !aligned(perm, 4) ||
      !aligned(inv, 4) || !aligned(tiles, 16))
    return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  return hip_status(launch_permute(T, d->n_experts, d->top_k, topk_idx, counts, offsets, perm, inv, tiles, stream));
}

moe_status moe_pack_act(int32_t K, int32_t rows, const void* a_bf16, void* a_packed, hipStream_t stream) {
  if (K <= 0 || rows < 0) return MOE_EINVAL;
  if (K % kKTile) return MOE_EUNSUPPORTED;
  if (!a_bf16 || !a_packed || !aligned(a_bf16, 16) || !aligned(a_packed, 16)) return MOE_EINVAL;
  if (rows == 0) return MOE_OK;
  return hip_status(launch_pack(K, rows, (const uint16_t*)a_bf16, (uint8_t*)a_packed, stream));
}

size_t moe_act4_pack_bytes(int32_t K, int32_t rows) {
  if (K <= 0 || K % kKTile || rows < 0) return 0;
  return (size_t)rows * act4_row_bytes(K);
}

moe_status moe_pack_act4(int32_t K, int32_t rows, const void* a_bf16, void* a_packed4, hipStream_t stream) {
  if (K <= 0 || rows < 0) return MOE_EINVAL;
  if (K % kKTile) return MOE_EUNSUPPORTED;
  if (!a_bf16 || !a_packed4 || !aligned(a_bf16, 16) || !aligned(a_packed4, 16)) return MOE_EINVAL;
  if (rows == 0) return MOE_OK;
  return hip_status(launch_pack(K, rows, (const uint16_t*)a_bf16, (uint8_t*)a_packed4, stream, kActFp4));
}

static moe_status expert_gemm(const moe_dims* d, int32_t T, moe_stage stage, const void* a_packed,
                              const int32_t* tiles, const uint8_t* codes, const uint8_t* scales,
                              const float* topk_w, void* out, hipStream_t stream, int af) {
  moe_status st = check_dims(d);
  if (st != MOE_OK) return st;
  if ((st = check_T(d, T)) != MOE_OK) return st;
  if (stage != MOE_STAGE_GATE_UP && stage != MOE_STAGE_DOWN) return MOE_EINVAL;
  if (!a_packed || !tiles || !codes || !scales || !out) return MOE_EINVAL;
  if (stage == MOE_STAGE_DOWN && !topk_w) return MOE_EINVAL;
  if (!aligned(a_packed, 16) || !aligned(codes, 16) || !aligned(scales, 4) || !aligned(out, 16) ||
      !aligned(tiles, 16) || (topk_w && !aligned(topk_w, 4)))
    return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  return hip_status(launch_gemm(stage == MOE_STAGE_GATE_UP ? 0 : 1, T, d->d_model, d->d_ff, d->n_experts,
                                d->top_k, d->swiglu_limit, (const uint8_t*)a_packed, tiles, codes, scales, topk_w,
                                out, stream, af));
}

moe_status moe_expert_gemm_mxfp4_packed(const moe_dims* d, int32_t T, moe_stage stage, const void* a_packed,
                                        const int32_t* tiles, const uint8_t* codes, const uint8_t* scales,
                                        const float* topk_w, void* out, hipStream_t stream) {
  return expert_gemm(d, T, stage, a_packed, tiles, codes, scales, topk_w, out, stream, kActSplit6);
}

// ---- the plain boundary: bf16 rows, perm and offsets, scratch from ws -----------------------

size_t moe_permute_workspace_bytes(const moe_dims* d, int32_t T) {
  if (check_dims(d) != MOE_OK || check_T(d, T) != MOE_OK) return 0;
  return tile_table_bytes(d, T);
}

moe_status moe_permute(const moe_dims* d, int32_t T, const int32_t* topk_idx, int32_t* counts, int32_t* offsets,
                       int32_t* perm, int32_t* inv, void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_dims(d);
  if (st != MOE_OK) return st;
  if ((st = check_T(d, T)) != MOE_OK) return st;
  if (!topk_idx || !counts || !offsets || !perm || !inv) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  if (!ws || !aligned(ws, kAlignWs)) return MOE_EINVAL;
  if (ws_bytes < tile_table_bytes(d, T)) return MOE_EWORKSPACE;
  return moe_permute_tiles(d, T, topk_idx, counts, offsets, perm, inv, (int32_t*)ws, stream);
}

// the plain expert GEMM's scratch: the row-tile table, then the packed activation rows
static size_t gemm_ws_packed_at(const moe_dims* d, int32_t T) { return round_up(tile_table_bytes(d, T), kAlignWs); }
static size_t gemm_ws_bytes(const moe_dims* d, int32_t T, moe_stage stage) {
  if (T == 0) return 0;
  const size_t rows = stage == MOE_STAGE_GATE_UP ? (size_t)T : (size_t)T * d->top_k;
  const int K = stage == MOE_STAGE_GATE_UP ? d->d_model : d->d_ff;
  return gemm_ws_packed_at(d, T) + rows * act_row_bytes(K);
}

size_t moe_expert_gemm_workspace_bytes(const moe_dims* d, int32_t T, moe_stage stage) {
  if (check_dims(d) != MOE_OK || check_T(d, T) != MOE_OK) return 0;
  if (stage != MOE_STAGE_GATE_UP && stage != MOE_STAGE_DOWN) return 0;
  return gemm_ws_bytes(d, T, stage);
}

moe_status moe_expert_gemm_mxfp4(const moe_dims* d, int32_t T, moe_stage stage, const void* a, const int32_t* perm,
                                 const int32_t* offsets, const uint8_t* codes, const uint8_t* scales,
                                 const float* topk_w, void* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_dims(d);
  if (st != MOE_OK) return st;
  if ((st = check_T(d, T)) != MOE_OK) return st;
  if (stage != MOE_STAGE_GATE_UP && stage != MOE_STAGE_DOWN) return MOE_EINVAL;
  if (!a || !perm || !offsets || !codes || !scales || !out) return MOE_EINVAL;
  if (stage == MOE_STAGE_DOWN && !topk_w) return MOE_EINVAL;
  if (!aligned(a, 16) || !aligned(perm, 4) || !aligned(offsets, 4) || !aligned(codes, 16) || !aligned(scales, 4) ||
      !aligned(out, 16) || (topk_w && !aligned(topk_w, 4)))
    return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  if (!ws || !aligned(ws, kAlignWs)) return MOE_EINVAL;
  if (ws_bytes < gemm_ws_bytes(d, T, stage)) return MOE_EWORKSPACE;
  const int D = d->d_model, I = d->d_ff, E = d->n_experts, k = d->top_k;
  int32_t* tiles = (int32_t*)ws;
  uint8_t* packed = (uint8_t*)ws + gemm_ws_packed_at(d, T);
  if (launch_tiles_from_groups(T, E, k, offsets, perm, tiles, stream)) return MOE_EHIP;
  const int s = stage == MOE_STAGE_GATE_UP ? 0 : 1;
  if (launch_pack(s == 0 ? D : I, s == 0 ? T : T * k, (const uint16_t*)a, packed, stream)) return MOE_EHIP;
  return hip_status(launch_gemm(s, T, D, I, E, k, d->swiglu_limit, packed, tiles, codes, scales, topk_w, out, stream,
                                kActSplit6, /*out_assign=*/0, /*dense_rows=*/0, /*h_bf16=*/s == 0));
}

moe_status moe_expert_gemm_mxfp4_act4(const moe_dims* d, int32_t T, moe_stage stage, const void* a_packed4,
                                      const int32_t* tiles, const uint8_t* codes, const uint8_t* scales,
                                      const float* topk_w, void* out, hipStream_t stream) {
  return expert_gemm(d, T, stage, a_packed4, tiles, codes, scales, topk_w, out, stream, kActFp4);
}

moe_status moe_combine(const moe_dims* d, int32_t T, const void* y_perm, const int32_t* inv, void* y,
                       moe_dtype y_dtype, hipStream_t stream) {
  moe_status st = check_dims(d);
  if (st != MOE_OK) return st;
  if ((st = check_T(d, T)) != MOE_OK) return st;
  if (y_dtype != MOE_BF16 && y_dtype != MOE_FP32) return MOE_EINVAL;
  if (!y_perm || !inv || !y || !aligned(y_perm, 16) || !aligned(inv, 4) || !aligned(y, 16)) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  return hip_status(launch_combine(T, d->d_model, d->top_k, (const _Float16*)y_perm, inv, nullptr, y,
                                   y_dtype == MOE_BF16, stream));
}

moe_status moe_combine_residual(const moe_dims* d, int32_t T, const void* y_perm, const int32_t* inv,
                                const void* residual_bf16, void* y, moe_dtype y_dtype, hipStream_t stream) {
  moe_status st = check_dims(d);
  if (st != MOE_OK) return st;
  if ((st = check_T(d, T)) != MOE_OK) return st;
  if (y_dtype != MOE_BF16 && y_dtype != MOE_FP32) return MOE_EINVAL;
  if (!y_perm || !inv || !residual_bf16 || !y || !aligned(y_perm, 16) || !aligned(inv, 4) ||
      !aligned(residual_bf16, 16) || !aligned(y, 16))
    return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  return hip_status(launch_combine(T, d->d_model, d->top_k, (const _Float16*)y_perm, inv,
                                   (const uint16_t*)residual_bf16, y, y_dtype == MOE_BF16, stream));
}

moe_status moe_rmsnorm(const moe_dims* d, int32_t T, const void* x_bf16, const float* gamma, float eps,
                       void* xn_bf16, hipStream_t stream) {
  moe_status st = check_dims(d);
  if (st != MOE_OK) return st;
  if ((st = check_T(d, T)) != MOE_OK) return st;
  if (!x_bf16 || !gamma || !xn_bf16 || !(eps > 0.0f) || !isfinite(eps)) return MOE_EINVAL;
  if (!aligned(x_bf16, 16) || !aligned(gamma, 16) || !aligned(xn_bf16, 16)) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  return hip_status(launch_rmsnorm(T, d->d_model, (const uint16_t*)x_bf16, gamma, eps, (uint16_t*)xn_bf16, stream));
}

moe_status moe_forward(const moe_dims* d, int32_t T, const void* x_bf16, const float* w_router,
                       const float* b_router, const moe_weights* wts, void* y, moe_dtype y_dtype, void* ws,
                       size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_forward(d, T, x_bf16, w_router, b_router, wts, y, y_dtype, ws);
  if (st != MOE_OK) return st;
  if (ws_bytes < ws_layout(d, T).total) return MOE_EWORKSPACE;
  if (T == 0) return MOE_OK;
  return forward_impl(d, T, (const uint16_t*)x_bf16, nullptr, w_router, b_router, wts, y, y_dtype,
                      (uint8_t*)ws, stream);
}

moe_status moe_forward_noalloc(const moe_dims* d, int32_t T, const void* x_bf16, const float* w_router,
                               const float* b_router, const moe_weights* wts, void* y, moe_dtype y_dtype,
                               hipStream_t stream) {
  // the checks of moe_forward, with the scratch array standing in for the workspace; all before
  // any HIP call
  moe_status st = check_layer_args(d, T, x_bf16, w_router, b_router, wts, y, y_dtype);
  if (st != MOE_OK) return st;
  if (ws_layout(d, T).total > kNoAllocScratchBytes) return MOE_EWORKSPACE;
  if (T == 0) return MOE_OK;
  uint8_t* base = nullptr;
  if ((st = scratch_of_current_device(stream, &base)) != MOE_OK) return st;
  return forward_impl(d, T, (const uint16_t*)x_bf16, nullptr, w_router, b_router, wts, y, y_dtype, base, stream);
}

size_t moe_workspace_bytes_act4(const moe_dims* d, int32_t T) {
  if (check_dims(d) != MOE_OK || check_T(d, T) != MOE_OK) return 0;
  return ws_layout(d, T, kActFp4).total;
}

moe_status moe_forward_act4(const moe_dims* d, int32_t T, const void* x_bf16, const float* w_router,
                            const float* b_router, const moe_weights* wts, void* y, moe_dtype y_dtype, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_forward(d, T, x_bf16, w_router, b_router, wts, y, y_dtype, ws);
  if (st != MOE_OK) return st;
  if (ws_bytes < ws_layout(d, T, kActFp4).total) return MOE_EWORKSPACE;
  if (T == 0) return MOE_OK;
  return forward_impl(d, T, (const uint16_t*)x_bf16, nullptr, w_router, b_router, wts, y, y_dtype,
                      (uint8_t*)ws, stream, kActFp4);
}

size_t moe_block_workspace_bytes(const moe_dims* d, int32_t T) {
  if (check_dims(d) != MOE_OK || check_T(d, T) != MOE_OK) return 0;
  return block_xn_bytes(d, T) + ws_layout(d, T).total;
}

moe_status moe_block_forward(const moe_dims* d, int32_t T, const void* x_bf16, const float* gamma, float eps,
                             const float* w_router, const float* b_router, const moe_weights* wts, void* y,
                             moe_dtype y_dtype, void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_forward(d, T, x_bf16, w_router, b_router, wts, y, y_dtype, ws);
  if (st != MOE_OK) return st;
  if (!gamma || !aligned(gamma, 16) || !(eps > 0.0f) || !isfinite(eps)) return MOE_EINVAL;
  const size_t xn_bytes = block_xn_bytes(d, T);
  if (ws_bytes < xn_bytes + ws_layout(d, T).total) return MOE_EWORKSPACE;
  if (T == 0) return MOE_OK;
  // the normalised rows go to the start of the workspace: written by the routing launch where
  // it folds the RMSNorm in, else by a launch of their own
  uint16_t* xn = (uint16_t*)ws;
  const FrontNorm fn = {(const uint16_t*)x_bf16, gamma, (double)eps};
  return forward_impl(d, T, xn, (const uint16_t*)x_bf16, w_router, b_router, wts, y, y_dtype,
                      (uint8_t*)ws + xn_bytes, stream, kActSplit6, &fn);
}

// ---- host-only ---------------------------------------------------------------

moe_status moe_mxfp4_quantize(const float* w, int64_t rows, int32_t K, uint8_t* codes, uint8_t* scales) {
  if (!w || !codes || !scales || rows < 0 || K <= 0) return MOE_EINVAL;
  if (K % kBlock) return MOE_EUNSUPPORTED;
  for (int64_t r = 0; r < rows; ++r) {
    for (int b = 0; b < K / kBlock; ++b) {
      const float* v = w + r * K + (int64_t)b * kBlock;
      float amax = 0.0f;
      for (int i = 0; i < kBlock; ++i) amax = fmaxf(amax, fabsf(v[i]));
      int sbyte = 0;
      if (amax > 0.0f) {
        int ex;
        frexpf(amax, &ex);                      // amax = m * 2^ex, m in [0.5, 1)
        sbyte = ex - 1 - 2 + 127;
        sbyte = sbyte < 0 ? 0 : (sbyte > 254 ? 254 : sbyte);
      }
      scales[r * (K / kBlock) + b] = (uint8_t)sbyte;
      const float inv = ldexpf(1.0f, 127 - sbyte);
      for (int i = 0; i < kBlock; ++i) {
        const float q = fabsf(v[i]) * inv;
        float c;
        if (q < 2.0f) c = rintf(q * 2.0f);
        else if (q < 4.0f) c = 4.0f + rintf(q - 2.0f);
        else c = 6.0f + rintf(fminf(q, 6.0f) * 0.5f - 2.0f);
        uint8_t code = (uint8_t)(c > 7.0f ? 7.0f : c);
        if (v[i] < 0.0f) code |= 8;
        const int64_t kk = (int64_t)b * kBlock + i;
        uint8_t* dst = codes + r * (K / 2) + kk / 2;
        if (kk % 2 == 0) *dst = code;
        else *dst = (uint8_t)(*dst | (code << 4));
      }
    }
  }
  return MOE_OK;
}

moe_status moe_mxfp4_prepack(const moe_dims* d, moe_stage stage, const uint8_t* codes, const uint8_t* scales,
                             uint8_t* codes_out, uint8_t* scales_out) {
  moe_status st = check_dims(d);
  if (st != MOE_OK) return st;
  if (stage != MOE_STAGE_GATE_UP && stage != MOE_STAGE_DOWN) return MOE_EINVAL;
  if (!codes || !scales || !codes_out || !scales_out) return MOE_EINVAL;
  const bool gu = stage == MOE_STAGE_GATE_UP;
  const int N = gu ? 2 * d->d_ff : d->d_model;
  const int K = gu ? d->d_model : d->d_ff;
  const int KT = K / kKTile, KG = w_kgroups(K), NQ = N / kNTile;
  const size_t cpe = w_codes_per_expert(N, K), spe = w_scales_per_expert(N, K);
  const size_t crow = K / 2, srow = K / kBlock;
  for (int e = 0; e < d->n_experts; ++e) {
    const uint8_t* ce = codes + (size_t)e * N * crow;
    const uint8_t* se = scales + (size_t)e * N * srow;
    uint8_t* co = codes_out + (size_t)e * cpe;
    uint8_t* so = scales_out + (size_t)e * spe;
    for (int q = 0; q < NQ; ++q) {
      const int base = gu ? ((q & 1) ? d->d_ff : 0) + 32 * (q >> 1) : 32 * q;
      for (int kt = 0; kt < KT; ++kt)
        for (int l = 0; l < 64; ++l) {
          const int row = base + (l & 31), blk = 2 * kt + (l >> 5);
          memcpy(co + (((size_t)q * KT + kt) * 64 + l) * 16, ce + (size_t)row * crow + (size_t)blk * 16, 16);
        }
      for (int g = 0; g < KG; ++g)
        for (int l = 0; l < 64; ++l)
          for (int j = 0; j < 4; ++j) {
            const int kt = 4 * g + j, row = base + (l & 31);
            const uint8_t v = kt < KT ? se[(size_t)row * srow + 2 * kt + (l >> 5)] : 0;
            so[(((size_t)q * KG + g) * 64 + l) * 4 + j] = v;
          }
    }
  }
  return MOE_OK;
}

}  // extern "C"
