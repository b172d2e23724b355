/*
 * moe_mxfp4.h — C ABI of the gpt-oss MoE feed-forward layer with MXFP4 experts
 * on one AMD Instinct MI355X (gfx950).
 *
 * The layer (sources: "gpt-oss architecture walk-through" (ewbang.com), sections
 * "Mixture of Experts" and "Quantization"; "From GPT-2 to gpt-oss" (qypowez.cn),
 * section 3 "Swish/SwiGLU" and section 4 "Mixture of Experts"; "GPT-OSS 20B"
 * model card (llm-atlas), config tables):
 *
 *   logits[t,e] = x[t,:] . Wr[e,:] + br[e]                        (router)
 *   S_t         = the top_k experts of token t                    (top-k)
 *   w[t,j]      = softmax over the selected logits                (gates, sum to 1)
 *   g, u        = x[t] W_gate[e]^T, x[t] W_up[e]^T                 (MXFP4 weights)
 *   h           = bf16( silu(clamp(g)) * clamp(u) ), clamp to +-swiglu_limit
 *   z           = h W_down[e]^T
 *   y[t]        = sum_j w[t,j] * z_{t, S_t[j]}                     (combine)
 *
 * Expert weights are MXFP4: E2M1 4-bit values with one E8M0 scale byte per 32
 * consecutive values along the reduction axis (4.25 bits per parameter).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All device pointers are caller-owned device memory; the library never
 *    allocates, frees or keeps them.  Host pointers are named so.
 *  - Every call validates its arguments on the host before any HIP call and
 *    returns MOE_EINVAL / MOE_EUNSUPPORTED without launching anything.  A
 *    launch failure returns MOE_EHIP.  Device faults appear at the caller's
 *    next synchronisation.  T == 0 is a no-op that returns MOE_OK.
 *  - Work is enqueued on `stream` (0 = the null stream); no call synchronises.
 *  - Supported shapes: d_model % 64 == 0, d_ff % 64 == 0, 1 <= top_k <= n_experts
 *    <= 256, 0 <= T, T * top_k < 2^24.  Inputs must be finite.
 *  - Index order: a token's k slots hold its experts in ascending id; an
 *    assignment id is a = t * top_k + j; the permutation lists assignment ids
 *    grouped by expert (ascending) and, within an expert, by token.
 *  - Calls that share no buffers may run concurrently on different streams.
 *
 * The step-by-step boundary
 * -------------------------
 * moe_route -> moe_permute -> moe_expert_gemm_mxfp4 (GATE_UP, then DOWN) ->
 * moe_combine computes what moe_forward computes, on bf16 rows: x [T][d_model],
 * h [T*top_k][d_ff] in grouped order, y_perm [T*top_k][d_model] fp16 with each
 * row already multiplied by its gate, and the grouping as perm and offsets.
 * Scratch comes from ws.  The same steps also exist on the operands the kernels
 * actually read, for callers that keep them between calls:
 *  - moe_permute_tiles writes, besides the grouping, the row-tile table
 *    (expert, first grouped row, row count and the assignment id of every row
 *    of each tile) that the expert GEMMs start from;
 *  - moe_expert_gemm_mxfp4_packed takes activations already packed ("split
 *    MX6", below): moe_pack_act packs x, and its gate/up stage writes h in the
 *    same packed format, which its down stage reads.  A packed row decodes to
 *    within 2^-8 of its 32-value block maximum of the bf16 row (hi + lo; the
 *    bf16 h the layer defines is rounded before it is packed).
 * moe_expert_gemm_mxfp4 builds the tile table from perm and offsets and packs
 * its input rows in ws, then runs the same kernels; its bf16 h is the value the
 * packed gate/up stage splits, so packing it gives the packed stage's bytes.
 *
 * Activation pack format ("split MX6")
 * ------------------------------------
 * The expert GEMMs consume activations that are already split into two MX
 * terms, hi + lo, each stored as FP6 E2M3 codes with one E8M0 scale per 32
 * values; hi + lo reproduces a bf16 row to about 2^-9 of its block maximum.
 * One packed row of K values (K % 64 == 0) is moe_act_pack_bytes(K, 1) = (K/64) * 112
 * bytes: one 112-byte chunk per 64-wide k-tile kt, holding
 *     [0,24) hi codes of block 2kt    [24,48) hi codes of block 2kt+1
 *     [48,72) lo codes of block 2kt   [72,96) lo codes of block 2kt+1
 *     [96],[97] hi scales of blocks 2kt, 2kt+1   [98],[99] lo scales   [100,112) unused
 * A block's 32 codes are 6-bit fields packed little-endian (element i at bits
 * 6i..6i+5); E2M3 = sign | 2 exponent bits (bias 1) | 3 mantissa bits.
 *
 * MXFP4 activation pack format (the activation-quantized entry points, *_act4)
 * ----------------------------------------------------------------------------
 * Activations quantized to MXFP4 with the OCP MX v1.0 conversion: per 32-value
 * block, shared exponent floor(log2 amax) - 2 as an E8M0 byte, elements rounded
 * to the nearest E2M1 value (ties to the even code), saturating at +-6; an
 * all-zero block gets scale byte 0.  A row of K values is (K/64) chunks of 48
 * bytes (moe_act4_pack_bytes): [0,16) codes of block 2kt (element i in nibble i,
 * low nibble first), [16,32) codes of block 2kt+1, [32] [33] their scales,
 * [34,48) unused.
 *
 * Prepacked weight format
 * -----------------------
 * moe_mxfp4_prepack reorders canonical MXFP4 bytes (codes [E][N][K/2], even K
 * in the low nibble; scales [E][N][K/32]; gate/up rows 0..I-1 gate and I..2I-1
 * up) into tiles of 32 output rows x 64 K values laid out in the order the
 * gfx950 scaled MFMA reads them, so each wavefront load is one contiguous
 * 1 KiB.  Sizes: moe_prepacked_codes_bytes / moe_prepacked_scales_bytes.
 */
#ifndef MOE_MXFP4_H
#define MOE_MXFP4_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = 1,          /* null pointer, negative size, misaligned pointer, bad enum */
  MOE_EUNSUPPORTED = 2,    /* shape outside the supported set above */
  MOE_EWORKSPACE = 3,      /* workspace smaller than moe_workspace_bytes */
  MOE_EHIP = 4             /* a HIP launch or runtime call failed */
} moe_status;

typedef enum { MOE_BF16 = 0, MOE_FP32 = 1 } moe_dtype;

typedef enum { MOE_STAGE_GATE_UP = 0, MOE_STAGE_DOWN = 1 } moe_stage;

/* MoE-relevant model configuration (model card fields hidden_size,
 * intermediate_size, num_local_experts, num_experts_per_tok, swiglu_limit). */
typedef struct {
  int32_t d_model;
  int32_t d_ff;
  int32_t n_experts;
  int32_t top_k;
  float swiglu_limit;
} moe_dims;

/* Prepacked expert weights of one layer (device pointers, 16-byte aligned). */
typedef struct {
  const uint8_t* gu_codes;
  const uint8_t* gu_scales;
  const uint8_t* dn_codes;
  const uint8_t* dn_scales;
} moe_weights;

/* Human-readable name of a status code (static string). */
const char* moe_status_str(moe_status s);

/* Bytes of `rows` packed activation rows of length K (0 if K % 64 != 0): the split-MX6
 * encoding above of the bf16 activations that enter the expert projections (the scaled
 * matrix instruction that reads the MXFP4 weights of "gpt-oss architecture walk-through",
 * section "Quantization", takes MX operands only). */
size_t moe_act_pack_bytes(int32_t K, int32_t rows);

/* Bytes of the prepacked codes / scales of all experts for one stage: 4 bits per weight plus
 * one scale byte per 32 weights, 4.25 bits per parameter ("gpt-oss architecture
 * walk-through", section "Quantization"); the scales are padded to whole groups of 4 k-tiles. */
size_t moe_prepacked_codes_bytes(const moe_dims* dims, moe_stage stage);
size_t moe_prepacked_scales_bytes(const moe_dims* dims, moe_stage stage);

/* Workspace bytes moe_forward needs for T tokens (0 on invalid dims or an unsupported T): the
 * scratch of the whole layer defined at the top of this file ("gpt-oss architecture
 * walk-through", sections "Mixture of Experts" and "Quantization"; "From GPT-2 to gpt-oss",
 * section 3): routing results, the grouping, packed x and h, y_perm, the router's float64
 * partials, in 256-byte aligned regions. */
size_t moe_workspace_bytes(const moe_dims* dims, int32_t T);

/*
 * Router, top-k and softmax gating ("gpt-oss architecture walk-through",
 * section "Mixture of Experts": the router scores experts, keeps several and
 * weights them; gpt-oss keeps 4).
 *   x_bf16    [T][d_model] bf16, row-major, 16-byte aligned
 *   w_router  [n_experts][d_model] fp32, 16-byte aligned;  b_router [n_experts] fp32
 *   topk_idx  out [T][top_k] int32: selected expert ids, ascending per token
 *   topk_w    out [T][top_k] fp32: softmax of the selected logits (same order)
 *   logits    out [T][n_experts] fp32 or NULL: router logits (rounded from float64)
 *   ws        device scratch of at least moe_route_workspace_bytes(dims, T)
 *             bytes, 256-byte aligned (float64 partial logits: of groups of 256
 *             K values for at most 32 tokens and 32 experts, of K slices beyond)
 * Logits are accumulated on the matrix cores (exact bf16 x split-fp32
 * products, 16-term fp32 partial sums, float64 accumulation); any expert
 * within 36 eps32 ||x_t|| max_e ||w_e|| of the k-th largest (twice the error
 * bound) is re-scored exactly in float64 before the final choice, so the
 * selection is the float64 one; exact ties go to the lower id.  Gates are the
 * softmax of the float64 scores.
 */
size_t moe_route_workspace_bytes(const moe_dims* dims, int32_t T);
moe_status moe_route(const moe_dims* dims, int32_t T, const void* x_bf16, const float* w_router,
                     const float* b_router, int32_t* topk_idx, float* topk_w, float* logits,
                     void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Group the T*top_k assignments by expert (deterministic, no atomics on order)
 * and cut every expert's rows into row tiles for the expert GEMMs.  Only the
 * selected experts run for a token, so each expert's feed-forward block works
 * on the rows routed to it ("From GPT-2 to gpt-oss", section 4 "Mixture of
 * Experts": the MoE module is sparse, not every expert is active for a token;
 * "gpt-oss architecture walk-through", section "Mixture of Experts").
 *   topk_idx  [T][top_k] int32, every entry in [0, n_experts) (precondition; an
 *             entry outside it is a caller error: that assignment gets no row,
 *             it is left out of counts, perm and the tiles, its inv entry is -1,
 *             offsets[n_experts] counts only the valid ones, and perm past
 *             offsets[n_experts] is left unwritten)
 *   counts    out [n_experts]; offsets out [n_experts + 1] (exclusive prefix sum)
 *   perm      out [T*top_k]: assignment id at each grouped position
 *   inv       out [T*top_k]: inv[perm[p]] = p
 *   ws        device scratch of at least moe_permute_workspace_bytes(dims, T)
 *             bytes (moe_workspace_bytes(dims, T) is always enough), 256-byte
 *             aligned; may be NULL when T == 0
 */
size_t moe_permute_workspace_bytes(const moe_dims* dims, int32_t T);
moe_status moe_permute(const moe_dims* dims, int32_t T, const int32_t* topk_idx, int32_t* counts,
                       int32_t* offsets, int32_t* perm, int32_t* inv, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_permute that also hands back the row-tile table the expert GEMMs start
 * from (the grouping of "From GPT-2 to gpt-oss", section 4 "Mixture of Experts":
 * only the selected experts run for a token, so each expert's GEMM takes the
 * rows routed to it):
 *   tiles     out, moe_tile_table_bytes(dims, T) bytes, 16-byte aligned: the
 *             row-tile table: 8-row tiles when T*top_k <= 6*n_experts (48
 *             int32 per slot), else 128-row tiles (132 int32 per slot).  A
 *             slot holds expert or -1, first grouped position, row count,
 *             number of tiles in use, then the assignment id of each row.
 */
size_t moe_tile_table_bytes(const moe_dims* dims, int32_t T);
moe_status moe_permute_tiles(const moe_dims* dims, int32_t T, const int32_t* topk_idx, int32_t* counts,
                             int32_t* offsets, int32_t* perm, int32_t* inv, int32_t* tiles, hipStream_t stream);

/*
 * Split bf16 rows into the packed hi/lo MX6 activation format above (the
 * activations entering an expert's projections are the bf16 rows of the layer;
 * the scaled matrix instruction that reads the MXFP4 weights, "gpt-oss
 * architecture walk-through", section "Quantization", takes no bf16 operand).
 *   a_bf16   [rows][K] bf16 row-major, 16-byte aligned;  K % 64 == 0
 *   a_packed out, moe_act_pack_bytes(K, rows) bytes, 16-byte aligned
 */
moe_status moe_pack_act(int32_t K, int32_t rows, const void* a_bf16, void* a_packed, hipStream_t stream);

/*
 * Grouped expert GEMM on MXFP4 weights with the CDNA4 scaled FP4 matrix cores.
 * Each expert is a SwiGLU feed-forward block ("From GPT-2 to gpt-oss", section 3
 * "Swish/SwiGLU", Figures 6-7: gate and up projections, silu(gate) * up, down
 * projection), its pre-activations clamped at swiglu_limit (7 in the "GPT-OSS
 * 20B" model card's raw config), its weights MXFP4 ("gpt-oss architecture
 * walk-through", section "Quantization").  On bf16 rows with the grouping as
 * perm and offsets (moe_permute):
 *  MOE_STAGE_GATE_UP:
 *    a         x [T][d_model] bf16; grouped position p reads token perm[p] / top_k
 *    out       h [T*top_k][d_ff] bf16, row p = grouped position p, the bf16
 *              round of silu(clamp(g)) * clamp(u) (g, u accumulated in fp32 over
 *              the hi/lo split of x)
 *    topk_w    unused (may be NULL)
 *  MOE_STAGE_DOWN:
 *    a         h [T*top_k][d_ff] bf16 in grouped order (the GATE_UP output)
 *    topk_w    [T][top_k] fp32 gates; row p is scaled by topk_w[perm[p]]
 *    out       y_perm [T*top_k][d_model] fp16 (round to nearest even), row p =
 *              gate-weighted expert output; its magnitude must stay below the
 *              fp16 maximum (65504)
 *  codes/scales  prepacked weights of the stage (moe_mxfp4_prepack)
 *  perm, offsets  moe_permute's outputs for the same T: offsets[0] = 0 <= ... <=
 *            offsets[E] = T*top_k and perm a permutation of [0, T*top_k)
 *            grouping the assignments by expert.  These are read on the device
 *            and not checked: other values can make the kernels read outside a
 *            and topk_w.
 *  ws        device scratch of at least moe_expert_gemm_workspace_bytes(dims, T,
 *            stage) bytes (moe_workspace_bytes(dims, T) is always enough),
 *            256-byte aligned: the row-tile table built from perm and offsets,
 *            then the packed input rows; may be NULL when T == 0
 *  Experts with no token have no tile (their weights are not read).
 */
size_t moe_expert_gemm_workspace_bytes(const moe_dims* dims, int32_t T, moe_stage stage);
moe_status moe_expert_gemm_mxfp4(const moe_dims* dims, int32_t T, moe_stage stage, const void* a,
                                 const int32_t* perm, const int32_t* offsets, const uint8_t* codes,
                                 const uint8_t* scales, const float* topk_w, void* out, void* ws, size_t ws_bytes,
                                 hipStream_t stream);

/*
 * The same GEMM on the packed activations and the row-tile table (see "The
 * step-by-step boundary" above): the SwiGLU expert of "From GPT-2 to gpt-oss",
 * section 3 "Swish/SwiGLU" (Figures 6-7), clamped at swiglu_limit (the "GPT-OSS
 * 20B" model card's raw config), on the MXFP4 weights of "gpt-oss architecture
 * walk-through", section "Quantization":
 *  MOE_STAGE_GATE_UP:
 *    a_packed  packed x, T rows of d_model (moe_pack_act output); the row of
 *              grouped position p is token perm[p] / top_k
 *    codes/scales  prepacked gate/up weights (moe_mxfp4_prepack, stage GATE_UP)
 *    out       packed h, T*top_k rows of d_ff, row p = grouped position p, with
 *              h = bf16(silu(clamp(g)) * clamp(u)) split into hi/lo MX6
 *    topk_w    unused (may be NULL)
 *  MOE_STAGE_DOWN:
 *    a_packed  packed h from the GATE_UP stage
 *    codes/scales  prepacked down weights (stage DOWN)
 *    topk_w    [T][top_k] fp32 gates; row p is scaled by topk_w[perm[p]]
 *    out       y_perm [T*top_k][d_model] fp16 (round to nearest even), row p =
 *              gate-weighted expert output; its magnitude must stay below the fp16
 *              maximum (65504)
 *  tiles is moe_permute_tiles's row-tile table for the same T.  Experts with no
 *  token have no tile (their weights are not read).
 */
moe_status moe_expert_gemm_mxfp4_packed(const moe_dims* dims, int32_t T, moe_stage stage, const void* a_packed,
                                        const int32_t* tiles, const uint8_t* codes, const uint8_t* scales,
                                        const float* topk_w, void* out, hipStream_t stream);

/*
 * Weighted combine: y[t] = sum over the token's slots j (ascending expert id)
 * of y_perm[inv[t*top_k + j]], summed in fp32: the gate-weighted sum of the
 * selected experts' outputs ("gpt-oss architecture walk-through", section
 * "Mixture of Experts": A = 0.7 x network 2 + 0.3 x network 4).  A slot whose
 * inv entry is negative (an invalid expert id given to moe_permute) adds nothing.
 *   y_perm [T*top_k][d_model] fp16 (gate already applied);  inv from moe_permute
 *   y      out [T][d_model], fp32 (MOE_FP32) or bf16 round-to-nearest-even (MOE_BF16)
 */
moe_status moe_combine(const moe_dims* dims, int32_t T, const void* y_perm, const int32_t* inv, void* y,
                       moe_dtype y_dtype, hipStream_t stream);

/*
 * Weighted combine plus the residual stream: y[t] = fp32(residual[t]) + (the
 * moe_combine sum of token t), one fp32 addition after the slot-order sum; the
 * bf16 output is its round to nearest even.  This is the end of the MoE half of
 * a pre-norm transformer block, y = x + MoE(RMSNorm(x)) (the block maps
 * [N x d_model] to [N x d_model]: "gpt-oss architecture walk-through",
 * section "Transformer Blocks").
 *   residual_bf16 [T][d_model] bf16, 16-byte aligned (the block input x)
 *   other arguments as moe_combine
 */
moe_status moe_combine_residual(const moe_dims* dims, int32_t T, const void* y_perm, const int32_t* inv,
                                const void* residual_bf16, void* y, moe_dtype y_dtype, hipStream_t stream);

/*
 * RMSNorm of the rows of x ("From GPT-2 to gpt-oss", section 7, Figures 11-12:
 * divide by the root mean square, multiply by a learned per-channel scale, no
 * mean and no bias; rms_norm_eps = 1e-5 in the model cards' config tables):
 *   r_t = 1 / sqrt(sum_d x[t,d]^2 / d_model + eps)
 *   xn[t,d] = bf16((x[t,d] * r_t) * gamma[d])
 * computed in float64 (eps widened from fp32) and rounded once, to nearest
 * even, from float64.
 *   x_bf16  [T][d_model] bf16, 16-byte aligned
 *   gamma   [d_model] fp32 scale, 16-byte aligned;  eps > 0 and finite
 *   xn_bf16 out [T][d_model] bf16, 16-byte aligned; must not overlap x_bf16
 */
moe_status moe_rmsnorm(const moe_dims* dims, int32_t T, const void* x_bf16, const float* gamma, float eps,
                       void* xn_bf16, hipStream_t stream);

/*
 * The whole layer: route -> permute -> pack x -> gate/up + SwiGLU -> down ->
 * combine, enqueued on `stream` with no host synchronisation.  This is the MoE
 * layer of a gpt-oss transformer block ("gpt-oss architecture walk-through",
 * sections "Transformer Blocks" and "Mixture of Experts": a router and several
 * expert networks replace the block's feed-forward network; [N x 2880] in and
 * out; the top 4 experts of 32 (20b) or 128 (120b) are active per token), with
 * the SwiGLU experts and MXFP4 weights of moe_expert_gemm_mxfp4.  y has the same
 * bits as the step-by-step entry points above give on the same inputs.  (Inside
 * the workspace the down stage writes each row at its assignment t*top_k + j
 * rather than at its permuted position, so the combine needs no inverse lookup.)
 *   ws / ws_bytes: device scratch of at least moe_workspace_bytes(dims, T)
 *   bytes, 256-byte aligned; its contents are undefined after the call.
 */
moe_status moe_forward(const moe_dims* dims, int32_t T, const void* x_bf16, const float* w_router,
                       const float* b_router, const moe_weights* weights, void* y, moe_dtype y_dtype,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_forward for callers that cannot allocate: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  The same kernels and
 * the same result bits as moe_forward, with no workspace argument: the scratch
 * is a file-scope device array of MOE_FORWARD_NOALLOC_MAX_WORKSPACE bytes that
 * each GPU holds from the library's load until the process ends (its device
 * address is looked up once per device, on the first call made with that
 * device current).  The call allocates and frees nothing, and calls no
 * allocating library routine.
 *  - Limit: T with moe_workspace_bytes(dims, T) > MOE_FORWARD_NOALLOC_MAX_WORKSPACE
 *    returns MOE_EWORKSPACE before anything is launched (at d_model = d_ff = 2880
 *    and top_k = 4: T up to 339 with 32 experts, 318 with 128; decode batches).
 *  - Every call on one GPU uses that GPU's one array: calls that overlap on one
 *    GPU (other streams, other threads) race and must be serialised by the
 *    caller.  Nothing in the array needs to start at zero; it keeps the last
 *    call's contents.
 *  - `stream` must belong to the current device (else MOE_EINVAL); other
 *    arguments and errors as moe_forward.
 */
#define MOE_FORWARD_NOALLOC_MAX_WORKSPACE ((size_t)16 << 20)
moe_status moe_forward_noalloc(const moe_dims* dims, int32_t T, const void* x_bf16, const float* w_router,
                               const float* b_router, const moe_weights* weights, void* y, moe_dtype y_dtype,
                               hipStream_t stream);

/*
 * The activation-quantized variant (W4A4): the expert GEMMs take their
 * activations as MXFP4 (format above) and run one FP4 x FP4 scaled matrix
 * instruction per weight tile, the full MXFP4 rate of the matrix cores (the
 * pages: the hardware supports MXFP4; "From GPT-2 to gpt-oss", section
 * "MXFP4").  The router and the permutation are those of the default path (on
 * the bf16 x); x is quantized for the gate/up GEMM and h = bf16(silu(clamp g) *
 * clamp u) is quantized in the gate/up epilogue for the down GEMM.  The result
 * is not the W4A16 layer of moe_forward: it is a different, lower-precision
 * contract.
 *   moe_pack_act4:               bf16 rows -> MXFP4 rows
 *   moe_expert_gemm_mxfp4_act4:  as moe_expert_gemm_mxfp4_packed with MXFP4 activations
 *                                (stage GATE_UP writes h in the MXFP4 format)
 *   moe_forward_act4:            the whole layer; ws of moe_workspace_bytes_act4
 */
size_t moe_act4_pack_bytes(int32_t K, int32_t rows);
moe_status moe_pack_act4(int32_t K, int32_t rows, const void* a_bf16, void* a_packed4, hipStream_t stream);
moe_status moe_expert_gemm_mxfp4_act4(const moe_dims* dims, int32_t T, moe_stage stage, const void* a_packed4,
                                      const int32_t* tiles, const uint8_t* codes, const uint8_t* scales,
                                      const float* topk_w, void* out, hipStream_t stream);
size_t moe_workspace_bytes_act4(const moe_dims* dims, int32_t T);
moe_status moe_forward_act4(const moe_dims* dims, int32_t T, const void* x_bf16, const float* w_router,
                            const float* b_router, const moe_weights* weights, void* y, moe_dtype y_dtype,
                            void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * The MoE half of a pre-norm transformer block ("From GPT-2 to gpt-oss", section 7
 * "RMSNorm replaces LayerNorm", Figures 11-12, for the normalisation; "gpt-oss
 * architecture walk-through", section "Transformer Blocks", for its place in the
 * block, [N x 2880] in and out): y = x + MoE(RMSNorm(x)), i.e.
 * moe_rmsnorm -> the moe_forward steps on the normalised rows ->
 * moe_combine_residual with x.  The bits equal those of that sequence of step
 * calls.  ws: at least moe_block_workspace_bytes(dims, T) bytes, 256-byte
 * aligned (the normalised rows, then moe_forward's workspace); contents
 * undefined after the call.  gamma / eps as moe_rmsnorm.
 */
size_t moe_block_workspace_bytes(const moe_dims* dims, int32_t T);
moe_status moe_block_forward(const moe_dims* dims, int32_t T, const void* x_bf16, const float* gamma, float eps,
                             const float* w_router, const float* b_router, const moe_weights* weights, void* y,
                             moe_dtype y_dtype, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---- host-only helpers (off the hot path; no HIP calls) ---------------- */

/*
 * Quantize fp32 rows [rows][K] (host memory, K % 32 == 0) to canonical MXFP4
 * (the MoE weights are quantized to 4-bit floats after training, one 8-bit
 * scale per 32 values: "gpt-oss architecture walk-through", section
 * "Quantization"; "From GPT-2 to gpt-oss", section "MXFP4") with the OCP
 * Microscaling v1.0 rule: scale exponent floor(log2(amax)) - 2,
 * elements rounded to nearest even on the E2M1 grid, saturating at +-6; an
 * all-zero block gets scale byte 0.  codes [rows][K/2], scales [rows][K/32].
 */
moe_status moe_mxfp4_quantize(const float* w, int64_t rows, int32_t K, uint8_t* codes, uint8_t* scales);

/*
 * Reorder canonical MXFP4 bytes of all n_experts experts (host memory) into
 * the device tile layout (the same 4.25-bit-per-parameter MXFP4 values of
 * "gpt-oss architecture walk-through", section "Quantization", only moved).  stage GATE_UP: N = 2*d_ff rows of K = d_model;
 * stage DOWN: N = d_model rows of K = d_ff.
 */
moe_status moe_mxfp4_prepack(const moe_dims* dims, moe_stage stage, const uint8_t* codes,
                             const uint8_t* scales, uint8_t* codes_out, uint8_t* scales_out);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MXFP4_H */
