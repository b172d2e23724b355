"""fp64 CPU oracle of the gpt-oss MoE feed-forward layer with MXFP4 experts.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
``cpu_baseline`` leg of the benchmark may import this module.  The GPU
library never calls it, and it shares no code, table or helper with the GPU
path: it has its own MXFP4 decoder, its own bf16 rounding and its own
routing.  Everything is computed in float64, step by step, in the order the
pages describe the layer:

  1. router: a small network scores every expert for every token
     [gpt-oss architecture walk-through (ewbang.com), section "Mixture of
     Experts": the router picks several experts and weights them];
  2. top-k: gpt-oss keeps the 4 best experts of 32 (20b) or 128 (120b)
     [same section; GPT-OSS 20B model card (llm-atlas), "feed-forward / MoE"];
  3. gates: softmax over the selected logits, so the weights sum to 1 as in
     the page's example A = 0.7 * NN2 + 0.3 * NN4 [same MoE section];
  4. experts: a SwiGLU feed-forward block (three linear maps, Swish = x *
     sigmoid(x) on the gate) [From GPT-2 to gpt-oss (qypowez.cn), section 3
     "Swish/SwiGLU", Fig. 6-7], width 2880 [model card config table], clamp
     limit swiglu_limit = 7 [model card raw config];
  5. expert weights in MXFP4: 4-bit values, one 8-bit scale per 32 values,
     4.25 bits per parameter [gpt-oss architecture walk-through, "Quantization"];
     element and scale formats E2M1 / E8M0 per the OCP Microscaling v1.0
     specification;
  6. combine: the weighted sum of the selected experts' outputs.

Around the layer, the MoE half of a pre-norm transformer block (block_forward):
  0. RMSNorm of the block input: divide by the root mean square, multiply by a
     learned per-channel scale, no mean, no bias [From GPT-2 to gpt-oss,
     section 7 "RMSNorm replaces LayerNorm", Fig. 11-12]; eps = rms_norm_eps =
     1e-5 [model card config tables]; every transformer block holds two such
     normalisations [walk-through, "Transformer Blocks"];
  7. residual: the block output adds the MoE output to the block input (the
     block maps [N x 2880] to [N x 2880]; residual/shortcut connections are
     named in the From-GPT-2 page's width-versus-depth discussion).

Readings where the pages are silent (each one is listed in the design notes):
router = linear map with bias; softmax over the k selected logits; exact
ties go to the lower expert id; the k slots of a token are stored in
ascending expert id; the permutation is stable by token within an expert;
the clamp applies to both gate and up pre-activations before silu(g) * u;
h is rounded to bf16 (round to nearest even) before the down projection;
the normalised activations are rounded once to bf16 (the expert path takes
bf16 activations), the RMS in float64 with eps widened from its fp32 value;
the residual block is pre-norm, y = x + MoE(RMSNorm(x)).

Parity status: every function here is pinned by the CPU tests
(exhaustive decode table, closed forms, the 0.7/0.3 example, brute force
on tiny inputs, permutation invariants).  The layer output values
themselves are not printed by the pages; they are pinned only through the
dense brute-force evaluation.
"""
from __future__ import annotations

import numpy as np

# E2M1 magnitudes for codes 0..7 (OCP MX v1.0, FP4 E2M1): bit 3 is the sign.
E2M1_MAGNITUDE = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)

NEAR_TIE = 1e-6      # logit gap below which a token's selection is flagged


# ----------------------------------------------------------------------------
# Formats
# ----------------------------------------------------------------------------
def mxfp4_decode(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Decode MXFP4 rows: codes uint8 [R][K/2], scales uint8 [R][K/32] -> f64 [R][K].

    value = E2M1(code) * 2^(s - 127); the low nibble holds the even K index;
    scale byte 255 is NaN (OCP MX v1.0 E8M0).  Exact in float64.
    """
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    R, half = codes.shape
    K = half * 2
    c = np.empty((R, K), dtype=np.uint8)
    c[:, 0::2] = codes & 0x0F
    c[:, 1::2] = codes >> 4
    mag = E2M1_MAGNITUDE[c & 7]
    val = np.where(c & 8, -mag, mag)
    s = scales.astype(np.int64)
    blk = np.where(s == 255, np.nan, np.ldexp(1.0, s - 127))
    return val * np.repeat(blk, 32, axis=1)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def round_to_bf16(v: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (8 significant bits), ties to even.

    Works on the float64 value directly (no intermediate fp32 rounding).
    Normal bf16 range only, which is all the layer produces (|h| <= 49).
    """
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)                     # v = m * 2^e, |m| in [0.5, 1)
    return np.ldexp(np.rint(m * 256.0), e - 8)


# ----------------------------------------------------------------------------
# Router, top-k and gates
# ----------------------------------------------------------------------------
def router_logits(x: np.ndarray, w_router: np.ndarray, b_router: np.ndarray) -> np.ndarray:
    """l[t, e] = sum_d x[t, d] * Wr[e, d] + br[e], float64 (bf16 x fp32 products are exact)."""
    x = np.asarray(x, dtype=np.float64)
    return x @ np.asarray(w_router, dtype=np.float64).T + np.asarray(b_router, dtype=np.float64)


def select_experts(logits: np.ndarray, k: int):
    """Top-k experts per token.

    Experts are ranked by (logit descending, id ascending) and the first k
    kept; the k ids are returned in ascending order.  A token is flagged as a
    near tie when the k-th and (k+1)-th largest logits differ by less than
    1e-6.  Returns (idx int32 [T][k], flagged bool [T], gap float64 [T]).
    """
    T, E = logits.shape
    order = np.argsort(-logits, axis=1, kind="stable")      # stable: ties keep ascending id
    idx = np.sort(order[:, :k], axis=1).astype(np.int32)
    srt = np.take_along_axis(logits, order, axis=1)
    gap = srt[:, k - 1] - srt[:, k] if k < E else np.full(T, np.inf)
    return idx, gap < NEAR_TIE, gap


def gate_weights(logits: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Softmax over the selected logits of each token (slot order = idx order)."""
    sel = np.take_along_axis(logits, idx.astype(np.int64), axis=1)
    ex = np.exp(sel - sel.max(axis=1, keepdims=True))
    return ex / ex.sum(axis=1, keepdims=True)


# ----------------------------------------------------------------------------
# Grouping of assignments by expert
# ----------------------------------------------------------------------------
def build_permutation(idx: np.ndarray, E: int):
    """Group the T*k assignments a = t*k + j by expert, stable by token.

    counts[e] = number of tokens routed to e; offsets = exclusive prefix sum
    (length E+1); perm[p] = assignment id at position p; inv[perm[p]] = p.
    """
    flat = idx.reshape(-1).astype(np.int64)
    n = flat.size
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    perm = np.lexsort((np.arange(n), flat)).astype(np.int32)   # key: expert, then assignment id
    inv = np.empty(n, dtype=np.int32)
    inv[perm] = np.arange(n, dtype=np.int32)
    return counts, offsets, perm, inv


# ----------------------------------------------------------------------------
# SwiGLU expert
# ----------------------------------------------------------------------------
def silu(v: np.ndarray) -> np.ndarray:
    """Swish / SiLU: v * sigmoid(v)."""
    return v / (1.0 + np.exp(-v))


def swiglu(g: np.ndarray, u: np.ndarray, limit: float) -> np.ndarray:
    """silu(clamp(g)) * clamp(u), both clamped to [-limit, limit]; float64, unrounded."""
    g = np.clip(g, -limit, limit)
    u = np.clip(u, -limit, limit)
    return silu(g) * u


def expert_ffn(xr: np.ndarray, gu_codes, gu_scales, dn_codes, dn_scales, limit: float, act4: bool = False,
               preact: bool = False):
    """One expert on rows xr [M][D]: returns (h [M][I] bf16-rounded f64, z [M][D] f64).

    act4: the activation-quantized variant; the rows entering each projection (x, then h) are
    quantized to MXFP4 first (mxfp4_quantize_rows), and the returned h is that quantized h.
    preact: also return the gate and up pre-activations g, u [M][I] (before the clamp), as
    (h, z, g, u); the arithmetic is the same either way."""
    w_gu = mxfp4_decode(gu_codes, gu_scales)        # [2I][D]
    I = w_gu.shape[0] // 2
    xa = mxfp4_quantize_rows(xr) if act4 else xr
    g = xa @ w_gu[:I].T
    u = xa @ w_gu[I:].T
    del w_gu
    h = round_to_bf16(swiglu(g, u, limit))
    if act4:
        h = mxfp4_quantize_rows(h)
    w_dn = mxfp4_decode(dn_codes, dn_scales)        # [D][I]
    z = h @ w_dn.T
    return (h, z, g, u) if preact else (h, z)


def mxfp4_quantize_rows(v: np.ndarray) -> np.ndarray:
    """MXFP4 values of rows [R][K] (K % 32 == 0) under the OCP MX v1.0 conversion, float64.

    Per 32-value block: shared exponent E = floor(log2 amax) - 2 (2 is the largest E2M1
    exponent), clamped to [-127, 127]; each element v / 2^E goes to the nearest E2M1 magnitude,
    ties to the one with the even code, magnitudes past 6 to 6; an all-zero block stays zero."""
    v = np.asarray(v, dtype=np.float64)
    R, K = v.shape
    b = v.reshape(R, K // 32, 32)
    amax = np.abs(b).max(axis=-1, keepdims=True)
    _, ex = np.frexp(amax)                          # amax = m 2^ex, m in [0.5, 1): floor(log2) = ex - 1
    E = np.clip(ex - 1 - 2, -127, 127)
    q = np.abs(b) / np.ldexp(1.0, E)
    d = np.abs(q[..., None] - E2M1_MAGNITUDE)      # distance to every grid value
    best = d.min(axis=-1, keepdims=True)
    even = np.arange(8) % 2 == 0
    # the nearest value; of two equally near (always neighbours, one code even) the even code
    pick = np.where(((d == best) & even).any(axis=-1), np.argmax((d == best) & even, axis=-1),
                    np.argmax(d == best, axis=-1))
    out = np.sign(b) * E2M1_MAGNITUDE[pick] * np.ldexp(1.0, E)
    out[np.broadcast_to(amax == 0, b.shape)] = 0.0
    return out.reshape(R, K)


# ----------------------------------------------------------------------------
# Whole layer
# ----------------------------------------------------------------------------
def combine(w: np.ndarray, z_perm: np.ndarray, inv: np.ndarray, tokens: np.ndarray, k: int) -> np.ndarray:
    """y[t] = sum_j w[t, j] * z[inv[t*k + j]], summed in slot (ascending expert id) order."""
    y = np.zeros((len(tokens), z_perm.shape[1]), dtype=np.float64)
    for j in range(k):
        y += w[tokens, j][:, None] * z_perm[inv[tokens * k + j]]
    return y


def forward(inp, tokens=None, override_idx: dict | None = None, act4: bool = False,
            preact: bool = False) -> dict:
    """Evaluate the layer.

    inp: object with T, D, E, k, I, swiglu_limit, x_bf16, w_router, b_router,
    gu_codes, gu_scales, dn_codes, dn_scales (canonical MXFP4 layout).
    tokens: optional array of token indices; routing and the permutation are
    always computed for all tokens, the experts and the combine only for
    these tokens (all tokens when None).
    override_idx: {token: k expert ids} replacing the oracle's own selection
    for those tokens (used for near-tie tokens only).
    act4: the activation-quantized variant (MXFP4 activations into both expert
    projections; routing on the unquantized x).
    preact: also keep each evaluated position's gate and up pre-activations
    (before the clamp) in g and u, by position p.

    Returns a dict with logits, idx, flagged, gap, w, counts, offsets, perm,
    inv, tokens, and for the evaluated tokens: h (by position p), z (by
    position p) and y [len(tokens)][D], all float64.
    """
    T, E, k = inp.T, inp.E, inp.k
    x = bf16_to_f64(inp.x_bf16)
    logits = router_logits(x, inp.w_router, inp.b_router)
    idx, flagged, gap = select_experts(logits, k)
    if override_idx:
        for t, ids in override_idx.items():
            idx[t] = np.sort(np.asarray(ids, dtype=np.int32))
    w = gate_weights(logits, idx)
    counts, offsets, perm, inv = build_permutation(idx, E)
    tokens = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)

    want = np.zeros(T, dtype=bool)
    want[tokens] = True
    h_all, z_all, g_all, u_all = {}, {}, {}, {}
    for e in range(E):
        seg = np.arange(offsets[e], offsets[e + 1])
        seg = seg[want[perm[seg] // k]]
        if seg.size == 0:
            continue
        rows = x[perm[seg] // k]
        res = expert_ffn(rows, inp.gu_codes[e], inp.gu_scales[e], inp.dn_codes[e],
                         inp.dn_scales[e], inp.swiglu_limit, act4=act4, preact=preact)
        h, z = res[0], res[1]
        for i, p in enumerate(seg):
            h_all[int(p)] = h[i]
            z_all[int(p)] = z[i]
            if preact:
                g_all[int(p)] = res[2][i]
                u_all[int(p)] = res[3][i]
    z_perm = np.zeros((T * k, inp.D), dtype=np.float64)
    for p, zz in z_all.items():
        z_perm[p] = zz
    y = combine(w, z_perm, inv, tokens, k)
    out = dict(logits=logits, idx=idx, flagged=flagged, gap=gap, w=w, counts=counts,
               offsets=offsets, perm=perm, inv=inv, tokens=tokens, h=h_all, z=z_all, y=y)
    if preact:
        out["g"], out["u"] = g_all, u_all
    return out


# ----------------------------------------------------------------------------
# The block around the layer: RMSNorm before it, the residual after it
# ----------------------------------------------------------------------------
def rms_norm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm of the rows of x [From GPT-2 to gpt-oss, section 7, Fig. 12]:
    x / sqrt(mean over the row of x^2 + eps), times the per-channel scale gamma,
    rounded to bf16.  float64 throughout; eps is the fp32 value the layer is given."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=1)
    r = 1.0 / np.sqrt(ms + float(np.float32(eps)))
    return round_to_bf16((x * r[:, None]) * np.asarray(gamma, dtype=np.float64)[None, :])


def f64_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of float64 values that are already bf16 values (exact)."""
    return (np.asarray(v, dtype=np.float64).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def block_forward(inp, tokens=None, override_idx: dict | None = None) -> dict:
    """The MoE half of a pre-norm transformer block: y = x + MoE(RMSNorm(x)).

    inp additionally carries norm_weight (gamma, fp32 [D]) and norm_eps.  Returns
    forward()'s dict computed on the normalised rows, with xn (float64 [T][D],
    bf16 values), y_moe (the layer output) and y = x + y_moe for the evaluated
    tokens."""
    import dataclasses
    x = bf16_to_f64(inp.x_bf16)
    xn = rms_norm(x, inp.norm_weight, inp.norm_eps)
    inner = dataclasses.replace(inp, x_bf16=f64_to_bf16_bits(xn))
    o = forward(inner, tokens=tokens, override_idx=override_idx)
    o["xn"] = xn
    o["y_moe"] = o["y"]
    o["y"] = x[o["tokens"]] + o["y_moe"]
    return o


# ----------------------------------------------------------------------------
# Closed forms printed by the pages
# ----------------------------------------------------------------------------
def mxfp4_bits_per_param(n_params: int, code_bytes: int, scale_bytes: int) -> float:
    """Storage bits per parameter of an MXFP4 tensor (4.25 on the pages)."""
    return 8.0 * (code_bytes + scale_bytes) / n_params


def gpt_oss_param_counts(n_layers: int, n_experts: int, top_k: int, d_model: int = 2880,
                         d_ff: int = 2880, n_q_heads: int = 64, n_kv_heads: int = 8,
                         head_dim: int = 64, vocab: int = 201088) -> dict:
    """Weight-matrix parameter counts of a gpt-oss model (biases and norms omitted).

    Per layer: experts 3 * d_model * d_ff each, router d_model * E, attention
    q/o d_model x (64*64) and k/v d_model x (8*64); untied embedding and
    unembedding vocab x d_model.  'active' counts the top_k experts, the
    attention, the router and the unembedding (the embedding is a lookup).
    """
    expert = 3 * d_model * d_ff
    attn = 2 * d_model * n_q_heads * head_dim + 2 * d_model * n_kv_heads * head_dim
    router = d_model * n_experts
    emb = vocab * d_model
    total = n_layers * (n_experts * expert + attn + router) + 2 * emb
    active = n_layers * (top_k * expert + attn + router) + emb
    return dict(total=total, active=active, expert=expert, attention=attn, router=router,
                embedding=emb, experts_all_layers=n_layers * n_experts * expert)
