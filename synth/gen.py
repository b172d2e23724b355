"""Seeded generator for MoE-layer inputs (activations, router, MXFP4 experts).

Shapes follow the gpt-oss pages: model width and expert width 2880, 32
experts for 20b and 128 for 120b, four active experts per token (P4 "gpt-oss
architecture walk-through", MoE section; P5 "GPT-OSS 20B" model card, config
table).  The SwiGLU clamp value 7 is the config field ``swiglu_limit`` of the
P5 raw-config table.  Expert weights are stored as MXFP4: 4-bit E2M1 values
with one 8-bit E8M0 scale per 32 consecutive values along the reduction axis
(P4, quantization section: 4 + 8/32 = 4.25 bits per parameter).

Distributions (the same for every workload):
  * x ~ N(0, 1) drawn in fp32, rounded to bf16 (round to nearest even);
  * RMSNorm scale gamma ~ 1 + N(0, 0.1), fp32, and eps = 1e-5 (model cards'
    rms_norm_eps), for the pre-norm block around the layer;
  * router weight ~ N(0, 0.02), router bias ~ N(0, 0.01), both fp32;
  * expert gate / up / down weights ~ N(0, 0.02) in fp32, then encoded to
    MXFP4 with the OCP Microscaling v1.0 conversion rule (shared exponent
    floor(log2 amax) - 2, elements rounded to nearest even on the E2M1 grid
    and saturated at +-6).

Random streams: numpy PCG64 seeded with SeedSequence([seed, tag, expert]) so
each tensor (and each expert's matrices) has its own reproducible substream.

Canonical weight layout produced here (the oracle reads it directly, the
GPU library re-orders it with its own prepack):
  gu_codes   uint8 [E][2I][D/2]  rows 0..I-1 gate, I..2I-1 up; K contiguous,
                                  even K index in the low nibble
  gu_scales  uint8 [E][2I][D/32] one E8M0 byte per 32 K values
  dn_codes   uint8 [E][D][I/2]
  dn_scales  uint8 [E][D][I/32]
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

SWIGLU_LIMIT = 7.0
RMS_NORM_EPS = 1e-5

# Substream tags.
_TAG_X, _TAG_WR, _TAG_BR, _TAG_GATE, _TAG_UP, _TAG_DOWN, _TAG_PERM, _TAG_NORM = range(8)

# Router-bias exponent of the skewed workload: expert popularity p(r) ~ r^-1.2
# for popularity rank r = 1..E.  The bias is beta * ln p(r) (up to a constant
# that cancels in the top-k); beta was calibrated offline so that the 10% most
# popular experts take about half of all assignments at T=8192, E=128, k=4.
ZIPF_S = 1.2
ZIPF_BETA = 0.42
ZIPF_N_EMPTY = 4          # least popular experts forced to receive no token
_EMPTY_BIAS = -1.0e4

CONFIGS = {
    0: dict(name="tiny", T=16, D=64, E=4, k=2, I=64, seed=0, bias="normal"),
    1: dict(name="gpt-oss-20b decode", T=32, D=2880, E=32, k=4, I=2880, seed=1, bias="normal"),
    2: dict(name="gpt-oss-20b prefill", T=4096, D=2880, E=32, k=4, I=2880, seed=2, bias="normal"),
    3: dict(name="gpt-oss-120b", T=4096, D=2880, E=128, k=4, I=2880, seed=3, bias="normal"),
    4: dict(name="gpt-oss-120b skewed", T=8192, D=2880, E=128, k=4, I=2880, seed=4, bias="zipf"),
}


@dataclasses.dataclass
class LayerInputs:
    T: int
    D: int
    E: int
    k: int
    I: int
    swiglu_limit: float
    x_bf16: np.ndarray      # uint16 [T][D] (bf16 bit patterns)
    w_router: np.ndarray    # float32 [E][D]
    b_router: np.ndarray    # float32 [E]
    gu_codes: np.ndarray    # uint8 [E][2I][D/2]
    gu_scales: np.ndarray   # uint8 [E][2I][D/32]
    dn_codes: np.ndarray    # uint8 [E][D][I/2]
    dn_scales: np.ndarray   # uint8 [E][D][I/32]
    desc: dict
    norm_weight: np.ndarray | None = None   # float32 [D]: RMSNorm scale of the block
    norm_eps: float = RMS_NORM_EPS

    @property
    def x_f32(self) -> np.ndarray:
        return bf16_bits_to_f32(self.x_bf16)


def _rng(seed: int, tag: int, sub: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tag, sub])))


def f32_to_bf16_bits(a) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def mxfp4_encode(w: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Encode fp32 rows [R][K] (K % 32 == 0) to MXFP4 (OCP MX v1.0 rule).

    Per block of 32: shared exponent X = floor(log2(amax)) - 2 (2 is the E2M1
    maximum exponent), stored as the E8M0 byte X + 127 clamped to [0, 254];
    an all-zero block stores byte 0.  Each element v/2^X is rounded to the
    nearest E2M1 magnitude {0, .5, 1, 1.5, 2, 3, 4, 6} with ties to the even
    code, saturating at 6; bit 3 of the code is the sign.
    Returns (codes uint8 [R][K/2], scales uint8 [R][K/32]).
    """
    w = np.ascontiguousarray(w, dtype=np.float32)
    R, K = w.shape
    assert K % 32 == 0
    b = w.reshape(R, K // 32, 32)
    amax = np.abs(b).max(axis=-1)
    _, e = np.frexp(amax)                          # amax = m * 2^e, m in [0.5, 1)
    sexp = np.where(amax > 0, e - 1 - 2, -127)
    sbyte = np.clip(sexp + 127, 0, 254)
    inv = np.ldexp(np.float32(1.0), (127 - sbyte).astype(np.int32)).astype(np.float32)
    q = np.abs(b) * inv[..., None]                 # exact: power-of-two scaling
    # piecewise-uniform E2M1 grid, np.rint rounds half to even (even code)
    code = np.where(q < 2.0, np.rint(q * 2.0),
           np.where(q < 4.0, 4.0 + np.rint(q - 2.0),
                    6.0 + np.rint(np.minimum(q, 6.0) * 0.5 - 2.0)))
    code = np.minimum(code, 7.0).astype(np.uint8)
    code |= np.where(b < 0, np.uint8(8), np.uint8(0))
    code = code.reshape(R, K)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return packed, sbyte.astype(np.uint8)


def _expert_weights(seed, e, D, I):
    g = _rng(seed, _TAG_GATE, e).standard_normal((I, D), dtype=np.float32) * np.float32(0.02)
    u = _rng(seed, _TAG_UP, e).standard_normal((I, D), dtype=np.float32) * np.float32(0.02)
    gc, gs = mxfp4_encode(g)
    uc, us = mxfp4_encode(u)
    del g, u
    d = _rng(seed, _TAG_DOWN, e).standard_normal((D, I), dtype=np.float32) * np.float32(0.02)
    dc, ds = mxfp4_encode(d)
    return e, np.concatenate([gc, uc]), np.concatenate([gs, us]), dc, ds


def _router_bias(seed, E, mode):
    br = _rng(seed, _TAG_BR).standard_normal(E, dtype=np.float32) * np.float32(0.01)
    if mode == "normal":
        return br
    if mode == "zipf":
        rank_of = _rng(seed, _TAG_PERM).permutation(E)      # expert id -> rank-1
        r = (rank_of + 1).astype(np.float64)
        br = (br.astype(np.float64) - ZIPF_BETA * ZIPF_S * np.log(r)).astype(np.float32)
        br[rank_of >= E - ZIPF_N_EMPTY] = _EMPTY_BIAS
        return br
    if mode.startswith("onehot"):
        # every token routes to expert `hot` (and the next k-1 by other logits)
        hot = int(mode[len("onehot"):] or 0)
        br = br.copy()
        br[hot] = 100.0
        return br
    raise ValueError(mode)


def make_inputs(cfg: int | dict = 0, *, T: int | None = None, x_scale: float = 1.0,
                bias: str | None = None, seed: int | None = None,
                threads: int | None = None, experts: bool = True) -> LayerInputs:
    """Build the inputs of one workload (a CONFIGS index or an explicit dict).

    T overrides the token count (same distributions, the first T rows of a
    longer draw are not guaranteed: x is drawn with shape [T][D]).  x_scale
    multiplies x before bf16 rounding (x8 drives most pre-activations into
    the +-7 clamp).  bias selects the router-bias recipe: "normal", "zipf" or
    "onehot<e>".  experts=False skips the expert weights (zero-size arrays),
    for routing-only checks.
    """
    c = dict(CONFIGS[cfg]) if isinstance(cfg, int) else dict(cfg)
    if T is not None:
        c["T"] = T
    if bias is not None:
        c["bias"] = bias
    if seed is not None:
        c["seed"] = seed
    c.setdefault("bias", "normal")
    Tn, D, E, k, I, s = c["T"], c["D"], c["E"], c["k"], c["I"], c["seed"]
    assert D % 32 == 0 and I % 32 == 0 and 1 <= k <= E
    x = _rng(s, _TAG_X).standard_normal((Tn, D), dtype=np.float32)
    if x_scale != 1.0:
        x = x * np.float32(x_scale)
    x_bf16 = f32_to_bf16_bits(x)
    wr = _rng(s, _TAG_WR).standard_normal((E, D), dtype=np.float32) * np.float32(0.02)
    br = _router_bias(s, E, c["bias"])

    Ew = E if experts else 0
    gu_codes = np.empty((Ew, 2 * I, D // 2), np.uint8)
    gu_scales = np.empty((Ew, 2 * I, D // 32), np.uint8)
    dn_codes = np.empty((Ew, D, I // 2), np.uint8)
    dn_scales = np.empty((Ew, D, I // 32), np.uint8)
    nthreads = threads or min(16, os.cpu_count() or 1)

    def store(res):
        e, gc, gs, dc, ds = res
        gu_codes[e], gu_scales[e], dn_codes[e], dn_scales[e] = gc, gs, dc, ds

    if Ew * D * I < 1 << 22 or nthreads == 1:
        for e in range(Ew):
            store(_expert_weights(s, e, D, I))
    else:
        with ThreadPoolExecutor(nthreads) as ex:
            for res in ex.map(lambda e: _expert_weights(s, e, D, I), range(Ew)):
                store(res)
    c["x_scale"] = x_scale
    gamma = np.float32(1.0) + _rng(s, _TAG_NORM).standard_normal(D, dtype=np.float32) * np.float32(0.1)
    return LayerInputs(Tn, D, E, k, I, SWIGLU_LIMIT, x_bf16, wr, br,
                       gu_codes, gu_scales, dn_codes, dn_scales, c, gamma, RMS_NORM_EPS)


def zipf_popularity(E: int) -> np.ndarray:
    """Normalised Zipf(ZIPF_S) shares by popularity rank (for reporting)."""
    p = np.arange(1, E + 1, dtype=np.float64) ** -ZIPF_S
    return p / p.sum()


__all__ = ["CONFIGS", "SWIGLU_LIMIT", "LayerInputs", "make_inputs", "mxfp4_encode",
           "f32_to_bf16_bits", "bf16_bits_to_f32", "zipf_popularity"]
