"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test names the fact it checks.  None of them re-types the oracle's own
formula: decode is checked against the bit-field definition, the layer
against an independent pure-Python dense brute force, the permutation against
a Python sort, closed forms against the numbers the pages print.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth
from tests import brute

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")))


# --------------------------------------------------------------------------- formats
def test_mxfp4_decode_exhaustive_16_codes_x_256_scales():
    """Every E2M1 code at every E8M0 scale byte equals the bit-field definition (OCP MX v1.0)."""
    codes = np.array([[c | (c << 4)] * 16 for c in range(16)], dtype=np.uint8)      # [16][16] -> 32 values
    for s in range(256):
        scales = np.full((16, 1), s, dtype=np.uint8)
        dec = oracle.mxfp4_decode(codes, scales)
        for c in range(16):
            want = brute.e2m1_value(c) * brute.e8m0_value(s)
            got = dec[c]
            if s == 255:
                assert np.all(np.isnan(got))
            else:
                assert np.all(got == want), (c, s, got[0], want)


def test_mxfp4_decode_nibble_order_and_block_scale():
    """Low nibble = even K index; scale byte j covers K in [32j, 32j+32)."""
    codes = np.zeros((1, 32), dtype=np.uint8)
    codes[0, 0] = 0x2 | (0x5 << 4)          # k=0 -> 1.0, k=1 -> 3.0
    codes[0, 16] = 0xF                       # k=32 -> -6
    scales = np.array([[127, 130]], dtype=np.uint8)
    d = oracle.mxfp4_decode(codes, scales)
    assert d[0, 0] == 1.0 and d[0, 1] == 3.0 and d[0, 32] == -48.0
    assert np.count_nonzero(d) == 3


def test_e2m1_magnitudes_are_the_format_grid():
    got = sorted({abs(brute.e2m1_value(c)) for c in range(16)})
    assert got == list(oracle.E2M1_MAGNITUDE)


def test_round_to_bf16_matches_bitwise_rounding():
    rng = np.random.default_rng(7)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-6, 3, 20000),
                        [1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 255.5, 0.0, 1 - 2 ** -10]])
    got = oracle.round_to_bf16(v)
    want = np.array([brute.bf16_round(float(a)) for a in v])
    assert np.array_equal(got, want)
    assert got[-6] == 1.0 and got[-5] == 1 + 2 ** -6 and got[-3] == 256.0


def test_storage_is_4_25_bits_per_parameter():
    fact = GOLD["mxfp4_bits_per_param"]["value"]
    inp = synth.make_inputs(0)
    n = inp.gu_codes.shape[0] * inp.gu_codes.shape[1] * inp.gu_codes.shape[2] * 2
    assert oracle.mxfp4_bits_per_param(n, inp.gu_codes.nbytes, inp.gu_scales.nbytes) == fact
    n = inp.dn_codes.size * 2
    assert oracle.mxfp4_bits_per_param(n, inp.dn_codes.nbytes, inp.dn_scales.nbytes) == fact
    # closed form per layer at the 20b / 120b shapes
    per_expert = 3 * 2880 * 2880 * fact / 8
    assert per_expert == 13_219_200
    assert 32 * per_expert == 423_014_400 and 128 * per_expert == 1_692_057_600


# --------------------------------------------------------------------------- quantizer used by the generator
def test_quantizer_round_to_nearest_even_ties_and_saturation():
    # block with amax in [4, 8) -> shared exponent 0, so the values are the E2M1 inputs themselves
    vals = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, 4.0, -0.25, -5.0, 0.0] + [0.0] * 20,
                    dtype=np.float32)
    codes, scales = synth.mxfp4_encode(vals[None, :])
    assert scales[0, 0] == 127
    dec = oracle.mxfp4_decode(codes, scales)[0]
    assert list(dec[:12]) == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0, 4.0, -0.0, -4.0, 0.0]


def test_quantizer_identity_on_grid_and_zero_block():
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float32)
    row = np.concatenate([grid, -grid, grid * 1.0, -grid]) * np.float32(2.0 ** -5)
    codes, scales = synth.mxfp4_encode(row[None, :])
    assert np.array_equal(oracle.mxfp4_decode(codes, scales)[0], row.astype(np.float64))
    codes, scales = synth.mxfp4_encode(np.zeros((1, 64), np.float32))
    assert np.all(codes == 0) and np.all(scales == 0)


def test_quantizer_error_bound():
    """|w - Q(w)| is at most half the local E2M1 step (times the block scale), or w is saturated."""
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    codes, scales = synth.mxfp4_encode(w)
    dec = oracle.mxfp4_decode(codes, scales)
    X = np.repeat(np.ldexp(1.0, scales.astype(int) - 127), 32, axis=1)
    q = np.abs(w) / X
    half_step = np.where(q < 2, 0.25, np.where(q < 4, 0.5, 1.0))
    err = np.abs(w - dec) / X
    assert np.all((err <= half_step + 1e-12) | (q > 6))
    amax = np.abs(w.reshape(64, -1, 32)).max(-1)
    assert np.all((amax / np.ldexp(1.0, scales.astype(int) - 127) >= 4) &
                  (amax / np.ldexp(1.0, scales.astype(int) - 127) < 8))


# --------------------------------------------------------------------------- activation and clamp
def test_silu_closed_forms():
    v = np.linspace(-30, 30, 1201)
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    assert np.allclose(oracle.silu(v) - oracle.silu(-v), v, rtol=0, atol=1e-12)
    assert np.allclose(oracle.silu(v), [x / (1 + math.exp(-x)) for x in v], rtol=1e-15, atol=0)


def test_swiglu_clamp_at_limit():
    L = GOLD["swiglu_limit"]["value"]
    g = np.array([0.5, -3.0, 6.99, 100.0, -100.0, 7.0])
    u = np.array([1.0, 2.0, -6.5, 100.0, 3.0, -50.0])
    got = oracle.swiglu(g, u, L)
    want = [brute_silu(min(max(a, -L), L)) * min(max(b, -L), L) for a, b in zip(g, u)]
    assert np.allclose(got, want, rtol=1e-15, atol=0)
    assert got[3] == pytest.approx(7.0 * 7.0 / (1 + math.exp(-7.0)) , rel=1e-15)
    # inside the limit the clamp is the identity
    assert got[0] == pytest.approx(brute_silu(0.5) * 1.0, rel=1e-15)


def brute_silu(x):
    return x / (1.0 + math.exp(-x))


# --------------------------------------------------------------------------- routing
def test_topk_and_gates_against_python_sort_with_exact_ties():
    rng = np.random.default_rng(11)
    T, E, k = 300, 16, 4
    L = np.round(rng.standard_normal((T, E)) * 4) / 4        # many exact ties
    idx, flagged, gap = oracle.select_experts(L, k)
    w = oracle.gate_weights(L, idx)
    for t in range(T):
        ranked = sorted(range(E), key=lambda e: (-L[t, e], e))
        assert list(idx[t]) == sorted(ranked[:k])
        assert len(set(idx[t])) == k
        assert flagged[t] == (L[t, ranked[k - 1]] - L[t, ranked[k]] < 1e-6)
        ex = [math.exp(L[t, e] - max(L[t, i] for i in idx[t])) for e in idx[t]]
        assert np.allclose(w[t], [a / sum(ex) for a in ex], rtol=1e-14, atol=0)
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-15)


def test_page_example_weights_0_7_0_3():
    """Top 2 of 4 experts with A = 0.7 NN2 + 0.3 NN4 (1-based on the page)."""
    ex = GOLD["router_example"]
    E, k = ex["n_experts"], ex["top_k"]
    inp = synth.make_inputs(dict(T=3, D=64, E=E, k=k, I=64, seed=5))
    inp.w_router[:] = 0.0
    inp.b_router[:] = np.array([0.0, math.log(7.0), -5.0, math.log(3.0)], dtype=np.float32)
    o = oracle.forward(inp)
    sel = [s - 1 for s in ex["selected_1based"]]
    assert all(list(r) == sel for r in o["idx"])
    # fp32 bias rounding moves the logits by < 1e-7 relative
    assert np.allclose(o["w"], [ex["weights"]] * 3, rtol=0, atol=2e-7)
    # y = w_a FFN_a(x) + w_b FFN_b(x), FFN evaluated by the independent brute force
    gu = [brute.decode_matrix(inp.gu_codes[e], inp.gu_scales[e]) for e in sel]
    dn = [brute.decode_matrix(inp.dn_codes[e], inp.dn_scales[e]) for e in sel]
    for t in range(3):
        xr = [brute.bf16_bits_value(int(b)) for b in inp.x_bf16[t]]
        z = [brute.expert_dense(xr, gu[i][:64], gu[i][64:], dn[i], 7.0)[1] for i in range(2)]
        want = np.array(z[0]) * o["w"][t, 0] + np.array(z[1]) * o["w"][t, 1]
        assert np.allclose(o["y"][t], want, rtol=1e-12, atol=1e-15 * np.abs(want).max())


def test_permutation_against_python_sort():
    rng = np.random.default_rng(2)
    for T, E, k in [(1, 4, 2), (37, 8, 3), (500, 32, 4), (64, 4, 4)]:
        L = rng.standard_normal((T, E))
        idx, _, _ = oracle.select_experts(L, k)
        counts, offsets, perm, inv = oracle.build_permutation(idx, E)
        pairs = sorted((int(idx[t, j]), t, t * k + j) for t in range(T) for j in range(k))
        assert list(perm) == [a for _, _, a in pairs]
        assert list(counts) == [sum(1 for e, _, _ in pairs if e == x) for x in range(E)]
        assert offsets[0] == 0 and offsets[-1] == T * k and np.all(np.diff(offsets) >= 0)
        assert np.array_equal(inv[perm], np.arange(T * k)) and np.array_equal(perm[inv], np.arange(T * k))
        for e in range(E):
            seg = perm[offsets[e]:offsets[e + 1]]
            assert np.all(idx.reshape(-1)[seg] == e) and np.all(np.diff(seg // k) > 0)


def test_router_special_cases():
    inp = synth.make_inputs(dict(T=8, D=64, E=4, k=2, I=64, seed=9), experts=False)
    inp.w_router[:] = 0.0
    L = oracle.router_logits(oracle.bf16_to_f64(inp.x_bf16), inp.w_router, inp.b_router)
    assert np.array_equal(L, np.tile(inp.b_router.astype(np.float64), (8, 1)))
    x = np.zeros((4, 64))
    x[np.arange(4), [0, 5, 17, 63]] = 1.0
    wr = np.random.default_rng(0).standard_normal((4, 64)).astype(np.float32)
    L = oracle.router_logits(x, wr, np.zeros(4, np.float32))
    assert np.array_equal(L, wr[:, [0, 5, 17, 63]].T.astype(np.float64))


# --------------------------------------------------------------------------- whole layer against the dense brute force
@pytest.mark.parametrize("case", [
    dict(cfg=0),
    dict(cfg=0, x_scale=64.0),                                       # clamp active (sigma ~10 at D=64)
    dict(cfg=dict(T=5, D=64, E=1, k=1, I=64, seed=21)),              # one expert: plain SwiGLU FFN
    dict(cfg=dict(T=6, D=64, E=3, k=3, I=64, seed=22)),              # k = E: dense MoE
    dict(cfg=dict(T=7, D=64, E=4, k=2, I=32 * 3, seed=23), bias="onehot2"),   # all tokens to one expert
    dict(cfg=dict(T=1, D=96, E=8, k=4, I=64, seed=24)),              # single token
])
def test_sparse_oracle_equals_dense_brute_force(case):
    inp = synth.make_inputs(case["cfg"], x_scale=case.get("x_scale", 1.0), bias=case.get("bias"))
    o = oracle.forward(inp)
    b = brute.brute_layer(inp)
    assert np.allclose(o["logits"], b["logits"], rtol=0, atol=1e-13)
    assert o["idx"].tolist() == b["idx"]
    assert np.allclose(o["w"], b["w"], rtol=1e-13, atol=0)
    yb = np.array(b["y"])
    scale = np.abs(yb).max()
    assert np.abs(o["y"] - yb).max() <= 1e-12 * scale
    if case.get("x_scale", 1.0) > 1.0:
        x = oracle.bf16_to_f64(inp.x_bf16)
        g = x @ oracle.mxfp4_decode(inp.gu_codes[0], inp.gu_scales[0]).T
        assert (np.abs(g) > 7).mean() > 0.2           # the clamp really binds


def test_one_expert_reduces_to_dense_swiglu():
    inp = synth.make_inputs(dict(T=9, D=128, E=1, k=1, I=64, seed=31))
    o = oracle.forward(inp)
    assert np.all(o["w"] == 1.0)
    x = np.array([[brute.bf16_bits_value(int(b)) for b in r] for r in inp.x_bf16])
    gu = np.array(brute.decode_matrix(inp.gu_codes[0], inp.gu_scales[0]))
    dn = np.array(brute.decode_matrix(inp.dn_codes[0], inp.dn_scales[0]))
    g = np.clip(x @ gu[:64].T, -7, 7)
    u = np.clip(x @ gu[64:].T, -7, 7)
    h = np.vectorize(brute.bf16_round)(g / (1 + np.exp(-g)) * u)
    assert np.allclose(o["y"], h @ dn.T, rtol=1e-12, atol=1e-16)


# --------------------------------------------------------------------------- closed forms
def test_param_counts_match_model_card():
    f = GOLD["params_20b"]
    a = GOLD["attention_shape"]
    c = oracle.gpt_oss_param_counts(f["n_layers"], GOLD["n_experts"]["gpt-oss-20b"], GOLD["top_k"]["value"],
                                    GOLD["d_model"]["value"], GOLD["intermediate_size"]["value"],
                                    a["n_q_heads"], a["n_kv_heads"], a["head_dim"], GOLD["vocab"]["value"])
    assert c["total"] == 20_907_786_240 and round(c["total"] / 1e9, 1) == f["total_billion"]
    assert c["active"] == 3_607_142_400 and round(c["active"] / 1e9, 1) == f["active_billion"]
    assert c["experts_all_layers"] / c["total"] > GOLD["moe_param_share"]["value_gt"]


def test_memory_fit_closed_form():
    fit = GOLD["memory_fit"]
    bits = GOLD["mxfp4_bits_per_param"]["value"]
    for name, layers, E, cap in (("20b", 24, 32, fit["gpt-oss-20b_GB"]), ("120b", 36, 128, fit["gpt-oss-120b_GB"])):
        c = oracle.gpt_oss_param_counts(layers, E, 4)
        moe_bytes = c["experts_all_layers"] * bits / 8
        rest_bytes = (c["total"] - c["experts_all_layers"]) * 2          # bf16
        total_gb = (moe_bytes + rest_bytes) / 1e9
        assert total_gb < cap, (name, total_gb)
        # without MXFP4 (bf16 experts) neither fits
        assert (c["total"] * 2) / 1e9 > cap


def test_swiglu_parameter_example():
    f = GOLD["swiglu_param_example"]
    assert 2 * f["d"] * f["ffn_hidden"] == f["ffn_fc1_plus_fc2"]
    assert f["d"] * f["d"] == f["glu_matrix"] and 3 * f["glu_matrix"] == f["glu_total"]


# --------------------------------------------------------------------------- workload structure
def test_skewed_workload_structure():
    """Top 10% of experts take about half of the assignments and 4 experts get no token."""
    inp = synth.make_inputs(4, experts=False)
    L = oracle.router_logits(oracle.bf16_to_f64(inp.x_bf16), inp.w_router, inp.b_router)
    idx, flagged, _ = oracle.select_experts(L, inp.k)
    counts = np.bincount(idx.ravel(), minlength=inp.E)
    top = np.sort(counts)[::-1]
    share = top[: round(0.1 * inp.E)].sum() / (inp.T * inp.k)
    assert 0.48 <= share <= 0.52, share
    assert (counts == 0).sum() == 4
    assert flagged.sum() <= 2


@pytest.mark.parametrize("cfg", [0, 1, 2, 3])
def test_workload_routing_has_no_near_ties(cfg):
    inp = synth.make_inputs(cfg, experts=False)
    L = oracle.router_logits(oracle.bf16_to_f64(inp.x_bf16), inp.w_router, inp.b_router)
    idx, flagged, gap = oracle.select_experts(L, inp.k)
    counts = np.bincount(idx.ravel(), minlength=inp.E)
    assert flagged.sum() <= 2
    if cfg == 1:
        assert (counts > 0).sum() >= 28          # near-uniform load at decode


# --------------------------------------------------------------------------- RMSNorm and residual block
def test_rms_norm_hand_computed_row():
    """[3, 4, 0, 0]: mean square 25/4, RMS 2.5, so 1.2 and 1.6; bf16 keeps 8 significant bits
    (1.0011001|1001.. and 1.1001100|1100.. both round up): 1.203125 and 1.6015625."""
    got = oracle.rms_norm(np.array([[3.0, 4.0, 0.0, 0.0]]), np.ones(4), 0.0)
    assert got.tolist() == [[1.203125, 1.6015625, 0.0, 0.0]]


def test_rms_norm_divides_by_the_mean_not_the_sum():
    """Fifteen ones and a seven: sum of squares 64 over 16 channels, mean 4, RMS 2 (exact)."""
    x = np.array([[1.0] * 15 + [7.0]])
    assert oracle.rms_norm(x, np.ones(16), 0.0).tolist() == [[0.5] * 15 + [3.5]]


def test_rms_norm_eps_is_added_to_the_mean_square():
    """Constant rows of 1/8 with eps = 3/64 (exact in fp32): sqrt(1/64 + 3/64) = 1/4, output 1/2."""
    x = np.full((3, 64), 0.125)
    assert np.all(oracle.rms_norm(x, np.ones(64), 3.0 / 64.0) == 0.5)


def test_rms_norm_scale_is_per_channel():
    """A constant row has RMS equal to its value, so with eps = 0 the output is gamma itself."""
    gamma = np.array([1.0, 2.0, 0.5, -1.0, 0.25, 3.0, -0.75, 1.5])
    assert np.array_equal(oracle.rms_norm(np.full((2, 8), 2.0), gamma, 0.0), np.tile(gamma, (2, 1)))


def test_rms_norm_is_invariant_to_power_of_two_scaling_and_has_unit_rms():
    """RMSNorm(2^j x) = RMSNorm(x) bit for bit when eps = 0 (every step scales exactly); the
    normalised rows have mean square 1 up to the bf16 rounding (relative 2^-8)."""
    x = synth.bf16_bits_to_f32(synth.make_inputs(0).x_bf16).astype(np.float64)
    base = oracle.rms_norm(x, np.ones(x.shape[1]), 0.0)
    for j in (-7, -1, 3, 20):
        assert np.array_equal(oracle.rms_norm(x * 2.0 ** j, np.ones(x.shape[1]), 0.0), base)
    assert np.allclose(np.mean(base ** 2, axis=1), 1.0, rtol=2.0 ** -7)


def test_block_with_zero_experts_returns_its_input():
    """All-zero expert weights (code 0 is +0): the MoE output is 0 and the block output is x."""
    inp = synth.make_inputs(0)
    inp.gu_codes[:] = 0
    inp.dn_codes[:] = 0
    o = oracle.block_forward(inp)
    assert np.all(o["y_moe"] == 0.0)
    assert np.array_equal(o["y"], oracle.bf16_to_f64(inp.x_bf16))


def test_block_is_the_layer_on_the_normalised_rows_plus_the_input():
    """block_forward = forward on bf16(RMSNorm(x)) (itself pinned by the dense brute force),
    plus x."""
    import dataclasses
    inp = synth.make_inputs(dict(T=9, D=64, E=4, k=2, I=64, seed=7))
    o = oracle.block_forward(inp)
    xn = oracle.rms_norm(oracle.bf16_to_f64(inp.x_bf16), inp.norm_weight, inp.norm_eps)
    inner = dataclasses.replace(inp, x_bf16=synth.f32_to_bf16_bits(xn.astype(np.float32)))
    ref = np.array(brute.brute_layer(inner)["y"])
    assert np.abs(o["y_moe"] - ref).max() <= 1e-12 * np.abs(ref).max()
    assert np.array_equal(o["y"], oracle.bf16_to_f64(inp.x_bf16) + o["y_moe"])


# --------------------------------------------------------------------------- activation-quantized variant
def test_act4_quantizer_ocp_ties_saturation_and_exponent():
    """OCP MX conversion to MXFP4: a block with amax 7 keeps exponent 0, so its values are the
    E2M1 inputs: ties 0.25 -> 0, 0.75 -> 1, 1.25 -> 1, 1.75 -> 2, 2.5 -> 2, 3.5 -> 4, 5 -> 4 (even
    codes), 7 saturates to 6.  A block with amax 0.3 takes exponent floor(log2 0.3) - 2 = -4:
    0.3 / 2^-4 = 4.8 -> 4, i.e. 0.25.  An all-zero block stays zero."""
    v = np.array([[0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, 4.0, -0.25, -5.0, 0.0] + [0.0] * 20
                  + [0.3, 0.03, -0.1] + [0.0] * 29 + [0.0] * 32])
    q = oracle.mxfp4_quantize_rows(v)[0]
    assert q[:12].tolist() == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0, 4.0, 0.0, -4.0, 0.0]
    # 0.03 / 2^-4 = 0.48 -> 0.5 (0.03125); -0.1 / 2^-4 = -1.6 -> -1.5 (-0.09375)
    assert q[32:35].tolist() == [0.25, 0.03125, -0.09375]
    assert np.all(q[64:] == 0.0)


def test_act4_quantizer_is_idempotent_and_within_half_a_step():
    """Quantizing twice changes nothing; every element is within half the local E2M1 step of
    its input (times the block scale), or saturated at 6 times the scale."""
    rng = np.random.default_rng(11)
    v = rng.standard_normal((8, 256)) * np.exp(rng.uniform(-8, 8, (8, 1)))
    q = oracle.mxfp4_quantize_rows(v)
    assert np.array_equal(oracle.mxfp4_quantize_rows(q), q)
    b = v.reshape(8, -1, 32)
    E = np.floor(np.log2(np.abs(b).max(-1, keepdims=True))) - 2
    r = np.abs(b) / 2.0 ** E
    half_step = np.where(r < 2, 0.25, np.where(r < 4, 0.5, 1.0))
    err = np.abs(b - q.reshape(b.shape)) / 2.0 ** E
    assert np.all((err <= half_step + 1e-12) | ((r > 6) & (np.abs(q.reshape(b.shape)) == 6 * 2.0 ** E)))


@pytest.mark.parametrize("case", [
    dict(cfg=0),
    dict(cfg=dict(T=5, D=64, E=1, k=1, I=64, seed=25)),              # one expert
    dict(cfg=dict(T=6, D=64, E=3, k=3, I=64, seed=26)),              # k = E
    dict(cfg=dict(T=1, D=96, E=8, k=4, I=64, seed=27)),              # single token
])
def test_act4_oracle_equals_dense_brute_force(case):
    """The activation-quantized layer against the pure-Python dense evaluation with its own
    element-by-element MXFP4 quantizer."""
    inp = synth.make_inputs(case["cfg"])
    o = oracle.forward(inp, act4=True)
    b = brute.brute_layer(inp, act4=True)
    assert o["idx"].tolist() == b["idx"]
    yb = np.array(b["y"])
    assert np.abs(o["y"] - yb).max() <= 1e-12 * np.abs(yb).max()
    # and it is not the W4A16 layer
    assert not np.allclose(o["y"], oracle.forward(inp)["y"], rtol=1e-3, atol=0)
