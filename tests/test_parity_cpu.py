"""CPU tests of the parity machinery (tests/parity.py) that the GPU tests rely on.

A host emulation of the library's arithmetic (the activation split of tests/actpack.py, float64
products, bf16 h, fp16 gated rows, an fp32 slot-order combine) stands in for the GPU results.
The derived bars must accept it, and must reject each planted mistake: a wrong expert, a
permutation swap, a perturbed h element, a perturbed y_perm element, a dropped gate.
Nothing here runs on the GPU or touches the HIP library.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import actpack, parity


def _f16(v):
    return v.astype(np.float16)


def _tiles(o, n, E):
    bm = 8 if n <= 6 * E else 128
    ints = max(48, 4 + bm)
    slots = -(-n // bm) + min(E, n)
    t = np.zeros((slots, ints), np.int32)
    s = 0
    for e in range(E):
        for p0 in range(int(o["offsets"][e]), int(o["offsets"][e + 1]), bm):
            rows = min(bm, int(o["offsets"][e + 1]) - p0)
            t[s, :3] = [e, p0, rows]
            t[s, 4:4 + rows] = o["perm"][p0:p0 + rows]
            s += 1
    t[:, 3] = s
    t[s:, 0] = -1
    return t.reshape(-1)


def emulate(inp, o):
    """GPU-shaped results computed on the host with the library's encodings."""
    T, k, D, I, E = inp.T, inp.k, inp.D, inp.I, inp.E
    x = oracle.bf16_to_f64(inp.x_bf16)
    xp = actpack.encode(x)
    xs = actpack.decode_sum(xp, D, T)
    n = T * k
    hp = np.zeros((n, actpack.row_bytes(I)), np.uint8)
    yp = np.zeros((n, D), np.float16)
    for e in range(E):
        seg = np.arange(o["offsets"][e], o["offsets"][e + 1])
        if seg.size == 0:
            continue
        a = o["perm"][seg]
        wgu = oracle.mxfp4_decode(inp.gu_codes[e], inp.gu_scales[e])
        gu = xs[a // k] @ wgu.T
        h = oracle.round_to_bf16(oracle.swiglu(gu[:, :I], gu[:, I:], inp.swiglu_limit))
        hp[seg] = actpack.encode(h)
        hs = actpack.decode_sum(hp[seg], I, len(seg))
        z = hs @ oracle.mxfp4_decode(inp.dn_codes[e], inp.dn_scales[e]).T
        w32 = o["w"].astype(np.float32)[a // k, a % k].astype(np.float64)
        yp[seg] = _f16((w32[:, None] * z).astype(np.float32))
    y32 = np.zeros((T, D), np.float32)
    for j in range(k):
        y32 = y32 + yp[o["inv"][np.arange(T) * k + j]].astype(np.float32)
    return dict(idx=o["idx"].copy(), w=o["w"].astype(np.float32), logits=o["logits"].astype(np.float32),
                counts=o["counts"].copy(), offsets=o["offsets"].copy(), perm=o["perm"].copy(),
                inv=o["inv"].copy(), tiles=_tiles(o, n, E), x_packed=xp.reshape(-1), h_packed=hp.reshape(-1),
                y_perm=yp, y32=y32, y16=parity.rne_bf16_bits(y32))


CASES = {
    "decode_tiles": dict(T=24, D=128, E=8, k=2, I=192, seed=90),
    "prefill_tiles": dict(T=200, D=256, E=4, k=2, I=128, seed=91),
    "clamp_x8": dict(T=32, D=128, E=4, k=2, I=64, seed=92),
}


@pytest.fixture(scope="module", params=list(CASES))
def case(request):
    c = CASES[request.param]
    inp = synth.make_inputs(c, x_scale=8.0 if request.param == "clamp_x8" else 1.0)
    o = parity.oracle_with_adoption(inp, oracle.forward(inp)["idx"])
    return inp, o, emulate(inp, o)


def test_bars_accept_the_emulated_path(case):
    inp, o, g = case
    stats = parity.compare(inp, g, o)
    assert stats["h_err_over_bar_max"] < 1.0 and stats["y_perm_err_over_bar_max"] < 1.0


def _fails(inp, g, o):
    with pytest.raises(AssertionError):
        parity.compare(inp, g, o)


def test_bars_reject_a_wrong_expert(case):
    inp, o, g = case
    g = dict(g, idx=g["idx"].copy())
    g["idx"][0, 0] = (g["idx"][0, 0] + 1) % inp.E
    _fails(inp, g, o)


def test_bars_reject_a_permutation_swap(case):
    inp, o, g = case
    g = dict(g, perm=g["perm"].copy())
    g["perm"][[0, 1]] = g["perm"][[1, 0]]
    _fails(inp, g, o)


def test_bars_reject_a_perturbed_h_element(case):
    inp, o, g = case
    I, n = inp.I, inp.T * inp.k
    rb = actpack.row_bytes(I)
    hp = g["h_packed"].reshape(n, rb).copy()
    # raise the hi code of element 3 of row 5 by a few steps: far more than one bf16 ulp
    hs = actpack.decode_sum(hp[5:6], I, 1)
    v = hs.copy()
    v[0, 3] += 0.25 * max(abs(v[0, 3]), 0.25)
    v = oracle.round_to_bf16(v)
    hp[5] = actpack.encode(v)[0]
    _fails(inp, dict(g, h_packed=hp.reshape(-1)), o)


def test_bars_reject_a_perturbed_y_perm_element(case):
    inp, o, g = case
    yp = g["y_perm"].copy()
    c = int(np.argmax(np.abs(yp[7].astype(np.float32))))
    yp[7, c] = -yp[7, c]                               # a sign error on the row's largest value
    _fails(inp, dict(g, y_perm=yp), o)


def test_bars_reject_a_dropped_gate(case):
    inp, o, g = case
    yp = g["y_perm"].copy()
    a = o["perm"][3]
    yp[3] = _f16(yp[3].astype(np.float32) / np.float32(o["w"][a // inp.k, a % inp.k]))
    _fails(inp, dict(g, y_perm=yp), o)


def test_tolerance_decoder_equals_the_oracle_decoder():
    rng = np.random.default_rng(93)
    codes = rng.integers(0, 256, size=(64, 96), dtype=np.uint8)
    scales = rng.integers(2, 252, size=(64, 6), dtype=np.uint8)        # 2^-125 .. 2^124 (x6 fits fp32)
    assert np.array_equal(parity.weights_f32(codes, scales).astype(np.float64), oracle.mxfp4_decode(codes, scales))
