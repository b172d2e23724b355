"""GPU parity of the activation-quantized variant (MXFP4 activations into the expert GEMMs)
against the oracle's act4 mode, through the C ABI.

Bars: routing, counts, offsets, the permutation and the tile table bit-exact (the routing of
the default path); the packed MXFP4 x equal in value to the oracle's quantization of x; the
quantized h equal to the oracle's except where the two bf16 h values (fp32 with hardware
transcendentals against float64) round differently next to an E2M1 rounding boundary (a
fraction below 1e-3 of the elements); y within 2e-2 x RMS(y) of the act4 oracle; the bf16
output equal to RNE(fp32); moe_forward_act4 equal to the step calls and deterministic.
"""
import json
import time

import numpy as np
import pytest

import oracle
import synth
from tests import actpack, parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu-marked tests need an MI355X")
    import mxfp4_expert_layer_moe_amd as M
    M.lib()                     # fails loudly if the HIP library is missing
    yield


def _record(name, stats):
    print(f"[act4] {name}: " + json.dumps(stats), flush=True)
    parity.record_stats("act4_" + name, stats)


def _u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _act4_check(name, inp, tokens=None):
    from mxfp4_expert_layer_moe_amd.device import DeviceLayer
    print(f"[act4] start {name} T={inp.T} D={inp.D} E={inp.E} k={inp.k} I={inp.I}", flush=True)
    t0 = time.time()
    layer = DeviceLayer(inp)
    T, D, I, k = inp.T, inp.D, inp.I, inp.k
    layer.steps_act4(bf16=False)
    layer.combine(bf16=True)
    torch.cuda.synchronize()
    g = dict(idx=layer.topk_idx.cpu().numpy(), w=layer.topk_w.cpu().numpy(), counts=layer.counts.cpu().numpy(),
             offsets=layer.offsets.cpu().numpy(), perm=layer.perm.cpu().numpy(), inv=layer.inv.cpu().numpy(),
             tiles=layer.tiles.cpu().numpy(), y32=layer.y32.cpu().numpy(), y16=_u16(layer.y16))
    x4 = actpack.decode4(layer.x_packed4.cpu().numpy(), D, T)
    h4 = actpack.decode4(layer.h_packed4.cpu().numpy(), I, T * k)
    o = parity.oracle_with_adoption(inp, g["idx"], tokens=tokens, act4=True)
    stats = dict(n_flagged=o["n_flagged"], n_adopted=o["n_adopted"])
    # routing and grouping: bit-exact
    for key in ("idx", "counts", "offsets", "perm", "inv"):
        assert np.array_equal(g[key], o[key]), key
    parity.check_tiles(g["tiles"], o["offsets"], o["perm"], T * k, inp.E)
    assert np.abs(g["w"].astype(np.float64) - o["w"]).max() <= parity.TOL_W
    # MXFP4 x: the oracle's quantization, exactly
    xq = oracle.mxfp4_quantize_rows(oracle.bf16_to_f64(inp.x_bf16))
    assert np.array_equal(x4, xq), int((x4 != xq).sum())
    # MXFP4 h at the evaluated positions
    pos = sorted(o["h"].keys())
    if pos:
        ho = np.array([o["h"][p] for p in pos])
        diff = h4[pos] != ho
        stats["h_code_mismatch_frac"] = float(diff.mean())
        assert diff.mean() <= 1e-3, diff.mean()
    # output
    rms_y = float(np.sqrt(np.mean(o["y"] ** 2)))
    dy = np.abs(g["y32"][o["tokens"]].astype(np.float64) - o["y"])
    stats["rms_y"] = rms_y
    stats["y_max_err_over_rms"] = float(dy.max() / rms_y)
    assert dy.max() <= parity.TOL_Y * rms_y, stats
    assert np.array_equal(g["y16"], parity.rne_bf16_bits(g["y32"]))
    # the act4 layer is a different contract from the default one: report how far it lands
    stats["seconds"] = round(time.time() - t0, 1)
    # forward = steps, deterministic
    f1 = layer.forward_act4(bf16=False).clone()
    f2 = layer.forward_act4(bf16=False).clone()
    torch.cuda.synchronize()
    assert torch.equal(f1, f2)
    assert np.array_equal(f1.cpu().numpy(), g["y32"])
    _record(name, stats)


SMALL = {
    "tiny": dict(cfg=0),
    "ragged": dict(cfg=dict(T=37, D=192, E=5, k=3, I=320, seed=43)),
    "single_token": dict(cfg=dict(T=1, D=128, E=8, k=4, I=128, seed=40)),
    "multi_tile": dict(cfg=dict(T=200, D=256, E=8, k=2, I=512, seed=46)),
    "k_tail_groups": dict(cfg=dict(T=70, D=320, E=4, k=2, I=448, seed=47)),
    # 8-row tiles up to 6 assignments per expert (48 = 6 x 8), 128-row tiles past it
    "decode_tiles_at_limit": dict(cfg=dict(T=24, D=64, E=8, k=2, I=64, seed=53)),
    "prefill_tiles_past_limit": dict(cfg=dict(T=25, D=64, E=8, k=2, I=64, seed=54)),
    # pre-activations far past the clamp, and MXFP4 block scales well above 2^0
    "large_activations_x8": dict(cfg=dict(T=24, D=128, E=8, k=2, I=128, seed=52), x_scale=8.0),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_act4_small_case_parity(name):
    c = SMALL[name]
    _act4_check(name, synth.make_inputs(c["cfg"], x_scale=c.get("x_scale", 1.0)))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg,n_tokens", [(1, None), (2, 32), (3, 32), (4, 512)])
def test_act4_full_size_workload(cfg, n_tokens):
    inp = synth.make_inputs(cfg)
    tokens = None if n_tokens is None else np.sort(np.random.default_rng(300 + cfg).choice(inp.T, n_tokens,
                                                                                         replace=False))
    _act4_check(f"config{cfg}", inp, tokens)
