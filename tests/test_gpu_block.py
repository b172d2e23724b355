"""GPU parity of the pre-norm block around the layer, y = x + MoE(RMSNorm(x)), through the C ABI.

Bars: the normalised rows bit-exact (both sides compute the RMS in float64 and round once to
bf16); on those rows, every bar of the layer tests (routing and permutation bit-exact, gates
within 1e-6, MoE output within 2e-2 x its RMS); the residual output equal to the fp32 sum
x + (MoE output) bit for bit, bf16 output its round to nearest even; moe_block_forward
equal to the step-by-step sequence bit for bit.
"""
import dataclasses
import json
import time

import numpy as np
import pytest

import oracle
import synth
from tests import parity

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
    print(f"[block] {name}: " + json.dumps(stats), flush=True)
    parity.record_stats("block_" + name, stats)


def _u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _block_check(name, inp, tokens=None):
    from mxfp4_expert_layer_moe_amd.device import DeviceLayer
    print(f"[block] start {name} T={inp.T} D={inp.D} E={inp.E} k={inp.k} I={inp.I}", flush=True)
    t0 = time.time()
    layer = DeviceLayer(inp)
    T, D = inp.T, inp.D
    x32 = synth.bf16_bits_to_f32(inp.x_bf16)
    # 1. RMSNorm: bit-exact against the oracle
    layer.rmsnorm()
    torch.cuda.synchronize()
    xn_bits = _u16(layer.xn)
    want = oracle.f64_to_bf16_bits(oracle.rms_norm(x32.astype(np.float64), inp.norm_weight, inp.norm_eps))
    mism = int((xn_bits != want).sum())
    assert mism == 0, f"{mism} normalised values differ"
    # 2. the layer on the normalised rows: every intermediate against the oracle
    inner = dataclasses.replace(inp, x_bf16=xn_bits)
    layer.route(x=layer.xn)
    layer.permute()
    layer.pack_x(x=layer.xn)
    layer.gate_up()
    layer.down()
    layer.combine(bf16=False)
    layer.combine(bf16=True)
    torch.cuda.synchronize()
    g = dict(idx=layer.topk_idx.cpu().numpy(), w=layer.topk_w.cpu().numpy(), counts=layer.counts.cpu().numpy(),
             offsets=layer.offsets.cpu().numpy(), perm=layer.perm.cpu().numpy(), inv=layer.inv.cpu().numpy(),
             tiles=layer.tiles.cpu().numpy(), x_packed=layer.x_packed.cpu().numpy(),
             h_packed=layer.h_packed.cpu().numpy(), y_perm=layer.y_perm.cpu().numpy(),
             y32=layer.y32.cpu().numpy(), y16=_u16(layer.y16), logits=layer.logits.cpu().numpy())
    o = parity.oracle_with_adoption(inner, g["idx"], tokens=tokens)
    stats = parity.compare(inner, g, o)
    moe32 = g["y32"].copy()
    # 3. residual: one fp32 addition, bit-exact; bf16 its rounding
    layer.combine(bf16=False, residual=layer.x)
    layer.combine(bf16=True, residual=layer.x)
    torch.cuda.synchronize()
    y32, y16 = layer.y32.cpu().numpy(), _u16(layer.y16)
    assert np.array_equal(y32, x32 + moe32)
    assert np.array_equal(y16, parity.rne_bf16_bits(y32))
    # 4. the block entry point gives the same bits as the steps
    b32 = layer.block_forward(bf16=False).clone()
    b16 = _u16(layer.block_forward(bf16=True))
    torch.cuda.synchronize()
    assert np.array_equal(b32.cpu().numpy(), y32)
    assert np.array_equal(b16, y16)
    # and against the oracle's block output on the evaluated tokens: oracle.block_forward is the
    # input row plus the layer on the normalised rows, which o already holds (same adoption)
    ob_y = x32[o["tokens"]].astype(np.float64) + o["y"]
    dy = np.abs(y32[o["tokens"]].astype(np.float64) - ob_y).max()
    rms_moe = float(np.sqrt(np.mean(o["y"] ** 2)))
    stats["block_y_max_err_over_rms_moe"] = float(dy / rms_moe)
    assert dy <= parity.TOL_Y * rms_moe
    stats["seconds"] = round(time.time() - t0, 1)
    _record(name, stats)


SMALL = {
    "tiny": dict(cfg=0),
    "ragged": dict(cfg=dict(T=37, D=192, E=5, k=3, I=320, seed=43)),
    "single_token": dict(cfg=dict(T=1, D=128, E=8, k=4, I=128, seed=40)),
    "multi_tile": dict(cfg=dict(T=200, D=256, E=8, k=2, I=512, seed=46)),
    "large_activations_x8": dict(cfg=dict(T=24, D=128, E=8, k=2, I=128, seed=52), x_scale=8.0),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_block_small_case_parity(name):
    c = SMALL[name]
    _block_check(name, synth.make_inputs(c["cfg"], x_scale=c.get("x_scale", 1.0)))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg,n_tokens", [(1, None), (2, 32), (3, 512), (4, 512)])
def test_block_full_size_workload(cfg, n_tokens):
    inp = synth.make_inputs(cfg)
    tokens = None if n_tokens is None else np.sort(np.random.default_rng(200 + cfg).choice(inp.T, n_tokens,
                                                                                         replace=False))
    _block_check(f"config{cfg}", inp, tokens)


@pytest.mark.parametrize("D,T", [(4096, 33), (4160, 5), (8192, 3)])
def test_rmsnorm_rows_at_and_past_the_one_wavefront_width(D, T):
    """moe_rmsnorm alone at d_model 4096 (the widest row one wavefront normalises), 4160 (the first
    width past it, normalised by a 512-thread workgroup per row) and 8192: bit-exact against the
    oracle."""
    import mxfp4_expert_layer_moe_amd as M
    inp = synth.make_inputs(dict(T=T, D=D, E=4, k=2, I=64, seed=70 + D % 97), experts=False)
    print(f"[block] rmsnorm T={T} D={D}", flush=True)
    d = M.dims(D, 64, 4, 2)
    x = torch.from_numpy(inp.x_bf16.view(np.int16)).to("cuda").view(torch.bfloat16)
    gamma = torch.from_numpy(np.ascontiguousarray(inp.norm_weight, dtype=np.float32)).to("cuda")
    xn = torch.empty_like(x)
    M.moe_rmsnorm(d, T, x, gamma, inp.norm_eps, xn)
    torch.cuda.synchronize()
    want = oracle.f64_to_bf16_bits(oracle.rms_norm(synth.bf16_bits_to_f32(inp.x_bf16).astype(np.float64),
                                                   inp.norm_weight, inp.norm_eps))
    got = _u16(xn)
    assert int((got != want).sum()) == 0
