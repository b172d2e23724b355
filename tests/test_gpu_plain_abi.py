"""GPU parity of the plain step-by-step boundary (bf16 rows, perm and offsets, scratch from ws),
through the C ABI.

Bars: moe_permute's counts, offsets, perm and inv equal to moe_permute_tiles's, and the tile table
it leaves in its scratch is the valid table for that grouping, as is the one moe_expert_gemm_mxfp4
builds from perm and offsets; moe_expert_gemm_mxfp4's bf16 h,
packed with moe_pack_act, equals the packed gate/up stage's bytes bit for bit (it is the value that
stage splits); its down stage on that h equals the packed down stage's y_perm bit for bit; and the
whole plain sequence holds every oracle bar of the layer tests (tests/parity.py), with h compared
through its packed form.
"""
import json
import time

import numpy as np
import pytest

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


def _np(t):
    return t.cpu().numpy()


def _bits16(t):
    return t.contiguous().view(torch.int16).cpu().numpy()


def _plain_check(name, inp, tokens=None):
    import mxfp4_expert_layer_moe_amd as M
    from mxfp4_expert_layer_moe_amd.device import DeviceLayer
    print(f"[plain] start {name} T={inp.T} D={inp.D} E={inp.E} k={inp.k} I={inp.I}", flush=True)
    t0 = time.time()
    layer = DeviceLayer(inp)
    T, k, D, I = inp.T, inp.k, inp.D, inp.I
    n = T * k
    # the packed operand path
    layer.route()
    layer.permute()
    layer.pack_x()
    layer.gate_up()
    layer.down()
    torch.cuda.synchronize()
    ref = dict(counts=_np(layer.counts), offsets=_np(layer.offsets), perm=_np(layer.perm), inv=_np(layer.inv),
               h_packed=_np(layer.h_packed)[: M.moe_act_pack_bytes(I, n)], y_perm=_bits16(layer.y_perm))
    # the plain path on the same routing, every output poisoned first
    for t in (layer.counts, layer.offsets, layer.perm, layer.inv):
        t.fill_(-7)
    layer.ws.fill_(0xA5)
    layer.y_perm.fill_(float("nan"))
    layer.permute_plain()
    torch.cuda.synchronize()
    tiles = layer.ws[: M.moe_tile_table_bytes(layer.dims, T)].view(torch.int32).cpu().numpy()
    h = torch.full((n, I), float("nan"), dtype=torch.bfloat16, device="cuda")
    layer.ws.fill_(0x5A)
    layer.gate_up_plain(h)
    torch.cuda.synchronize()
    # the table the expert GEMM built in its scratch from perm and offsets
    parity.check_tiles(layer.ws[: M.moe_tile_table_bytes(layer.dims, T)].view(torch.int32).cpu().numpy(),
                       ref["offsets"], ref["perm"], n, inp.E)
    layer.down_plain(h)
    hp = torch.empty(max(M.moe_act_pack_bytes(I, n), 16), dtype=torch.uint8, device="cuda")
    M.moe_pack_act(I, n, h, hp)
    torch.cuda.synchronize()
    for key in ("counts", "offsets", "perm", "inv"):
        assert np.array_equal(_np(getattr(layer, key)), ref[key]), key
    # the packed rows' defined bytes: per 112-byte chunk, codes and scales [0, 100); bytes [100, 112)
    # are unused and left unwritten by both writers
    rb = M.moe_act_pack_bytes(I, 1)
    used = (np.arange(rb) % 112) < 100
    got = _np(hp)[: M.moe_act_pack_bytes(I, n)].reshape(n, rb)[:, used]
    want = ref["h_packed"].reshape(n, rb)[:, used]
    assert not np.isnan(h.float().cpu().numpy()).any(), "the plain gate/up left h values unwritten"
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        raise AssertionError(f"packed plain h differs: {len(bad)} bytes in rows {np.unique(bad[:, 0])[:12]}")
    assert np.array_equal(_bits16(layer.y_perm), ref["y_perm"]), "plain y_perm differs"
    # the plain outputs against the oracle
    layer.pack_x()
    layer.combine(bf16=False)
    layer.combine(bf16=True)
    torch.cuda.synchronize()
    g = dict(idx=_np(layer.topk_idx), w=_np(layer.topk_w), logits=_np(layer.logits), counts=_np(layer.counts),
             offsets=_np(layer.offsets), perm=_np(layer.perm), inv=_np(layer.inv), tiles=tiles,
             x_packed=_np(layer.x_packed), h_packed=_np(hp), y_perm=_np(layer.y_perm), y32=_np(layer.y32),
             y16=_bits16(layer.y16).view(np.uint16))
    o = parity.oracle_with_adoption(inp, g["idx"], tokens=tokens)
    stats = parity.compare(inp, g, o)
    stats["seconds"] = round(time.time() - t0, 1)
    print(f"[plain] {name}: " + json.dumps(stats), flush=True)
    parity.record_stats("plain_" + name, stats)


CASES = {
    "tiny": dict(cfg=0),
    "single_token": dict(cfg=dict(T=1, D=128, E=8, k=4, I=128, seed=40)),
    "ragged": dict(cfg=dict(T=37, D=192, E=5, k=3, I=320, seed=43)),
    "prefill_tiles": dict(cfg=dict(T=200, D=256, E=8, k=2, I=512, seed=46)),
    "skewed_small": dict(cfg=dict(T=96, D=128, E=16, k=4, I=192, seed=47)),
}


@pytest.mark.parametrize("name", list(CASES))
def test_plain_boundary_small(name):
    _plain_check(name, synth.make_inputs(CASES[name]["cfg"]))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg,n_tokens", [(1, None), (2, 32)])
def test_plain_boundary_full_size(cfg, n_tokens):
    inp = synth.make_inputs(cfg)
    tokens = None if n_tokens is None else np.sort(np.random.default_rng(300 + cfg).choice(inp.T, n_tokens,
                                                                                         replace=False))
    _plain_check(f"config{cfg}", inp, tokens)
