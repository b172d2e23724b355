"""GPU parity of the HIP path against the float64 oracle, through the C ABI.

Bars: routing indices, counts, offsets and the permutation bit-exact (near-tie
tokens handled by adoption, see tests/parity.py); gates within 1e-6; layer
output within 2e-2 x RMS(y); the bf16 output equal to RNE(fp32 output).
Intermediates: h and y_perm element by element within the derived bars of
tests/parity.py.  Every case compares every token except the batches larger
than the benchmark workloads, which compare routing for all tokens and the
expert outputs on a seeded sample.  The full-size workloads also run the
whole-layer entry point the benchmark times (moe_forward) and require its
output to equal the step-by-step calls bit for bit.
"""
import dataclasses
import json
import sys
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
    print(f"[parity] {name}: " + json.dumps(stats), flush=True)
    parity.record_stats(name, stats)


def _layer(inp):
    from mxfp4_expert_layer_moe_amd.device import DeviceLayer
    return DeviceLayer(inp)


def _full_check(name, inp, tokens=None):
    """Every intermediate of the step calls against the oracle, then moe_forward (the whole-layer
    entry point: fused routing front end, the dense decode path where it applies, rows written at
    their assignment index) equal to the step calls bit for bit."""
    from mxfp4_expert_layer_moe_amd import _dense_decode
    print(f"[parity] start {name} T={inp.T} D={inp.D} E={inp.E} k={inp.k} I={inp.I}", flush=True)
    t0 = time.time()
    layer = _layer(inp)
    g = parity.run_gpu(layer)
    o = parity.oracle_with_adoption(inp, g["idx"], tokens=tokens)
    stats = parity.compare(inp, g, o)
    y32 = layer.forward(bf16=False).clone()
    y16 = layer.forward(bf16=True).clone()
    torch.cuda.synchronize()
    assert np.array_equal(y32.cpu().numpy(), g["y32"]), "moe_forward differs from the step calls"
    assert np.array_equal(y16.view(torch.int16).cpu().numpy().view(np.uint16), g["y16"])
    stats["forward_path"] = "dense" if _dense_decode(inp.T, inp.E, inp.k, inp.D) else "routed"
    stats["seconds"] = round(time.time() - t0, 1)
    _record(name, stats)
    return layer, g


SMALL = {
    "tiny": dict(cfg=0),
    "tiny_clamp_x64": dict(cfg=0, x_scale=64.0),
    "single_token": dict(cfg=dict(T=1, D=128, E=8, k=4, I=128, seed=40)),
    "k_equals_E": dict(cfg=dict(T=9, D=64, E=3, k=3, I=64, seed=41)),
    "one_hot_expert_two_tiles": dict(cfg=dict(T=40, D=128, E=6, k=2, I=128, seed=42), bias="onehot3"),
    "ragged": dict(cfg=dict(T=37, D=192, E=5, k=3, I=320, seed=43)),
    "mostly_empty_experts": dict(cfg=dict(T=5, D=64, E=16, k=2, I=64, seed=44)),
    "max_experts_256": dict(cfg=dict(T=20, D=64, E=256, k=8, I=64, seed=45)),
    "multi_tile_multi_group": dict(cfg=dict(T=200, D=256, E=8, k=2, I=512, seed=46)),
    "k_tail_groups": dict(cfg=dict(T=70, D=320, E=4, k=2, I=448, seed=47)),
    "skew_small": dict(cfg=dict(T=300, D=128, E=32, k=4, I=128, seed=48), bias="zipf"),
    # degenerate routing: a single expert (every gate 1), and top-1 of 8
    "one_expert": dict(cfg=dict(T=5, D=64, E=1, k=1, I=64, seed=60)),
    "top1_of_8": dict(cfg=dict(T=40, D=64, E=8, k=1, I=64, seed=61)),
    # size thresholds of the path, each met exactly and passed by one:
    # 8-row tiles up to 6 assignments per expert (here 48 = 6 x 8), 128-row tiles past it
    "decode_tiles_at_limit": dict(cfg=dict(T=24, D=64, E=8, k=2, I=64, seed=53)),
    "prefill_tiles_past_limit": dict(cfg=dict(T=25, D=64, E=8, k=2, I=64, seed=54)),
    # grouping in one 256-thread workgroup up to 256 assignments, one 1024-thread workgroup up
    # to 1024, three kernels past that
    "grouping_256_threads_at_limit": dict(cfg=dict(T=64, D=64, E=16, k=4, I=64, seed=58)),
    "grouping_1024_threads_past_256": dict(cfg=dict(T=65, D=64, E=16, k=4, I=64, seed=59)),
    "grouping_one_workgroup_at_limit": dict(cfg=dict(T=256, D=64, E=16, k=4, I=64, seed=55)),
    "grouping_three_kernels_past_limit": dict(cfg=dict(T=257, D=64, E=16, k=4, I=64, seed=56)),
    # the one-workgroup selection takes at most 32 tokens and 32 experts
    "selection_one_workgroup_at_limit": dict(cfg=dict(T=32, D=64, E=32, k=4, I=64, seed=62)),
    "tokens_33_general_selection": dict(cfg=dict(T=33, D=64, E=32, k=4, I=64, seed=63)),
    "experts_33_general_selection": dict(cfg=dict(T=32, D=64, E=33, k=4, I=64, seed=57)),
    # the dense decode path of moe_forward (every (expert, token) pair through gate/up, the selection
    # beside it): used from (1 - k/E)^T <= 0.15; at 14 tokens of 32 experts it is not, at 15 it is
    "dense_threshold_routed": dict(cfg=dict(T=14, D=128, E=32, k=4, I=128, seed=66)),
    "dense_threshold_dense": dict(cfg=dict(T=15, D=128, E=32, k=4, I=128, seed=67)),
    "dense_ragged_k_tail": dict(cfg=dict(T=29, D=320, E=20, k=3, I=192, seed=68)),
    "dense_model_width_20_tokens": dict(cfg=dict(T=20, D=2880, E=32, k=4, I=2880, seed=69)),
    # full 8-row tiles whose activations do not fit LDS whole (K = 3072 and 4096): the small-batch
    # GEMMs stage K in chunks and their weight ring runs across the chunk boundaries
    "chunked_k_full_small_tiles": dict(cfg=dict(T=24, D=3072, E=8, k=2, I=4096, seed=64), bias="onehot3"),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_case_parity(name):
    c = SMALL[name]
    inp = synth.make_inputs(c["cfg"], x_scale=c.get("x_scale", 1.0), bias=c.get("bias"))
    _full_check(name, inp)


@pytest.mark.parametrize("T", [24, 200])          # 8-row (decode) tiles / 128-row tiles
def test_forward_equals_steps_and_is_deterministic(T):
    inp = synth.make_inputs(dict(T=T, D=128, E=8, k=2, I=192, seed=50))
    layer = _layer(inp)
    g = parity.run_gpu(layer)
    y1 = layer.forward(bf16=False).clone()
    y2 = layer.forward(bf16=False).clone()
    yb = layer.forward(bf16=True).clone()
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    assert np.array_equal(y1.cpu().numpy(), g["y32"])
    assert np.array_equal(yb.view(torch.int16).cpu().numpy().view(np.uint16), g["y16"])
    g2 = parity.run_gpu(layer)
    for key in ("idx", "w", "perm", "inv", "x_packed", "y_perm"):
        assert np.array_equal(g[key], g2[key]), key


def test_identity_activation_probe_down_gemm_is_exact():
    """One-hot h rows: y_perm row p equals the dequantized down-weight column p, exactly.

    Checks the prepacked weight layout, the scaled FP4 decode of all 16 codes and
    the E8M0 scales through the matrix cores against the oracle's decoder.  Scales
    span 2^-14 .. 2^13, where every decoded weight is exact in fp16 (y_perm's type).
    """
    import mxfp4_expert_layer_moe_amd as M
    import oracle
    D, I = 64, 1024
    rng = np.random.default_rng(60)
    codes = rng.integers(0, 256, size=(1, D, I // 2), dtype=np.uint8)
    scales = rng.integers(113, 141, size=(1, D, I // 32), dtype=np.uint8)
    d = M.dims(D, I, 1, 1)
    dc, ds = M.moe_mxfp4_prepack(d, M.MOE_STAGE_DOWN, codes, scales)
    dev = "cuda"
    h = np.zeros((I, I), np.float32)
    h[np.arange(I), np.arange(I)] = 1.0
    hb = torch.from_numpy(synth.f32_to_bf16_bits(h).view(np.int16)).to(dev).view(torch.bfloat16)
    hp = torch.empty(M.moe_act_pack_bytes(I, I), dtype=torch.uint8, device=dev)
    M.moe_pack_act(I, I, hb, hp)
    # one expert, k = 1: every token routes to expert 0, so row p of y is token p (32-row tiles)
    idx = torch.zeros((I, 1), dtype=torch.int32, device=dev)
    i32 = dict(dtype=torch.int32, device=dev)
    counts, offsets = torch.empty(1, **i32), torch.empty(2, **i32)
    perm, inv = torch.empty(I, **i32), torch.empty(I, **i32)
    tiles = torch.empty(M.moe_tile_table_bytes(d, I) // 4, **i32)
    M.moe_permute_tiles(d, I, idx, counts, offsets, perm, inv, tiles)
    w = torch.ones(I, dtype=torch.float32, device=dev)
    y = torch.empty((I, D), dtype=torch.float16, device=dev)
    M.moe_expert_gemm_mxfp4_packed(d, I, M.MOE_STAGE_DOWN, hp, tiles, torch.from_numpy(dc).to(dev),
                            torch.from_numpy(ds).to(dev), w, y)
    torch.cuda.synchronize()
    from tests import actpack
    hs = actpack.decode_sum(hp.cpu().numpy(), I, I)
    assert np.array_equal(hs, h.astype(np.float64))          # the split of a one-hot row is exact
    want = oracle.mxfp4_decode(codes[0], scales[0]).T          # [I][D]
    assert np.array_equal(y.cpu().numpy().astype(np.float64), want)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_full_size_workload(cfg):
    """The four model-shape workloads, every token, and moe_forward (the benchmark's entry point, in
    the benchmark's launch configuration) equal to the step calls bit for bit."""
    t0 = time.time()
    inp = synth.make_inputs(cfg)
    print(f"[parity] config {cfg} generated in {time.time() - t0:.1f}s", flush=True)
    _full_check(f"config{cfg}", inp)


@pytest.mark.parametrize("T", [24, 300])           # one-workgroup selection / 16-token workgroups
def test_duplicate_router_rows_force_exact_rescoring(T):
    """Experts 2j and 2j+1 get the same router row and bias, so their logits tie exactly; with an
    odd k the k-th and (k+1)-th places are always such a pair, so every token is flagged and
    re-scored in float64, and the tie must go to the lower expert id, as in the oracle."""
    inp = synth.make_inputs(dict(T=T, D=128, E=16, k=3, I=128, seed=62))
    wr, br = inp.w_router.copy(), inp.b_router.copy()
    wr[1::2], br[1::2] = wr[0::2], br[0::2]
    inp = dataclasses.replace(inp, w_router=wr, b_router=br)
    o = oracle.forward(inp)
    assert o["flagged"].all()                           # every token goes through the re-scoring
    _full_check(f"duplicate_router_rows_T{T}", inp)


def test_large_batch_full_shape():
    """32768 tokens at the 20b shape (131072 assignments, four times the largest benchmark
    workload's): routing, grouping and the tile table bit-exact for every token, the expert
    outputs on 32 sampled tokens."""
    t0 = time.time()
    inp = synth.make_inputs(dict(T=32768, D=2880, E=32, k=4, I=2880, seed=71))
    print(f"[parity] large batch generated in {time.time() - t0:.1f}s", flush=True)
    tokens = np.sort(np.random.default_rng(171).choice(inp.T, 32, replace=False))
    _full_check("large_batch_T32768", inp, tokens)


def test_maximum_batch_full_shape():
    """The largest batch the C ABI accepts at the 20b shape: T*k*(packed row bytes) < 2^32, the
    reach of the GEMMs' 32-bit buffer offsets, so the packed h buffer ends 256 bytes short of
    4 GiB.  Routing, grouping and the tile table are checked for every token (852176 assignments),
    the outputs on 16 sampled tokens."""
    from mxfp4_expert_layer_moe_amd import moe_dims, moe_workspace_bytes, moe_act_pack_bytes
    D, k = 2880, 4
    T = ((1 << 32) - 1) // (k * moe_act_pack_bytes(D, 1))
    assert T == 213044 and moe_act_pack_bytes(D, T * k) == 4294967040
    dims = moe_dims(d_model=D, d_ff=D, n_experts=32, top_k=k, swiglu_limit=7.0)
    assert moe_workspace_bytes(dims, T) > 0 and moe_workspace_bytes(dims, T + 1) == 0
    t0 = time.time()
    inp = synth.make_inputs(dict(T=T, D=D, E=32, k=k, I=D, seed=72))
    print(f"[parity] maximum batch generated in {time.time() - t0:.1f}s", flush=True)
    tokens = np.sort(np.random.default_rng(172).choice(inp.T, 16, replace=False))
    _full_check("maximum_batch_T213044", inp, tokens)


def test_invalid_expert_ids_get_no_row():
    """moe_permute_tiles with expert ids outside [0, E) (a caller error): those assignments are left out
    of counts, perm and the tiles, their inv entry is -1, and moe_combine skips them."""
    import mxfp4_expert_layer_moe_amd as M
    T, E, k, D = 40, 6, 2, 64
    rng = np.random.default_rng(65)
    idx = np.sort(np.stack([rng.choice(E, k, replace=False) for _ in range(T)]), axis=1).astype(np.int32)
    bad = [(3, 0, -1), (7, 1, E), (20, 0, 1 << 20)]
    for t, j, v in bad:
        idx[t, j] = v
    d = M.dims(D, 64, E, k)
    dev = "cuda"
    i32 = dict(dtype=torch.int32, device=dev)
    n = T * k
    counts, offsets = torch.empty(E, **i32), torch.empty(E + 1, **i32)
    perm, inv = torch.full((n,), 12345, **i32), torch.full((n,), 12345, **i32)
    tiles = torch.empty(M.moe_tile_table_bytes(d, T) // 4, **i32)
    M.moe_permute_tiles(d, T, torch.from_numpy(idx).to(dev), counts, offsets, perm, inv, tiles)
    yp = torch.from_numpy(rng.standard_normal((n, D)).astype(np.float16)).to(dev)
    y = torch.empty((T, D), dtype=torch.float32, device=dev)
    M.moe_combine(d, T, yp, inv, y, M.MOE_FP32)
    torch.cuda.synchronize()
    flat = idx.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    want_counts = np.bincount(flat[valid], minlength=E)
    assert np.array_equal(counts.cpu().numpy(), want_counts)
    assert offsets.cpu().numpy()[-1] == valid.sum()
    pv = perm.cpu().numpy()[: valid.sum()]
    assert np.array_equal(pv, np.nonzero(valid)[0][np.argsort(flat[valid], kind="stable")])
    iv = inv.cpu().numpy()
    assert np.all(iv[~valid] == -1)
    assert np.array_equal(iv[pv], np.arange(valid.sum()))
    ypn = yp.cpu().numpy().astype(np.float32)
    want = np.zeros((T, D), np.float32)
    for t in range(T):
        for j in range(k):
            if valid[t * k + j]:
                want[t] = want[t] + ypn[iv[t * k + j]]
    assert np.array_equal(y.cpu().numpy(), want)


def test_clamp_stress_prefill_shape():
    inp = synth.make_inputs(dict(T=512, D=2880, E=32, k=4, I=2880, seed=70), x_scale=8.0)
    tokens = np.arange(0, 512, 16)
    layer, g = _full_check("clamp_stress_x8", inp, tokens)
