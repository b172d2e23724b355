"""The whole-layer entry points under HIP graph capture.

moe_forward and moe_block_forward allocate nothing and clear nothing with memset calls, so a
caller can capture them into a graph.  Each case captures the call on a side stream, then
replays the graph several times; between replays the program overwrites the output with eager
work and synchronizes.  Every replay must equal the eager call bit for bit.
"""
import time

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu-marked tests need an MI355X")
    import mxfp4_expert_layer_moe_amd as M
    M.lib()                     # fails loudly if the HIP library is missing
    yield


CASES = {
    # 8-row tiles, one-workgroup selection and grouping
    "decode_size": dict(T=24, D=128, E=8, k=2, I=192, seed=80),
    # 128-row tiles, per-token selection, three-kernel grouping
    "prefill_size": dict(T=600, D=256, E=8, k=2, I=256, seed=81),
}


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("entry", ["forward", "block_forward"])
def test_graph_replays_equal_the_eager_call(name, entry):
    from mxfp4_expert_layer_moe_amd.device import DeviceLayer
    print(f"[graph] start {entry} {name}", flush=True)
    t0 = time.time()
    layer = DeviceLayer(synth.make_inputs(CASES[name]))
    call = getattr(layer, entry)
    eager = call(bf16=False).clone()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        out = call(bf16=False)
    torch.cuda.synchronize()
    for i in range(3):
        out.fill_(float("nan"))            # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i} differs from the eager call"
    # the eager call still gives the same bits after the replays
    again = call(bf16=False)
    torch.cuda.synchronize()
    assert np.array_equal(again.cpu().numpy(), eager.cpu().numpy())
    print(f"[graph] {entry} {name}: 3 replays equal, {time.time() - t0:.1f}s", flush=True)
