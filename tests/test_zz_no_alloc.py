"""GPU test of moe_forward_noalloc, the whole layer with its scratch in a file-scope device array
(for callers that cannot allocate): through the C ABI, two calls in a row, the second on a smaller
batch, each bit for bit equal to moe_forward on the same inputs with a caller workspace; and the
device's free memory unchanged by the calls once the library's device code is loaded (the runtime
loads each code object, the one holding the array among them, at its first use)."""
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
    M.lib()
    yield


def _case(T, seed):
    from mxfp4_expert_layer_moe_amd.device import DeviceLayer
    inp = synth.make_inputs(dict(T=T, D=2880, E=32, k=4, I=2880, seed=seed))
    return DeviceLayer(inp)


def test_noalloc_forward_equals_forward_on_two_calls_the_second_smaller():
    import mxfp4_expert_layer_moe_amd as M
    big = _case(300, 80)          # 1200 assignments: 128-row tiles, the separate grouping kernels
    small = _case(24, 81)         # 96 assignments: 8-row tiles, the one-workgroup selection
    torch.cuda.synchronize()
    for layer in (big, small):
        assert M.moe_workspace_bytes(layer.dims, layer.T) <= M.MOE_FORWARD_NOALLOC_MAX_WORKSPACE
    outs = []
    for layer in (big, small):
        for bf16 in (False, True):
            y = torch.full((layer.T, layer.D), float("nan"), dtype=torch.bfloat16 if bf16 else torch.float32,
                           device="cuda")
            outs.append((layer, bf16, y))
    # the first call on the device looks up the array's address, and the runtime loads each of the
    # library's device code objects (the array's among them) at the first launch of one of its
    # kernels, once per process: one call of each size runs first, and free memory is read after it
    for layer in (big, small):
        warm = torch.empty((layer.T, layer.D), dtype=torch.float32, device="cuda")
        M.moe_forward_noalloc(layer.dims, layer.T, layer.x, layer.w_router, layer.b_router, layer.weights.struct(),
                              warm, M.MOE_FP32)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    for layer, bf16, y in outs:
        M.moe_forward_noalloc(layer.dims, layer.T, layer.x, layer.w_router, layer.b_router,
                              layer.weights.struct(), y, M.MOE_BF16 if bf16 else M.MOE_FP32)
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    for layer, bf16, y in outs:
        want = layer.forward(bf16=bf16).clone()
        torch.cuda.synchronize()
        a = y.view(torch.int16) if bf16 else y.view(torch.int32)
        b = want.view(torch.int16) if bf16 else want.view(torch.int32)
        assert torch.equal(a, b), (layer.T, bf16)
    # every buffer was allocated before free0 was read: the calls themselves took no device memory
    assert free1 == free0


def test_noalloc_forward_refuses_a_batch_past_its_array():
    import mxfp4_expert_layer_moe_amd as M
    layer = _case(340, 82)
    assert M.moe_workspace_bytes(layer.dims, 340) > M.MOE_FORWARD_NOALLOC_MAX_WORKSPACE
    y = torch.empty((340, 2880), dtype=torch.float32, device="cuda")
    with pytest.raises(M.MoeError) as e:
        M.moe_forward_noalloc(layer.dims, 340, layer.x, layer.w_router, layer.b_router, layer.weights.struct(), y,
                              M.MOE_FP32)
    assert e.value.status == M.MOE_EWORKSPACE
