"""CPU tests of the C ABI: the library loads, exports what the header declares,
rejects bad arguments before any HIP call, and its host-side helpers (MXFP4
quantizer, prepack, size functions) are right.  No GPU needed: no call here
reaches a kernel launch.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import mxfp4_expert_layer_moe_amd as M
import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    return M.lib()


def header_functions(header="moe_mxfp4.h"):
    src = open(os.path.join(ROOT, "include", header)).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_header_symbol(L):
    names = header_functions()
    assert len(names) >= 12
    assert sorted(M.EXPORTS) == names
    for n in names:
        assert hasattr(L, n), n


def test_probe_library_exports_every_header_symbol():
    from mxfp4_expert_layer_moe_amd import peaks
    P = peaks.lib()
    names = header_functions("moe_peaks.h")
    assert sorted(peaks.EXPORTS) == names
    for n in names:
        assert hasattr(P, n), n
    # the work each probe reports, and argument checks before any launch
    assert P.moe_peak_mfma_flops(peaks.FP6_FP4, 10, 3) == 10 * 4 * 3 * 4 * 2 * 32 * 32 * 64
    assert P.moe_peak_mfma_flops(peaks.BF16, 10, 3) == 10 * 4 * 3 * 4 * 2 * 32 * 32 * 16
    assert P.moe_peak_mfma(peaks.FP6_FP4, 0, 1, 16, None) == 1
    assert P.moe_peak_mfma(9, 1, 1, 16, None) == 1
    assert P.moe_peak_stream_read(16, 24, 1, 1, 16, None) == 1           # not a multiple of 16 bytes
    assert P.moe_peak_stream_read(None, 32, 1, 1, 16, None) == 1


def test_status_strings(L):
    for s in range(5):
        assert M.moe_status_str(s).startswith("MOE_")


D = M.dims(2880, 2880, 32, 4)


def test_size_functions_closed_forms():
    assert M.moe_act_pack_bytes(2880, 1) == 45 * 112
    assert M.moe_act_pack_bytes(64, 3) == 3 * 112
    assert M.moe_act_pack_bytes(96, 1) == 0                    # K % 64 != 0
    # prepacked codes are exactly the MXFP4 code bytes: 4 bits per weight
    assert M.moe_prepacked_codes_bytes(D, M.MOE_STAGE_GATE_UP) == 32 * 5760 * 2880 // 2
    assert M.moe_prepacked_codes_bytes(D, M.MOE_STAGE_DOWN) == 32 * 2880 * 2880 // 2
    # scales: 45 k-tiles padded to 48 per 32-row tile
    assert M.moe_prepacked_scales_bytes(D, M.MOE_STAGE_GATE_UP) == 32 * (5760 // 32) * 12 * 256
    ws = M.moe_workspace_bytes(D, 4096)
    # per assignment: fp16 y_perm row + packed h row; per token: packed x row
    assert ws >= 4096 * 4 * (2880 * 2 + M.moe_act_pack_bytes(2880, 1)) + 4096 * M.moe_act_pack_bytes(2880, 1)


@pytest.mark.parametrize("bad,status", [
    (dict(d_model=2880 + 32), M.MOE_EUNSUPPORTED),
    (dict(d_ff=100), M.MOE_EUNSUPPORTED),
    (dict(top_k=0), M.MOE_EINVAL),
    (dict(top_k=33), M.MOE_EUNSUPPORTED),
    (dict(n_experts=257, top_k=4), M.MOE_EUNSUPPORTED),
    (dict(swiglu_limit=0.0), M.MOE_EINVAL),
    (dict(swiglu_limit=float("inf")), M.MOE_EINVAL),
])
def test_bad_dims_rejected(L, bad, status):
    args = dict(d_model=2880, d_ff=2880, n_experts=32, top_k=4, swiglu_limit=7.0)
    args.update(bad)
    d = M.moe_dims(**args)
    st = L.moe_route(ctypes.byref(d), 4, 16, 16, 16, 16, 16, None, 256, 1 << 30, None)
    assert st == status
    assert L.moe_workspace_bytes(ctypes.byref(d), 4) == 0


def test_bad_arguments_rejected_before_launch(L):
    d = ctypes.byref(D)
    A = 1 << 20                                   # fake, aligned, never dereferenced
    # at most 32 tokens and 32 experts: the score groups, [ceil(d_model / 256)] x (8 KiB float64 tile +
    # 256 B norms); larger batches: K-partial tiles
    assert L.moe_route_workspace_bytes(d, 4) == 12 * 8192 + 12 * 256
    R = L.moe_route_workspace_bytes(d, 64)
    assert R > 0 and L.moe_route_workspace_bytes(d, 0) == 0
    assert L.moe_route(None, 64, A, A, A, A, A, None, A, R, None) == M.MOE_EINVAL
    assert L.moe_route(d, -1, A, A, A, A, A, None, A, R, None) == M.MOE_EINVAL
    assert L.moe_route(d, 1 << 22, A, A, A, A, A, None, A, R, None) == M.MOE_EUNSUPPORTED   # T*k >= 2^24
    assert L.moe_route(d, 64, None, A, A, A, A, None, A, R, None) == M.MOE_EINVAL
    assert L.moe_route(d, 64, A + 2, A, A, A, A, None, A, R, None) == M.MOE_EINVAL          # misaligned x
    assert L.moe_route(d, 64, A, A, A, A, A, None, None, R, None) == M.MOE_EINVAL           # no workspace
    assert L.moe_route(d, 64, A, A, A, A, A, None, A + 16, R, None) == M.MOE_EINVAL         # misaligned ws
    assert L.moe_route(d, 64, A, A, A, A, A, None, A, R - 1, None) == M.MOE_EWORKSPACE
    assert L.moe_route(d, 0, A, A, A, A, A, None, None, 0, None) == M.MOE_OK               # T = 0: no-op
    assert L.moe_permute_tiles(d, 4, A, A, A, None, A, A, None) == M.MOE_EINVAL
    assert L.moe_permute_tiles(d, 4, A, A, A, A, A, None, None) == M.MOE_EINVAL       # no tile table
    assert L.moe_permute_tiles(d, 4, A, A, A, A, A, A + 4, None) == M.MOE_EINVAL      # misaligned tiles
    assert L.moe_permute_tiles(d, 0, A, A, A, A, A, A, None) == M.MOE_OK
    # the plain form: scratch instead of the tile table
    P = L.moe_permute_workspace_bytes(d, 4)
    assert P == L.moe_tile_table_bytes(d, 4) and P <= L.moe_workspace_bytes(d, 4)
    assert L.moe_permute(d, 4, A, A, A, None, A, A, P, None) == M.MOE_EINVAL
    assert L.moe_permute(d, 4, A, A, A, A, A, None, P, None) == M.MOE_EINVAL              # no workspace
    assert L.moe_permute(d, 4, A, A, A, A, A, A + 16, P, None) == M.MOE_EINVAL            # misaligned workspace
    assert L.moe_permute(d, 4, A, A, A, A, A, A, P - 1, None) == M.MOE_EWORKSPACE
    assert L.moe_permute(d, 0, A, A, A, A, A, None, 0, None) == M.MOE_OK
    # tile table: 8-row tiles (48-int slots) up to 6 assignments per expert on average, 128-row
    # tiles (132-int slots) beyond
    # followed by the grouping's scratch: [G][E] counts (G = ceil(n / 1024)) and E + 1 tile starts,
    # the whole rounded up to 16 bytes
    def table(n, E, bm, ints):
        words = (-(-n // bm) + min(E, n)) * ints + (-(-n // 1024)) * E + E + 1
        return -(-words // 4) * 16
    assert L.moe_tile_table_bytes(d, 32) == table(128, 32, 8, 48)
    assert L.moe_tile_table_bytes(d, 48) == table(192, 32, 8, 48)         # 6 per expert: 8-row tiles
    assert L.moe_tile_table_bytes(d, 49) == table(196, 32, 128, 132)      # past it: 128-row tiles
    assert L.moe_tile_table_bytes(d, 4096) == table(16384, 32, 128, 132)
    assert L.moe_tile_table_bytes(d, 4097) == table(16388, 32, 128, 132)
    assert L.moe_pack_act(96, 4, A, A, None) == M.MOE_EUNSUPPORTED
    assert L.moe_pack_act(64, 4, A, A + 8, None) == M.MOE_EINVAL
    assert L.moe_pack_act(64, 0, A, A, None) == M.MOE_OK
    assert L.moe_expert_gemm_mxfp4_packed(d, 4, 7, A, A, A, A, A, A, None) == M.MOE_EINVAL
    assert L.moe_expert_gemm_mxfp4_packed(d, 4, M.MOE_STAGE_DOWN, A, A, A, A, None, A, None) == M.MOE_EINVAL
    assert L.moe_expert_gemm_mxfp4_packed(d, 4, M.MOE_STAGE_GATE_UP, A, A, A + 4, A, None, A, None) == M.MOE_EINVAL
    assert L.moe_expert_gemm_mxfp4_packed(d, 4, M.MOE_STAGE_GATE_UP, A, A + 8, A, A, None, A, None) == M.MOE_EINVAL
    assert L.moe_expert_gemm_mxfp4_packed(d, 0, M.MOE_STAGE_GATE_UP, A, A, A, A, None, A, None) == M.MOE_OK
    # the plain form: bf16 rows, perm and offsets, scratch = the tile table + the packed rows
    for st, rows, K in ((M.MOE_STAGE_GATE_UP, 4, 2880), (M.MOE_STAGE_DOWN, 16, 2880)):
        G = L.moe_expert_gemm_workspace_bytes(d, 4, st)
        assert G == -(-L.moe_tile_table_bytes(d, 4) // 256) * 256 + L.moe_act_pack_bytes(K, rows)
        assert G <= L.moe_workspace_bytes(d, 4)
    G = L.moe_expert_gemm_workspace_bytes(d, 4, M.MOE_STAGE_DOWN)
    assert L.moe_expert_gemm_workspace_bytes(d, 4, 7) == 0
    gemm = L.moe_expert_gemm_mxfp4
    assert gemm(d, 4, 7, A, A, A, A, A, A, A, A, G, None) == M.MOE_EINVAL
    assert gemm(d, 4, M.MOE_STAGE_DOWN, A, A, A, A, A, None, A, A, G, None) == M.MOE_EINVAL   # no gates
    assert gemm(d, 4, M.MOE_STAGE_DOWN, A, None, A, A, A, A, A, A, G, None) == M.MOE_EINVAL   # no perm
    assert gemm(d, 4, M.MOE_STAGE_DOWN, A + 2, A, A, A, A, A, A, A, G, None) == M.MOE_EINVAL  # misaligned rows
    assert gemm(d, 4, M.MOE_STAGE_DOWN, A, A, A, A, A, A, A, None, G, None) == M.MOE_EINVAL   # no workspace
    assert gemm(d, 4, M.MOE_STAGE_DOWN, A, A, A, A, A, A, A, A, G - 1, None) == M.MOE_EWORKSPACE
    assert gemm(d, 0, M.MOE_STAGE_GATE_UP, A, A, A, A, A, None, A, None, 0, None) == M.MOE_OK
    assert L.moe_combine(d, 4, A, A, A, 5, None) == M.MOE_EINVAL
    assert L.moe_combine(d, 4, A, A, A + 4, M.MOE_FP32, None) == M.MOE_EINVAL
    # the inverse permutation is required: only the whole-layer path reads rows without it
    assert L.moe_combine(d, 4, A, None, A, M.MOE_FP32, None) == M.MOE_EINVAL
    assert L.moe_combine_residual(d, 4, A, None, A, A, M.MOE_FP32, None) == M.MOE_EINVAL
    w = M.moe_weights(A, A, A, A)
    need = L.moe_workspace_bytes(d, 4)
    assert L.moe_forward(d, 4, A, A, A, ctypes.byref(w), A, M.MOE_FP32, A, need - 1, None) == M.MOE_EWORKSPACE
    assert L.moe_forward(d, 4, A, A, A, ctypes.byref(w), A, M.MOE_FP32, A + 16, need, None) == M.MOE_EINVAL
    w0 = M.moe_weights(A, None, A, A)
    assert L.moe_forward(d, 4, A, A, A, ctypes.byref(w0), A, M.MOE_FP32, A, need, None) == M.MOE_EINVAL
    assert L.moe_forward(d, 0, A, A, A, ctypes.byref(w), A, M.MOE_FP32, A, need, None) == M.MOE_OK


def test_host_quantizer_matches_generator_encoder():
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    w[3, :32] = 0.0                                   # zero block
    w[5, 40] = 1e3                                    # wide block
    w[7, :32] = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0] * 4, np.float32)   # ties
    c1, s1 = M.moe_mxfp4_quantize(w)
    c2, s2 = synth.mxfp4_encode(w)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
    # decodes within the quantizer bound: half a step, or up to 2X when amax/X in (6, 8) saturates
    dec = oracle.mxfp4_decode(c1, s1)
    X = np.repeat(np.ldexp(1.0, s1.astype(int) - 127), 32, axis=1)
    assert np.all(np.abs(dec - w) <= 2.0 * X)


def prepack_reference(codes, scales, N, K, I, gate_up):
    """Independent statement of the device tile layout (see include/moe_mxfp4.h)."""
    E = codes.shape[0]
    KT, KG, NQ = K // 64, (K // 64 + 3) // 4, N // 32
    co = np.zeros((E, NQ, KT, 64, 16), np.uint8)
    so = np.zeros((E, NQ, KG, 64, 4), np.uint8)
    for q in range(NQ):
        base = ((I if q % 2 else 0) + 32 * (q // 2)) if gate_up else 32 * q
        rows = base + np.arange(64) % 32
        for kt in range(KT):
            blk = 2 * kt + np.arange(64) // 32
            for l in range(64):
                co[:, q, kt, l] = codes[:, rows[l], blk[l] * 16:(blk[l] + 1) * 16]
                so[:, q, kt // 4, l, kt % 4] = scales[:, rows[l], blk[l]]
    return co.reshape(-1), so.reshape(-1)


@pytest.mark.parametrize("D_,I_", [(64, 64), (128, 192)])
def test_prepack_layout(D_, I_):
    inp = synth.make_inputs(dict(T=4, D=D_, E=3, k=2, I=I_, seed=8))
    d = M.dims(D_, I_, 3, 2)
    co, so = M.moe_mxfp4_prepack(d, M.MOE_STAGE_GATE_UP, inp.gu_codes, inp.gu_scales)
    rc, rs = prepack_reference(inp.gu_codes, inp.gu_scales, 2 * I_, D_, I_, True)
    assert np.array_equal(co, rc) and np.array_equal(so, rs)
    co, so = M.moe_mxfp4_prepack(d, M.MOE_STAGE_DOWN, inp.dn_codes, inp.dn_scales)
    rc, rs = prepack_reference(inp.dn_codes, inp.dn_scales, D_, I_, I_, False)
    assert np.array_equal(co, rc) and np.array_equal(so, rs)


def test_block_and_act4_entry_points_reject_bad_arguments(L):
    """The pre-norm block and the MXFP4-activation entry points validate before any launch."""
    d = ctypes.byref(D)
    A = 1 << 20                                   # fake, aligned, never dereferenced
    w = M.moe_weights(A, A, A, A)
    # RMSNorm: eps must be positive and finite; pointers 16-byte aligned; T = 0 is a no-op
    assert L.moe_rmsnorm(d, 4, A, A, 0.0, A, None) == M.MOE_EINVAL
    assert L.moe_rmsnorm(d, 4, A, A, -1e-5, A, None) == M.MOE_EINVAL
    assert L.moe_rmsnorm(d, 4, A, A, float("nan"), A, None) == M.MOE_EINVAL
    assert L.moe_rmsnorm(d, 4, A, A + 4, 1e-5, A, None) == M.MOE_EINVAL            # misaligned gamma
    assert L.moe_rmsnorm(d, 4, None, A, 1e-5, A, None) == M.MOE_EINVAL
    assert L.moe_rmsnorm(d, 0, A, A, 1e-5, A, None) == M.MOE_OK
    # combine with residual
    assert L.moe_combine_residual(d, 4, A, A, None, A, M.MOE_FP32, None) == M.MOE_EINVAL
    assert L.moe_combine_residual(d, 4, A, A, A + 8, A, M.MOE_FP32, None) == M.MOE_EINVAL
    assert L.moe_combine_residual(d, 4, A, A, A, A, 9, None) == M.MOE_EINVAL
    assert L.moe_combine_residual(d, 0, A, A, A, A, M.MOE_BF16, None) == M.MOE_OK
    # block forward: its workspace is the normalised rows (256-byte rounded) + moe_forward's
    for T in (1, 4, 32, 4096):
        assert L.moe_block_workspace_bytes(d, T) == -(-T * 2880 * 2 // 256) * 256 + L.moe_workspace_bytes(d, T)
    need = L.moe_block_workspace_bytes(d, 4)
    assert L.moe_block_forward(d, 4, A, A, 1e-5, A, A, ctypes.byref(w), A, M.MOE_FP32, A, need - 1,
                               None) == M.MOE_EWORKSPACE
    assert L.moe_block_forward(d, 4, A, None, 1e-5, A, A, ctypes.byref(w), A, M.MOE_FP32, A, need,
                               None) == M.MOE_EINVAL
    assert L.moe_block_forward(d, 4, A, A, 0.0, A, A, ctypes.byref(w), A, M.MOE_FP32, A, need,
                               None) == M.MOE_EINVAL
    assert L.moe_block_forward(d, 0, A, A, 1e-5, A, A, ctypes.byref(w), A, M.MOE_FP32, A, need,
                               None) == M.MOE_OK
    # MXFP4 activations: 48 bytes per row and 64-wide k-tile
    assert L.moe_act4_pack_bytes(2880, 7) == 7 * 45 * 48
    assert L.moe_act4_pack_bytes(96, 7) == 0
    assert L.moe_pack_act4(96, 4, A, A, None) == M.MOE_EUNSUPPORTED
    assert L.moe_pack_act4(64, 4, A, A + 8, None) == M.MOE_EINVAL
    assert L.moe_pack_act4(64, 0, A, A, None) == M.MOE_OK
    assert L.moe_expert_gemm_mxfp4_act4(d, 4, 7, A, A, A, A, A, A, None) == M.MOE_EINVAL
    assert L.moe_expert_gemm_mxfp4_act4(d, 4, M.MOE_STAGE_DOWN, A, A, A, A, None, A, None) == M.MOE_EINVAL
    assert L.moe_expert_gemm_mxfp4_act4(d, 0, M.MOE_STAGE_GATE_UP, A, A, A, A, None, A, None) == M.MOE_OK
    # the act4 workspace holds smaller packed rows than the default one
    for T in (4, 32, 4096):
        assert 0 < L.moe_workspace_bytes_act4(d, T) < L.moe_workspace_bytes(d, T)
    need4 = L.moe_workspace_bytes_act4(d, 4)
    assert L.moe_forward_act4(d, 4, A, A, A, ctypes.byref(w), A, M.MOE_FP32, A, need4 - 1,
                              None) == M.MOE_EWORKSPACE
    assert L.moe_forward_act4(d, 0, A, A, A, ctypes.byref(w), A, M.MOE_FP32, A, need4, None) == M.MOE_OK


def test_largest_batch_is_accepted_and_one_more_token_is_not(L):
    """The packed activation rows are addressed with 32-bit buffer offsets: T*k*(packed row
    bytes) must stay below 2^32.  At the 20b shape (5040 packed bytes per 2880-wide row, top-4)
    that is T = 213044; the entry points accept it and reject T + 1 before any launch."""
    d = M.moe_dims(d_model=2880, d_ff=2880, n_experts=32, top_k=4, swiglu_limit=7.0)
    assert L.moe_act_pack_bytes(2880, 1) == 5040
    T = ((1 << 32) - 1) // (4 * 5040)
    assert T == 213044
    assert L.moe_workspace_bytes(ctypes.byref(d), T) > 0
    assert L.moe_workspace_bytes(ctypes.byref(d), T + 1) == 0
    A = 1 << 20                                              # fake, aligned, never dereferenced
    w = M.moe_weights(A, A, A, A)
    dp = ctypes.byref(d)
    assert L.moe_route(dp, T + 1, A, A, A, A, A, None, A, 1 << 40, None) == M.MOE_EUNSUPPORTED
    assert L.moe_forward(dp, T + 1, A, A, A, ctypes.byref(w), A, M.MOE_FP32, A, 1 << 40, None) == M.MOE_EUNSUPPORTED
    # with T itself the arguments pass and only the (too small) workspace is refused
    assert L.moe_forward(dp, T, A, A, A, ctypes.byref(w), A, M.MOE_FP32, A, 256, None) == M.MOE_EWORKSPACE


def test_noalloc_forward_rejects_before_any_device_call(L):
    """moe_forward_noalloc checks its arguments and its scratch limit on the host first: a batch
    whose workspace passes the 16 MiB array is refused with MOE_EWORKSPACE, bad arguments with
    MOE_EINVAL, and T = 0 returns MOE_OK, all without a device (none in this process)."""
    d = M.dims(2880, 2880, 32, 4)
    assert M.MOE_FORWARD_NOALLOC_MAX_WORKSPACE == 16 << 20
    big = 340                                   # the first T past the limit at this shape
    assert M.moe_workspace_bytes(d, big) > M.MOE_FORWARD_NOALLOC_MAX_WORKSPACE >= M.moe_workspace_bytes(d, big - 1)
    w = M.moe_weights(256, 256, 256, 256)
    args = lambda T, y=256: (ctypes.byref(d), T, 256, 256, 256, ctypes.byref(w), y, M.MOE_FP32, None)
    assert L.moe_forward_noalloc(*args(big)) == M.MOE_EWORKSPACE
    assert L.moe_forward_noalloc(*args(8, y=None)) == M.MOE_EINVAL
    assert L.moe_forward_noalloc(*args(8, y=258)) == M.MOE_EINVAL            # misaligned output
    assert L.moe_forward_noalloc(*args(-1)) == M.MOE_EINVAL
    assert L.moe_forward_noalloc(*args(0)) == M.MOE_OK
