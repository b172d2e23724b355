"""Python binding of libmoe_mxfp4.so, the MI355X MoE layer with MXFP4 experts.

Argument marshalling only: every function forwards to the C entry point of the
same name (declared in include/moe_mxfp4.h).  Device buffers are anything with
``data_ptr()`` (torch tensors on the GPU); streams default to torch's current
stream.  There is no CPU fallback: if the library is not built, loading it
raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "libmoe_mxfp4.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP = range(5)
MOE_BF16, MOE_FP32 = 0, 1
MOE_STAGE_GATE_UP, MOE_STAGE_DOWN = 0, 1

# Symbols the header declares (checked by the CPU tests).
EXPORTS = ("moe_status_str", "moe_act_pack_bytes", "moe_prepacked_codes_bytes", "moe_prepacked_scales_bytes",
           "moe_workspace_bytes", "moe_route_workspace_bytes", "moe_tile_table_bytes", "moe_route", "moe_permute",
           "moe_permute_workspace_bytes", "moe_permute_tiles", "moe_expert_gemm_workspace_bytes",
           "moe_expert_gemm_mxfp4_packed",
           "moe_pack_act", "moe_expert_gemm_mxfp4", "moe_combine", "moe_forward", "moe_mxfp4_quantize",
           "moe_mxfp4_prepack", "moe_combine_residual", "moe_rmsnorm", "moe_block_workspace_bytes",
           "moe_block_forward", "moe_act4_pack_bytes", "moe_pack_act4", "moe_expert_gemm_mxfp4_act4",
           "moe_workspace_bytes_act4", "moe_forward_act4", "moe_forward_noalloc")
MOE_FORWARD_NOALLOC_MAX_WORKSPACE = 16 << 20


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {moe_status_str(status)}")
        self.status = status


class moe_dims(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("swiglu_limit", ctypes.c_float)]


class moe_weights(ctypes.Structure):
    _fields_ = [("gu_codes", ctypes.c_void_p), ("gu_scales", ctypes.c_void_p),
                ("dn_codes", ctypes.c_void_p), ("dn_scales", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m mxfp4_expert_layer_moe_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz, f32p, i32p = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p
        dp = ctypes.POINTER(moe_dims)
        L.moe_status_str.restype = ctypes.c_char_p
        L.moe_status_str.argtypes = [ctypes.c_int]
        L.moe_act_pack_bytes.restype = sz
        L.moe_act_pack_bytes.argtypes = [i32, i32]
        for name in ("moe_prepacked_codes_bytes", "moe_prepacked_scales_bytes"):
            getattr(L, name).restype = sz
            getattr(L, name).argtypes = [dp, ctypes.c_int]
        for name in ("moe_workspace_bytes", "moe_route_workspace_bytes", "moe_tile_table_bytes",
                     "moe_block_workspace_bytes", "moe_workspace_bytes_act4", "moe_permute_workspace_bytes"):
            getattr(L, name).restype = sz
            getattr(L, name).argtypes = [dp, i32]
        L.moe_route.argtypes = [dp, i32, vp, f32p, f32p, i32p, f32p, f32p, vp, sz, vp]
        L.moe_expert_gemm_workspace_bytes.restype = sz
        L.moe_expert_gemm_workspace_bytes.argtypes = [dp, i32, ctypes.c_int]
        L.moe_permute.argtypes = [dp, i32, i32p, i32p, i32p, i32p, i32p, vp, sz, vp]
        L.moe_permute_tiles.argtypes = [dp, i32, i32p, i32p, i32p, i32p, i32p, i32p, vp]
        L.moe_pack_act.argtypes = [i32, i32, vp, vp, vp]
        L.moe_expert_gemm_mxfp4.argtypes = [dp, i32, ctypes.c_int, vp, i32p, i32p, vp, vp, f32p, vp, vp, sz, vp]
        L.moe_expert_gemm_mxfp4_packed.argtypes = [dp, i32, ctypes.c_int, vp, i32p, vp, vp, f32p, vp, vp]
        L.moe_combine.argtypes = [dp, i32, f32p, i32p, vp, ctypes.c_int, vp]
        L.moe_forward.argtypes = [dp, i32, vp, f32p, f32p, ctypes.POINTER(moe_weights), vp, ctypes.c_int, vp, sz, vp]
        L.moe_combine_residual.argtypes = [dp, i32, vp, i32p, vp, vp, ctypes.c_int, vp]
        L.moe_act4_pack_bytes.restype = sz
        L.moe_act4_pack_bytes.argtypes = [i32, i32]
        L.moe_pack_act4.argtypes = [i32, i32, vp, vp, vp]
        L.moe_expert_gemm_mxfp4_act4.argtypes = [dp, i32, ctypes.c_int, vp, i32p, vp, vp, f32p, vp, vp]
        L.moe_forward_act4.argtypes = [dp, i32, vp, f32p, f32p, ctypes.POINTER(moe_weights), vp, ctypes.c_int, vp,
                                       sz, vp]
        L.moe_forward_noalloc.argtypes = [dp, i32, vp, f32p, f32p, ctypes.POINTER(moe_weights), vp, ctypes.c_int, vp]
        L.moe_rmsnorm.argtypes = [dp, i32, vp, f32p, ctypes.c_float, vp, vp]
        L.moe_block_forward.argtypes = [dp, i32, vp, f32p, ctypes.c_float, f32p, f32p, ctypes.POINTER(moe_weights),
                                        vp, ctypes.c_int, vp, sz, vp]
        L.moe_mxfp4_quantize.argtypes = [vp, ctypes.c_int64, i32, vp, vp]
        L.moe_mxfp4_prepack.argtypes = [dp, ctypes.c_int, vp, vp, vp, vp]
        for name in ("moe_route", "moe_permute", "moe_permute_tiles", "moe_pack_act", "moe_expert_gemm_mxfp4",
                     "moe_expert_gemm_mxfp4_packed", "moe_combine",
                     "moe_forward", "moe_mxfp4_quantize", "moe_mxfp4_prepack", "moe_combine_residual",
                     "moe_rmsnorm", "moe_block_forward", "moe_pack_act4", "moe_expert_gemm_mxfp4_act4",
                     "moe_forward_act4", "moe_forward_noalloc"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _dense_decode(T: int, E: int, k: int, D: int) -> bool:
    """Whether moe_forward takes the dense decode path (the library's rule, for tests and reports):
    at most 32 tokens and 32 experts, at most 6 assignments per expert, d_model up to 2880, and an
    expert left untouched with probability (1 - k/E)^T <= 0.15."""
    if T < 1 or T > 32 or E > 32 or T * k > 6 * E or D // 64 > 45:
        return False
    untouched = 1.0
    for _ in range(T):
        untouched *= 1.0 - k / E
    return untouched <= 0.15


def _p(t):
    """Device/host pointer of a tensor, ndarray, int or None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _s(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _check(st: int, where: str):
    if st != MOE_OK:
        raise MoeError(st, where)


def dims(d_model: int, d_ff: int, n_experts: int, top_k: int, swiglu_limit: float = 7.0) -> moe_dims:
    return moe_dims(d_model, d_ff, n_experts, top_k, swiglu_limit)


def moe_status_str(status: int) -> str:
    return lib().moe_status_str(status).decode()


def moe_act_pack_bytes(K: int, rows: int) -> int:
    return lib().moe_act_pack_bytes(K, rows)


def moe_prepacked_codes_bytes(d: moe_dims, stage: int) -> int:
    return lib().moe_prepacked_codes_bytes(ctypes.byref(d), stage)


def moe_prepacked_scales_bytes(d: moe_dims, stage: int) -> int:
    return lib().moe_prepacked_scales_bytes(ctypes.byref(d), stage)


def moe_workspace_bytes(d: moe_dims, T: int) -> int:
    return lib().moe_workspace_bytes(ctypes.byref(d), T)


def moe_route_workspace_bytes(d: moe_dims, T: int) -> int:
    return lib().moe_route_workspace_bytes(ctypes.byref(d), T)


def moe_route(d, T, x, w_router, b_router, topk_idx, topk_w, logits, ws, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(lib().moe_route(ctypes.byref(d), T, _p(x), _p(w_router), _p(b_router), _p(topk_idx), _p(topk_w),
                           _p(logits), _p(ws), ws_bytes, _s(stream)), "moe_route")


def moe_tile_table_bytes(d: moe_dims, T: int) -> int:
    return lib().moe_tile_table_bytes(ctypes.byref(d), T)


def moe_permute_workspace_bytes(d: moe_dims, T: int) -> int:
    return lib().moe_permute_workspace_bytes(ctypes.byref(d), T)


def moe_permute(d, T, topk_idx, counts, offsets, perm, inv, ws, ws_bytes, stream=None):
    _check(lib().moe_permute(ctypes.byref(d), T, _p(topk_idx), _p(counts), _p(offsets), _p(perm), _p(inv),
                             _p(ws), ws_bytes, _s(stream)), "moe_permute")


def moe_permute_tiles(d, T, topk_idx, counts, offsets, perm, inv, tiles, stream=None):
    _check(lib().moe_permute_tiles(ctypes.byref(d), T, _p(topk_idx), _p(counts), _p(offsets), _p(perm), _p(inv),
                                   _p(tiles), _s(stream)), "moe_permute_tiles")


def moe_pack_act(K, rows, a, a_packed, stream=None):
    _check(lib().moe_pack_act(K, rows, _p(a), _p(a_packed), _s(stream)), "moe_pack_act")


def moe_expert_gemm_workspace_bytes(d: moe_dims, T: int, stage: int) -> int:
    return lib().moe_expert_gemm_workspace_bytes(ctypes.byref(d), T, stage)


def moe_expert_gemm_mxfp4(d, T, stage, a, perm, offsets, codes, scales, topk_w, out, ws, ws_bytes, stream=None):
    _check(lib().moe_expert_gemm_mxfp4(ctypes.byref(d), T, stage, _p(a), _p(perm), _p(offsets), _p(codes),
                                       _p(scales), _p(topk_w), _p(out), _p(ws), ws_bytes, _s(stream)),
           "moe_expert_gemm_mxfp4")


def moe_expert_gemm_mxfp4_packed(d, T, stage, a_packed, tiles, codes, scales, topk_w, out, stream=None):
    _check(lib().moe_expert_gemm_mxfp4_packed(ctypes.byref(d), T, stage, _p(a_packed), _p(tiles), _p(codes),
                                              _p(scales), _p(topk_w), _p(out), _s(stream)),
           "moe_expert_gemm_mxfp4_packed")


def moe_combine(d, T, y_perm, inv, y, y_dtype, stream=None):
    _check(lib().moe_combine(ctypes.byref(d), T, _p(y_perm), _p(inv), _p(y), y_dtype, _s(stream)), "moe_combine")


def moe_forward(d, T, x, w_router, b_router, weights: moe_weights, y, y_dtype, ws, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(lib().moe_forward(ctypes.byref(d), T, _p(x), _p(w_router), _p(b_router), ctypes.byref(weights), _p(y),
                             y_dtype, _p(ws), ws_bytes, _s(stream)), "moe_forward")


def moe_forward_noalloc(d, T, x, w_router, b_router, weights: moe_weights, y, y_dtype, stream=None):
    _check(lib().moe_forward_noalloc(ctypes.byref(d), T, _p(x), _p(w_router), _p(b_router), ctypes.byref(weights),
                                     _p(y), y_dtype, _s(stream)), "moe_forward_noalloc")


def moe_combine_residual(d, T, y_perm, inv, residual, y, y_dtype, stream=None):
    _check(lib().moe_combine_residual(ctypes.byref(d), T, _p(y_perm), _p(inv), _p(residual), _p(y), y_dtype,
                                      _s(stream)), "moe_combine_residual")


def moe_rmsnorm(d, T, x, gamma, eps, xn, stream=None):
    _check(lib().moe_rmsnorm(ctypes.byref(d), T, _p(x), _p(gamma), float(eps), _p(xn), _s(stream)), "moe_rmsnorm")


def moe_block_workspace_bytes(d: moe_dims, T: int) -> int:
    return lib().moe_block_workspace_bytes(ctypes.byref(d), T)


def moe_block_forward(d, T, x, gamma, eps, w_router, b_router, weights: moe_weights, y, y_dtype, ws, ws_bytes=None,
                      stream=None):
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(lib().moe_block_forward(ctypes.byref(d), T, _p(x), _p(gamma), float(eps), _p(w_router), _p(b_router),
                                   ctypes.byref(weights), _p(y), y_dtype, _p(ws), ws_bytes, _s(stream)),
           "moe_block_forward")


def moe_act4_pack_bytes(K: int, rows: int) -> int:
    return lib().moe_act4_pack_bytes(K, rows)


def moe_pack_act4(K, rows, a, a_packed4, stream=None):
    _check(lib().moe_pack_act4(K, rows, _p(a), _p(a_packed4), _s(stream)), "moe_pack_act4")


def moe_expert_gemm_mxfp4_act4(d, T, stage, a_packed4, tiles, codes, scales, topk_w, out, stream=None):
    _check(lib().moe_expert_gemm_mxfp4_act4(ctypes.byref(d), T, stage, _p(a_packed4), _p(tiles), _p(codes),
                                            _p(scales), _p(topk_w), _p(out), _s(stream)), "moe_expert_gemm_mxfp4_act4")


def moe_workspace_bytes_act4(d: moe_dims, T: int) -> int:
    return lib().moe_workspace_bytes_act4(ctypes.byref(d), T)


def moe_forward_act4(d, T, x, w_router, b_router, weights: moe_weights, y, y_dtype, ws, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(lib().moe_forward_act4(ctypes.byref(d), T, _p(x), _p(w_router), _p(b_router), ctypes.byref(weights),
                                  _p(y), y_dtype, _p(ws), ws_bytes, _s(stream)), "moe_forward_act4")


def moe_mxfp4_quantize(w: np.ndarray):
    """Host: fp32 [rows][K] -> (codes uint8 [rows][K/2], scales uint8 [rows][K/32])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, K = w.shape
    codes = np.zeros((rows, K // 2), np.uint8)
    scales = np.zeros((rows, max(K // 32, 0)), np.uint8)
    _check(lib().moe_mxfp4_quantize(_p(w), rows, K, _p(codes), _p(scales)), "moe_mxfp4_quantize")
    return codes, scales


def moe_mxfp4_prepack(d: moe_dims, stage: int, codes: np.ndarray, scales: np.ndarray):
    """Host: canonical MXFP4 bytes of all experts -> device tile layout (numpy uint8 arrays)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    co = np.empty(moe_prepacked_codes_bytes(d, stage), np.uint8)
    so = np.empty(moe_prepacked_scales_bytes(d, stage), np.uint8)
    _check(lib().moe_mxfp4_prepack(ctypes.byref(d), stage, _p(codes), _p(scales), _p(co), _p(so)),
           "moe_mxfp4_prepack")
    return co, so
