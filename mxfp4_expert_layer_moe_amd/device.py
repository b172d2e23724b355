"""Device-side buffers of one MoE layer (torch for memory and streams only).

``DeviceLayer`` uploads a layer's inputs (bf16 x, fp32 router, MXFP4 experts
prepacked by the C library) to the GPU, owns the workspace and output buffers,
and calls the C entry points, either one step at a time or as ``moe_forward``.
"""
from __future__ import annotations

import numpy as np
import torch

from . import (MOE_BF16, MOE_FP32, MOE_STAGE_DOWN, MOE_STAGE_GATE_UP, dims, moe_act4_pack_bytes, moe_act_pack_bytes,
               moe_block_forward, moe_block_workspace_bytes, moe_combine, moe_combine_residual,
               moe_expert_gemm_mxfp4, moe_expert_gemm_mxfp4_act4, moe_expert_gemm_mxfp4_packed, moe_forward,
               moe_forward_act4, moe_mxfp4_prepack, moe_pack_act, moe_pack_act4, moe_permute, moe_permute_tiles,
               moe_rmsnorm, moe_route, moe_route_workspace_bytes, moe_tile_table_bytes, moe_weights,
               moe_workspace_bytes, moe_workspace_bytes_act4)


def _u8(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).reshape(-1)).to(device)


class DeviceWeights:
    """Prepacked MXFP4 expert weights of one layer on the device."""

    def __init__(self, d, gu_codes, gu_scales, dn_codes, dn_scales, device="cuda"):
        gc, gs = moe_mxfp4_prepack(d, MOE_STAGE_GATE_UP, gu_codes, gu_scales)
        dc, ds = moe_mxfp4_prepack(d, MOE_STAGE_DOWN, dn_codes, dn_scales)
        self.gu_codes, self.gu_scales = _u8(gc, device), _u8(gs, device)
        self.dn_codes, self.dn_scales = _u8(dc, device), _u8(ds, device)

    @classmethod
    def from_prepacked(cls, tensors):
        obj = cls.__new__(cls)
        obj.gu_codes, obj.gu_scales, obj.dn_codes, obj.dn_scales = tensors
        return obj

    def clone(self):
        return DeviceWeights.from_prepacked([t.clone() for t in
                                             (self.gu_codes, self.gu_scales, self.dn_codes, self.dn_scales)])

    def struct(self) -> moe_weights:
        return moe_weights(self.gu_codes.data_ptr(), self.gu_scales.data_ptr(), self.dn_codes.data_ptr(),
                           self.dn_scales.data_ptr())

    @property
    def nbytes(self) -> int:
        return sum(t.numel() for t in (self.gu_codes, self.gu_scales, self.dn_codes, self.dn_scales))


class DeviceLayer:
    def __init__(self, inp, device="cuda", weights: DeviceWeights | None = None):
        self.T, self.D, self.E, self.k, self.I = inp.T, inp.D, inp.E, inp.k, inp.I
        self.dims = dims(inp.D, inp.I, inp.E, inp.k, inp.swiglu_limit)
        self.device = device
        self.x = torch.from_numpy(inp.x_bf16.view(np.int16)).to(device).view(torch.bfloat16)
        self.w_router = torch.from_numpy(np.ascontiguousarray(inp.w_router)).to(device)
        self.b_router = torch.from_numpy(np.ascontiguousarray(inp.b_router)).to(device)
        self.weights = weights or DeviceWeights(self.dims, inp.gu_codes, inp.gu_scales, inp.dn_codes,
                                                inp.dn_scales, device)
        T, k, D, I, E = self.T, self.k, self.D, self.I, self.E
        n = T * k
        i32 = dict(dtype=torch.int32, device=device)
        self.topk_idx = torch.empty((T, k), **i32)
        self.topk_w = torch.empty((T, k), dtype=torch.float32, device=device)
        self.logits = torch.empty((T, E), dtype=torch.float32, device=device)
        self.counts = torch.empty(E, **i32)
        self.offsets = torch.empty(E + 1, **i32)
        self.perm = torch.empty(n, **i32)
        self.inv = torch.empty(n, **i32)
        self.tiles = torch.empty(max(moe_tile_table_bytes(self.dims, T) // 4, 4), **i32)
        self.x_packed = torch.empty(max(moe_act_pack_bytes(D, T), 16), dtype=torch.uint8, device=device)
        self.h_packed = torch.empty(max(moe_act_pack_bytes(I, n), 16), dtype=torch.uint8, device=device)
        self.y_perm = torch.empty((n, D), dtype=torch.float16, device=device)
        self.y32 = torch.empty((T, D), dtype=torch.float32, device=device)
        self.y16 = torch.empty((T, D), dtype=torch.bfloat16, device=device)
        self.ws = torch.empty(max(moe_workspace_bytes(self.dims, T), 256), dtype=torch.uint8, device=device)
        self.route_ws = torch.empty(max(moe_route_workspace_bytes(self.dims, T), 256), dtype=torch.uint8,
                                    device=device)
        # the pre-norm block around the layer: RMSNorm scale, normalised rows, block workspace
        gamma = inp.norm_weight if getattr(inp, "norm_weight", None) is not None else np.ones(D, np.float32)
        self.gamma = torch.from_numpy(np.ascontiguousarray(gamma, dtype=np.float32)).to(device)
        self.eps = float(getattr(inp, "norm_eps", 1e-5))
        self.xn = torch.empty((T, D), dtype=torch.bfloat16, device=device)
        self.block_ws = None
        # the activation-quantized variant (MXFP4 activations), allocated on first use
        self.x_packed4 = self.h_packed4 = self.ws4 = None

    # ---- step by step (the C entry points in order) ---------------------------
    def route(self, logits=True, stream=None, x=None):
        moe_route(self.dims, self.T, self.x if x is None else x, self.w_router, self.b_router, self.topk_idx,
                  self.topk_w, self.logits if logits else None, self.route_ws, None, stream)

    def permute(self, stream=None):
        moe_permute_tiles(self.dims, self.T, self.topk_idx, self.counts, self.offsets, self.perm, self.inv,
                          self.tiles, stream)

    def pack_x(self, stream=None, x=None):
        moe_pack_act(self.D, self.T, self.x if x is None else x, self.x_packed, stream)

    def gate_up(self, weights: DeviceWeights | None = None, stream=None):
        w = weights or self.weights
        moe_expert_gemm_mxfp4_packed(self.dims, self.T, MOE_STAGE_GATE_UP, self.x_packed, self.tiles, w.gu_codes,
                                     w.gu_scales, None, self.h_packed, stream)

    def down(self, weights: DeviceWeights | None = None, stream=None):
        w = weights or self.weights
        moe_expert_gemm_mxfp4_packed(self.dims, self.T, MOE_STAGE_DOWN, self.h_packed, self.tiles, w.dn_codes,
                                     w.dn_scales, self.topk_w, self.y_perm, stream)

    def combine(self, bf16=False, stream=None, residual=None):
        y, dt = (self.y16, MOE_BF16) if bf16 else (self.y32, MOE_FP32)
        if residual is None:
            moe_combine(self.dims, self.T, self.y_perm, self.inv, y, dt, stream)
        else:
            moe_combine_residual(self.dims, self.T, self.y_perm, self.inv, residual, y, dt, stream)

    # ---- the plain boundary: bf16 rows, perm and offsets, scratch from the workspace ----------
    def permute_plain(self, stream=None):
        moe_permute(self.dims, self.T, self.topk_idx, self.counts, self.offsets, self.perm, self.inv, self.ws,
                    self.ws.numel(), stream)

    def gate_up_plain(self, h_bf16, weights: DeviceWeights | None = None, stream=None, x=None):
        w = weights or self.weights
        moe_expert_gemm_mxfp4(self.dims, self.T, MOE_STAGE_GATE_UP, self.x if x is None else x, self.perm,
                              self.offsets, w.gu_codes, w.gu_scales, None, h_bf16, self.ws, self.ws.numel(), stream)

    def down_plain(self, h_bf16, weights: DeviceWeights | None = None, stream=None):
        w = weights or self.weights
        moe_expert_gemm_mxfp4(self.dims, self.T, MOE_STAGE_DOWN, h_bf16, self.perm, self.offsets, w.dn_codes,
                              w.dn_scales, self.topk_w, self.y_perm, self.ws, self.ws.numel(), stream)

    def steps(self, bf16=False, stream=None):
        self.route(stream=stream)
        self.permute(stream)
        self.pack_x(stream)
        self.gate_up(stream=stream)
        self.down(stream=stream)
        self.combine(bf16, stream)

    # ---- the activation-quantized variant (MXFP4 activations) -----------------
    def _act4_buffers(self):
        if self.x_packed4 is None:
            T, k, D, I = self.T, self.k, self.D, self.I
            u8 = dict(dtype=torch.uint8, device=self.device)
            self.x_packed4 = torch.empty(max(moe_act4_pack_bytes(D, T), 16), **u8)
            self.h_packed4 = torch.empty(max(moe_act4_pack_bytes(I, T * k), 16), **u8)
            self.ws4 = torch.empty(max(moe_workspace_bytes_act4(self.dims, T), 256), **u8)

    def steps_act4(self, bf16=False, stream=None):
        self._act4_buffers()
        w = self.weights
        self.route(stream=stream)
        self.permute(stream)
        moe_pack_act4(self.D, self.T, self.x, self.x_packed4, stream)
        moe_expert_gemm_mxfp4_act4(self.dims, self.T, MOE_STAGE_GATE_UP, self.x_packed4, self.tiles, w.gu_codes,
                                   w.gu_scales, None, self.h_packed4, stream)
        moe_expert_gemm_mxfp4_act4(self.dims, self.T, MOE_STAGE_DOWN, self.h_packed4, self.tiles, w.dn_codes,
                                   w.dn_scales, self.topk_w, self.y_perm, stream)
        self.combine(bf16, stream)

    def forward_act4(self, bf16=False, weights: DeviceWeights | None = None, stream=None):
        self._act4_buffers()
        w = weights or self.weights
        y, dt = (self.y16, MOE_BF16) if bf16 else (self.y32, MOE_FP32)
        moe_forward_act4(self.dims, self.T, self.x, self.w_router, self.b_router, w.struct(), y, dt, self.ws4, None,
                         stream)
        return y

    # ---- the pre-norm block: y = x + MoE(RMSNorm(x)) --------------------------
    def rmsnorm(self, stream=None):
        moe_rmsnorm(self.dims, self.T, self.x, self.gamma, self.eps, self.xn, stream)

    def block_steps(self, bf16=False, stream=None):
        self.rmsnorm(stream)
        self.route(stream=stream, x=self.xn)
        self.permute(stream)
        self.pack_x(stream, x=self.xn)
        self.gate_up(stream=stream)
        self.down(stream=stream)
        self.combine(bf16, stream, residual=self.x)

    def block_forward(self, bf16=False, weights: DeviceWeights | None = None, stream=None):
        w = weights or self.weights
        if self.block_ws is None:
            self.block_ws = torch.empty(max(moe_block_workspace_bytes(self.dims, self.T), 256), dtype=torch.uint8,
                                        device=self.device)
        y, dt = (self.y16, MOE_BF16) if bf16 else (self.y32, MOE_FP32)
        moe_block_forward(self.dims, self.T, self.x, self.gamma, self.eps, self.w_router, self.b_router, w.struct(),
                          y, dt, self.block_ws, None, stream)
        return y

    def forward(self, bf16=False, weights: DeviceWeights | None = None, stream=None):
        w = weights or self.weights
        moe_forward(self.dims, self.T, self.x, self.w_router, self.b_router, w.struct(),
                    self.y16 if bf16 else self.y32, MOE_BF16 if bf16 else MOE_FP32, self.ws, None, stream)
        return self.y16 if bf16 else self.y32
