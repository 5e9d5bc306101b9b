"""One GPU's MoE layer: device buffers plus the six entry points in order.

torch provides device memory and the stream; every step of the layer runs
in libmoe_ep.so:

    moe_dispatch_layout -> moe_permute -> moe_grouped_gemm_w13 (fused SiLU*up)
      -> moe_grouped_gemm_w2 -> moe_combine

or, unfused, moe_grouped_gemm_w13 (G) -> moe_silu_mul -> moe_grouped_gemm_w2.
Buffers are sized from capacity bounds once, so a step never allocates and
its launch shapes never depend on the routing.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import (MOE_EPI_SILU_MUL, MOE_EPI_STORE_G, moe_combine, moe_dispatch_layout,
               moe_dispatch_layout_workspace_bytes, moe_grouped_gemm_w2, moe_grouped_gemm_w13,
               moe_grouped_gemm_workspace_bytes, moe_pack_w13, MOE_W_PACKED, MOE_W_ROW_MAJOR,
               moe_combine_backward, moe_silu_mul_backward, moe_permute_backward,
               moe_transpose_weights, moe_grouped_gemm_wgrad, moe_grouped_gemm_w13_silu_backward,
               moe_permute, moe_silu_mul)

_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}


@dataclass(frozen=True)
class LayerShape:
    T: int
    K: int
    E: int              # global experts
    expert_begin: int
    L: int              # local experts
    H: int
    I: int
    R: int              # capacity per local expert, 0 = exact-fit
    act: str            # token activations: "f32" | "bf16"
    wdt: str            # expert weights: "f32" | "bf16" | "fp8"
    BM: int = 128

    @property
    def rows_cap(self) -> int:
        return self.L * self.R if self.R > 0 else self.T * self.K

    @property
    def buf_dt(self) -> str:
        return "fp8" if self.wdt == "fp8" else self.act

    @property
    def z_dt(self) -> str:
        return "fp8" if self.wdt == "fp8" else ("f32" if self.wdt == "f32" else "bf16")

    @property
    def out_dt(self) -> str:
        return "f32" if self.act == "f32" else "bf16"


class MoELayer:
    def __init__(self, shape: LayerShape, device="cuda", fused: bool = True):
        s = self.shape = shape
        self.fused = fused
        dev = torch.device(device)
        i32 = dict(dtype=torch.int32, device=dev)
        rc = s.rows_cap
        self.counts = torch.zeros(s.L, **i32)
        self.offsets = torch.zeros(s.L + 1, **i32)
        self.slot_of = torch.zeros(s.T, s.K, **i32)
        self.row_src = torch.zeros(max(rc, 1), **i32)[:rc]
        self.tile_offsets = torch.zeros(s.L + 1, **i32)
        self.dev_status = torch.zeros(2, **i32)
        ws = moe_dispatch_layout_workspace_bytes(s.T, s.K, s.L)
        self.workspace = torch.zeros(max(ws, 4), dtype=torch.uint8, device=dev)
        # K-split partial sums of the GEMMs' last round (both GEMMs run on one
        # stream, one after the other, so they share it)
        self.gemm_workspace = torch.empty(moe_grouped_gemm_workspace_bytes(), dtype=torch.uint8,
                                          device=dev)
        self.buf = torch.empty(rc, s.H, dtype=_TORCH[s.buf_dt], device=dev)
        self.buf_scales = (torch.empty(rc, s.H // 128, dtype=torch.float32, device=dev)
                           if s.buf_dt == "fp8" else None)
        self.g = None if fused else torch.empty(rc, 2 * s.I, dtype=torch.float32, device=dev)
        self.z = torch.empty(rc, s.I, dtype=_TORCH[s.z_dt], device=dev)
        self.z_scales = (torch.empty(rc, s.I // 128, dtype=torch.float32, device=dev)
                         if s.z_dt == "fp8" else None)
        self.out = torch.empty(rc, s.H, dtype=_TORCH[s.out_dt], device=dev)
        self.y = torch.empty(s.T, s.H, dtype=_TORCH[s.out_dt], device=dev)
        self.w13 = self.w13_scales = self.w2 = self.w2_scales = self.w13_packed = None

    def set_fused(self, fused: bool):
        """Switch the gate/up GEMM between the fused SiLU*up epilogue (the
        inference forward; a backward recomputes G) and the unfused pair
        (stores fp32 G, which the backward then reuses)."""
        s = self.shape
        if not fused and self.g is None:
            g = getattr(self, "g_saved", None)
            self.g = g if g is not None else torch.empty(s.rows_cap, 2 * s.I, dtype=torch.float32,
                                                         device=self.buf.device)
        if fused:
            self.g = None
        self.fused = fused

    def set_weights(self, w13, w2, w13_scales=None, w2_scales=None, pack_w13=True):
        """Device weights in the pages' layouts.  With pack_w13 (the default)
        the gate/up weights are also packed once into the GEMM's staging
        order (moe_pack_w13), which the gate/up GEMM then reads."""
        self.w13, self.w2, self.w13_scales, self.w2_scales = w13, w2, w13_scales, w2_scales
        self.w13_packed = None
        if pack_w13:
            self.w13_packed = torch.empty_like(w13)
            moe_pack_w13(w13, self.w13_packed)

    # ---- the six steps
    def layout(self, topk_ids):
        s = self.shape
        moe_dispatch_layout(topk_ids, s.E, s.expert_begin, s.L, s.R, s.BM, self.counts,
                            self.offsets, self.slot_of, self.row_src, self.tile_offsets,
                            self.dev_status, self.workspace)

    def permute(self, x):
        moe_permute(x, self.slot_of, self.buf, self.buf_scales)

    def gemm_w13(self):
        w, lay = ((self.w13_packed, MOE_W_PACKED) if self.w13_packed is not None
                  else (self.w13, MOE_W_ROW_MAJOR))
        if self.fused:
            moe_grouped_gemm_w13(self.buf, self.buf_scales, w, self.w13_scales, self.counts,
                                 self.offsets, MOE_EPI_SILU_MUL, self.z, self.z_scales,
                                 workspace=self.gemm_workspace, w13_layout=lay)
        else:
            moe_grouped_gemm_w13(self.buf, self.buf_scales, w, self.w13_scales, self.counts,
                                 self.offsets, MOE_EPI_STORE_G, self.g,
                                 workspace=self.gemm_workspace, w13_layout=lay)

    def silu_mul(self):
        if not self.fused:
            moe_silu_mul(self.g, self.counts, self.offsets, self.z, self.z_scales)

    def gemm_w2(self):
        moe_grouped_gemm_w2(self.z, self.z_scales, self.w2, self.w2_scales, self.counts,
                            self.offsets, self.out, workspace=self.gemm_workspace)

    def combine(self, topk_weights):
        moe_combine(self.out, self.slot_of, topk_weights, self.y)

    # ---- backward (bf16 / fp32 layers)
    def prepare_backward(self):
        """Transposed weights and gradient buffers, made once (the weights are
        transposed again when set_weights installs new tensors; in-place
        updates need refresh_transposed_weights)."""
        s = self.shape
        if s.wdt == "fp8":
            raise ValueError("the backward covers bf16 and fp32 layers")
        dev = self.buf.device
        gdt = self.out.dtype                       # gradients stored like the expert output
        src = getattr(self, "_wt_src", None)
        if src is None or src[0] is not self.w13 or src[1] is not self.w2:
            self.w2_t = torch.empty(s.L, s.I, s.H, dtype=self.w2.dtype, device=dev)
            self.w13_t = torch.empty(s.L, s.H, 2 * s.I, dtype=self.w13.dtype, device=dev)
            self._wt_src = (self.w13, self.w2)
            self.refresh_transposed_weights()
        rc = s.rows_cap
        if getattr(self, "d_out", None) is None:
            self.d_out = torch.empty(rc, s.H, dtype=gdt, device=dev)
            self.d_w = torch.empty(s.T, s.K, dtype=torch.float32, device=dev)
            self.dz = torch.empty(rc, s.I, dtype=gdt, device=dev)
            self.dg = torch.empty(rc, 2 * s.I, dtype=gdt, device=dev)
            self.da = torch.empty(rc, s.H, dtype=gdt, device=dev)
            self.dx = torch.empty(s.T, s.H, dtype=gdt, device=dev)
            self.dw2 = torch.empty(s.L, s.H, s.I, dtype=torch.float32, device=dev)
            self.dw13 = torch.empty(s.L, 2 * s.I, s.H, dtype=torch.float32, device=dev)

    def refresh_transposed_weights(self):
        """Rewrite W2^T and W13^T from the current weights.  prepare_backward
        does it when set_weights installs new weight tensors; a caller that
        updates the weights in place (an optimizer step) calls this before
        the next backward."""
        moe_transpose_weights(self.w2, self.w2_t)
        moe_transpose_weights(self.w13, self.w13_t)

    def backward_stages(self, dy, topk_weights, weight_grads=True, fuse_silu=True):
        """The backward as (name, launch) pairs in run order, for dy [T,H]:
        combine backward, dZ = d_out W2 (on W2^T), dG, dA = dG W13 (on
        W13^T), permute backward, then with weight_grads dW2 = d_out^T Z and
        dW13 = dG^T A per expert.  dG comes from G and dZ: after the unfused
        forward, which kept G, the SiLU*up backward reads it; after the fused
        forward the gate/up GEMM recomputes G with the SiLU*up gradient in its
        epilogue ("gemm_g_silu_bw"), or, with fuse_silu=False, stores fp32 G
        (g_saved) for a separate SiLU*up backward (the same values)."""
        self.prepare_backward()
        s = self.shape
        w, lay = ((self.w13_packed, MOE_W_PACKED) if self.w13_packed is not None
                  else (self.w13, MOE_W_ROW_MAJOR))
        st = [
            ("combine_bw", lambda: moe_combine_backward(dy, self.out, self.slot_of, topk_weights,
                                                        self.d_out, self.d_w)),
            ("gemm_dz", lambda: moe_grouped_gemm_w2(self.d_out, None, self.w2_t, None, self.counts,
                                                    self.offsets, self.dz, workspace=self.gemm_workspace)),
        ]
        if self.g is None and fuse_silu:
            st.append(("gemm_g_silu_bw", lambda: moe_grouped_gemm_w13_silu_backward(
                self.buf, w, self.counts, self.offsets, self.dz, self.dg, workspace=self.gemm_workspace,
                w13_layout=lay)))
        else:
            if self.g is not None:
                self.g_saved = self.g                # kept by the unfused forward
            else:
                if getattr(self, "g_saved", None) is None:
                    self.g_saved = torch.empty(s.rows_cap, 2 * s.I, dtype=torch.float32,
                                               device=self.buf.device)
                st.append(("gemm_g", lambda: moe_grouped_gemm_w13(
                    self.buf, self.buf_scales, w, self.w13_scales, self.counts, self.offsets,
                    MOE_EPI_STORE_G, self.g_saved, workspace=self.gemm_workspace, w13_layout=lay)))
            st.append(("silu_mul_bw", lambda: moe_silu_mul_backward(self.g_saved, self.dz, self.counts,
                                                                    self.offsets, self.dg)))
        st += [
            ("gemm_da", lambda: moe_grouped_gemm_w2(self.dg, None, self.w13_t, None, self.counts,
                                                    self.offsets, self.da, workspace=self.gemm_workspace)),
            ("permute_bw", lambda: moe_permute_backward(self.da, self.slot_of, self.dx)),
        ]
        if weight_grads:
            st += [
                ("wgrad_w2", lambda: moe_grouped_gemm_wgrad(self.d_out, self.z, self.counts,
                                                            self.offsets, self.dw2)),
                ("wgrad_w13", lambda: moe_grouped_gemm_wgrad(self.dg, self.buf, self.counts,
                                                             self.offsets, self.dw13)),
            ]
        return st

    def backward(self, dy, topk_weights, weight_grads=True, fuse_silu=True):
        """Gradients of the last forward for dy [T,H]: returns (dx [T,H],
        d_w [T,K]); with weight_grads also fills dw2 [L,H,I] = d_out^T Z and
        dw13 [L,2I,H] = dG^T A per expert.  Reuses the forward's routing
        (slot_of, counts, offsets), its permuted activations, Z and expert
        outputs; G is the unfused forward's, else recomputed."""
        for _, f in self.backward_stages(dy, topk_weights, weight_grads, fuse_silu):
            f()
        return self.dx, self.d_w

    def bind_forward(self, x, topk_ids, topk_weights):
        """The forward's launches as (name, callable) pairs, each marshalled
        once (shapes checked, pointers and the current stream looked up), so
        calling them runs the path with a few microseconds of host time per
        launch.  The tensors must stay alive and unchanged in shape."""
        s = self.shape
        w, lay = ((self.w13_packed, MOE_W_PACKED) if self.w13_packed is not None
                  else (self.w13, MOE_W_ROW_MAJOR))
        st = [
            ("layout", moe_dispatch_layout(topk_ids, s.E, s.expert_begin, s.L, s.R, s.BM, self.counts,
                                           self.offsets, self.slot_of, self.row_src, self.tile_offsets,
                                           self.dev_status, self.workspace, bind=True)),
            ("permute", moe_permute(x, self.slot_of, self.buf, self.buf_scales, bind=True)),
        ]
        if self.fused:
            st.append(("gemm_w13", moe_grouped_gemm_w13(self.buf, self.buf_scales, w, self.w13_scales,
                                                         self.counts, self.offsets, MOE_EPI_SILU_MUL, self.z,
                                                         self.z_scales, workspace=self.gemm_workspace,
                                                         w13_layout=lay, bind=True)))
        else:
            st.append(("gemm_w13", moe_grouped_gemm_w13(self.buf, self.buf_scales, w, self.w13_scales,
                                                         self.counts, self.offsets, MOE_EPI_STORE_G, self.g,
                                                         workspace=self.gemm_workspace, w13_layout=lay,
                                                         bind=True)))
            st.append(("silu_mul", moe_silu_mul(self.g, self.counts, self.offsets, self.z, self.z_scales,
                                                bind=True)))
        st += [
            ("gemm_w2", moe_grouped_gemm_w2(self.z, self.z_scales, self.w2, self.w2_scales, self.counts,
                                            self.offsets, self.out, workspace=self.gemm_workspace,
                                            bind=True)),
            ("combine", moe_combine(self.out, self.slot_of, topk_weights, self.y, bind=True)),
        ]
        return st

    def forward(self, x, topk_ids, topk_weights):
        """The whole path on the current stream; returns y [T,H] (no sync)."""
        self.layout(topk_ids)
        self.permute(x)
        self.gemm_w13()
        self.silu_mul()
        self.gemm_w2()
        self.combine(topk_weights)
        return self.y
