"""MoeLayer: holds one layer's weights and a workspace, allocates outputs with
torch and calls the C ABI through `binding`.  All computation runs in libmoe."""
from __future__ import annotations

from typing import Optional

import torch

from . import binding as B

_ACT = {B.MOE_F32: torch.float32, B.MOE_BF16: torch.bfloat16}


class MoeLayer:
    def __init__(self, cfg: B.MoeCfg, w_router: torch.Tensor, w_gate, w_up, w_down, *,
                 logit_bias: Optional[torch.Tensor] = None, select_bias: Optional[torch.Tensor] = None,
                 s_gate=None, s_up=None, s_down=None, sh_gate=None, sh_up=None, sh_down=None,
                 shs_gate=None, shs_up=None, shs_down=None):
        st = B.validate(cfg)
        if st != B.MOE_OK:
            raise B.MoeError(st, B.lib.moe_last_error().decode())
        self.cfg = B.MoeCfg.from_buffer_copy(cfg)
        self.w_router, self.logit_bias, self.select_bias = w_router, logit_bias, select_bias
        self._keep = (w_gate, w_up, w_down, s_gate, s_up, s_down, sh_gate, sh_up, sh_down, shs_gate, shs_up,
                      shs_down)
        self.experts = B.experts(*self._keep)
        self.device = w_router.device
        self.act_dtype = _ACT[cfg.act_dtype]
        self._ws = None

    # ------------------------------------------------------------ sizes
    def cfg_for(self, T: int) -> B.MoeCfg:
        return B.cfg_with_T(self.cfg, T)

    def workspace(self, cfg: B.MoeCfg) -> torch.Tensor:
        need = B.workspace_bytes(cfg)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(max(need, 256), dtype=torch.uint8, device=self.device)
        return self._ws

    # ------------------------------------------------------------ fused path
    def forward(self, x: torch.Tensor, out=None, topk_idx=None, topk_w=None, drop_mask=None, stream=None):
        c = self.cfg_for(x.shape[0])
        T, k, d = c.T, c.k, c.d
        dev = self.device
        out = torch.empty((T, d), dtype=self.act_dtype, device=dev) if out is None else out
        topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev) if topk_idx is None else topk_idx
        topk_w = torch.empty((T, k), dtype=torch.float32, device=dev) if topk_w is None else topk_w
        drop_mask = torch.empty((T, k), dtype=torch.uint8, device=dev) if drop_mask is None else drop_mask
        B.moe_forward(c, x, self.w_router, self.logit_bias, self.select_bias, self.experts, out, topk_idx, topk_w,
                      drop_mask, self.workspace(c), stream)
        return out, topk_idx, topk_w, drop_mask

    def forward_with_routes(self, x: torch.Tensor, topk_idx: torch.Tensor, topk_w: torch.Tensor, out=None,
                            drop_mask=None, stream=None):
        """Route replay: the layer from the given [T, k] indices and gates (no router)."""
        c = self.cfg_for(x.shape[0])
        dev = self.device
        assert topk_idx.shape == (c.T, c.k) and topk_idx.dtype == torch.int32 and topk_idx.is_contiguous()
        assert topk_w.shape == (c.T, c.k) and topk_w.dtype == torch.float32 and topk_w.is_contiguous()
        out = torch.empty((c.T, c.d), dtype=self.act_dtype, device=dev) if out is None else out
        drop_mask = torch.empty((c.T, c.k), dtype=torch.uint8, device=dev) if drop_mask is None else drop_mask
        B.moe_forward_with_routes(c, x, topk_idx, topk_w, self.experts, out, drop_mask, self.workspace(c), stream)
        return out, drop_mask

    # ------------------------------------------------------------ split path
    def route(self, x: torch.Tensor, want_scores: bool = True, stream=None):
        c = self.cfg_for(x.shape[0])
        dev = self.device
        idx = torch.empty((c.T, c.k), dtype=torch.int32, device=dev)
        gates = torch.empty((c.T, c.k), dtype=torch.float32, device=dev)
        scores = torch.empty((c.T, c.E), dtype=torch.float32, device=dev) if want_scores else None
        B.moe_route(c, x, self.w_router, self.logit_bias, self.select_bias, idx, gates, scores, self.workspace(c),
                    stream)
        return idx, gates, scores

    def permute(self, topk_idx: torch.Tensor, stream=None):
        c = self.cfg_for(topk_idx.shape[0])
        dev = self.device
        R = B.rows(c)
        counts = torch.empty(c.E, dtype=torch.int32, device=dev)
        offsets = torch.empty(c.E + 1, dtype=torch.int32, device=dev)
        row_token = torch.full((max(R, 1),), -1, dtype=torch.int32, device=dev)
        slot_row = torch.empty((c.T, c.k), dtype=torch.int32, device=dev)
        drop = torch.empty((c.T, c.k), dtype=torch.uint8, device=dev)
        B.moe_permute(c, topk_idx, counts, offsets, row_token, slot_row, drop, self.workspace(c), stream)
        return counts, offsets, row_token, slot_row, drop

    def expert_ffn(self, x: torch.Tensor, offsets: torch.Tensor, row_token: torch.Tensor, stream=None):
        c = self.cfg_for(x.shape[0])
        dev = self.device
        R = B.rows(c)
        y_rows = torch.zeros((max(R, 1), c.d), dtype=self.act_dtype, device=dev)
        y_shared = torch.empty((c.T, c.d), dtype=self.act_dtype, device=dev) if c.n_shared else None
        B.moe_expert_ffn(c, x, offsets, row_token, self.experts, y_rows, y_shared, self.workspace(c), stream)
        return y_rows, y_shared

    def combine(self, y_rows, slot_row, topk_w, y_shared, stream=None):
        c = self.cfg_for(slot_row.shape[0])
        out = torch.empty((c.T, c.d), dtype=self.act_dtype, device=self.device)
        B.moe_combine(c, y_rows, slot_row, topk_w, y_shared, out, stream)
        return out
