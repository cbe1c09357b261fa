"""MoeLayer: holds one layer's weights and a workspace, allocates outputs with
torch and calls the C ABI through `binding`.  All computation runs in libmoe.

Stream ownership.  Every call takes an optional `stream` (default: torch's
current stream).  Outputs and the workspace are allocated while that stream is
current, so torch's caching allocator orders their reuse after the kernels the
call enqueues; a workspace made on one stream and used on another is marked
with `record_stream`, so its memory is not handed out again before that
stream's work ends.  A workspace that a HIP graph capture used is never freed
while the layer lives (a larger T grows a new one beside it), since the graph
keeps its address."""
from __future__ import annotations

import contextlib
from typing import Optional

import torch

from . import binding as B

_ACT = {B.MOE_F32: torch.float32, B.MOE_BF16: torch.bfloat16}


def _resolve(stream, device: torch.device):
    if device.type != "cuda":
        return None
    return torch.cuda.current_stream(device) if stream is None else stream


def _on(stream):
    """Context in which torch allocations are made for `stream`."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _capturing(stream) -> bool:
    return stream is not None and torch.cuda.is_current_stream_capturing()


class Workspace:
    """The layer's workspace buffer and the rules for when it may be freed.

    get(nbytes, stream) returns a buffer of at least nbytes, allocated on
    `stream` when it has to grow.  A buffer used on another stream than the one
    it was allocated on is recorded on that stream.  Once a capture has used a
    buffer, growing keeps the old one in `retained` for the life of the layer."""

    def __init__(self, device):
        self.device = torch.device(device)
        self.buf: Optional[torch.Tensor] = None
        self.alloc_stream = None
        self.captured = False
        self.retained: list = []

    def get(self, nbytes: int, stream=None, capturing: bool = False) -> torch.Tensor:
        if self.buf is None or self.buf.numel() < nbytes:
            if self.buf is not None and self.captured:
                self.retained.append(self.buf)
            with _on(stream):
                self.buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
            self.alloc_stream, self.captured = stream, False
        elif stream is not None and stream != self.alloc_stream and not capturing:
            self.buf.record_stream(stream)
        self.captured = self.captured or capturing
        return self.buf


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
        self._ws = Workspace(self.device)

    # ------------------------------------------------------------ sizes
    def cfg_for(self, T: int) -> B.MoeCfg:
        return B.cfg_with_T(self.cfg, T)

    def workspace(self, cfg: B.MoeCfg, stream=None) -> torch.Tensor:
        s = _resolve(stream, self.device)
        return self._ws.get(B.workspace_bytes(cfg), s, _capturing(s))

    def _empty(self, shape, dtype, s, fill=None):
        with _on(s):
            if fill is None:
                return torch.empty(shape, dtype=dtype, device=self.device)
            return torch.full(shape, fill, dtype=dtype, device=self.device)

    # ------------------------------------------------------------ fused path
    def forward(self, x: torch.Tensor, out=None, topk_idx=None, topk_w=None, drop_mask=None, stream=None):
        c = self.cfg_for(x.shape[0])
        T, k, d = c.T, c.k, c.d
        s = _resolve(stream, self.device)
        out = self._empty((T, d), self.act_dtype, s) if out is None else out
        topk_idx = self._empty((T, k), torch.int32, s) if topk_idx is None else topk_idx
        topk_w = self._empty((T, k), torch.float32, s) if topk_w is None else topk_w
        drop_mask = self._empty((T, k), torch.uint8, s) if drop_mask is None else drop_mask
        B.moe_forward(c, x, self.w_router, self.logit_bias, self.select_bias, self.experts, out, topk_idx, topk_w,
                      drop_mask, self.workspace(c, s), s)
        return out, topk_idx, topk_w, drop_mask

    def forward_with_routes(self, x: torch.Tensor, topk_idx: torch.Tensor, topk_w: torch.Tensor, out=None,
                            drop_mask=None, stream=None):
        """Route replay: the layer from the given [T, k] indices and gates (no router)."""
        c = self.cfg_for(x.shape[0])
        s = _resolve(stream, self.device)
        assert topk_idx.shape == (c.T, c.k) and topk_idx.dtype == torch.int32 and topk_idx.is_contiguous()
        assert topk_w.shape == (c.T, c.k) and topk_w.dtype == torch.float32 and topk_w.is_contiguous()
        out = self._empty((c.T, c.d), self.act_dtype, s) if out is None else out
        drop_mask = self._empty((c.T, c.k), torch.uint8, s) if drop_mask is None else drop_mask
        B.moe_forward_with_routes(c, x, topk_idx, topk_w, self.experts, out, drop_mask, self.workspace(c, s), s)
        return out, drop_mask

    # ------------------------------------------------------------ split path
    def route(self, x: torch.Tensor, want_scores: bool = True, stream=None):
        c = self.cfg_for(x.shape[0])
        s = _resolve(stream, self.device)
        idx = self._empty((c.T, c.k), torch.int32, s)
        gates = self._empty((c.T, c.k), torch.float32, s)
        scores = self._empty((c.T, c.E), torch.float32, s) if want_scores else None
        B.moe_route(c, x, self.w_router, self.logit_bias, self.select_bias, idx, gates, scores,
                    self.workspace(c, s), s)
        return idx, gates, scores

    def permute(self, topk_idx: torch.Tensor, stream=None):
        c = self.cfg_for(topk_idx.shape[0])
        s = _resolve(stream, self.device)
        R = B.rows(c)
        counts = self._empty(c.E, torch.int32, s)
        offsets = self._empty(c.E + 1, torch.int32, s)
        row_token = self._empty((max(R, 1),), torch.int32, s, fill=-1)
        slot_row = self._empty((c.T, c.k), torch.int32, s)
        drop = self._empty((c.T, c.k), torch.uint8, s)
        B.moe_permute(c, topk_idx, counts, offsets, row_token, slot_row, drop, self.workspace(c, s), s)
        return counts, offsets, row_token, slot_row, drop

    def expert_ffn(self, x: torch.Tensor, offsets: torch.Tensor, row_token: torch.Tensor, stream=None):
        c = self.cfg_for(x.shape[0])
        s = _resolve(stream, self.device)
        R = B.rows(c)
        y_rows = self._empty((max(R, 1), c.d), self.act_dtype, s, fill=0)
        y_shared = self._empty((c.T, c.d), self.act_dtype, s) if c.n_shared else None
        B.moe_expert_ffn(c, x, offsets, row_token, self.experts, y_rows, y_shared, self.workspace(c, s), s)
        return y_rows, y_shared

    def combine(self, y_rows, slot_row, topk_w, y_shared, stream=None):
        c = self.cfg_for(slot_row.shape[0])
        s = _resolve(stream, self.device)
        out = self._empty((c.T, c.d), self.act_dtype, s)
        B.moe_combine(c, y_rows, slot_row, topk_w, y_shared, out, s)
        return out
