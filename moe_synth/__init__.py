"""Seeded synthetic inputs for a top-k MoE SwiGLU layer.

This module only DRAWS inputs: random normals, the fixed scaling of their
distribution, rounding to the storage dtype and (for the INT4 layer) the
quantiser that produces the stored nibbles and scales.  It holds none of the
layer's own arithmetic (no router product, scoring, selection, permutation,
expert FFN or combine).  Both the CPU oracle and the GPU path consume what it
produces; neither shares any other code.

Layers are shaped like the models the pages study (OLMoE-1B-7B,
DeepSeek-V2-Lite, Qwen3-30B-A3B, DeepSeek-V3) plus a tiny fp32 layer.  Weights
are random (no checkpoints): W ~ N(0, 1/fan_in) (variance 1/fan_in), router
skew and selection biases ~ N(0, std).

Storage layout (what the library consumes):
  x            [T][d]          act dtype (fp32 or bf16)
  w_router     [E][d]          act dtype (one K-contiguous row per expert)
  logit_bias   [E]             fp32 or None (added to router logits)
  select_bias  [E]             fp32 or None (selection only, sigmoid scoring)
  w_gate/w_up  [E][ffn][d]     expert dtype (K-contiguous rows per output channel)
  w_down       [E][d][ffn]
  INT4 experts: packed uint8 [E][N][K/2] (low nibble = even k) and bf16 scales
  [E][N][K/128]; shared experts [S][...] in the same layout.

Generation runs with torch on the requested device so the 22.5 GB DeepSeek-V3
layer can be drawn in seconds on the GPU; the same recipe runs on the CPU for
small layers.  A torch.Generator is seeded per (seed, layer, tensor) so every
tensor is reproducible on its own.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

__all__ = ["LayerSpec", "SPECS", "Layer", "make_layer", "make_tokens", "spec"]


@dataclasses.dataclass(frozen=True)
class LayerSpec:
    name: str
    cfg_id: int
    d: int
    E: int
    k: int
    ffn: int
    n_shared: int
    ffn_shared: int
    act: str              # 'f32' | 'bf16'  (x, router weight, outputs)
    expert: str           # 'f32' | 'bf16' | 'int4' | 'fp8' | 'fp8a8' (fp8 weights, FP8 activations)
    score: str            # 'softmax' | 'sigmoid'
    renorm: bool          # gates /= sum over the selected k
    gate_scale: float     # multiplies routed gates (2.5 for DeepSeek-V3)
    logit_bias_std: float  # 0 -> no router skew bias
    select_bias_std: float  # 0 -> no selection-only bias
    rms_norm_x: bool
    tokens: tuple         # token counts the layer is exercised at
    capacity: Optional[tuple] = None  # (num, den) for C = num/den, None = dropless
    groups: Optional[tuple] = None    # (n_groups, topk_groups) for group-limited selection, None = none

    def replace(self, **kw) -> "LayerSpec":
        return dataclasses.replace(self, **kw)


SPECS = {
    "tiny_f32": LayerSpec("tiny_f32", 0, d=128, E=8, k=2, ffn=256, n_shared=0, ffn_shared=0,
                          act="f32", expert="f32", score="softmax", renorm=False, gate_scale=1.0,
                          logit_bias_std=0.5, select_bias_std=0.0, rms_norm_x=False,
                          tokens=(64,)),
    "olmoe": LayerSpec("olmoe", 1, d=2048, E=64, k=8, ffn=1024, n_shared=0, ffn_shared=0,
                       act="bf16", expert="bf16", score="softmax", renorm=False, gate_scale=1.0,
                       logit_bias_std=0.5, select_bias_std=0.0, rms_norm_x=True,
                       tokens=(1, 8, 32, 64, 4096)),
    "dsv2_lite": LayerSpec("dsv2_lite", 2, d=2048, E=64, k=6, ffn=1408, n_shared=2, ffn_shared=1408,
                           act="bf16", expert="bf16", score="softmax", renorm=False, gate_scale=1.0,
                           logit_bias_std=0.7, select_bias_std=0.0, rms_norm_x=False,
                           tokens=(8192,)),
    "qwen3_int4": LayerSpec("qwen3_int4", 3, d=2048, E=128, k=8, ffn=768, n_shared=0, ffn_shared=0,
                            act="bf16", expert="int4", score="softmax", renorm=True, gate_scale=1.0,
                            logit_bias_std=0.0, select_bias_std=0.0, rms_norm_x=False,
                            tokens=(32, 4096)),
    "dsv3": LayerSpec("dsv3", 4, d=7168, E=256, k=8, ffn=2048, n_shared=1, ffn_shared=2048,
                      act="bf16", expert="bf16", score="sigmoid", renorm=True, gate_scale=2.5,
                      logit_bias_std=0.0, select_bias_std=0.1, rms_norm_x=False,
                      tokens=(1, 16, 256, 4096, 16384)),
}
# DeepSeek-V2-Lite is also run with a fixed capacity C = 1.25.
SPECS["dsv2_lite_cap"] = SPECS["dsv2_lite"].replace(name="dsv2_lite_cap", capacity=(5, 4))
# the OLMoE-shaped layer with FP8 (E4M3) expert weights and per-channel scales (decode sizes)
SPECS["olmoe_fp8"] = SPECS["olmoe"].replace(name="olmoe_fp8", cfg_id=5, expert="fp8", tokens=(1, 8, 32, 64, 4096))
# the DeepSeek-V2-Lite-shaped layer with FP8 routed and shared experts (prefill)
SPECS["dsv2_lite_fp8"] = SPECS["dsv2_lite"].replace(name="dsv2_lite_fp8", cfg_id=6, expert="fp8")
# FP8 weights with FP8 activations (the same weights as the fp8 layers of the same cfg_id): the
# OLMoE-shaped layer and the DeepSeek-V3-shaped layer (one shared expert)
SPECS["olmoe_fp8a8"] = SPECS["olmoe_fp8"].replace(name="olmoe_fp8a8", expert="fp8a8")
SPECS["dsv3_fp8a8"] = SPECS["dsv3"].replace(name="dsv3_fp8a8", expert="fp8a8")
# the DeepSeek-V2-Lite-shaped layer (two shared experts) with FP8 activations, on the weights of
# dsv2_lite_fp8
SPECS["dsv2_lite_fp8a8"] = SPECS["dsv2_lite_fp8"].replace(name="dsv2_lite_fp8a8", expert="fp8a8")


def spec(name: str) -> LayerSpec:
    return SPECS[name]


INT4_GROUP = 128

# tensor ids for seeding
_T_X, _T_WR, _T_BL, _T_BS, _T_WG, _T_WU, _T_WD, _T_SG, _T_SU, _T_SD = range(10)


def _gen(device, seed: int, cfg_id: int, tensor_id: int, extra: int = 0) -> torch.Generator:
    g = torch.Generator(device=device)
    # fixed mixing of the identifying integers into one 63-bit seed
    h = (seed * 1_000_003 + cfg_id) * 1_000_033 + tensor_id
    h = (h * 1_000_037 + extra) & ((1 << 63) - 1)
    g.manual_seed(h)
    return g


def _dt(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def _normal(shape, std, g, device) -> torch.Tensor:
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).mul_(std)


def _quantise_int4(w: torch.Tensor):
    """Symmetric per-output-channel INT4 quantiser with groups of 128 along K.

    Data generation only: s = bf16(absmax/7), q = clamp(rint_half_even(w/s), -8, 7),
    s == 0 -> q = 0.  Packing: byte i of a row holds k = 2i in its low nibble and
    k = 2i+1 in its high nibble, both two's complement."""
    N, K = w.shape[-2], w.shape[-1]
    assert K % INT4_GROUP == 0
    wg = w.reshape(*w.shape[:-1], K // INT4_GROUP, INT4_GROUP)
    s = (wg.abs().amax(dim=-1) / 7.0).to(torch.bfloat16)
    sf = s.to(torch.float32).unsqueeze(-1)
    q = torch.where(sf > 0, torch.round(wg / torch.where(sf > 0, sf, torch.ones_like(sf))),
                    torch.zeros_like(wg))
    q = q.clamp_(-8, 7).to(torch.int16).reshape(*w.shape)
    lo = (q[..., 0::2] & 0xF)
    hi = (q[..., 1::2] & 0xF)
    packed = (lo | (hi << 4)).to(torch.uint8)
    return packed, s


def _quantise_fp8(w: torch.Tensor):
    """Per-output-channel FP8 (OCP E4M3, the "fn" variant) quantiser.

    Data generation only: s = absmax over the channel's K values / 448 (fp32), codes =
    torch's round-to-nearest-even conversion of w / s to float8_e4m3fn, stored as bytes;
    s == 0 -> codes 0."""
    s = w.abs().amax(dim=-1) / 448.0
    sf = torch.where(s > 0, s, torch.ones_like(s)).unsqueeze(-1)
    codes = (w / sf).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, s.to(torch.float32)


@dataclasses.dataclass
class Layer:
    """All weights of one synthetic MoE layer (tokens are drawn separately)."""
    spec: LayerSpec
    w_router: torch.Tensor
    logit_bias: Optional[torch.Tensor]
    select_bias: Optional[torch.Tensor]
    w_gate: torch.Tensor
    w_up: torch.Tensor
    w_down: torch.Tensor
    s_gate: Optional[torch.Tensor] = None
    s_up: Optional[torch.Tensor] = None
    s_down: Optional[torch.Tensor] = None
    sh_gate: Optional[torch.Tensor] = None
    sh_up: Optional[torch.Tensor] = None
    sh_down: Optional[torch.Tensor] = None
    shs_gate: Optional[torch.Tensor] = None   # FP8 shared-expert scales [S][N] (None otherwise)
    shs_up: Optional[torch.Tensor] = None
    shs_down: Optional[torch.Tensor] = None


def _expert_mats(sp: LayerSpec, n: int, ffn: int, ids, seed, device, chunk):
    """Draw gate/up [n][ffn][d] and down [n][d][ffn] in the spec's expert dtype."""
    d = sp.d
    out = []
    for tid, shape_tail, fan_in in ((ids[0], (ffn, d), d), (ids[1], (ffn, d), d),
                                    (ids[2], (d, ffn), ffn)):
        std = 1.0 / math.sqrt(fan_in)
        g = _gen(device, seed, sp.cfg_id, tid)
        if sp.expert == "int4":
            packed = torch.empty((n, shape_tail[0], shape_tail[1] // 2), dtype=torch.uint8, device=device)
            scales = torch.empty((n, shape_tail[0], shape_tail[1] // INT4_GROUP), dtype=torch.bfloat16,
                                 device=device)
            for e0 in range(0, n, chunk):
                e1 = min(n, e0 + chunk)
                w = _normal((e1 - e0,) + shape_tail, std, g, device)
                packed[e0:e1], scales[e0:e1] = _quantise_int4(w)
                del w
            out.append((packed, scales))
        elif sp.expert in ("fp8", "fp8a8"):
            codes = torch.empty((n,) + shape_tail, dtype=torch.uint8, device=device)
            scales = torch.empty((n, shape_tail[0]), dtype=torch.float32, device=device)
            for e0 in range(0, n, chunk):
                e1 = min(n, e0 + chunk)
                w = _normal((e1 - e0,) + shape_tail, std, g, device)
                codes[e0:e1], scales[e0:e1] = _quantise_fp8(w)
                del w
            out.append((codes, scales))
        else:
            t = torch.empty((n,) + shape_tail, dtype=_dt(sp.expert), device=device)
            for e0 in range(0, n, chunk):
                e1 = min(n, e0 + chunk)
                t[e0:e1] = _normal((e1 - e0,) + shape_tail, std, g, device).to(t.dtype)
            out.append((t, None))
    return out


def make_layer(sp: LayerSpec, device="cpu", seed: int = 0, chunk: int = 16) -> Layer:
    """Draw the weights of layer `sp` on `device` (seeded, deterministic per device)."""
    if isinstance(sp, str):
        sp = SPECS[sp]
    act = _dt(sp.act)
    g = _gen(device, seed, sp.cfg_id, _T_WR)
    w_router = _normal((sp.E, sp.d), 1.0 / math.sqrt(sp.d), g, device).to(act)
    logit_bias = None
    if sp.logit_bias_std > 0:
        logit_bias = _normal((sp.E,), sp.logit_bias_std, _gen(device, seed, sp.cfg_id, _T_BL), device)
    select_bias = None
    if sp.select_bias_std > 0:
        select_bias = _normal((sp.E,), sp.select_bias_std, _gen(device, seed, sp.cfg_id, _T_BS), device)
    (wg, sg), (wu, su), (wd, sd) = _expert_mats(sp, sp.E, sp.ffn, (_T_WG, _T_WU, _T_WD), seed, device, chunk)
    lay = Layer(sp, w_router, logit_bias, select_bias, wg, wu, wd, sg, su, sd)
    if sp.n_shared:
        (a, sa), (b, sb), (c, sc) = _expert_mats(sp.replace(expert="bf16" if sp.expert == "int4" else sp.expert),
                                                 sp.n_shared, sp.ffn_shared, (_T_SG, _T_SU, _T_SD), seed,
                                                 device, chunk)
        lay.sh_gate, lay.sh_up, lay.sh_down = a, b, c
        if sp.expert in ("fp8", "fp8a8"):
            lay.shs_gate, lay.shs_up, lay.shs_down = sa, sb, sc
    return lay


def make_tokens(sp: LayerSpec, T: int, device="cpu", seed: int = 0) -> torch.Tensor:
    """Draw the hidden states x [T][d] ~ N(0,1); RMS-normalise rows where the layer says so."""
    if isinstance(sp, str):
        sp = SPECS[sp]
    g = _gen(device, seed, sp.cfg_id, _T_X, extra=T)
    x = torch.randn((T, sp.d), generator=g, device=device, dtype=torch.float32)
    if sp.rms_norm_x and T > 0:
        xd = x.to(torch.float64)
        xd = xd / torch.sqrt((xd * xd).mean(dim=1, keepdim=True))
        x = xd.to(torch.float32) if sp.act == "f32" else xd
    return x.to(_dt(sp.act))


def make_bf16_twin(sp: LayerSpec, device="cpu", seed: int = 0, chunk: int = 16):
    """Pre-quantisation expert weights of an INT4 layer, rounded to bf16 (quality context)."""
    if isinstance(sp, str):
        sp = SPECS[sp]
    twin = sp.replace(expert="bf16")
    (wg, _), (wu, _), (wd, _) = _expert_mats(twin, sp.E, sp.ffn, (_T_WG, _T_WU, _T_WD), seed, device, chunk)
    return wg, wu, wd
