"""GPU pins of the INT4 expert path against the GPU's own bf16 path.

With power-of-two group scales and |q| <= 8, every dequantised weight q*s is
exact in bf16, so an INT4 layer and a bf16 layer holding those exact weights
compute the same function: their outputs may differ only by fp32
accumulation order, and by the bf16 roundings of h and of the expert rows
that such a difference can flip (one bf16 step is 2^-8 of the value), so the
bar here is 1e-2 per row and 1e-3 on average, against 5e-2 for INT4 against
the oracle; a misplaced nibble, row or scale group moves an output by O(1).
One-hot weights (a single non-zero nibble) then pin the nibble order inside a
byte, the scale group a K index reads and the output row or column it lands
in, in both weight layouts and in both the streaming (decode) and the tiled
(prefill) kernels."""
import numpy as np
import pytest
import torch

import moe_synth as S
from gpu_harness import layer_of, row_rel_err

pytestmark = pytest.mark.gpu

# a small layer with the Qwen3-30B-A3B routing (softmax, renormalised top-k, INT4 g128 experts)
SP = S.SPECS["qwen3_int4"].replace(name="int4_pins", cfg_id=41, d=512, E=16, k=4, ffn=256)
BF = SP.replace(expert="bf16")
PAIR_MAX, PAIR_MEAN = 1e-2, 1e-3


def _pack(q: torch.Tensor) -> torch.Tensor:
    """[..., K] int nibbles in [-8, 7] -> [..., K/2] bytes (even k in the low nibble)."""
    q = q.to(torch.int16)
    return ((q[..., 0::2] & 0xF) | ((q[..., 1::2] & 0xF) << 4)).to(torch.uint8)


def _pow2_int4(n: int, rows: int, K: int, g: torch.Generator, zero: bool = False):
    """Random nibbles (or zeros) and power-of-two bf16 scales 2^-9 .. 2^-5 per 128-K group."""
    q = torch.zeros((n, rows, K), dtype=torch.int16) if zero else \
        torch.randint(-8, 8, (n, rows, K), generator=g, dtype=torch.int16)
    p = torch.randint(-9, -4, (n, rows, K // 128), generator=g)
    s = torch.pow(2.0, p.to(torch.float32)).to(torch.bfloat16)
    return q, s


def _dequant(q: torch.Tensor, s: torch.Tensor) -> torch.Tensor:
    w = q.to(torch.float32) * s.to(torch.float32).repeat_interleave(128, dim=-1)
    wb = w.to(torch.bfloat16)
    assert torch.equal(wb.to(torch.float32), w)  # exact by construction
    return wb


def _layers(mats, seed: int):
    """The INT4 layer and its exact bf16 twin over nibble/scale pairs (gate, up, down)."""
    base = S.make_layer(SP, device="cpu", seed=seed)  # router weight and logit bias
    (qg, sg), (qu, su), (qd, sd) = mats
    dev = "cuda"
    lay4 = S.Layer(SP, base.w_router.to(dev), None, None, _pack(qg).to(dev), _pack(qu).to(dev), _pack(qd).to(dev),
                   sg.to(dev), su.to(dev), sd.to(dev))
    layb = S.Layer(BF, base.w_router.to(dev), None, None, _dequant(qg, sg).to(dev), _dequant(qu, su).to(dev),
                   _dequant(qd, sd).to(dev))
    return lay4, layb


def _run_pair(lay4, layb, T: int, layout: str, seed: int):
    x = S.make_tokens(SP, T, device="cuda", seed=seed)
    o4 = layer_of(SP, lay4, layout).forward(x)
    ob = layer_of(BF, layb, layout).forward(x)
    torch.cuda.synchronize()
    assert torch.equal(o4[1], ob[1]), "routing must not depend on the expert dtype"
    assert torch.equal(o4[2], ob[2])
    return o4[0].float().cpu().numpy().astype(np.float64), ob[0].float().cpu().numpy().astype(np.float64), \
        o4[1].cpu().numpy()


@pytest.mark.parametrize("layout", ["rows", "tiled"])
@pytest.mark.parametrize("T", [1, 32, 300, 1000])
def test_power_of_two_scales_match_the_bf16_path(T, layout):
    g = torch.Generator().manual_seed(1000 + T)
    mats = [_pow2_int4(SP.E, SP.ffn, SP.d, g), _pow2_int4(SP.E, SP.ffn, SP.d, g), _pow2_int4(SP.E, SP.d, SP.ffn, g)]
    lay4, layb = _layers(mats, seed=T)
    y4, yb, _ = _run_pair(lay4, layb, T, layout, seed=T)
    assert np.abs(yb).max() > 0
    rel = row_rel_err(y4, yb)
    assert rel.max() <= PAIR_MAX and rel.mean() <= PAIR_MEAN, (rel.max(), rel.mean())


# one-hot positions: expert, row, K index.  K = 165 is odd (the high nibble of
# byte 82) and lies in scale group 1; row 77 sits inside a 16-row tile.
@pytest.mark.parametrize("which", ["gate", "up", "down"])
@pytest.mark.parametrize("T,layout", [(8, "rows"), (8, "tiled"), (600, "rows"), (600, "tiled")])
def test_one_hot_nibble_lands_on_its_weight(which, T, layout):
    g = torch.Generator().manual_seed(7)
    mats = [_pow2_int4(SP.E, SP.ffn, SP.d, g), _pow2_int4(SP.E, SP.ffn, SP.d, g), _pow2_int4(SP.E, SP.d, SP.ffn, g)]
    m = {"gate": 0, "up": 1, "down": 2}[which]
    q, s = _pow2_int4(*mats[m][0].shape, g, zero=True)
    # the expert most tokens pick, found from a bf16 run of the random layer
    lay4, layb = _layers(mats, seed=3)
    _, _, idx = _run_pair(lay4, layb, T, layout, seed=3)
    e = int(np.bincount(idx.ravel(), minlength=SP.E).argmax())
    row, kk, val = 77, 165, 3
    q[e, row, kk] = val
    s[e, row, :] = torch.tensor(2.0 ** -6, dtype=torch.bfloat16)
    s[e, row, kk // 128] = torch.tensor(2.0 ** -4, dtype=torch.bfloat16)  # a wrong group reads 4x less
    mats[m] = (q, s)
    lay4, layb = _layers(mats, seed=3)
    y4, yb, idx = _run_pair(lay4, layb, T, layout, seed=3)
    hit = (idx == e).any(axis=1)
    assert hit.any()
    # Everything but expert e's one weight is zero.  The bf16 path then gives exact zeros; the
    # INT4 streaming kernels form sum(q x) as sum((136 + q) x) - 136 sum(x), so theirs are zero up
    # to that fp32 cancellation (measured up to 6e-4 of the one-hot signal here): bounded at 1e-2
    # of the signal, which a misplaced weight (the whole signal in the wrong place) exceeds 100x.
    small = 1e-2 * np.abs(yb[hit]).max()
    assert small > 0
    # tokens that did not pick e get nothing (gate/up: silu(0) * u = 0 and g * 0 = 0)
    assert np.all(yb[~hit] == 0) and np.abs(y4[~hit]).max(initial=0) <= small
    if which == "down":
        # only output column `row` of expert e is non-zero
        cols = np.ones(SP.d, dtype=bool)
        cols[row] = False
        assert np.all(yb[:, cols] == 0) and np.abs(y4[:, cols]).max() <= small
    # one h element carries the whole signal, so a flipped bf16 rounding of it is a 2^-8 step
    rel = row_rel_err(y4[hit], yb[hit])
    assert rel.max() <= PAIR_MAX, rel.max()
