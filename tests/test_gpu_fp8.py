"""GPU tests of FP8 (OCP E4M3) expert weights with per-channel fp32 scales
("MoE at the inference level", workarounds: fp8 expert weights halve the bytes),
on the decode (streaming) and prefill (tiled) kernels, routed and shared experts.

- Parity against the FP64 oracle, which decodes every byte exactly, on
  OLMoE- and Qwen3-shaped layers at decode sizes, in both weight layouts.
- Every one of the 254 finite codes through the kernel: weights that make each
  output a single product, so the FP8 layer and its exact bf16 twin (every E4M3
  value times a power-of-two scale is exact in bf16) must agree bit for bit."""
import dataclasses

import numpy as np
import pytest
import torch

import moe_synth as S
import oracle as O
from gpu_harness import compare_routes, layer_of, oracle_run, row_rel_err, tol_of

pytestmark = pytest.mark.gpu

FP8 = S.SPECS["olmoe_fp8"]
QW8 = S.SPECS["qwen3_int4"].replace(name="qwen3_fp8", cfg_id=32, expert="fp8")
_LAY = {}


def _layer(sp):
    if sp.name not in _LAY:
        _LAY.clear()
        torch.cuda.empty_cache()
        _LAY[sp.name] = S.make_layer(sp, device="cuda")
    return _LAY[sp.name]


@pytest.mark.parametrize("layout", ["rows", "tiled"])
@pytest.mark.parametrize("name,T", [("olmoe", 1), ("olmoe", 8), ("olmoe", 32), ("olmoe", 64), ("qwen3", 32),
                                    ("qwen3", 5)])
def test_fp8_forward_matches_oracle(name, T, layout):
    sp = FP8 if name == "olmoe" else QW8
    lay = _layer(sp)
    ml = layer_of(sp, lay, layout)
    x = S.make_tokens(sp, T, device="cuda", seed=T)
    out, idx, gates, drop = ml.forward(x)
    torch.cuda.synchronize()
    ref = oracle_run(sp, lay, x)
    rep = compare_routes(idx.cpu().numpy(), ref, sp.k)
    assert rep.set_mismatch_strict == 0 and rep.order_mismatch == 0
    ok = rep.matched
    rel = row_rel_err(out.float().cpu().numpy().astype(np.float64)[ok], ref["out"][ok])
    print(f"  {sp.name} T={T} {layout}: max row rel err {rel.max(initial=0):.2e}")
    assert rel.max(initial=0) <= tol_of(sp)


def _codes_layers(layout):
    """An FP8 layer (E=16, k=1) whose outputs are single products, and its bf16 twin.
    Gate and up: row 165 of every expert holds code 0x38 (1.0) at K = 7 and zeros
    elsewhere, so h[165] = silu(x_7) * x_7 and every other h is 0.  Down: expert e's
    output column n holds code (512 e + n) mod 256 at K = 165 (NaN codes 0x7F, 0xFF
    replaced by 0), with scale 2^-(n mod 4), so y[n] = h[165] * fp8(code) * 2^-(n mod 4):
    each expert carries every code twice."""
    sp = S.SPECS["olmoe_fp8"].replace(name="fp8_codes", cfg_id=33, d=512, E=16, k=1, ffn=256)
    base = S.make_layer(sp, device="cpu")
    E, d, F = sp.E, sp.d, sp.ffn
    gu = torch.zeros((E, F, d), dtype=torch.uint8)
    gu[:, 165, 7] = 0x38
    dn = torch.zeros((E, d, F), dtype=torch.uint8)
    codes = (torch.arange(E)[:, None] * 512 + torch.arange(d)[None, :]) % 256
    codes[(codes == 0x7F) | (codes == 0xFF)] = 0
    dn[:, :, 165] = codes.to(torch.uint8)
    ones = torch.ones((E, F), dtype=torch.float32)
    sd = torch.pow(2.0, -(torch.arange(d) % 4).to(torch.float32))[None, :].repeat(E, 1)
    dev = "cuda"
    lay8 = dataclasses.replace(base, w_router=base.w_router.to(dev), logit_bias=base.logit_bias.to(dev),
                               w_gate=gu.to(dev), w_up=gu.clone().to(dev), w_down=dn.to(dev), s_gate=ones.to(dev),
                               s_up=ones.clone().to(dev), s_down=sd.to(dev))

    def deq(q, s):
        w = O.fp8_dequant(q.numpy(), s.numpy())
        wb = torch.from_numpy(w).to(torch.bfloat16)
        assert torch.equal(wb.to(torch.float64), torch.from_numpy(w))  # exact by construction
        return wb.to(dev)
    spb = sp.replace(expert="bf16")
    layb = dataclasses.replace(lay8, spec=spb, w_gate=deq(gu, ones), w_up=deq(gu, ones), w_down=deq(dn, sd),
                               s_gate=None, s_up=None, s_down=None)
    return sp, lay8, spb, layb


@pytest.mark.parametrize("T", [64, 100])
@pytest.mark.parametrize("layout", ["rows", "tiled"])
def test_every_fp8_code_decodes_exactly(layout, T):
    """T = 64 runs the streaming (decode) kernels, T = 100 the tiled (prefill) ones,
    with non-temporal weight loads."""
    sp, lay8, spb, layb = _codes_layers(layout)
    m8, mb = layer_of(sp, lay8, layout), layer_of(spb, layb, layout)
    x = S.make_tokens(sp, T, device="cuda", seed=5)
    o8, ob = m8.forward(x), mb.forward(x)
    torch.cuda.synchronize()
    assert torch.equal(o8[1], ob[1])
    assert torch.equal(o8[0], ob[0])
    # the products are there: in each output row the decoded codes times the row's constant
    y = ob[0].float().cpu().numpy().astype(np.float64)
    e = o8[1].cpu().numpy()[:, 0]
    n = np.arange(sp.d)
    for t in range(8):
        c = (e[t] * 512 + n) % 256
        c[(c == 0x7F) | (c == 0xFF)] = 0
        ref = O.fp8_e4m3_to_f64(c.astype(np.uint8)) * 2.0 ** -(n % 4)
        nz = ref != 0
        ratio = y[t, nz] / ref[nz]
        assert np.allclose(ratio, ratio[0], rtol=1e-2), t  # y = const * fp8(code) * scale, to bf16 rounding


def _sample(T, n, seed=0):
    return np.arange(T) if T <= n else np.sort(np.random.default_rng(seed).choice(T, n, replace=False))


@pytest.mark.parametrize("layout", ["rows", "tiled"])
@pytest.mark.parametrize("name,T", [("olmoe_fp8", 4096), ("dsv2_lite_fp8", 3000), ("dsv2_lite_fp8", 40),
                                    ("olmoe_fp8", 300)])
def test_fp8_prefill_and_shared_experts_match_oracle(name, T, layout):
    """The tiled FP8 kernels (T > 64: OLMoE-shaped at T = 4096 and 300, the latter with
    non-temporal weight loads; DeepSeek-V2-Lite-shaped with two FP8 shared experts at
    T = 3000) and the streaming ones with FP8 shared experts (T = 40), against the
    oracle on a token sample."""
    sp = S.SPECS[name]
    lay = _layer(sp)
    ml = layer_of(sp, lay, layout)
    x = S.make_tokens(sp, T, device="cuda", seed=T)
    out, idx, gates, drop = ml.forward(x)
    torch.cuda.synchronize()
    rows = _sample(T, 128)
    ref = oracle_run(sp, lay, x, ffn_rows=rows)
    rep = compare_routes(idx.cpu().numpy(), ref, sp.k)
    assert rep.set_mismatch_strict == 0 and rep.order_mismatch == 0
    ok = rows[rep.matched[rows]]
    assert len(ok) >= 0.9 * len(rows)
    rel = row_rel_err(out.float().cpu().numpy().astype(np.float64)[ok], ref["out"][ok])
    print(f"  {name} T={T} {layout}: max row rel err {rel.max(initial=0):.2e} over {len(ok)} tokens")
    assert rel.max(initial=0) <= tol_of(sp)
