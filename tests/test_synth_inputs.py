"""The seeded input generator: determinism, shapes, dtypes, distributions and the INT4
quantiser's stored format.  CPU only."""
import numpy as np
import torch

import moe_synth as S
import oracle as O


def test_specs_match_layer_shapes():
    sp = S.SPECS
    assert (sp["tiny_f32"].d, sp["tiny_f32"].E, sp["tiny_f32"].k, sp["tiny_f32"].ffn) == (128, 8, 2, 256)
    assert (sp["olmoe"].d, sp["olmoe"].E, sp["olmoe"].k, sp["olmoe"].ffn) == (2048, 64, 8, 1024)
    assert (sp["dsv2_lite"].E, sp["dsv2_lite"].k, sp["dsv2_lite"].ffn, sp["dsv2_lite"].n_shared) == (64, 6, 1408, 2)
    assert sp["dsv2_lite_cap"].capacity == (5, 4)
    assert (sp["qwen3_int4"].E, sp["qwen3_int4"].k, sp["qwen3_int4"].ffn, sp["qwen3_int4"].expert) == \
        (128, 8, 768, "int4")
    assert (sp["dsv3"].d, sp["dsv3"].E, sp["dsv3"].ffn, sp["dsv3"].n_shared, sp["dsv3"].gate_scale) == \
        (7168, 256, 2048, 1, 2.5)


def _small(name, **kw):
    return S.SPECS[name].replace(**kw)


def test_generation_is_deterministic_and_seeded():
    sp = _small("olmoe", d=256, E=8, ffn=128)
    a, b = S.make_layer(sp), S.make_layer(sp)
    c = S.make_layer(sp, seed=1)
    for f in ("w_router", "w_gate", "w_up", "w_down", "logit_bias"):
        assert torch.equal(getattr(a, f), getattr(b, f))
        assert not torch.equal(getattr(a, f), getattr(c, f))
    assert torch.equal(S.make_tokens(sp, 5), S.make_tokens(sp, 5))
    assert a.w_gate.shape == (8, 128, 256) and a.w_down.shape == (8, 256, 128)
    assert a.w_gate.dtype == torch.bfloat16 and a.logit_bias.dtype == torch.float32


def test_weight_variance_is_one_over_fan_in_and_rms_rows():
    sp = _small("olmoe", d=512, E=4, ffn=256)
    lay = S.make_layer(sp)
    assert abs(lay.w_gate.float().var().item() * 512 - 1) < 0.02
    assert abs(lay.w_down.float().var().item() * 256 - 1) < 0.02
    assert abs(lay.logit_bias.std().item() - 0.5) < 0.35   # only 4 draws
    x = S.make_tokens(sp, 16).double()
    rms = x.pow(2).mean(1).sqrt()
    assert torch.allclose(rms, torch.ones_like(rms), atol=1e-2)


def test_int4_quantiser_format():
    sp = _small("qwen3_int4", d=256, E=2, ffn=128)
    lay = S.make_layer(sp)
    assert lay.w_gate.dtype == torch.uint8 and lay.w_gate.shape == (2, 128, 128)
    assert lay.s_gate.dtype == torch.bfloat16 and lay.s_gate.shape == (2, 128, 2)
    assert lay.w_down.shape == (2, 256, 64) and lay.s_down.shape == (2, 256, 1)
    twin = S.make_bf16_twin(sp)
    # the dequantised weight is within half a step of the bf16 twin, per group
    packed = lay.w_gate.numpy()
    sbits = lay.s_gate.view(torch.int16).numpy()
    w = O.int4_dequant(packed, sbits)
    ref = twin[0].float().numpy().astype(np.float64)
    step = np.repeat(O.bf16_to_f64(sbits), 128, axis=-1)
    # twin is bf16-rounded and the scale is bf16-rounded: allow a little beyond half a step
    assert (np.abs(w - ref) <= 0.5 * step + 2e-2 * np.abs(ref) + 1e-6).all()
    q = O.int4_unpack(packed)
    assert q.min() >= -8 and q.max() <= 7 and (np.abs(q) == 7).any()
