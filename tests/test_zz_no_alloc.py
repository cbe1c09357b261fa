"""moe_forward_noalloc (the forward with the library's built-in device workspace)
against moe_forward with a caller-owned workspace, through the C ABI: bit for bit
on two calls in a row, the second with fewer tokens (the built-in array keeps the
first call's contents)."""
import pytest
import torch

import moe_synth as S
from gpu_harness import cfg_of, layer_of

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.uint8) if t.dtype == torch.bfloat16 else t


@pytest.mark.parametrize("name,Ts", [("olmoe", (300, 7)), ("qwen3_int4", (64, 1)), ("dsv2_lite_cap", (256, 33)),
                                     ("olmoe_fp8a8", (200, 5))])
def test_noalloc_forward_matches_forward(name, Ts):
    from mixture_experts_layer_13_amd import binding as B
    sp = S.SPECS[name]
    lay = S.make_layer(sp, device="cuda")
    ml = layer_of(sp, lay)
    for T in Ts:
        x = S.make_tokens(sp, T, device="cuda")
        ref = [t.clone() for t in ml.forward(x)]
        c = cfg_of(sp, T)
        assert B.workspace_bytes(c) <= B.lib.moe_noalloc_scratch_bytes()
        outs = [torch.full_like(t, 7) for t in ref]
        B.moe_forward_noalloc(c, x, lay.w_router, lay.logit_bias, lay.select_bias, ml.experts, *outs)
        torch.cuda.synchronize()
        for u, v in zip(ref, outs):
            assert torch.equal(_bits(u), _bits(v)), (name, T)
