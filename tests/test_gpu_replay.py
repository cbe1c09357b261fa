"""GPU tests of route replay (moe_forward_with_routes): the layer run from given
expert indices and gates, with no router (the launch-bound study's Sub-study 2:
a model's routes replayed through a layer; replaying the layer's own routes must
return its baseline exactly).

- The control: the layer's own routes give moe_forward's output and drop mask
  bit for bit, on both permutation paths (one-block small-T and multi-block),
  with capacity, shared experts and INT4 experts.
- Foreign routes: routes from an INT4-quantised copy of the router (drift is
  non-zero and reported in swaps per token), replayed through the bf16 layer,
  against the oracle run on the same routes (outputs within the layer's bar,
  drop masks exact)."""
import dataclasses

import numpy as np
import pytest
import torch

import moe_synth as S
import oracle as O
from gpu_harness import layer_of, oracle_run, row_rel_err, tol_of

pytestmark = pytest.mark.gpu

SMALL = {
    "olmoe": S.SPECS["olmoe"].replace(name="replay_olmoe", cfg_id=21, d=512, ffn=256),
    "dsv2_lite_cap": S.SPECS["dsv2_lite_cap"].replace(name="replay_dsv2_cap", cfg_id=22, d=512, ffn=256,
                                                      ffn_shared=256),
    "qwen3_int4": S.SPECS["qwen3_int4"].replace(name="replay_qwen3", cfg_id=23, d=512, ffn=256),
    "dsv3": S.SPECS["dsv3"].replace(name="replay_dsv3", cfg_id=24, d=512, ffn=256, ffn_shared=256),
    # d >= 4096 with >= 128 rows per expert: the gate/up GEMM on 256-row items, the down GEMM on
    # its own 128-row tile map
    "dsv3_wide": S.SPECS["dsv3"].replace(name="replay_dsv3_wide", cfg_id=26, d=4096, ffn=256, ffn_shared=256),
}


@pytest.mark.parametrize("name,T", [("olmoe", 1), ("olmoe", 300), ("olmoe", 5000), ("dsv2_lite_cap", 200),
                                    ("dsv2_lite_cap", 3000), ("qwen3_int4", 32), ("qwen3_int4", 2000),
                                    ("dsv3", 16), ("dsv3", 9000), ("dsv3_wide", 4096)])
def test_own_routes_replay_bitwise(name, T):
    sp = SMALL[name]
    lay = S.make_layer(sp, device="cuda")
    ml = layer_of(sp, lay)
    x = S.make_tokens(sp, T, device="cuda", seed=T)
    out, idx, gates, drop = ml.forward(x)
    out2, drop2 = ml.forward_with_routes(x, idx, gates)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    assert torch.equal(drop, drop2)


def _int4_router(w: torch.Tensor) -> torch.Tensor:
    """w [E][d] bf16 -> symmetric INT4 per 128-wide group (scale absmax / 7, round half even),
    dequantised back to bf16: a quantised router for the drift study."""
    E, d = w.shape
    g = w.float().reshape(E, d // 128, 128)
    s = g.abs().amax(dim=2, keepdim=True) / 7.0
    q = torch.clamp(torch.round(g / torch.where(s > 0, s, torch.ones_like(s))), -8, 7)
    return (q * s).reshape(E, d).to(torch.bfloat16)


@pytest.mark.parametrize("name,T", [("olmoe", 300), ("olmoe", 5000), ("dsv2_lite_cap", 3000), ("dsv3", 256)])
def test_quantised_router_routes_replayed_match_oracle(name, T):
    sp = SMALL[name]
    lay = S.make_layer(sp, device="cuda")
    ml = layer_of(sp, lay)
    lay_q = dataclasses.replace(lay, w_router=_int4_router(lay.w_router))
    ml_q = layer_of(sp, lay_q)
    x = S.make_tokens(sp, T, device="cuda", seed=T + 1)
    _, idx0, _, _ = ml.forward(x)
    idx_q, gates_q, _ = ml_q.route(x, want_scores=False)
    out, drop = ml.forward_with_routes(x, idx_q, gates_q)
    torch.cuda.synchronize()
    swaps = O.swaps_per_token(idx0.cpu().numpy(), idx_q.cpu().numpy())
    print(f"  {name} T={T}: INT4 router drift {swaps.mean():.3f} swaps per token out of {sp.k}")
    assert swaps.sum() > 0  # the quantised router moves some picks
    rows = np.arange(T) if T <= 400 else np.sort(np.random.default_rng(3).choice(T, 400, replace=False))
    ref = oracle_run(sp, lay, x, ffn_rows=rows, routes=(idx_q.cpu().numpy(), gates_q.cpu().numpy()))
    # the drops follow the given routes only: integer work, compared exactly on every pair
    assert np.array_equal(drop.cpu().numpy().astype(bool), ref["drop"].astype(bool))
    rel = row_rel_err(out.float().cpu().numpy().astype(np.float64)[rows], ref["out"][rows])
    assert rel.max() <= tol_of(sp), rel.max()
