"""GPU tests of FP8 expert weights with FP8 activations on the FP8 matrix unit
("MoE at the inference level", Fields, weight_dtype, and workarounds: fp8
expert weights): each GEMM row quantised to E4M3 with an fp32 row scale.

- Parity against the FP64 oracle, which quantises the same bf16 rows with the
  same fp32 arithmetic (oracle.quantize_rows_e4m3), on the OLMoE-shaped layer at
  decode sizes (the streaming kernels up to T = 32) and prefill sizes (the tiled
  FP8 MFMA kernels; a ragged T among them), on the DeepSeek-V3-shaped layer with
  its shared expert and on the DeepSeek-V2-Lite-shaped one with two.
- The two weight layouts, and the split path (route -> permute -> expert_ffn ->
  combine) against the fused forward, bit for bit; the forward captured in a HIP
  graph (seven launches, no memset nodes) replays to the eager result."""
import numpy as np
import pytest
import torch

import moe_synth as S
from gpu_harness import A8_MEDIAN_TOL, compare_routes, layer_of, oracle_run, row_rel_err, tol_of

pytestmark = pytest.mark.gpu

_LAY = {}


def _layer(name):
    sp = S.SPECS[name]
    if name not in _LAY:
        _LAY.clear()
        torch.cuda.empty_cache()
        _LAY[name] = S.make_layer(sp, device="cuda")
    return sp, _LAY[name]


def _check(sp, lay, ml, T, seed, nsamp=None):
    x = S.make_tokens(sp, T, device="cuda", seed=seed)
    out, idx, gates, drop = ml.forward(x)
    torch.cuda.synchronize()
    rows = None
    if nsamp is not None and nsamp < T:
        rows = np.sort(np.random.default_rng(T).choice(T, size=nsamp, replace=False))
    ref = oracle_run(sp, lay, x, ffn_rows=rows)
    rep = compare_routes(idx.cpu().numpy(), ref, sp.k)
    assert rep.set_mismatch_strict == 0 and rep.order_mismatch == 0
    ok = rep.matched.copy()
    if rows is not None:
        sel = np.zeros(T, bool)
        sel[rows] = True
        ok &= sel
    rel = row_rel_err(out.float().cpu().numpy().astype(np.float64)[ok], ref["out"][ok])
    print(f"  {sp.name} T={T}: {ok.sum()} rows, max row rel err {rel.max(initial=0):.2e}, "
          f"median {np.median(rel) if rel.size else 0:.2e}")
    assert rel.size > 0
    assert rel.max() <= tol_of(sp) and np.median(rel) <= A8_MEDIAN_TOL
    return out


@pytest.mark.parametrize("T,layout", [(1, "rows"), (8, "tiled"), (64, "rows"), (300, "tiled"), (300, "rows"),
                                      (4096, "tiled")])
def test_a8_forward_matches_oracle(T, layout):
    sp, lay = _layer("olmoe_fp8a8")
    ml = layer_of(sp, lay, layout)
    print(f"case olmoe_fp8a8 T={T} {layout}", flush=True)
    _check(sp, lay, ml, T, seed=T)


def test_a8_layouts_and_split_path_bitwise():
    sp, lay = _layer("olmoe_fp8a8")
    rows, tiled = layer_of(sp, lay, "rows"), layer_of(sp, lay, "tiled")
    for T in (100, 4096):
        x = S.make_tokens(sp, T, device="cuda", seed=7)
        a = rows.forward(x)[0].clone()
        b = tiled.forward(x)[0]
        idx2, gates2, _ = tiled.route(x)
        counts, offsets, row_token, slot_row, drop2 = tiled.permute(idx2)
        y_rows, y_sh = tiled.expert_ffn(x, offsets, row_token)
        c = tiled.combine(y_rows, slot_row, gates2, y_sh)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
        assert torch.equal(b.view(torch.int16), c.view(torch.int16))


@pytest.mark.parametrize("T,nsamp", [(16, None), (4096, 12), (16384, 8)])
def test_a8_deepseek_v3_with_shared_expert(T, nsamp):
    sp, lay = _layer("dsv3_fp8a8")
    ml = layer_of(sp, lay, "tiled")
    print(f"case dsv3_fp8a8 T={T}", flush=True)
    _check(sp, lay, ml, T, seed=T, nsamp=nsamp)


def test_a8_graph_replay_matches_eager():
    sp, lay = _layer("olmoe_fp8a8")
    ml = layer_of(sp, lay, "tiled")
    for T in (8, 300):
        x = S.make_tokens(sp, T, device="cuda", seed=3)
        ref = [t.clone() for t in ml.forward(x)]
        outs = [torch.empty_like(t) for t in ref]
        ml.workspace(ml.cfg_for(T))
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            ml.forward(x, *outs)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            ml.forward(x, *outs)
        for rep in range(3):
            for t in outs:
                t.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for u, v in zip(ref, outs):
                assert torch.equal(u.view(torch.uint8) if u.dtype == torch.bfloat16 else u,
                                   v.view(torch.uint8) if v.dtype == torch.bfloat16 else v), (T, rep)
        del g


def test_a8_capacity_drops_match_oracle():
    """FP8 activations with a capacity (C = 5/4): the down GEMM's operand is quantised over
    all of its R rows (stale rows past the kept count included, which no tile reads).  The
    oracle replays the GPU's own routes, so the drop mask must equal the capacity rule on
    them exactly, and every token's output must match."""
    sp = S.SPECS["olmoe_fp8a8"].replace(capacity=(5, 4))
    _, lay = _layer("olmoe_fp8a8")
    ml = layer_of(sp, lay, "tiled")
    x = S.make_tokens(sp, 4096, device="cuda", seed=11)
    out, idx, gates, drop = ml.forward(x)
    torch.cuda.synchronize()
    ref = oracle_run(sp, lay, x, routes=(idx.cpu().numpy(), gates.cpu().numpy().astype(np.float64)))
    assert np.array_equal(drop.cpu().numpy(), ref["drop"]) and int(ref["drop"].sum()) > 0
    rel = row_rel_err(out.float().cpu().numpy().astype(np.float64), ref["out"])
    print(f"  olmoe_fp8a8 C=5/4 T=4096: {int(ref['drop'].sum())} pairs dropped, max row rel err "
          f"{rel.max():.2e}, median {np.median(rel):.2e}")
    assert rel.max() <= tol_of(sp) and np.median(rel) <= A8_MEDIAN_TOL


@pytest.mark.parametrize("T,layout", [(20, "tiled"), (40, "rows"), (300, "tiled"), (3000, "tiled")])
def test_a8_two_shared_experts_match_oracle(T, layout):
    """The DeepSeek-V2-Lite-shaped layer with FP8 activations: two shared experts, whose SwiGLU
    rows are quantised as one concatenated row and whose down GEMM walks their two K slabs, each
    with its own channel scales (T = 20: the streaming kernels; from T = 40: the tiled ones)."""
    sp, lay = _layer("dsv2_lite_fp8a8")
    ml = layer_of(sp, lay, layout)
    print(f"case dsv2_lite_fp8a8 T={T} {layout}", flush=True)
    _check(sp, lay, ml, T, seed=T)
