"""The tiled expert-weight layout.  moe_pack_weights must be exactly the byte
permutation the header defines (checked against that formula written out in
numpy), and a layer run on packed weights must return the same outputs,
indices, gates and drop masks, bit for bit, as the same layer on row-layout
weights: the layout changes where a lane finds its bytes, not the order of any
accumulation.  Parity of the row layout with the oracle is tested elsewhere;
two cases here also compare the tiled layout with the oracle directly."""
import numpy as np
import pytest
import torch

import moe_synth as S
from gpu_harness import compare_routes, layer_of, oracle_run, row_rel_err, tol_of

pytestmark = pytest.mark.gpu


def _B():
    from mixture_experts_layer_13_amd import binding
    return binding


def tiled_positions(rows: int, R: int) -> np.ndarray:
    """Destination byte of (row n, byte b): ((n/16)(R/64) + b/64) KB + 256 ((b%64)/16) + 16 (n%16) + b%16."""
    n = np.arange(rows, dtype=np.int64)[:, None]
    b = np.arange(R, dtype=np.int64)[None, :]
    return ((n // 16) * (R // 64) + b // 64) * 1024 + ((b % 64) // 16) * 256 + (n % 16) * 16 + b % 16


@pytest.mark.parametrize("expert,rows,K", [("bf16", 16, 32), ("bf16", 48, 2048), ("int4", 32, 128),
                                           ("int4", 16, 768), ("f32", 32, 16), ("f32", 16, 272), ("fp8", 32, 128),
                                           ("fp8", 16, 1408)])
def test_pack_is_the_documented_permutation(expert, rows, K):
    R = {"bf16": 2 * K, "int4": K // 2, "f32": 4 * K, "fp8": K}[expert]
    g = torch.Generator().manual_seed(rows * 1000 + K)
    src = torch.randint(0, 256, (rows, R), dtype=torch.uint8, generator=g)
    dst = torch.empty_like(src.cuda())
    _B().moe_pack_weights(_B()._DTYPES[expert], src.cuda(), dst, rows, K)
    torch.cuda.synchronize()
    expect = np.empty(rows * R, np.uint8)
    expect[tiled_positions(rows, R).ravel()] = src.numpy().ravel()
    assert np.array_equal(dst.cpu().numpy().ravel(), expect)


def test_pack_of_nothing_is_ok():
    t = torch.empty(0, dtype=torch.uint8, device="cuda")
    _B().moe_pack_weights(_B().MOE_BF16, t, t, 0, 64)


# a layer whose d is an odd multiple of 128: the last 256-column down block is half past d
ODD = S.SPECS["dsv2_lite"].replace(name="odd_d", cfg_id=21, d=640, E=16, k=4, ffn=384, ffn_shared=256)
MID = S.SPECS["olmoe"].replace(name="mid_l", cfg_id=22, d=1024, E=32, k=4, ffn=512)
INT4S = S.SPECS["qwen3_int4"].replace(name="int4_s", cfg_id=23, E=32)
DSV3S = S.SPECS["dsv3"].replace(name="dsv3_s", cfg_id=24, E=32)
ODD8 = ODD.replace(name="odd_d_fp8", cfg_id=25, expert="fp8")   # FP8 routed and shared experts

CASES = [("tiny_f32", None, 64), ("olmoe", None, 1), ("olmoe", None, 8), ("olmoe", None, 64), ("olmoe", None, 4096),
         ("mid", MID, 33), ("mid", MID, 300), ("odd", ODD, 7), ("odd", ODD, 500), ("dsv2_lite", None, 8192),
         ("dsv2_lite_cap", None, 8192), ("qwen3_int4", None, 32), ("qwen3_int4", None, 4096), ("int4_s", INT4S, 200),
         ("dsv3_s", DSV3S, 16), ("dsv3_s", DSV3S, 100), ("dsv3_s", DSV3S, 1000), ("odd8", ODD8, 7),
         ("odd8", ODD8, 500), ("olmoe_fp8", None, 4096)]

_LAYERS = {}


def layers(name, spec):
    if name not in _LAYERS:
        _LAYERS.clear()
        torch.cuda.empty_cache()
        sp = spec if spec is not None else S.SPECS[name]
        lay = S.make_layer(sp, device="cuda")
        _LAYERS[name] = (sp, lay, layer_of(sp, lay), layer_of(sp, lay, layout="tiled"))
    return _LAYERS[name]


@pytest.mark.parametrize("name,spec,T", CASES, ids=[f"{n}-T{t}" for n, _, t in CASES])
def test_tiled_layout_is_bitwise_equal(name, spec, T):
    sp, lay, rows_layer, tiled_layer = layers(name, spec)
    x = S.make_tokens(sp, T, device="cuda", seed=T)
    a = rows_layer.forward(x)
    b = tiled_layer.forward(x)
    torch.cuda.synchronize()
    for u, v, what in zip(a, b, ("out", "idx", "gates", "drop")):
        assert torch.equal(u, v), f"{name} T={T}: {what} differs between the row and tiled layouts"


# T = 100 and 80 sit in the tiled mode with at most 32 rows per expert on average, where the
# tiled kernels load weights non-temporally
@pytest.mark.parametrize("name,spec,T", [("odd", ODD, 300), ("int4_s", INT4S, 100), ("dsv3_s", DSV3S, 100),
                                         ("int4_s", INT4S, 80)])
def test_tiled_layout_matches_oracle(name, spec, T):
    sp, lay, _, tiled_layer = layers(name, spec)
    x = S.make_tokens(sp, T, device="cuda", seed=1)
    out, idx, _, _ = tiled_layer.forward(x)
    torch.cuda.synchronize()
    ref = oracle_run(sp, lay, x, ffn_rows=np.arange(T))
    rep = compare_routes(idx.cpu().numpy(), ref, sp.k)
    assert rep.set_mismatch_strict == 0 and rep.order_mismatch == 0
    ok = np.nonzero(rep.matched)[0]
    rel = row_rel_err(out.float().cpu().numpy().astype(np.float64)[ok], ref["out"][ok])
    assert rel.max(initial=0) <= tol_of(sp), rel.max()
