"""GPU edge cases and degenerate layers: empty and ragged token counts across
every mode boundary, the dense and soft-mixture limits, exact ties, a capacity
that drops everything, extreme routing skew, invalid indices handed to the
permutation, caller-built row maps, gate sums, and the INT4 routing-drift
report.  Every comparison is against the FP64 oracle or a closed form."""
import numpy as np
import pytest
import torch
from scipy import special

import moe_synth as S
import oracle as O
from gpu_harness import compare_routes, layer_of, oracle_run, row_rel_err, to_f64, tol_of

pytestmark = pytest.mark.gpu

# a mid-size layer keeps the oracle fast while crossing every tile boundary
MID = S.SPECS["olmoe"].replace(name="mid", cfg_id=11, d=1024, E=32, k=4, ffn=512)


def run_and_check(sp, lay, ml, x, nsamp=None, tol=None):
    T = x.shape[0]
    out, idx, gates, drop = ml.forward(x)
    torch.cuda.synchronize()
    rows = np.arange(T) if nsamp is None or T <= nsamp else \
        np.sort(np.random.default_rng(1).choice(T, nsamp, replace=False))
    ref = oracle_run(sp, lay, x, ffn_rows=rows)
    gi = idx.cpu().numpy()
    rep = compare_routes(gi, ref, sp.k)
    assert rep.set_mismatch_strict == 0 and rep.order_mismatch == 0
    ok = rows[rep.matched[rows]]
    rel = row_rel_err(out.float().cpu().numpy().astype(np.float64)[ok], ref["out"][ok])
    assert rel.max(initial=0) <= (tol or tol_of(sp)), rel.max()
    return out, idx, gates, drop, ref


@pytest.fixture(scope="module")
def mid():
    lay = S.make_layer(MID, device="cuda")
    return MID, lay, layer_of(MID, lay)


def test_zero_tokens_is_a_noop(mid):
    sp, lay, ml = mid
    x = torch.empty((0, sp.d), dtype=torch.bfloat16, device="cuda")
    out, idx, gates, drop = ml.forward(x)
    torch.cuda.synchronize()
    assert out.shape == (0, sp.d) and idx.shape == (0, sp.k)


@pytest.mark.parametrize("T", [1, 3, 17, 33, 63, 64, 65, 100, 255, 256, 257, 300, 1000])
def test_ragged_token_counts(mid, T):
    """Crosses the small/large routing boundary (256), the streaming/tiled GEMM
    boundary (64), the 16/32/64-row streaming items and partial 128-row tiles."""
    sp, lay, ml = mid
    x = S.make_tokens(sp, T, device="cuda", seed=T)
    run_and_check(sp, lay, ml, x, nsamp=300)


@pytest.mark.parametrize("T", [2100, 3001])
def test_partly_filled_items_skip_idle_row_tiles(mid, T):
    """From T*k >= 256 E on (experts averaging two 128-row items), the tiled
    kernels skip the idle 32-row tiles of items that are not full.  An expert's
    32-row tiles are spread evenly over its ceil(rows / 128) items; every row is
    checked, and the items cover several counts of active row tiles."""
    sp, lay, ml = mid
    assert T * sp.k >= 256 * sp.E
    x = S.make_tokens(sp, T, device="cuda", seed=T)
    _, idx, _, _, _ = run_and_check(sp, lay, ml, x)
    counts = np.bincount(idx.cpu().numpy().ravel(), minlength=sp.E)
    active = set()
    for c in counts[counts > 0]:
        n, tiles = -(-int(c) // 128), -(-int(c) // 32)
        active |= {tiles // n, -(-tiles // n)}
    assert len(active) >= 2 and min(active) < 4, active


@pytest.mark.parametrize("T", [64, 2100])
def test_token_permutation_permutes_outputs_bitwise(mid, T):
    """Dropless, every token's routing and FFN are its own: permuting the token
    order permutes idx, gates and out, bit for bit (streaming and tiled paths,
    including the partly filled items whose rows then change places)."""
    sp, lay, ml = mid
    x = S.make_tokens(sp, T, device="cuda", seed=T + 7)
    perm = torch.randperm(T, generator=torch.Generator().manual_seed(T)).to("cuda")
    a = ml.forward(x)
    b = ml.forward(x[perm].contiguous())
    torch.cuda.synchronize()
    for u, v, what in zip(a[:3], b[:3], ("out", "idx", "gates")):
        u = u[perm]
        assert torch.equal(u.view(torch.int16) if u.dtype == torch.bfloat16 else u,
                           v.view(torch.int16) if v.dtype == torch.bfloat16 else v), what


def test_combine_is_linear_in_the_gates(mid):
    """Scaling every gate by a power of two scales the combined output by it
    exactly (fp32 accumulation, one rounding); zero gates give exact zeros."""
    sp, lay, ml = mid
    x = S.make_tokens(sp, 300, device="cuda", seed=5)
    idx, gates, _ = ml.route(x, want_scores=False)
    _, offsets, row_token, slot_row, _ = ml.permute(idx)
    y_rows, y_sh = ml.expert_ffn(x, offsets, row_token)
    base = ml.combine(y_rows, slot_row, gates, y_sh).float()
    twice = ml.combine(y_rows, slot_row, gates * 2, y_sh).float()
    zero = ml.combine(y_rows, slot_row, gates * 0, y_sh).float()
    torch.cuda.synchronize()
    assert base.abs().max() > 0
    assert torch.equal(twice, base * 2)
    assert torch.equal(zero, torch.zeros_like(zero))


def test_several_router_tiles_per_block(mid):
    """Above 512 router tiles each router and permute block takes several
    consecutive tiles (T=20000: 1250 tiles of 16 tokens, 3 per block)."""
    sp, lay, ml = mid
    x = S.make_tokens(sp, 20000, device="cuda", seed=11)
    run_and_check(sp, lay, ml, x, nsamp=300)


# the largest token count the library accepts, on a small layer
MAXT = S.SPECS["olmoe"].replace(name="maxt", cfg_id=12, d=128, E=64, k=8, ffn=128, rms_norm_x=False)


def _check_permutation(idx: np.ndarray, counts, offsets, row_token, slot_row, drop):
    """Dropless permutation by its definition: pairs walked token-major fill each
    expert's rows in order, and every row maps back to its token."""
    T, k = idx.shape
    E = counts.shape[0]
    flat = idx.reshape(-1).astype(np.int64)
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts)
    assert not drop.any()
    order = np.argsort(flat, kind="stable")  # expert-major, token-major inside an expert
    expect = np.empty(T * k, np.int64)
    expect[order] = np.arange(T * k)
    assert np.array_equal(slot_row.reshape(-1), expect)
    assert np.array_equal(row_token[expect], np.repeat(np.arange(T), k))


def test_largest_token_count():
    """T = 2^20 (the API's limit): 65536 router tiles, 128 per block.  The GPU's own
    routing must be a valid top-k that agrees with the oracle on sampled tokens
    (dropless routing is per token), its permutation must follow the definition
    exactly, and sampled outputs must match the oracle."""
    from mixture_experts_layer_13_amd import binding as B
    sp = MAXT
    T = 1 << 20
    lay = S.make_layer(sp, device="cuda")
    ml = layer_of(sp, lay)
    x = S.make_tokens(sp, T, device="cuda", seed=3)
    out, idx, gates, drop = ml.forward(x)
    counts, offsets, row_token, slot_row, drop2 = ml.permute(idx)
    torch.cuda.synchronize()
    gi = idx.cpu().numpy()
    _check_permutation(gi, counts.cpu().numpy(), offsets.cpu().numpy(), row_token.cpu().numpy(),
                       slot_row.cpu().numpy(), drop2.cpu().numpy())
    assert not drop.cpu().numpy().any()
    rows = np.sort(np.random.default_rng(2).choice(T, 256, replace=False))
    ref = oracle_run(sp, lay, x[torch.from_numpy(rows).to("cuda")])
    rep = compare_routes(gi[rows], ref, sp.k)
    assert rep.set_mismatch_strict == 0 and rep.order_mismatch == 0
    ok = rep.matched
    rel = row_rel_err(out[torch.from_numpy(rows).to("cuda")].float().cpu().numpy().astype(np.float64)[ok],
                      ref["out"][ok])
    assert rel.max(initial=0) <= tol_of(sp), rel.max()
    assert B.forward_launches(ml.cfg_for(T)) == 5


# DeepSeek-V3 routing (sigmoid, selection bias, 2.5 x renormalised gates, a shared expert)
# with more than 128 experts, where from T = 8192 on the router takes 64-token tiles and splits
# the experts over its waves (T = 8492: a ragged last tile); E = 160 leaves one wave half and
# one wave wholly past E; T = 1000 stays on 16-token tiles
WIDE = S.SPECS["dsv3"].replace(name="wide_router", cfg_id=13, d=512, E=256, ffn=256, ffn_shared=256)


@pytest.mark.parametrize("E,T,cap", [(256, 1000, None), (256, 8492, None), (160, 9000, None), (256, 8492, (5, 4))])
def test_wide_router_many_experts(E, T, cap):
    sp = WIDE.replace(E=E, capacity=cap)
    lay = S.make_layer(sp, device="cuda")
    ml = layer_of(sp, lay)
    x = S.make_tokens(sp, T, device="cuda", seed=E + T)
    out, idx, gates, drop, ref = run_and_check(sp, lay, ml, x, nsamp=300)
    if cap is None:
        assert not drop.cpu().numpy().any()
    else:
        # drops follow every earlier token's routing: compared when the routing agrees everywhere
        if np.array_equal(idx.cpu().numpy(), ref["idx"]):
            assert np.array_equal(drop.cpu().numpy().astype(bool), ref["drop"].astype(bool))


# Group-limited selection ("MoE Research", section 2, node-limited routing; "MoE at the
# inference level", workarounds, device-limited routing with M = 4): DeepSeek-V3 routing with
# 256 experts in 8 groups, 4 kept, through every router path (the one-launch small-T route at
# T = 1, 16, 300; 16-token tiles at T = 1000; 64-token tiles at T = 8492); 160 experts in
# groups of 20 that straddle the waves' 64-expert blocks; softmax over 64 experts in 8 groups
# with 2 kept (k = 8 of the 16 experts left) on the small route and on 16-token tiles.
GROUPED = WIDE.replace(name="grouped", cfg_id=14, groups=(8, 4))
GROUPED_SM = S.SPECS["olmoe"].replace(name="grouped_softmax", cfg_id=15, d=512, ffn=256, groups=(8, 2))


@pytest.mark.parametrize("which,E,G,M,T", [("sig", 256, 8, 4, 1), ("sig", 256, 8, 4, 16), ("sig", 256, 8, 4, 300),
                                           ("sig", 256, 8, 4, 1000), ("sig", 256, 8, 4, 8492),
                                           ("sig", 160, 8, 3, 9000), ("sm", 64, 8, 2, 1), ("sm", 64, 8, 2, 64),
                                           ("sm", 64, 8, 2, 5000)])
def test_group_limited_selection(which, E, G, M, T):
    sp = (GROUPED if which == "sig" else GROUPED_SM).replace(E=E, groups=(G, M))
    lay = S.make_layer(sp, device="cuda")
    ml = layer_of(sp, lay)
    x = S.make_tokens(sp, T, device="cuda", seed=E + T)
    out, idx, gates, drop, ref = run_and_check(sp, lay, ml, x, nsamp=300)
    gi = idx.cpu().numpy()
    gsz = E // G
    # every token, whatever its margins: its picks come from at most M groups
    assert max(len(set((row // gsz).tolist())) for row in gi) <= M
    if T >= 64:
        # the limit binds: plain top-k would spread some tokens over more groups
        free = oracle_run(sp.replace(groups=None), lay, x, ffn_rows=np.arange(0))["idx"]
        assert max(len(set((row // gsz).tolist())) for row in free) > M


def test_groups_of_one_expert_keep_plain_topk():
    """Groups of one expert with M = k select exactly the plain top-k: bitwise the
    same indices, gates and outputs as the layer without a group limit."""
    sp = GROUPED_SM.replace(groups=(64, 8))
    lay = S.make_layer(sp, device="cuda")
    a, b = layer_of(sp, lay), layer_of(sp.replace(groups=None), lay)
    for T in (1, 300, 5000):
        x = S.make_tokens(sp, T, device="cuda", seed=T)
        ra, rb = a.forward(x), b.forward(x)
        torch.cuda.synchronize()
        for u, v in zip(ra, rb):
            assert torch.equal(u, v)


def test_dense_limit_matches_textbook_swiglu():
    """E = 1, k = 1: the gate is softmax of one logit = 1, so the layer is a dense
    SwiGLU FFN.  Checked against the formula written out with scipy's expit."""
    sp = MID.replace(name="dense", cfg_id=12, E=1, k=1)
    lay = S.make_layer(sp, device="cuda")
    ml = layer_of(sp, lay)
    for T in (5, 300):
        x = S.make_tokens(sp, T, device="cuda")
        out, idx, gates, _ = ml.forward(x)
        torch.cuda.synchronize()
        assert (idx.cpu() == 0).all() and torch.equal(gates.cpu(), torch.ones_like(gates.cpu()))
        xf = to_f64(x)
        wg, wu, wd = to_f64(lay.w_gate[0]), to_f64(lay.w_up[0]), to_f64(lay.w_down[0])
        a = xf @ wg.T
        ref = (a * special.expit(a) * (xf @ wu.T)) @ wd.T
        assert row_rel_err(to_f64(out), ref).max() <= 2e-2


def test_k_equals_E_soft_mixture():
    sp = MID.replace(name="soft", cfg_id=13, E=8, k=8)
    lay = S.make_layer(sp, device="cuda")
    ml = layer_of(sp, lay)
    for T in (40, 400):
        x = S.make_tokens(sp, T, device="cuda")
        out, idx, gates, _, ref = run_and_check(sp, lay, ml, x)
        # every token uses every expert; gates are the full softmax, summing to 1
        assert (np.sort(idx.cpu().numpy(), 1) == np.arange(8)).all()
        assert np.abs(gates.cpu().numpy().sum(1) - 1).max() <= 1e-5


def test_zero_router_gives_lowest_indices_on_gpu():
    """All logits equal (W_r = 0, no bias): exact ties everywhere, so every token
    selects experts 0..k-1 with softmax gates 1/E (sigmoid: 2.5/k after renorm)."""
    for sp, T in ((MID.replace(name="ties", cfg_id=14, logit_bias_std=0.0), 300),
                  (S.SPECS["dsv3"].replace(name="ties3", cfg_id=15, d=512, E=64, ffn=256, select_bias_std=0.0), 40)):
        lay = S.make_layer(sp, device="cuda")
        lay.w_router.zero_()
        ml = layer_of(sp, lay)
        x = S.make_tokens(sp, T, device="cuda")
        _, idx, gates, _ = ml.forward(x)
        torch.cuda.synchronize()
        assert (idx.cpu().numpy() == np.arange(sp.k)[None, :]).all()
        expect = 1.0 / sp.E if sp.score == "softmax" else sp.gate_scale / sp.k
        assert np.abs(gates.cpu().numpy() - expect).max() <= 1e-6


def test_capacity_zero_leaves_shared_experts():
    """C = 0 drops every routed pair; the output is the shared experts' FFN."""
    sp = S.SPECS["dsv2_lite"].replace(name="capzero", cfg_id=16, d=512, E=16, ffn=256, ffn_shared=256,
                                      capacity=(0, 1))
    lay = S.make_layer(sp, device="cuda")
    ml = layer_of(sp, lay)
    x = S.make_tokens(sp, 200, device="cuda")
    out, idx, gates, drop, ref = run_and_check(sp, lay, ml, x)
    assert drop.cpu().numpy().all()
    assert ref["drop"].all()


def test_capacity_zero_at_decode_sizes():
    """Decode sizes (T = 1 takes the single-token permutation): C = 0 drops every
    routed pair.  With a shared expert the output is the shared FFN (checked
    against the oracle); with none, no expert block is live and the combine
    must still write the output, as exact zeros."""
    sp = S.SPECS["dsv2_lite"].replace(name="capzero_dec", cfg_id=18, d=512, E=16, ffn=256, ffn_shared=256,
                                      capacity=(0, 1))
    lay = S.make_layer(sp, device="cuda")
    ml = layer_of(sp, lay)
    for T in (1, 40):
        x = S.make_tokens(sp, T, device="cuda", seed=T)
        out, idx, gates, drop, ref = run_and_check(sp, lay, ml, x)
        assert drop.cpu().numpy().all()
    sp0 = S.SPECS["olmoe"].replace(name="capzero_dec_noshared", cfg_id=19, d=512, E=16, ffn=256, capacity=(0, 1))
    lay0 = S.make_layer(sp0, device="cuda")
    ml0 = layer_of(sp0, lay0)
    for T in (1, 40):
        x = S.make_tokens(sp0, T, device="cuda", seed=T)
        o = torch.full((T, sp0.d), float("nan"), dtype=torch.bfloat16, device="cuda")
        out, idx, gates, drop = ml0.forward(x, o)
        torch.cuda.synchronize()
        assert drop.cpu().numpy().all()
        assert (out.float() == 0).all()


def test_extreme_skew_single_hot_set():
    """Every token identical: every token picks the same k experts, so k experts
    each get all T rows (many tiles per expert) and the rest get none."""
    sp = MID
    lay = S.make_layer(sp, device="cuda")
    ml = layer_of(sp, lay)
    x1 = S.make_tokens(sp, 1, device="cuda")
    for T in (64, 700):
        x = x1.repeat(T, 1).contiguous()
        out, idx, *_ = run_and_check(sp, lay, ml, x, nsamp=20)
        assert (idx.cpu() == idx[0].cpu()).all()
        assert (out.float() == out[0:1].float()).all()


@pytest.mark.parametrize("T", [40, 100, 600])
def test_permute_treats_invalid_indices_as_dropped(mid, T):
    sp, lay, ml = mid
    r = np.random.default_rng(T)
    idx = np.stack([r.choice(sp.E, sp.k, replace=False) for _ in range(T)]).astype(np.int32)
    idx[3, 1] = -1
    idx[5, 0] = sp.E
    idx[7, 2] = 1 << 20
    counts, offsets, row_token, slot_row, drop = ml.permute(torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    valid = (idx >= 0) & (idx < sp.E)
    assert np.array_equal(drop.cpu().numpy(), (~valid).astype(np.uint8))
    assert np.array_equal(counts.cpu().numpy(), np.bincount(idx[valid], minlength=sp.E))
    sr, rt, off = slot_row.cpu().numpy(), row_token.cpu().numpy(), offsets.cpu().numpy()
    assert (sr[~valid] == -1).all() and off[-1] == valid.sum()
    for t in range(T):
        for j in range(sp.k):
            if valid[t, j]:
                e = idx[t, j]
                assert off[e] <= sr[t, j] < off[e + 1] and rt[sr[t, j]] == t
    # rows of an expert are ascending in t (stable token-major ranking)
    for e in range(sp.E):
        seg = rt[off[e]:off[e + 1]]
        assert (np.diff(seg) > 0).all()


def test_expert_ffn_on_caller_row_map(mid):
    """moe_expert_ffn on a row map built on the host (not by moe_permute): each
    row equals the oracle's FFN of its token through its expert."""
    sp, lay, ml = mid
    T = 90
    x = S.make_tokens(sp, T, device="cuda")
    r = np.random.default_rng(5)
    idx = np.stack([r.choice(sp.E, sp.k, replace=False) for _ in range(T)]).astype(np.int32)
    a = O.assign_rows(idx, sp.E)
    offsets = torch.tensor(a["offsets"], dtype=torch.int32, device="cuda")
    row_token = torch.tensor(a["row_token"], dtype=torch.int32, device="cuda")
    y_rows, _ = ml.expert_ffn(x, offsets, row_token)
    torch.cuda.synchronize()
    xf = to_f64(x)
    y = to_f64(y_rows)
    for e in (0, 7, 31):
        rows = np.arange(a["offsets"][e], a["offsets"][e + 1])
        if rows.size == 0:
            continue
        wg, wu, wd = to_f64(lay.w_gate[e]), to_f64(lay.w_up[e]), to_f64(lay.w_down[e])
        ref = O.swiglu_ffn(xf[a["row_token"][rows]], wg, wu, wd)
        assert row_rel_err(y[rows], ref).max() <= 2e-2


def test_gate_sums_on_gpu():
    for name, T, target in (("dsv3", 16, 2.5), ("qwen3_int4", 32, 1.0)):
        sp = S.SPECS[name]
        if name == "dsv3":
            sp = sp.replace(name="dsv3s", cfg_id=17, d=1024, ffn=256, E=256)
        lay = S.make_layer(sp, device="cuda")
        ml = layer_of(sp, lay)
        x = S.make_tokens(sp, T, device="cuda")
        _, _, gates, _ = ml.forward(x)
        torch.cuda.synchronize()
        assert np.abs(gates.cpu().numpy().sum(1) - target).max() <= 1e-5 * target


def test_int4_routing_drift_report():
    """INT4 experts with a bf16 router: routing is the bf16-weight layer's routing,
    so drift (mean swaps out of k) is 0 up to near-ties.  Also reports the INT4
    vs bf16-twin output difference as quality context (not a pass/fail bar)."""
    sp = S.SPECS["qwen3_int4"]
    lay = S.make_layer(sp, device="cuda")
    ml = layer_of(sp, lay)
    twin_sp = sp.replace(expert="bf16")
    wg, wu, wd = S.make_bf16_twin(sp, device="cuda")
    twin = S.Layer(twin_sp, lay.w_router, lay.logit_bias, lay.select_bias, wg, wu, wd)
    mt = layer_of(twin_sp, twin)
    for T in (32, 4096):
        x = S.make_tokens(sp, T, device="cuda")
        o4, i4, _, _ = ml.forward(x)
        ob, ib, _, _ = mt.forward(x)
        torch.cuda.synchronize()
        swaps = O.swaps_per_token(i4.cpu().numpy(), ib.cpu().numpy())
        rel = float((o4.float() - ob.float()).pow(2).mean().sqrt() / ob.float().pow(2).mean().sqrt())
        print(f"\nqwen3 INT4 T={T}: routing drift {swaps.mean():.4f} swaps/token (of {sp.k}); "
              f"INT4 vs bf16-twin output rel RMS {rel:.3f}")
        assert swaps.mean() == 0.0
