"""Pins of the FP64 oracle against facts that do not come from the oracle itself:
closed forms, invariants, brute force on tiny inputs, special cases that reduce
to a textbook formula or a library routine.  CPU only."""
import itertools
import math

import numpy as np
import pytest
from scipy import special

import oracle as O

rng = np.random.default_rng(1234)


# ---------------------------------------------------------------- decoding
def test_bf16_decoding_closed_forms():
    # 0x3F80 = 1.0, 0xC000 = -2.0, 0x3E80 = 0.25, 0x7F7F = largest finite bf16
    bits = np.array([0x3F80, 0xC000, 0x3E80, 0x0000, 0x8000, 0x7F7F], np.uint16)
    v = O.bf16_to_f64(bits)
    assert v[0] == 1.0 and v[1] == -2.0 and v[2] == 0.25 and v[3] == 0.0
    assert v[4] == 0.0 and math.copysign(1, v[4]) == -1.0
    assert v[5] == (2 - 2 ** -7) * 2.0 ** 127


def _f32_from_fields(bits: int) -> float:
    """IEEE-754 binary32 decoded field by field (sign, 8-bit biased exponent,
    23-bit fraction; exponent 0 is subnormal), in exact Python arithmetic."""
    sign = -1.0 if bits >> 31 else 1.0
    exp, frac = (bits >> 23) & 0xFF, bits & 0x7FFFFF
    if exp == 0:
        return sign * math.ldexp(frac, -149)
    return sign * math.ldexp((1 << 23) | frac, exp - 150)


def test_f32_widening_closed_forms():
    # 0x3F800000 = 1, 0xC0200000 = -2.5, 0x00000001 = 2^-149 (smallest subnormal),
    # 0x7F7FFFFF = largest finite, 0x3DCCCCCD = float32(0.1), 0x80000000 = -0
    bits = np.array([0x3F800000, 0xC0200000, 0x00000001, 0x7F7FFFFF, 0x3DCCCCCD, 0x80000000], np.uint32)
    v = O.f32_to_f64(bits.view(np.float32))
    assert v.dtype == np.float64
    assert v[0] == 1.0 and v[1] == -2.5 and v[2] == 2.0 ** -149
    assert v[3] == (2 - 2 ** -23) * 2.0 ** 127
    assert v[4] == 13421773 * 2.0 ** -27 and v[4] != 0.1
    assert v[5] == 0.0 and math.copysign(1, v[5]) == -1.0
    # random finite bit patterns, every one against the field-by-field decoding
    rb = rng.integers(0, 1 << 32, size=2000, dtype=np.uint64).astype(np.uint32)
    rb = rb[((rb >> 23) & 0xFF) != 0xFF]
    w = O.f32_to_f64(rb.view(np.float32).reshape(-1, 1))
    assert w.shape == (len(rb), 1)
    assert all(w[i, 0] == _f32_from_fields(int(b)) for i, b in enumerate(rb))


def test_int4_unpack_bit_by_bit():
    packed = rng.integers(0, 256, size=(3, 5), dtype=np.uint8)
    q = O.int4_unpack(packed)
    for r in range(3):
        for i in range(5):
            byte = int(packed[r, i])
            for half, shift in ((0, 0), (1, 4)):
                nib = (byte >> shift) & 0xF
                val = nib - 16 if nib & 0x8 else nib   # two's complement nibble
                assert q[r, 2 * i + half] == val


def test_fp8_decoding_matches_library_and_closed_forms():
    """Every one of the 256 E4M3 codes against torch's own float8_e4m3fn decoding (a
    library routine), plus closed forms: 0x38 = 1, 0x7E = 448 (largest), 0x08 = 2^-6
    (smallest normal), 0x01 = 2^-9 (smallest subnormal), 0x80 = -0, 0x7F / 0xFF NaN."""
    import torch
    codes = np.arange(256, dtype=np.uint8)
    got = O.fp8_e4m3_to_f64(codes)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(got), np.isnan(lib)) and np.isnan(got).sum() == 2
    ok = ~np.isnan(lib)
    assert np.array_equal(got[ok], lib[ok])
    assert got[0x38] == 1.0 and got[0x7E] == 448.0 and got[0x08] == 2.0 ** -6 and got[0x01] == 2.0 ** -9
    assert got[0x80] == 0.0 and np.signbit(got[0x80]) and got[0xB8] == -1.0
    assert np.nanmax(got) == 448.0 and np.nanmin(got) == -448.0
    # per-channel scales multiply whole rows
    c = np.array([[0x38, 0x40], [0x30, 0xB8]], np.uint8)
    assert np.array_equal(O.fp8_dequant(c, np.array([0.5, 3.0])), np.array([[0.5, 1.0], [1.5, -3.0]]))


def test_int4_one_hot_selects_exactly_one_weight():
    """A single non-zero nibble at a known (n, k) selects exactly q * s of its group:
    pins nibble order (low nibble = even k) and the group index k // 128."""
    N, K = 4, 384
    for n, kk, qv in ((0, 0, 3), (1, 1, -8), (2, 129, 7), (3, 383, -1)):
        q = np.zeros((N, K), np.int64)
        q[n, kk] = qv
        packed = np.zeros((N, K // 2), np.uint8)
        for r in range(N):
            for i in range(K // 2):
                packed[r, i] = (q[r, 2 * i] & 0xF) | ((q[r, 2 * i + 1] & 0xF) << 4)
        # power-of-two scales that differ per (row, group): 2^-(r + 3g)
        s = np.array([[2.0 ** -(r + 3 * g) for g in range(K // 128)] for r in range(N)], np.float32)
        sbits = (s.view(np.uint32) >> 16).astype(np.uint16)
        w = O.int4_dequant(packed, sbits)
        expect = np.zeros((N, K))
        expect[n, kk] = qv * 2.0 ** -(n + 3 * (kk // 128))
        assert np.array_equal(w, expect)


# ---------------------------------------------------------------- scores
def test_softmax_rows_sum_to_one_and_match_library():
    L = rng.normal(size=(50, 64)) * 4
    P = O.softmax_scores(L)
    assert np.abs(P.sum(1) - 1).max() <= 1e-12
    assert np.allclose(P, special.softmax(L, axis=1), rtol=1e-13, atol=0)
    # closed form: logits (0, ln 3) -> (1/4, 3/4); shift invariance
    P2 = O.softmax_scores(np.array([[0.0, math.log(3.0)], [100.0, 100.0 + math.log(3.0)]]))
    assert np.allclose(P2, [[0.25, 0.75], [0.25, 0.75]], rtol=1e-14, atol=0)
    # large logits do not overflow (max-subtract form)
    assert np.isfinite(O.softmax_scores(np.array([[1000.0, 999.0]]))).all()


def test_sigmoid_matches_library():
    L = rng.normal(size=(20, 16)) * 3
    assert np.allclose(O.sigmoid_scores(L), special.expit(L), rtol=1e-14, atol=0)
    assert O.sigmoid_scores(np.zeros((1, 1)))[0, 0] == 0.5


def test_router_logits_bias_and_orientation():
    # non-square: x [3,5], w_router stored [E=4][d=5]; logits[t,e] = sum_i x[t,i] w[e,i] + b[e]
    x = rng.normal(size=(3, 5))
    w = rng.normal(size=(4, 5))
    b = rng.normal(size=4)
    L = O.router_logits(x, w, b)
    for t in range(3):
        for e in range(4):
            assert math.isclose(L[t, e], sum(x[t, i] * w[e, i] for i in range(5)) + b[e], rel_tol=1e-12,
                                abs_tol=1e-12)


# ---------------------------------------------------------------- top-k
def _brute_topk(row, k):
    order = sorted(range(len(row)), key=lambda e: (-(row[e] + 0.0), e))
    return order[:k]


@pytest.mark.parametrize("E,k", [(4, 1), (8, 2), (16, 4), (16, 16), (5, 3)])
def test_topk_matches_brute_force_full_sort_with_ties(E, k):
    # integer-valued keys with few distinct values force many exact ties
    key = rng.integers(0, 4, size=(64, E)).astype(np.float64)
    key[0] = 0.0
    key[1, :] = -0.0  # -0 ties with +0
    key[1, ::2] = 0.0
    idx, margin = O.select_topk(key, k)
    for t in range(key.shape[0]):
        assert idx[t].tolist() == _brute_topk(key[t].tolist(), k)
        assert len(set(idx[t].tolist())) == k
        if k < E:
            srt = sorted(key[t], reverse=True)
            assert margin[t] == srt[k - 1] - srt[k]
        else:
            assert margin[t] == np.inf


# ---------------------------------------------------------------- group-limited selection
def test_group_limit_worked_example():
    """E = 8 in 4 groups of 2, M = 2, k = 3, worked by hand.  Group maxima are
    0.30, 0.22, 0.25, 0.05, so groups 0 and 2 stay and the picks are 0, 4, 5;
    plain top-3 is 0, 4, 2.  Scoring groups by their sum (0.31, 0.43, 0.27, 0.05)
    would keep groups 1 and 0 (picks 0, 2, 3), and interleaved groups (e mod 4)
    would allow {0, 2, 4, 6} (picks 0, 4, 2): both fail here."""
    key = np.array([[0.30, 0.01, 0.22, 0.21, 0.25, 0.02, 0.05, 0.00]])
    masked, gm = O.limit_groups(key, 4, 2)
    assert np.isneginf(masked[0, [2, 3, 6, 7]]).all()
    assert (masked[0, [0, 1, 4, 5]] == key[0, [0, 1, 4, 5]]).all()
    assert O.select_topk(masked, 3)[0][0].tolist() == [0, 4, 5]
    assert O.select_topk(key, 3)[0][0].tolist() == [0, 4, 2]
    assert gm[0] == pytest.approx(0.25 - 0.22)  # 2nd and 3rd group maxima
    # equal group maxima: the lower group stays
    tie = np.array([[0.5, 0.1, 0.2, 0.5, 0.4, 0.5]])
    m2, gm2 = O.limit_groups(tie, 3, 2)
    assert np.isneginf(m2[0, 4:]).all() and np.isfinite(m2[0, :4]).all() and gm2[0] == 0.0


@pytest.mark.parametrize("E,G,M", [(8, 4, 2), (12, 3, 1), (16, 8, 3), (6, 6, 4)])
def test_group_limit_brute_force(E, G, M):
    """Every kept group's maximum is >= every dropped group's (on equal maxima the
    kept group has the lower index); keys inside kept groups are untouched, all
    others -inf; at most M groups carry a pick, and the overall best expert is
    always picked."""
    key = rng.integers(0, 6, size=(200, E)).astype(np.float64)  # many exact ties
    masked, gm = O.limit_groups(key, G, M)
    gsz = E // G
    for t in range(key.shape[0]):
        gmax = [max(key[t, g * gsz:(g + 1) * gsz]) for g in range(G)]
        kept = [g for g in range(G) if np.isfinite(masked[t, g * gsz])]
        assert len(kept) == M
        for g in range(G):
            inside = masked[t, g * gsz:(g + 1) * gsz]
            if g in kept:
                assert (inside == key[t, g * gsz:(g + 1) * gsz]).all()
            else:
                assert np.isneginf(inside).all()
                for h in kept:
                    assert gmax[h] > gmax[g] or (gmax[h] == gmax[g] and h < g)
        srt = sorted(gmax, reverse=True)
        assert gm[t] == (srt[M - 1] - srt[M] if M < G else np.inf)
        for k in range(1, M * gsz + 1):
            picks = O.select_topk(masked[t:t + 1], k)[0][0]
            assert len({int(e) // gsz for e in picks}) <= M
            assert int(picks[0]) == _brute_topk(key[t].tolist(), 1)[0]


def test_group_limit_special_cases():
    """M = n_groups and n_groups = 1 change nothing; groups of one expert with
    M = k reduce to the plain top-k."""
    key = rng.normal(size=(50, 16))
    assert (O.limit_groups(key, 4, 4)[0] == key).all()
    assert (O.limit_groups(key, 1, 1)[0] == key).all()
    for k in (1, 3, 8):
        assert (O.select_topk(O.limit_groups(key, 16, k)[0], k)[0] == O.select_topk(key, k)[0]).all()
    with pytest.raises(ValueError):
        O.limit_groups(key, 5, 2)
    with pytest.raises(ValueError):
        O.limit_groups(key, 4, 5)


def test_group_limited_layer():
    """Through the whole layer: M = n_groups gives the ungrouped result; M < n_groups
    keeps each token's picks inside M groups, and its gates still follow the
    unbiased scores of the picks."""
    E, d, k = 16, 8, 4
    x = rng.normal(size=(40, d))
    wr = rng.normal(size=(E, d))
    ex = _experts_fn(_rand_experts(E, d, 5))
    sb = rng.normal(size=E) * 0.1
    base = O.moe_layer(x, wr, ex, E, k, score="sigmoid", select_bias=sb, renorm=True, gate_scale=2.5)
    same = O.moe_layer(x, wr, ex, E, k, score="sigmoid", select_bias=sb, renorm=True, gate_scale=2.5,
                       groups=(4, 4))
    assert (same["idx"] == base["idx"]).all() and np.array_equal(same["out"], base["out"])
    lim = O.moe_layer(x, wr, ex, E, k, score="sigmoid", select_bias=sb, renorm=True, gate_scale=2.5,
                      groups=(4, 1))
    assert all(len(set((lim["idx"][t] // 4).tolist())) == 1 for t in range(40))
    assert (lim["idx"] != base["idx"]).any()
    g = np.take_along_axis(lim["scores"], lim["idx"].astype(np.int64), axis=1)
    assert np.allclose(lim["gates"], 2.5 * g / g.sum(axis=1, keepdims=True))


def test_zero_router_gives_lowest_indices():
    """W_r = 0 and no bias: every key ties, so every token selects experts 0..k-1."""
    x = rng.normal(size=(10, 6))
    for score in ("softmax", "sigmoid"):
        res = O.moe_layer(x, np.zeros((8, 6)), _experts_fn(_rand_experts(8, 6, 3)), 8, 3, score=score,
                          ffn_rows=np.arange(0))
        assert (res["idx"] == np.arange(3)[None, :]).all()


# ---------------------------------------------------------------- gates
def test_gate_sums_and_order():
    L = rng.normal(size=(40, 16)) * 2
    P = O.softmax_scores(L)
    idx, _ = O.select_topk(P, 4)
    g = O.gate_weights(P, idx, renorm=False, scale=1.0)
    assert (g.sum(1) <= 1 + 1e-15).all()
    assert (np.diff(g, axis=1) <= 0).all()          # non-increasing in slot order
    gr = O.gate_weights(P, idx, renorm=True, scale=1.0)
    assert np.abs(gr.sum(1) - 1).max() <= 1e-15
    S = O.sigmoid_scores(L)
    gs = O.gate_weights(S, idx, renorm=True, scale=2.5)
    assert np.abs(gs.sum(1) - 2.5).max() <= 1e-14


def test_selection_bias_selects_but_does_not_weight():
    """Sigmoid scoring with a selection-only bias: the bias decides which experts win,
    the gate uses the unbiased score.  Hand-worked: logits (2, 0, 0.5), bias (0, 3, 0), k=2
    -> keys (s(2), s(0)+3, s(0.5)) picks experts 1 then 0; gates 2.5*s_e / (s(0)+s(2))."""
    x = np.array([[1.0]])
    w = np.array([[2.0], [0.0], [0.5]])
    res = O.moe_layer(x, w, _experts_fn(_rand_experts(3, 1, 1)), 3, 2, score="sigmoid", renorm=True,
                      gate_scale=2.5, select_bias=np.array([0.0, 3.0, 0.0]), ffn_rows=np.arange(0))
    assert res["idx"][0].tolist() == [1, 0]
    s0, s2 = 0.5, 1 / (1 + math.exp(-2.0))
    assert np.allclose(res["gates"][0], [2.5 * s0 / (s0 + s2), 2.5 * s2 / (s0 + s2)], rtol=1e-14)


# ---------------------------------------------------------------- permutation
def test_capacity_rows_exact_integer_ceil():
    assert O.capacity_rows(8192, 6, 64, 5, 4) == 960        # DeepSeek-V2-Lite at C = 1.25
    assert O.capacity_rows(8, 2, 4, 5, 4) == 5               # exactly 5.0, must not round up
    assert O.capacity_rows(10, 1, 4, 1, 1) == 3              # ceil(2.5)
    assert O.capacity_rows(3, 1, 4, 1, 1) == 1               # ceil(0.75)
    assert O.capacity_rows(5, 2, 3, 0, 1) == 0


def _brute_assign(idx, E, cap):
    # group pairs by expert with a dict, keep the first `cap` in (t, j) order
    groups = {}
    for t, j in itertools.product(range(idx.shape[0]), range(idx.shape[1])):
        groups.setdefault(int(idx[t, j]), []).append((t, j))
    kept = {e: (v if cap is None else v[:cap]) for e, v in groups.items()}
    return groups, kept


@pytest.mark.parametrize("T,E,k,cap", [(1, 4, 2, None), (13, 5, 2, None), (40, 8, 3, None),
                                       (40, 8, 3, 7), (40, 8, 3, 1), (40, 8, 3, 40), (17, 3, 3, 0)])
def test_assignment_matches_brute_force(T, E, k, cap):
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    a = O.assign_rows(idx, E, cap)
    groups, kept = _brute_assign(idx, E, cap)
    assert a["counts"].sum() == T * k
    for e in range(E):
        assert a["counts"][e] == len(groups.get(e, []))
        assert a["kept"][e] == len(kept.get(e, []))
        rows = list(range(a["offsets"][e], a["offsets"][e + 1]))
        # rows of expert e map back, in order, to the kept pairs of e
        assert [int(a["row_token"][r]) for r in rows] == [t for t, _ in kept.get(e, [])]
        for r, (t, j) in zip(rows, kept.get(e, [])):
            assert a["slot_row"][t, j] == r
    # round trip and drop accounting
    for t in range(T):
        for j in range(k):
            if a["drop"][t, j]:
                assert a["slot_row"][t, j] == -1
            else:
                assert a["row_token"][a["slot_row"][t, j]] == t
    n_drop = int(a["drop"].sum())
    expect = 0 if cap is None else sum(max(0, len(v) - cap) for v in groups.values())
    assert n_drop == expect
    assert int(a["offsets"][E]) == T * k - n_drop
    if cap is not None and cap >= T:
        assert n_drop == 0            # an expert receives each token at most once
    if cap == 1:
        for e, v in groups.items():   # exactly the first pair in (t, j) order survives
            t, j = v[0]
            assert a["drop"][t, j] == 0 and a["offsets"][e + 1] - a["offsets"][e] == 1


# ---------------------------------------------------------------- experts / whole layer
def _rand_experts(E, d, F, scale=0.5):
    return [(rng.normal(size=(F, d)) * scale, rng.normal(size=(F, d)) * scale, rng.normal(size=(d, F)) * scale)
            for _ in range(E)]


def _experts_fn(lst):
    return lambda e: lst[e]


def _textbook_swiglu(x, Wg_dF, Wu_dF, Wd_Fd):
    # logical [d, ffn] / [ffn, d] matrices, silu via the library logistic function
    a = x @ Wg_dF
    return (a * special.expit(a) * (x @ Wu_dF)) @ Wd_Fd


def test_swiglu_scalar_closed_form():
    # d = ffn = 1: x = 1, Wg = 1, Wu = 2, Wd = 3 -> silu(1) * 2 * 3 = 6 / (1 + e^-1)
    y = O.swiglu_ffn(np.array([[1.0]]), np.array([[1.0]]), np.array([[2.0]]), np.array([[3.0]]))
    assert math.isclose(y[0, 0], 6.0 / (1.0 + math.exp(-1.0)), rel_tol=1e-15)
    # silu is odd-symmetric around its definition: silu(-z) = silu(z) - z
    z = rng.normal(size=100) * 5
    assert np.allclose(O.silu(-z), O.silu(z) - z, rtol=1e-12, atol=1e-12)


def test_single_expert_reduces_to_dense_swiglu():
    """E = 1, k = 1: the softmax of one logit is 1, so the layer is a dense SwiGLU FFN."""
    T, d, F = 9, 5, 7
    x = rng.normal(size=(T, d))
    Wg, Wu, Wd = rng.normal(size=(d, F)), rng.normal(size=(d, F)), rng.normal(size=(F, d))
    # stored layout: one K-contiguous row per output channel
    ex = [(Wg.T.copy(), Wu.T.copy(), Wd.T.copy())]
    res = O.moe_layer(x, rng.normal(size=(1, d)), _experts_fn(ex), 1, 1,
                      logit_bias=np.array([0.3]))
    assert np.allclose(res["gates"], 1.0, rtol=0, atol=1e-15)
    assert np.allclose(res["out"], _textbook_swiglu(x, Wg, Wu, Wd), rtol=1e-12, atol=1e-12)


def test_k_equals_E_is_soft_mixture():
    """k = E, softmax, no renorm: out = sum_e p_e FFN_e(x) (every gate applied)."""
    T, d, F, E = 6, 4, 3, 5
    x = rng.normal(size=(T, d))
    wr = rng.normal(size=(E, d))
    ex = _rand_experts(E, d, F)
    res = O.moe_layer(x, wr, _experts_fn(ex), E, E)
    L = x @ wr.T
    P = np.exp(L) / np.exp(L).sum(1, keepdims=True)
    expect = np.zeros((T, d))
    for e in range(E):
        Wg, Wu, Wd = ex[e]
        expect += P[:, e:e + 1] * _textbook_swiglu(x, Wg.T, Wu.T, Wd.T)
    assert np.allclose(res["out"], expect, rtol=1e-12, atol=1e-12)


def test_everything_dropped_leaves_shared_experts_only():
    T, d, F, E = 7, 4, 3, 4
    x = rng.normal(size=(T, d))
    ex, sh = _rand_experts(E, d, F), _rand_experts(2, d, 6)
    res = O.moe_layer(x, rng.normal(size=(E, d)), _experts_fn(ex), E, 2, capacity=(0, 1),
                      shared=_experts_fn(sh), n_shared=2)
    assert res["drop"].all()
    expect = sum(_textbook_swiglu(x, a.T, b.T, c.T) for a, b, c in sh)
    assert np.allclose(res["out"], expect, rtol=1e-12, atol=1e-12)
    res0 = O.moe_layer(x, rng.normal(size=(E, d)), _experts_fn(ex), E, 2, capacity=(0, 1))
    assert (res0["out"] == 0).all()


def test_capacity_drop_skips_ffn_and_keeps_other_gates():
    """A dropped pair contributes nothing; kept gates are not renormalised."""
    T, d, F, E, k = 30, 4, 3, 3, 2
    x = rng.normal(size=(T, d))
    wr = rng.normal(size=(E, d))
    ex = _rand_experts(E, d, F)
    res = O.moe_layer(x, wr, _experts_fn(ex), E, k, capacity=(1, 2))
    assert res["drop"].any()
    for t in range(T):
        y = np.zeros(d)
        for j in range(k):
            if not res["drop"][t, j]:
                Wg, Wu, Wd = ex[res["idx"][t, j]]
                y += res["gates"][t, j] * _textbook_swiglu(x[t:t + 1], Wg.T, Wu.T, Wd.T)[0]
        assert np.allclose(res["out"][t], y, rtol=1e-12, atol=1e-12)


def test_linearity_in_gates_and_route_replay_control():
    T, d, F, E, k = 12, 6, 5, 6, 2
    x = rng.normal(size=(T, d))
    wr = rng.normal(size=(E, d))
    ex, sh = _rand_experts(E, d, F), _rand_experts(1, d, 4)
    kw = dict(shared=_experts_fn(sh), n_shared=1)
    base = O.moe_layer(x, wr, _experts_fn(ex), E, k, **kw)
    # control: replaying the layer's own routes returns the baseline exactly
    rep = O.moe_layer(x, wr, _experts_fn(ex), E, k, routes=(base["idx"], base["gates"]), **kw)
    assert np.array_equal(rep["out"], base["out"])
    shared_part = _textbook_swiglu(x, sh[0][0].T, sh[0][1].T, sh[0][2].T)
    scaled = O.moe_layer(x, wr, _experts_fn(ex), E, k, routes=(base["idx"], 3.0 * base["gates"]), **kw)
    assert np.allclose(scaled["out"] - shared_part, 3.0 * (base["out"] - shared_part), rtol=1e-11, atol=1e-11)


def test_token_permutation_equivariance():
    T, d, F, E, k = 15, 5, 4, 6, 3
    x = rng.normal(size=(T, d))
    wr = rng.normal(size=(E, d))
    ex = _rand_experts(E, d, F)
    perm = rng.permutation(T)
    a = O.moe_layer(x, wr, _experts_fn(ex), E, k)
    b = O.moe_layer(x[perm], wr, _experts_fn(ex), E, k)
    assert np.allclose(b["out"], a["out"][perm], rtol=1e-13, atol=1e-13)
    assert (b["idx"] == a["idx"][perm]).all()


def test_ffn_row_subset_matches_full():
    T, d, F, E, k = 20, 4, 3, 5, 2
    x = rng.normal(size=(T, d))
    wr = rng.normal(size=(E, d))
    ex = _rand_experts(E, d, F)
    full = O.moe_layer(x, wr, _experts_fn(ex), E, k)
    rows = np.array([0, 3, 19])
    sub = O.moe_layer(x, wr, _experts_fn(ex), E, k, ffn_rows=rows)
    assert np.allclose(sub["out"][rows], full["out"][rows], rtol=1e-13, atol=1e-14)
    assert np.isnan(sub["out"][1]).all()


def test_experts_touched_formula_statistics():
    """Unbiased router on random tokens: distinct experts touched by B tokens averages
    E (1 - (1 - k/E)^B)  (within 4 standard errors over 200 draws).  Orthonormal router
    rows and isotropic tokens make the logits i.i.d. per (token, expert), which is the
    uniform independent routing the formula assumes."""
    E, k, d = 64, 8, 64
    for B in (1, 4, 16):
        touched = []
        for s in range(200):
            r = np.random.default_rng(10_000 + s)
            x = r.normal(size=(B, d))
            wr = np.linalg.qr(r.normal(size=(d, E)))[0].T
            L = O.router_logits(x, wr)
            idx, _ = O.select_topk(O.softmax_scores(L), k)
            touched.append(len(np.unique(idx)))
        m, se = np.mean(touched), np.std(touched) / math.sqrt(len(touched))
        expect = O.experts_touched_expected(E, k, B)
        assert abs(m - expect) <= 4 * se + 1e-9, (B, m, expect, se)
    assert O.experts_touched_expected(64, 8, 1) == 8
    assert math.isclose(O.experts_touched_expected(64, 8, 32), 64 * (1 - (7 / 8) ** 32))


def test_swaps_per_token():
    a = np.array([[0, 1, 2, 3], [4, 5, 6, 7]])
    b = np.array([[3, 2, 1, 0], [4, 5, 9, 8]])
    assert O.swaps_per_token(a, b).tolist() == [0, 2]


def test_logit_bias_steers_selection_and_gates():
    """The skew bias is part of the logits: a large bias on one expert makes every token
    select it, and its softmax gate is exp(l + b) / sum exp(l' + b')."""
    T, d, E, k = 8, 4, 5, 2
    x = rng.normal(size=(T, d)) * 0.1
    wr = rng.normal(size=(E, d))
    bias = np.zeros(E)
    bias[3] = 20.0
    res = O.moe_layer(x, wr, _experts_fn(_rand_experts(E, d, 2)), E, k, logit_bias=bias,
                      ffn_rows=np.arange(0))
    assert (res["idx"][:, 0] == 3).all()
    L = x @ wr.T + bias
    expect = np.exp(L[:, 3]) / np.exp(L).sum(1)
    assert np.allclose(res["gates"][:, 0], expect, rtol=1e-13)


# --------------------------------------------------------------------------
# FP8 activations: bf16 rounding, E4M3 rounding, per-row quantisation
# --------------------------------------------------------------------------
def test_bf16_rounding_matches_library():
    """round_to_bf16 against torch's float32 -> bfloat16 cast (round to nearest even, a
    library routine) on fp32 values of every magnitude; bf16 values map to themselves;
    exact midpoints go to the even significand."""
    import torch
    v = (rng.normal(size=20000) * np.exp2(rng.integers(-40, 40, size=20000))).astype(np.float32)
    lib = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.round_to_bf16(v.astype(np.float64)), lib)
    b = O.bf16_to_f64(np.arange(0x0080, 0x7F00, 7, dtype=np.uint16))
    assert np.array_equal(O.round_to_bf16(b), b)
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties to even -> 1; 1 + 3 2^-8 -> 1 + 2^-6
    assert O.round_to_bf16(np.array([1 + 2.0 ** -8]))[0] == 1.0
    assert O.round_to_bf16(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2.0 ** -6
    assert O.round_to_bf16(np.array([-(1 + 2.0 ** -8)]))[0] == -1.0


def _e4m3_finite_values():
    v = O.fp8_e4m3_to_f64(np.arange(256, dtype=np.uint8))
    return v[~np.isnan(v)]


def test_e4m3_rounding_round_trips_every_value_and_ties_to_even():
    vals = _e4m3_finite_values()
    assert np.array_equal(O.round_to_e4m3(vals), vals)
    pos = np.unique(vals[vals >= 0])
    codes = {float(O.fp8_e4m3_to_f64(np.uint8(c))): c for c in range(0x7F)}
    for a, b in zip(pos[:-1], pos[1:]):
        mid = (a + b) / 2
        even = a if codes[float(a)] % 2 == 0 else b   # the code with mantissa bit 0
        assert O.round_to_e4m3(np.array([mid]))[0] == even
        assert O.round_to_e4m3(np.array([-mid]))[0] == -even
        # just off the midpoint: the nearer neighbour
        assert O.round_to_e4m3(np.array([mid - (b - a) / 64]))[0] == a
        assert O.round_to_e4m3(np.array([mid + (b - a) / 64]))[0] == b
    # beyond the largest finite value: held at 448
    assert np.array_equal(O.round_to_e4m3(np.array([448.0 * (1 + 2.0 ** -23), 463.9, 1e6, -500.0])),
                          np.array([448.0, 448.0, 448.0, -448.0]))


def test_e4m3_rounding_matches_library():
    """Against torch's float32 -> float8_e4m3fn cast (round to nearest even) over the whole
    finite range, subnormals included."""
    import torch
    v = (rng.uniform(-1, 1, size=50000) * np.exp2(rng.uniform(-12, 8.8, size=50000))).astype(np.float32)
    v = v[np.abs(v) <= 448]
    lib = torch.from_numpy(v).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(O.round_to_e4m3(v.astype(np.float64)), lib)


def test_row_quantisation_exact_cases_and_bounds():
    vals = _e4m3_finite_values()
    # a row of E4M3 values times 2^j holding +-448 2^j: codes are the values, scale is 2^j
    for j in (-20, -3, 0, 5):
        row = rng.choice(vals, size=(3, 200))
        row[:, 7] = 448.0
        row[1, 9] = -448.0
        codes, scale = O.quantize_rows_e4m3(row * 2.0 ** j)
        assert np.array_equal(codes, row) and np.array_equal(scale, np.full(3, 2.0 ** j))
    # an all-zero row: codes 0, scale 0
    codes, scale = O.quantize_rows_e4m3(np.zeros((2, 64)))
    assert not codes.any() and not scale.any()
    # random bf16 rows: the largest magnitude always lands on +-448; every element within half an
    # E4M3 step (2^-4 of its magnitude, or 2^-10 in the subnormal range) times the fp32 scale
    bits = rng.integers(0, 0x7F00, size=(50, 300)) | (rng.integers(0, 2, size=(50, 300)) << 15)
    x = O.bf16_to_f64(bits.astype(np.uint16))   # every finite bf16 magnitude, both signs
    codes, scale = O.quantize_rows_e4m3(x)
    top = np.abs(x).argmax(axis=1)
    assert np.array_equal(np.abs(codes[np.arange(50), top]), np.full(50, 448.0))
    assert np.all(np.abs(codes) <= 448.0)
    err = np.abs(codes * scale[:, None] - x)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * scale[:, None]) * (1 + 2.0 ** -20) + 1e-300
    assert np.all(err <= bound)
    # the scale is amax / 448 in fp32
    assert np.array_equal(scale, (np.abs(x).max(axis=1).astype(np.float32) / np.float32(448)).astype(np.float64))


def test_a8_ffn_in_the_code_domain():
    """swiglu_ffn_a8 against the same layer computed from the integer codes: with every E4M3
    value times 2^9 an integer, a GEMM of quantised rows is the exact integer sum of code
    products, times the row scale and the weight's own scale, times 2^-18."""
    T, d, F = 5, 16, 12
    vals = _e4m3_finite_values()
    wq = [rng.choice(vals, size=(F, d)), rng.choice(vals, size=(F, d)), rng.choice(vals, size=(d, F))]
    ws = [rng.uniform(0.5, 2, size=F) / 448, rng.uniform(0.5, 2, size=F) / 448, rng.uniform(0.5, 2, size=d) / 448]
    W = [q * s[:, None] for q, s in zip(wq, ws)]
    x = O.bf16_to_f64(rng.integers(0x3C00, 0x4100, size=(T, d)).astype(np.uint16) ^ (rng.integers(0, 2, size=(T, d)) << 15).astype(np.uint16))
    got = O.swiglu_ffn_a8(x, *W)

    def gemm_codes(rows, wi):
        codes, scale = O.quantize_rows_e4m3(rows)
        ci = (codes * 512).astype(np.int64)
        wi_int = (wq[wi] * 512).astype(np.int64)
        out = np.empty((rows.shape[0], wi_int.shape[0]))
        for t in range(rows.shape[0]):
            for n in range(wi_int.shape[0]):
                acc = sum(int(ci[t, k]) * int(wi_int[n, k]) for k in range(ci.shape[1]))
                out[t, n] = acc * 2.0 ** -18 * scale[t] * ws[wi][n]
        return out
    g, u = gemm_codes(x, 0), gemm_codes(x, 1)
    h = O.round_to_bf16(g / (1 + np.exp(-g)) * u)
    ref = gemm_codes(h, 2)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_a8_layer_structure_and_size_of_the_quantisation_error():
    """E = 1, k = 1 and a shared expert: the FP8-activation layer is swiglu_ffn_a8 plus the
    shared expert's own FP8-activation FFN; against the bf16-activation layer it differs, by
    an amount of the order of E4M3's relative precision (2^-4 per element at most)."""
    T, d, F = 64, 128, 96
    x = O.round_to_bf16(rng.normal(size=(T, d)))
    mk = lambda *s: O.round_to_bf16(rng.normal(size=s) / math.sqrt(s[-1]))
    ex = [(mk(F, d), mk(F, d), mk(d, F))]
    sh = [(mk(F, d), mk(F, d), mk(d, F))]
    kw = dict(logit_bias=np.array([0.1]), shared=_experts_fn(sh), n_shared=1)
    a8 = O.moe_layer(x, rng.normal(size=(1, d)), _experts_fn(ex), 1, 1, act_fp8=True, **kw)["out"]
    ref = O.swiglu_ffn_a8(x, *ex[0]) + O.swiglu_ffn_a8(x, *sh[0])
    assert np.allclose(a8, ref, rtol=1e-13, atol=1e-13)
    plain = O.moe_layer(x, rng.normal(size=(1, d)), _experts_fn(ex), 1, 1, **kw)["out"]
    rel = np.abs(a8 - plain).max(axis=1) / np.abs(plain).max(axis=1)
    assert 1e-3 < np.median(rel) < 6e-2 and rel.max() < 0.15


def test_a8_shared_experts_quantise_one_concatenated_row():
    """Two shared experts share one quantised row per token: a second expert of zeros changes
    nothing (its h is 0, the row maximum is the first's), and a second copy of the first
    doubles the shared output exactly (the same maximum, the same codes)."""
    T, d, F = 16, 128, 64
    x = O.round_to_bf16(rng.normal(size=(T, d)))
    mk = lambda *s: O.round_to_bf16(rng.normal(size=s) / math.sqrt(s[-1]))
    ex = [(mk(F, d), mk(F, d), mk(d, F))]
    sh = (mk(F, d), mk(F, d), mk(d, F))
    zero = tuple(np.zeros_like(w) for w in sh)
    wr = rng.normal(size=(1, d))
    run = lambda shs: O.moe_layer(x, wr, _experts_fn(ex), 1, 1, act_fp8=True, shared=_experts_fn(shs),
                                  n_shared=len(shs))["out"]
    one = run([sh])
    assert np.array_equal(run([sh, zero]), one)
    routed = O.swiglu_ffn_a8(x, *ex[0])
    assert np.allclose(run([sh, sh]) - routed, 2 * (one - routed), rtol=1e-13, atol=1e-13)
