"""Plain, slow FP64 CPU oracle for the forward pass of a top-k MoE SwiGLU FFN layer.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
the benchmark's CPU-baseline leg may import this module.  It shares no code
with the HIP library and imports nothing from it.

Every function computes its step in float64 from the exact bit patterns the
GPU receives (bf16 / fp32 / INT4 nibbles + bf16 scales, FP8 bytes + fp32
scales), one step at a time and in the order the pages describe, with numpy
matmuls and sorts as the only library primitives.  The one exception is the
per-row FP8 quantisation of activations, whose scale and product are defined
in IEEE fp32 (the reading in quantize_rows_e4m3) and are computed here in
numpy float32, so that both sides take the same rounding decisions.

Sources (the pages this follows):
  [MoE-dyn]  "MoE: dynamism the compiler cannot remove" -- the natural
             implementation (router logits -> top-k -> per-expert FFN ->
             accumulate into the token's output), the capacity section
             (buffers of C*T*k/E rows, overflow dropped and skipping the FFN),
             the grouped-GEMM section and the batch-1 recipe (fixed-shape
             scatter into preallocated buffers).
  [Ceil]     picx.dev summary of the MoE launch-bound study, "Sub-study 1:
             Triton Kernel Engineering" (FP32 gate probabilities from a
             max-subtract-expsum softmax before top-k) and "Sub-study 2"
             (route replay; the replay of a model's own routes must return the
             baseline exactly).
  [MoE-inf]  "MoE at the inference level ..." -- Workarounds (int4 / fp8
             expert weights, auxiliary-loss-free bias term) and Fields
             (weight_dtype).
  [MoE-res]  "MoE Research", section 2 (shared always-on experts;
             loss-free balancing bias used for selection; node-limited
             routing: a token's experts come from at most M nodes) and
             section 7A (experts-touched formula E*(1-(1-k/E)^B)).
Readings where the pages are silent (the SwiGLU definition, gate
renormalisation, capacity priority, INT4 format, ...) are listed in the
repository's design notes and restated at each function below.
"""
from __future__ import annotations

import math
from typing import Callable, Optional, Sequence

import numpy as np

INT4_GROUP = 128


# --------------------------------------------------------------------------
# exact decoding of stored bit patterns
# --------------------------------------------------------------------------
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16/int16) -> exact float64 values.

    A bf16 value is the upper half of an IEEE binary32, so widening is exact."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f32_to_f64(a: np.ndarray) -> np.ndarray:
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def int4_unpack(packed: np.ndarray) -> np.ndarray:
    """Packed INT4 -> signed integers in [-8, 7].

    Format (reading of "INT4 symmetric ... groups of 128 with bf16 scales"):
    byte i of a row holds element 2i in its low nibble and element 2i+1 in its
    high nibble, each a two's-complement 4-bit integer."""
    p = np.asarray(packed, dtype=np.uint8)
    lo = (p & 0x0F).astype(np.int16)
    hi = (p >> 4).astype(np.int16)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    q = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.int16)
    q[..., 0::2] = lo
    q[..., 1::2] = hi
    return q


def int4_dequant(packed: np.ndarray, scale_bits: np.ndarray, group: int = INT4_GROUP) -> np.ndarray:
    """w[n, k] = q[n, k] * s[n, k // group], exactly, in float64 ([MoE-inf] int4 expert weights)."""
    q = int4_unpack(packed).astype(np.float64)
    s = bf16_to_f64(scale_bits)
    return q * np.repeat(s, group, axis=-1)


def fp8_e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """FP8 E4M3 bytes (the OCP 8-bit floating-point format, "fn" variant: sign,
    4 exponent bits with bias 7, 3 mantissa bits, no infinities) to float64,
    exactly ([MoE-inf] workarounds: fp8 expert weights).  Exponent field 0 is
    subnormal, m/8 * 2^-6; field 15 with mantissa 7 is NaN; every other code is
    (1 + m/8) * 2^(e - 7), so the largest finite value is 448."""
    c = np.asarray(codes, np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    return np.where((e == 15) & (m == 7), np.nan, sign * mag)


def fp8_dequant(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """w[n, k] = fp8(code[n, k]) * s[n] with one fp32 scale per output channel, exactly."""
    return fp8_e4m3_to_f64(codes) * np.asarray(scales, np.float64)[..., None]


def round_to_bf16(v: np.ndarray) -> np.ndarray:
    """float64 -> the nearest bf16 value (8 significant bits, ties to even), as float64.

    v = m 2^e with 0.5 <= |m| < 1; m 2^8 rounded half-to-even is the bf16
    significand.  (Normal range only: the values here are far from bf16's
    subnormals and its overflow threshold.)"""
    m, e = np.frexp(np.asarray(v, np.float64))
    return np.ldexp(np.rint(m * 256.0), e - 8)


E4M3_MAX = 448.0


def round_to_e4m3(v: np.ndarray) -> np.ndarray:
    """float64 -> the nearest OCP E4M3 ("fn") value, ties to the even significand, as float64.

    In the binade [2^b, 2^(b+1)) with b >= -6 the values are spaced 2^(b-3);
    below 2^-6 (subnormals) they are spaced 2^-9.  Magnitudes past the largest
    finite value 448 are held at 448 (reading: the format has no infinity and
    the quantiser below never produces more than 448 (1 + 2^-23))."""
    v = np.asarray(v, np.float64)
    a = np.abs(v)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    b = np.clip(ex - 1, -6, 8)              # binade exponent (frexp's exponent is one above it)
    step = np.exp2(b - 3.0)
    q = np.minimum(np.rint(a / step) * step, E4M3_MAX)
    return np.where(v < 0, -q, q)


def quantize_rows_e4m3(v: np.ndarray):
    """Per-row symmetric E4M3 quantisation of activations, with fp32 scale arithmetic.

    Reading of "fp8 expert weights" run on an FP8 matrix unit ([MoE-inf]
    workarounds and Fields, weight_dtype): the matrix unit takes both operands
    in FP8, so each row of a GEMM's activation operand (a token's x, or its
    SwiGLU output h) is quantised on its own.  With v the row's values (exact
    fp32 values: bf16 here) and amax = max |v|, in IEEE fp32:
        inv = 448 / amax,  code_i = E4M3(v_i * inv),  scale = amax / 448;
    the row stands for code_i * scale.  An all-zero row has codes 0, scale 0.
    Returns (codes as float64 values [.., n], scale float64 [..])."""
    v32 = np.asarray(v, np.float64).astype(np.float32)
    if not np.array_equal(v32.astype(np.float64), np.asarray(v, np.float64)):
        raise ValueError("quantize_rows_e4m3 takes fp32-representable values")
    amax = np.abs(v32).max(axis=-1)
    nz = amax > 0
    safe = np.where(nz, amax, np.float32(1))
    inv = np.where(nz, np.float32(448.0) / safe, np.float32(0)).astype(np.float32)
    prod = (v32 * inv[..., None]).astype(np.float32)
    codes = round_to_e4m3(prod.astype(np.float64))
    scale = np.where(nz, safe / np.float32(448.0), np.float32(0)).astype(np.float32)
    return codes, scale.astype(np.float64)


def dequant_rows_e4m3(v: np.ndarray) -> np.ndarray:
    """The row as the FP8 matrix unit sees it: code_i * scale (exact in float64)."""
    codes, scale = quantize_rows_e4m3(v)
    return codes * scale[..., None]


# --------------------------------------------------------------------------
# router: logits, scores, selection, gates
# --------------------------------------------------------------------------
def router_logits(x: np.ndarray, w_router: np.ndarray,
                  logit_bias: Optional[np.ndarray] = None) -> np.ndarray:
    """logits[t, e] = sum_i x[t, i] * w_router[e, i] (+ logit_bias[e])   ([MoE-dyn] `router(x)`, [T, E]).

    w_router is stored one row per expert.  The per-expert skew bias is a
    router parameter added to the logits (so it shapes the gates as well)."""
    logits = np.asarray(x, np.float64) @ np.asarray(w_router, np.float64).T
    if logit_bias is not None:
        logits = logits + np.asarray(logit_bias, np.float64)[None, :]
    return logits


def softmax_scores(logits: np.ndarray) -> np.ndarray:
    """Row softmax in the max-subtract-expsum form ([Ceil] Sub-study 1):
    p[t, e] = exp(l[t, e] - max_e l[t]) / sum_e exp(l[t, e] - max_e l[t])."""
    m = logits.max(axis=1, keepdims=True)
    z = np.exp(logits - m)
    return z / z.sum(axis=1, keepdims=True)


def sigmoid_scores(logits: np.ndarray) -> np.ndarray:
    """s[t, e] = 1 / (1 + exp(-l[t, e]))  (DeepSeek-V3-style sigmoid scoring)."""
    return 1.0 / (1.0 + np.exp(-logits))


def select_topk(key: np.ndarray, k: int):
    """Top-k expert indices per row.

    Order: descending key; equal keys go to the lower expert index first.
    -0.0 and +0.0 are treated as equal.  Returns (idx [T, k] int32 in slot
    order, margin [T] = key of the k-th pick minus the best key not picked,
    +inf when k == E)."""
    key = np.asarray(key, np.float64) + 0.0  # canonicalise -0.0
    T, E = key.shape
    idx = np.empty((T, k), np.int32)
    margin = np.full(T, np.inf)
    cols = np.arange(E)
    for t in range(T):
        # lexsort sorts by the last key first: primary -key, secondary index
        order = np.lexsort((cols, -key[t]))
        idx[t] = order[:k]
        if k < E:
            margin[t] = key[t, order[k - 1]] - key[t, order[k]]
    return idx, margin


def limit_groups(key: np.ndarray, n_groups: int, topk_groups: int):
    """Group-limited selection ([MoE-res] section 2, node-limited routing; [MoE-inf]
    workarounds, device-limited routing with M = 4): a token's k experts must come
    from at most M = topk_groups of the n_groups groups.

    Reading (the pages name the constraint, not the rule that picks the groups):
    the experts form n_groups equal groups of consecutive indices (group of e is
    e // (E / n_groups)); a group's score is the largest selection key in it; the
    M groups with the largest scores are kept (equal scores: the lower group
    first); every expert outside them gets key -inf, so the top-k that follows
    picks only inside them.  Returns (masked key, group margin [T] = M-th group
    score minus the (M+1)-th, +inf when M == n_groups)."""
    key = np.asarray(key, np.float64) + 0.0
    T, E = key.shape
    if E % n_groups or not 1 <= topk_groups <= n_groups:
        raise ValueError((E, n_groups, topk_groups))
    gsz = E // n_groups
    gscore = key.reshape(T, n_groups, gsz).max(axis=2)
    keep, gmargin = select_topk(gscore, topk_groups)
    allowed = np.zeros((T, n_groups), bool)
    np.put_along_axis(allowed, keep.astype(np.int64), True, axis=1)
    masked = np.where(np.repeat(allowed, gsz, axis=1), key, -np.inf)
    return masked, gmargin


def gate_weights(scores: np.ndarray, idx: np.ndarray, renorm: bool, scale: float) -> np.ndarray:
    """g[t, j] = scale * score[t, idx[t, j]] (/ sum_j' score[t, idx[t, j']] when renorm).

    The combine weights each selected expert by its gate (the pages' "weighted"
    combine; the printed loop adds expert outputs unweighted, read as an
    omission).  Scores are the unbiased ones: a selection-only bias never
    enters a gate."""
    g = np.take_along_axis(np.asarray(scores, np.float64), idx.astype(np.int64), axis=1)
    if renorm:
        g = g / g.sum(axis=1, keepdims=True)
    return g * scale


# --------------------------------------------------------------------------
# permutation: histogram, prefix sum, capacity, fixed-shape assignment
# --------------------------------------------------------------------------
def capacity_rows(T: int, k: int, E: int, cap_num: int, cap_den: int) -> int:
    """cap = ceil(C * T * k / E) with C = cap_num / cap_den, in exact integer arithmetic
    ([MoE-dyn] capacity: each expert's buffer holds C*T*k/E rows)."""
    num = cap_num * T * k
    den = cap_den * E
    return -(-num // den)


def assign_rows(idx: np.ndarray, E: int, cap: Optional[int] = None):
    """Fixed-shape assignment of (token, slot) pairs to expert-major rows.

    Walk the pairs in token-major order (t ascending, then slot j ascending);
    the r-th pair routed to expert e gets rank r.  With a capacity, a pair with
    rank >= cap overflows: it is dropped and skips the expert FFN
    ([MoE-dyn] capacity).  Kept pairs of expert e fill rows
    offsets[e] .. offsets[e+1]-1 in walk order, so rows are stable in t.

    Returns dict(counts [E] (routed pairs per expert, before capacity),
    kept [E], offsets [E+1] (prefix sum of kept), row_token [R] (token of each
    row), slot_row [T, k] (row of each pair, -1 if dropped), drop [T, k] uint8)."""
    T, k = idx.shape
    counts = np.zeros(E, np.int64)
    rank = np.empty((T, k), np.int64)
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            rank[t, j] = counts[e]
            counts[e] += 1
    kept = counts.copy() if cap is None else np.minimum(counts, cap)
    offsets = np.zeros(E + 1, np.int64)
    offsets[1:] = np.cumsum(kept)
    drop = np.zeros((T, k), np.uint8)
    slot_row = np.full((T, k), -1, np.int64)
    row_token = np.full(int(offsets[E]), -1, np.int64)
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            if cap is not None and rank[t, j] >= cap:
                drop[t, j] = 1
                continue
            r = offsets[e] + rank[t, j]
            slot_row[t, j] = r
            row_token[r] = t
    return dict(counts=counts, kept=kept, offsets=offsets, row_token=row_token,
                slot_row=slot_row, drop=drop)


# --------------------------------------------------------------------------
# experts
# --------------------------------------------------------------------------
def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z * sigma(z) = z / (1 + exp(-z))."""
    return z / (1.0 + np.exp(-z))


def swiglu_ffn(x: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """One expert: (silu(x W_gate) * (x W_up)) W_down, no biases (reading of "SwiGLU
    expert ffn, W_gate, W_up [d, ffn], W_down [ffn, d]").

    Weights arrive as stored: w_gate, w_up [ffn][d] and w_down [d][ffn], one
    K-contiguous row per output channel, so x W_gate is x @ w_gate.T."""
    x = np.asarray(x, np.float64)
    g = x @ np.asarray(w_gate, np.float64).T
    u = x @ np.asarray(w_up, np.float64).T
    return (silu(g) * u) @ np.asarray(w_down, np.float64).T


def swiglu_ffn_a8(x: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """One expert with FP8 activations on both GEMMs (weights as given, e.g. fp8 * channel scale):
    x rows quantised per row (quantize_rows_e4m3) before x W_gate and x W_up; the SwiGLU output
    rounded to bf16 (the intermediate's storage type) and quantised per row before the down GEMM."""
    xa = dequant_rows_e4m3(x)
    g = xa @ np.asarray(w_gate, np.float64).T
    u = xa @ np.asarray(w_up, np.float64).T
    h = round_to_bf16(silu(g) * u)
    return dequant_rows_e4m3(h) @ np.asarray(w_down, np.float64).T


# An expert provider maps an expert number to its float64 (w_gate, w_up, w_down).
ExpertFn = Callable[[int], Sequence[np.ndarray]]


def moe_layer(x: np.ndarray, w_router: np.ndarray, experts: ExpertFn, E: int, k: int, *,
              score: str = "softmax", renorm: bool = False, gate_scale: float = 1.0,
              logit_bias: Optional[np.ndarray] = None, select_bias: Optional[np.ndarray] = None,
              capacity: Optional[tuple] = None, shared: Optional[ExpertFn] = None, n_shared: int = 0,
              ffn_rows: Optional[np.ndarray] = None, routes: Optional[tuple] = None,
              groups: Optional[tuple] = None, act_fp8: bool = False) -> dict:
    """The whole layer, step by step.

    1. logits = x W_r (+ skew bias); 2. scores (softmax, or sigmoid);
    3. selection key = score (+ selection-only bias for sigmoid scoring);
    3b. groups = (n_groups, M): keys outside the token's M best groups -> -inf;
    4. top-k with lowest-index ties; 5. gates; 6. capacity / assignment;
    7. every kept (t, j): y = FFN_{idx[t,j]}(x_t); 8. out_t = sum over kept j of
    g[t,j] * y + sum over shared experts of FFN_s(x_t) (weight 1, never dropped).
    A dropped pair contributes nothing and the remaining gates are not
    renormalised; the residual add belongs to the caller.

    ffn_rows: optional sorted token subset for steps 7-8 (routing always runs
    over every token); out rows outside the subset are NaN.
    routes: optional (idx, gates) that replace steps 2-5 (route replay).
    act_fp8: the expert GEMMs take FP8 activations (swiglu_ffn_a8); the shared
    experts' SwiGLU outputs are quantised as one row per token over all of them
    (their down GEMMs form one sum over the concatenated intermediate).
    """
    x = np.asarray(x, np.float64)
    T = x.shape[0]
    logits = router_logits(x, w_router, logit_bias)
    if score == "softmax":
        scores = softmax_scores(logits)
        key = scores
    elif score == "sigmoid":
        scores = sigmoid_scores(logits)
        key = scores if select_bias is None else scores + np.asarray(select_bias, np.float64)[None, :]
    else:
        raise ValueError(score)
    group_margin = np.full(T, np.inf)
    if groups is not None:
        key, group_margin = limit_groups(key, groups[0], groups[1])
    idx, margin = select_topk(key, k)
    gates = gate_weights(scores, idx, renorm, gate_scale)
    if routes is not None:
        idx = np.asarray(routes[0]).astype(np.int32)
        gates = np.asarray(routes[1], np.float64)
    cap = None
    if capacity is not None:
        cap = capacity_rows(T, k, E, capacity[0], capacity[1])
    asg = assign_rows(idx, E, cap)

    rows = np.arange(T) if ffn_rows is None else np.asarray(ffn_rows)
    in_set = np.zeros(T, bool)
    in_set[rows] = True
    out = np.full((T, x.shape[1]), np.nan)
    out[rows] = 0.0
    # per-expert evaluation over the expert's gathered tokens (one matmul per expert)
    for e in range(E):
        sel_t, sel_j = np.nonzero((idx == e) & (asg["drop"] == 0) & in_set[:, None])
        if sel_t.size == 0:
            continue
        wg, wu, wd = experts(e)
        y = (swiglu_ffn_a8 if act_fp8 else swiglu_ffn)(x[sel_t], wg, wu, wd)
        np.add.at(out, sel_t, gates[sel_t, sel_j][:, None] * y)
    if act_fp8 and n_shared > 0:
        xa = dequant_rows_e4m3(x[rows])
        ws = [shared(s) for s in range(n_shared)]
        h = np.concatenate([round_to_bf16(silu(xa @ np.asarray(wg, np.float64).T) * (xa @ np.asarray(wu, np.float64).T))
                            for wg, wu, _ in ws], axis=1)
        ha = dequant_rows_e4m3(h)
        wd_cat = np.concatenate([np.asarray(wd, np.float64) for _, _, wd in ws], axis=1)
        out[rows] += ha @ wd_cat.T
    else:
        for s in range(n_shared):
            wg, wu, wd = shared(s)
            out[rows] += swiglu_ffn(x[rows], wg, wu, wd)
    return dict(out=out, logits=logits, scores=scores, key=key, idx=idx, gates=gates,
                margin=margin, group_margin=group_margin, cap=cap, **asg)


def experts_touched_expected(E: int, k: int, B: int) -> float:
    """Expected number of distinct experts touched by B tokens under uniform
    routing: E * (1 - (1 - k/E)^B)  ([MoE-res] section 7, exercise A)."""
    return E * (1.0 - (1.0 - k / E) ** B)


def swaps_per_token(idx_a: np.ndarray, idx_b: np.ndarray) -> np.ndarray:
    """Routing drift per token: k - |S_a intersect S_b| (selection shift times k,
    [Ceil] "Swaps per token")."""
    k = idx_a.shape[1]
    return np.array([k - len(set(a.tolist()) & set(b.tolist())) for a, b in zip(idx_a, idx_b)])
