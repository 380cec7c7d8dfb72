"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test states what fixes the expected value: a closed form, a textbook or
library routine, a brute-force enumeration, an exact rational computation, or a
number printed on the pages (tests/golden/beam_page_facts.json).  CPU only.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from beam_inputs import WORKLOADS, make_inputs, normal

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# helpers that do exact arithmetic independently of the oracle
# ---------------------------------------------------------------------------
def round_f32(q: Fraction) -> float:
    """Round an exact rational to the nearest float32 (ties to even), no double rounding."""
    if q == 0:
        return 0.0
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum = Fraction(2) ** (max(e, -126) - 23)
    m = a / quantum
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * float(fl * quantum)


def fma_f32(a, b, c) -> float:
    return round_f32(Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c)))


def ulp32(x: np.ndarray) -> np.ndarray:
    """ulp of a float32 at |x| (normal range)."""
    _, e = np.frexp(np.abs(x))
    return np.ldexp(1.0, e - 24)


# ---------------------------------------------------------------------------
# exp / sigmoid
# ---------------------------------------------------------------------------
def test_exp_within_2ulp_of_double_exp_strided_sweep():
    """Own FP32 exp vs float64 exp: <= 2 ulp over a strided sweep of every FP32 in
    [-87, 87] (every 13th bit pattern: ~170M values)."""
    hi = np.float32(87.0).view(np.uint32)
    worst = 0.0
    for sign in (0, 0x80000000):
        for start in range(0, int(hi) + 1, 13 * (1 << 22)):
            bits = np.arange(start, min(start + 13 * (1 << 22), int(hi) + 1), 13, dtype=np.uint32)
            x = (bits | np.uint32(sign)).view(np.float32)
            y = oracle.expf(x).astype(np.float64)
            ref = np.exp(x.astype(np.float64))
            err = np.abs(y - ref) / ulp32(ref)
            worst = max(worst, float(err.max()))
    assert worst <= 2.0, worst


def test_exp_dense_near_zero_and_special_values():
    x = np.linspace(-1, 1, 2_000_001, dtype=np.float32)
    y = oracle.expf(x).astype(np.float64)
    ref = np.exp(x.astype(np.float64))
    assert (np.abs(y - ref) / ulp32(ref)).max() <= 2.0
    assert oracle.expf(np.array([0.0], np.float32))[0] == 1.0
    # clamp: values beyond +-87 behave as +-87, results stay normal and finite
    big = oracle.expf(np.array([87.0, 1000.0, -87.0, -1000.0], np.float32))
    assert big[0] == big[1] and big[2] == big[3]
    assert np.isfinite(big).all() and big[2] >= np.finfo(np.float32).tiny


def test_sigmoid_closed_forms():
    s = oracle.sigmoidf(np.array([0.0, math.log(3.0), -math.log(3.0)], np.float32))
    assert s[0] == 0.5                                   # sigma(0) = 1/2 exactly
    assert abs(s[1] - 0.75) < 2e-7 and abs(s[2] - 0.25) < 2e-7
    z = np.linspace(-30, 30, 100001, dtype=np.float32)
    ref = 1.0 / (1.0 + np.exp(-z.astype(np.float64)))
    got = oracle.sigmoidf(z).astype(np.float64)
    assert (np.abs(got - ref) / ref).max() < 4e-7
    # symmetry sigma(z) + sigma(-z) = 1
    assert np.abs(got + oracle.sigmoidf(-z).astype(np.float64) - 1.0).max() < 2e-7


# ---------------------------------------------------------------------------
# router logits
# ---------------------------------------------------------------------------
def test_logits_order_contract_exact_rationals():
    """Bit-exact against exact rational emulation of the order contract: 64 contiguous
    chunks, each acc = fma(x_h, w_h, acc) over its h ascending, chunk sums added in
    ascending order, then + bias (one rounding each)."""
    rs = np.random.default_rng(7)
    T, H, E = 2, 192, 3
    x = rs.standard_normal((T, H)).astype(np.float32)
    w = rs.standard_normal((H, E)).astype(np.float32)
    b = rs.standard_normal(E).astype(np.float32)
    z = oracle.router_logits(x, w, b)
    ch = H // 64
    for t in range(T):
        for e in range(E):
            tot = 0.0
            for c in range(64):
                acc = 0.0
                for h in range(c * ch, (c + 1) * ch):
                    acc = fma_f32(x[t, h], w[h, e], acc)
                tot = round_f32(Fraction(tot) + Fraction(acc))
            tot = round_f32(Fraction(tot) + Fraction(float(b[e])))
            assert z[t, e] == np.float32(tot), (t, e)


def test_logits_within_rounding_bound_of_exact_dot():
    """|z - exact| <= gamma_H * sum |x w| (standard error bound of a length-H
    floating-point dot product)."""
    w = WORKLOADS["beam_decode_t16"]
    x = normal(0, (99,), (8, w.H))
    wr = normal(0, (98,), (w.H, w.E), std=1 / math.sqrt(w.H))
    z = oracle.router_logits(x, wr).astype(np.float64)
    exact = x.astype(np.float64) @ wr.astype(np.float64)
    u = 2.0 ** -24
    gamma = w.H * u / (1 - w.H * u)
    bound = gamma * (np.abs(x.astype(np.float64)) @ np.abs(wr.astype(np.float64)))
    assert (np.abs(z - exact) <= bound).all()


# ---------------------------------------------------------------------------
# group-limited selection
# ---------------------------------------------------------------------------
def brute_route(s: np.ndarray, G: int, Kg: int, K: int):
    """Brute force for one token: group score = best pair sum in the group (max over
    all pairs i<j of fl(s_i + s_j)), kept groups and experts by enumerating every
    subset and taking the one whose members, sorted by (value desc, index asc),
    form the lexicographically best sequence."""
    E = s.size
    S = E // G
    gs = []
    for g in range(G):
        vals = s[g * S:(g + 1) * S]
        gs.append(max(np.float32(vals[i] + vals[j]) for i in range(S) for j in range(i + 1, S)))

    def key(items, val):
        return sorted(((-float(val[i]), i) for i in items))

    best_groups = min(itertools.combinations(range(G), Kg), key=lambda c: key(c, gs))
    cand = [e for e in range(E) if e // S in best_groups]
    best_exp = min(itertools.combinations(cand, K), key=lambda c: key(c, s))
    ordered = [i for _, i in key(best_exp, s)]
    return ordered, sorted(best_groups, key=lambda g: (-float(gs[g]), g))


@pytest.mark.parametrize("seed", range(6))
def test_route_matches_brute_force_tiny_layer(seed):
    w = WORKLOADS["tiny_f32"]
    rs = np.random.default_rng(seed)
    T = 48
    z = rs.standard_normal((T, w.E)).astype(np.float32)
    if seed % 2:          # force exact ties across and within groups
        z = np.round(z * 2) / 2
    ids, wts, d = oracle.route(z, w.G, w.Kg, w.K, w.alpha, details=True)
    s = d["scores"]
    for t in range(T):
        exp_ids, exp_groups = brute_route(s[t], w.G, w.Kg, w.K)
        assert list(ids[t]) == exp_ids, (t, ids[t], exp_ids)
        assert list(d["kept_groups"][t]) == exp_groups


# Selection-only bias (auxiliary-loss-free balancing; reading: ranking value r = s + b in
# FP32, weights from the unbiased scores s).
@pytest.mark.parametrize("seed", range(4))
def test_select_bias_matches_brute_force_tiny_layer(seed):
    w = WORKLOADS["tiny_f32"]
    rs = np.random.default_rng(100 + seed)
    T = 48
    z = rs.standard_normal((T, w.E)).astype(np.float32)
    b = (rs.standard_normal(w.E) * 0.3).astype(np.float32)
    if seed % 2:          # ties in the ranking values
        b = np.round(b * 4) / 4
        z = np.round(z * 2) / 2
    ids, wts, d = oracle.route(z, w.G, w.Kg, w.K, w.alpha, details=True, select_bias=b)
    s = d["scores"]
    for t in range(T):
        r = (s[t] + b).astype(np.float32)       # IEEE single-precision adds
        exp_ids, exp_groups = brute_route(r, w.G, w.Kg, w.K)
        assert list(ids[t]) == exp_ids, (t, ids[t], exp_ids)
        assert list(d["kept_groups"][t]) == exp_groups
        sel = s[t][ids[t]].astype(np.float64)
        assert np.allclose(wts[t], w.alpha * sel / sel.sum(), rtol=1e-6, atol=0)


def test_select_bias_zero_is_the_unbiased_route():
    w = WORKLOADS["beam_decode_t16"]
    z = np.random.default_rng(7).standard_normal((64, w.E)).astype(np.float32)
    i0, w0 = oracle.route(z, w.G, w.Kg, w.K, w.alpha)
    i1, w1 = oracle.route(z, w.G, w.Kg, w.K, w.alpha, select_bias=np.zeros(w.E, np.float32))
    assert np.array_equal(i0, i1) and np.array_equal(w0, w1)


def test_select_bias_dominant_bias_forces_the_picks():
    """A bias of +8 on two experts in each of Kg chosen groups (scores lie in (0, 1))
    forces exactly those K experts whatever the logits; -8 on the natural winner
    removes it.  Weights normalise the unbiased scores of the forced picks."""
    w = WORKLOADS["beam_decode_t16"]
    S = w.E // w.G
    rs = np.random.default_rng(11)
    z = rs.standard_normal((32, w.E)).astype(np.float32)
    forced = np.array([g * S + j for g in (1, 3, 4, 6) for j in (5, 17)])
    b = np.zeros(w.E, np.float32)
    b[forced] = 8.0
    ids, wts, d = oracle.route(z, w.G, w.Kg, w.K, w.alpha, details=True, select_bias=b)
    s = d["scores"]
    for t in range(z.shape[0]):
        r = (s[t][forced] + np.float32(8.0)).astype(np.float32)
        order = sorted(range(len(forced)), key=lambda i: (-float(r[i]), int(forced[i])))
        assert list(ids[t]) == [int(forced[i]) for i in order]
        assert sorted(d["kept_groups"][t]) == [1, 3, 4, 6]
        sel = s[t][ids[t]].astype(np.float64)
        assert np.allclose(wts[t], w.alpha * sel / sel.sum(), rtol=1e-6, atol=0)
    top, _ = oracle.route(z, w.G, w.Kg, w.K, w.alpha)
    b2 = np.zeros(w.E, np.float32)
    b2[top[0, 0]] = -8.0
    ids2, _ = oracle.route(z[:1], w.G, w.Kg, w.K, w.alpha, select_bias=b2)
    assert top[0, 0] not in ids2[0]


def dominance_ok(s, gs, kept, ids, G, K):
    E = s.size
    S = E // G
    order = lambda v, i: (-float(v), i)
    keptset = set(int(g) for g in kept)
    for g in keptset:
        for h in set(range(G)) - keptset:
            if not order(gs[g], g) < order(gs[h], h):
                return False
    chosen = set(int(e) for e in ids)
    cand = [e for e in range(E) if e // S in keptset]
    for e in chosen:
        if e // S not in keptset:
            return False
        for f in set(cand) - chosen:
            if not order(s[e], e) < order(s[f], f):
                return False
    seq = [order(s[e], e) for e in ids]
    return seq == sorted(seq) and len(chosen) == K


def test_route_dominance_certificate_beam_size():
    w = WORKLOADS["beam_prefill_t4096"]
    rs = np.random.default_rng(3)
    T = 256
    z = rs.standard_normal((T, w.E)).astype(np.float32)
    ids, wts, d = oracle.route(z, w.G, w.Kg, w.K, w.alpha, details=True)
    s, gs, kept = d["scores"], d["group_scores"], d["kept_groups"]
    for t in range(T):
        # group scores: independent recomputation via a sort
        grp = np.sort(s[t].reshape(w.G, -1), axis=1)
        assert np.array_equal(gs[t], (grp[:, -1] + grp[:, -2]).astype(np.float32))
        assert dominance_ok(s[t], gs[t], kept[t], ids[t], w.G, w.K)
    # group choice brute-forced over all C(8,4) = 70 subsets
    for t in range(0, T, 17):
        best = min(itertools.combinations(range(w.G), w.Kg),
                   key=lambda c: sorted((-float(gs[t][g]), g) for g in c))
        assert sorted(best) == sorted(kept[t])


def test_route_all_ties_closed_form():
    """Wr = 0 -> every score is sigma(0) = 0.5 -> groups 0..Kg-1, experts 0..K-1,
    every weight exactly alpha / K."""
    for name in ("tiny_f32", "beam_decode_t16"):
        w = WORKLOADS[name]
        z = oracle.router_logits(np.ones((4, w.H), np.float32), np.zeros((w.H, w.E), np.float32))
        ids, wts, d = oracle.route(z, w.G, w.Kg, w.K, w.alpha, details=True)
        assert (ids == np.arange(w.K)).all()
        assert (d["kept_groups"] == np.arange(w.Kg)).all()
        assert (wts == np.float32(w.alpha / w.K)).all()


def test_route_single_group_is_plain_topk():
    """G = 1 (or Kg = G) reduces to plain top-K over all experts: compare with a
    stable numpy sort on (-s, index)."""
    rs = np.random.default_rng(11)
    z = np.round(rs.standard_normal((64, 32)).astype(np.float32) * 4) / 4
    for G, Kg in ((1, 1), (4, 4)):
        ids, _, d = oracle.route(z, G, Kg, 6, 2.5, details=True)
        s = d["scores"]
        ref = np.argsort(-s, axis=1, kind="stable")[:, :6]
        assert np.array_equal(ids, ref)


def test_route_top2_sum_not_max():
    """A group with the single highest score but a weak runner-up loses to a group
    with two strong scores."""
    E, G = 16, 4
    z = np.full((1, E), -5.0, np.float32)
    z[0, 0] = 4.0          # group 0: max 4.0, runner-up -5
    z[0, 4] = 3.0          # group 1: 3.0 + 3.0
    z[0, 5] = 3.0
    ids, _, d = oracle.route(z, G, 1, 2, 2.5, details=True)
    assert list(d["kept_groups"][0]) == [1]
    assert sorted(ids[0]) == [4, 5]


def test_route_k1_weight_is_alpha():
    rs = np.random.default_rng(5)
    z = rs.standard_normal((32, 16)).astype(np.float32)
    _, wts = oracle.route(z, 4, 2, 1, 2.5)
    assert (wts == np.float32(2.5)).all()


def test_route_weights_normalised_and_scaled():
    w = WORKLOADS["beam_prefill_t4096"]
    rs = np.random.default_rng(9)
    z = rs.standard_normal((512, w.E)).astype(np.float32) * 2
    ids, wts, d = oracle.route(z, w.G, w.Kg, w.K, w.alpha, details=True)
    assert np.allclose(wts.astype(np.float64).sum(1), 2.5, rtol=1e-6, atol=0)
    s = np.take_along_axis(d["scores"], ids, 1).astype(np.float64)
    ref = 2.5 * s / s.sum(1, keepdims=True)
    assert (np.abs(wts - ref) / ref).max() < 1e-6
    # the selected experts lie inside the kept groups, 8 distinct ids
    assert ((ids // (w.E // w.G))[:, :, None] == d["kept_groups"][:, None, :]).any(2).all()
    assert all(len(set(r)) == w.K for r in ids)


# ---------------------------------------------------------------------------
# expert MLP and combine
# ---------------------------------------------------------------------------
def test_expert_impulse_closed_form():
    """x = c e_h0, Wg = a at (j0,h0), Wu = b at (j0,h0), Wd = d at (m0,j0), zero elsewhere:
    o[m0] = d * SiLU(a c) * (b c), o = 0 elsewhere.  With a c = ln 3,
    SiLU(ln 3) = 0.75 ln 3.  Pins the layout (gate rows first, Wd[m, j]) and that the
    SiLU applies to the gate, not to the up projection."""
    H, I = 12, 5
    h0, j0, m0 = 7, 3, 2
    c, a, b, dd = 2.0, math.log(3.0) / 2.0, -1.5, 0.25
    x = np.zeros((1, H)); x[0, h0] = c
    w13 = np.zeros((2 * I, H)); w13[j0, h0] = a; w13[I + j0, h0] = b
    w2 = np.zeros((H, I)); w2[m0, j0] = dd
    o = oracle.expert_ffn(x, w13, w2)
    expect = np.zeros(H); expect[m0] = dd * 0.75 * math.log(3.0) * (b * c)
    assert np.allclose(o[0], expect, rtol=1e-14, atol=1e-15)


def _tiny_bank(rs, E, H, I, same=False):
    w13 = rs.standard_normal((1 if same else E, 2 * I, H)) / math.sqrt(H)
    w2 = rs.standard_normal((1 if same else E, H, I)) / math.sqrt(I)
    if same:
        w13 = np.repeat(w13, E, 0); w2 = np.repeat(w2, E, 0)
    return oracle.ExpertBank(w13.astype(np.float32), w2.astype(np.float32), "f32")


def test_identical_experts_give_alpha_times_ffn():
    w = WORKLOADS["tiny_f32"]
    rs = np.random.default_rng(2)
    bank = _tiny_bank(rs, w.E, w.H, w.I, same=True)
    x = rs.standard_normal((16, w.H)).astype(np.float32)
    wr = rs.standard_normal((w.H, w.E)).astype(np.float32)
    r = oracle.moe_forward(x, wr, None, bank, w.G, w.Kg, w.K, w.alpha)
    w13, w2 = bank.expert(0)
    ref = 2.5 * oracle.expert_ffn(x.astype(np.float64), w13, w2)
    assert np.allclose(r["y"], ref, rtol=1e-6, atol=1e-6)


def test_dense_gate_vector_cross_check():
    """y[t] = sum over ALL experts e of G[t,e] FFN_e(x_t), with G the sparse gate
    vector (weights at the chosen ids, 0 elsewhere), computed token by token."""
    w = WORKLOADS["tiny_f32"]
    inp = make_inputs(w)
    bank = oracle.ExpertBank(inp.w13, inp.w2, "f32")
    x = inp.x
    r = oracle.moe_forward(x, inp.w_router, None, bank, w.G, w.Kg, w.K, w.alpha)
    for t in range(0, w.T, 5):
        gate = np.zeros(w.E)
        gate[r["ids"][t]] = r["w"][t]
        acc = np.zeros(w.H)
        for e in range(w.E):
            w13, w2 = bank.expert(e)
            acc += gate[e] * oracle.expert_ffn(x[t:t + 1].astype(np.float64), w13, w2)[0]
        assert np.allclose(r["y"][t], acc, rtol=1e-12, atol=1e-12)


def test_combine_linear_in_down_projection():
    w = WORKLOADS["tiny_f32"]
    inp = make_inputs(w)
    b1 = oracle.ExpertBank(inp.w13, inp.w2, "f32")
    b2 = oracle.ExpertBank(inp.w13, inp.w2 * 2, "f32")
    r1 = oracle.moe_forward(inp.x, inp.w_router, None, b1, w.G, w.Kg, w.K, w.alpha)
    r2 = oracle.moe_forward(inp.x, inp.w_router, None, b2, w.G, w.Kg, w.K, w.alpha)
    assert np.allclose(r2["y"], 2 * r1["y"], rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# dense SwiGLU MLP (first decoder layers)
# ---------------------------------------------------------------------------
def _one_slot(w13, w2):
    return oracle.ExpertBank(w13[None].astype(np.float32), w2[None].astype(np.float32), "f32")


def test_dense_impulse_closed_form_and_token_subset():
    """Token 0 = c e_h0, token 1 = 0: y[0] = d SiLU(a c) (b c) e_m0 with a c = ln 3
    (SiLU(ln 3) = 0.75 ln 3), y[1] = 0; a token subset returns just those rows."""
    H, I = 10, 6
    h0, j0, m0 = 4, 5, 9
    c, a, b, dd = 3.0, math.log(3.0) / 3.0, 0.5, -2.0
    x = np.zeros((2, H), np.float32); x[0, h0] = c
    w13 = np.zeros((2 * I, H)); w13[j0, h0] = a; w13[I + j0, h0] = b
    w2 = np.zeros((H, I)); w2[m0, j0] = dd
    bank = oracle.ExpertBank(w13[None].astype(np.float64), w2[None].astype(np.float64), "f32")
    bank.w13, bank.w2 = w13[None], w2[None]          # exact float64 values
    r = oracle.dense_forward(x, bank)
    expect = np.zeros((2, H)); expect[0, m0] = dd * 0.75 * math.log(3.0) * (b * c)
    assert np.allclose(r["y"], expect, rtol=1e-14, atol=1e-15)
    r1 = oracle.dense_forward(x, bank, token_subset=np.array([1]))
    assert r1["y"].shape == (1, H) and np.all(r1["y"] == 0.0) and list(r1["tokens"]) == [1]


def test_dense_is_the_moe_with_identical_experts_over_alpha():
    """A MoE layer whose experts all hold the dense weights returns alpha * dense(x)
    whatever the routing (the combine weights sum to alpha)."""
    w = WORKLOADS["tiny_f32"]
    rs = np.random.default_rng(5)
    bank = _tiny_bank(rs, w.E, w.H, w.I, same=True)
    x = rs.standard_normal((24, w.H)).astype(np.float32)
    wr = rs.standard_normal((w.H, w.E)).astype(np.float32)
    moe = oracle.moe_forward(x, wr, None, bank, w.G, w.Kg, w.K, w.alpha)
    dense = oracle.dense_forward(x, oracle.ExpertBank(bank.w13[:1], bank.w2[:1], "f32"))
    assert np.allclose(moe["y"], w.alpha * dense["y"], rtol=1e-6, atol=1e-6)


def test_dense_sublayer_zero_down_projection_keeps_the_scaled_stream():
    """Wd = 0 gives y = 0, RMSNorm(0) = 0, so h' = sqrt((k-1)/k) h exactly."""
    rs = np.random.default_rng(6)
    H, I, k = 64, 32, 7
    h = rs.standard_normal((5, H)).astype(np.float32)
    bank = _one_slot(rs.standard_normal((2 * I, H)), np.zeros((H, I)))
    r = oracle.dense_sublayer_forward(h, None, None, k, 1e-6, bank)
    assert np.all(r["y"] == 0.0)
    assert np.array_equal(r["h_new"], math.sqrt((k - 1) / k) * h.astype(np.float64))


def test_dense_sublayer_matches_moe_sublayer_with_identical_experts():
    """With alpha = 1 and every expert holding the dense weights, the MoE sublayer and
    the dense sublayer compute the same h' (up to the FP32 combine weights)."""
    w = WORKLOADS["tiny_f32"]
    rs = np.random.default_rng(7)
    bank = _tiny_bank(rs, w.E, w.H, w.I, same=True)
    h = rs.standard_normal((12, w.H)).astype(np.float32)
    wr = rs.standard_normal((w.H, w.E)).astype(np.float32)
    g1 = (1 + 0.1 * rs.standard_normal(w.H)).astype(np.float32)
    g2 = (1 + 0.1 * rs.standard_normal(w.H)).astype(np.float32)
    moe = oracle.sublayer_forward(h, g1, g2, 5, 1e-6, wr, None, bank, w.G, w.Kg, w.K, 1.0)
    dense = oracle.dense_sublayer_forward(h, g1, g2, 5, 1e-6,
                                          oracle.ExpertBank(bank.w13[:1], bank.w2[:1], "f32"))
    assert np.allclose(moe["h_new"], dense["h_new"], rtol=1e-6, atol=1e-6)


# ---------------------------------------------------------------------------
# storage formats
# ---------------------------------------------------------------------------
def test_e4m3_decode_matches_spec_facts_and_torch():
    import torch
    tab = oracle.E4M3_TABLE
    assert tab[0x7E] == 448.0 and tab[0xFE] == -448.0       # max normal
    assert tab[0x08] == 2.0 ** -6                             # min normal
    assert tab[0x01] == 2.0 ** -9                             # min subnormal
    assert tab[0x38] == 1.0 and tab[0x40] == 2.0 and tab[0x3F] == 1.875
    assert np.isnan(tab[0x7F]) and np.isnan(tab[0xFF])
    pos = tab[:0x7F]
    assert (np.diff(pos) > 0).all()                           # monotone code order
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.nan_to_num(tab, nan=1e9), np.nan_to_num(t, nan=1e9))


def test_e2m1_and_e8m0_decode_match_the_mx_spec():
    """OCP Microscaling Formats v1.0: FP4 E2M1 magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6
    (max normal 6 = 1.5 * 2^2, min normal 1, min subnormal 0.5), sign in bit 3; the E8M0
    scale is 2^(code - 127) with code 255 = NaN (checked against torch's float8_e8m0fnu)."""
    import torch
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert list(oracle.E2M1_TABLE[:8]) == mags
    assert list(oracle.E2M1_TABLE[8:]) == [-m for m in mags]
    codes = np.arange(255, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float32).numpy().astype(np.float64)
    assert np.array_equal(oracle.e8m0_to_f64(codes), ref)
    assert np.isnan(oracle.e8m0_to_f64(np.array([255], np.uint8)))[0]


def test_mxfp4_dequant_layout_and_blocks():
    """Packed layout (element 2j low nibble, 2j+1 high nibble of byte j) and one scale per
    32 consecutive elements along K, on a hand-built matrix."""
    packed = np.zeros((2, 32), np.uint8)          # 2 rows x 64 elements
    packed[0, 0] = 0x2 | (0x7 << 4)               # row 0: e0 = 1.0, e1 = 6.0
    packed[1, 20] = 0xB << 4                      # row 1: e41 = -1.5
    scales = np.array([[127, 130], [126, 120]], np.uint8)   # 2^0, 2^3; 2^-1, 2^-7
    v = oracle.dequant_mxfp4(packed, scales)
    exp = np.zeros((2, 64))
    exp[0, 0], exp[0, 1] = 1.0, 6.0
    exp[1, 41] = -1.5 * 2.0 ** -7
    assert np.array_equal(v, exp)


def test_e4m3_encode_matches_torch_and_spec():
    """The oracle's E4M3 rounding (activation operands) against torch's float8_e4m3fn
    conversion (round to nearest even) on values from the subnormal range to 448, on every
    midpoint between neighbouring codes (the ties) and on every code value; magnitudes
    past 448 saturate to 448 (torch returns NaN from 464 on)."""
    import torch
    rs = np.random.default_rng(5)
    v = (rs.standard_normal(400_000) * np.exp(rs.uniform(-14, 6, 400_000))).astype(np.float32)
    v = np.clip(v, -448, 448)
    pos = oracle.E4M3_TABLE[:0x7F]
    mid = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    v = np.concatenate([v, mid, -mid, pos.astype(np.float32), -pos.astype(np.float32)])
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode(v), ref)
    # ties go to the even code: 1 + 1/16 (between 1 and 1.125) -> 1.0, 1 + 3/16 -> 1.25
    assert oracle.e4m3_encode(np.float32([1.0625, 1.1875])).tolist() == [0x38, 0x3A]
    assert oracle.e4m3_encode(np.float32([460.0, 500.0, -1e9, 0.0, -0.0])).tolist() == [0x7E, 0x7E, 0xFE, 0x00, 0x80]


def test_bf16_round_matches_torch_including_ties():
    import torch
    rs = np.random.default_rng(6)
    b = rs.integers(0, 2 ** 32, 300_000, dtype=np.uint64).astype(np.uint32)
    b = b[np.isfinite(b.view(np.float32))]
    ties = (b & np.uint32(0xFFFF0000)) | np.uint32(0x8000)        # exactly half way
    v = np.concatenate([b, ties[np.isfinite(ties.view(np.float32))]]).view(np.float32)
    v = v[np.abs(v) < 3e38]
    ref = torch.from_numpy(v).to(torch.bfloat16).float().numpy()
    assert np.array_equal(oracle.bf16_round(v).view(np.uint32), ref.view(np.uint32))


def test_quant_rows_e4m3_closed_forms():
    """Row E4M3 quantisation: a row whose amax is 448 * 2^k has the scale 2^k exactly and
    its E4M3-representable multiples come back unchanged; an all-zero row gets scale 1
    and zero codes; the amax element becomes +-448; negating a row flips only sign bits;
    every value is within half an E4M3 step of its input (relative 2^-4 in the normal
    range, 2^-10 s below it)."""
    rs = np.random.default_rng(7)
    grid = oracle.E4M3_TABLE[:0x7F]
    k = np.array([-20, -3, 0, 5], np.int64)
    rows = rs.choice(grid, size=(4, 256)) * rs.choice([-1.0, 1.0], size=(4, 256))
    rows[:, 7] = 448.0
    rows = (rows * np.exp2(k)[:, None]).astype(np.float32)
    codes, s = oracle.quant_rows_e4m3(rows)
    assert np.array_equal(s, np.exp2(k).astype(np.float32))
    assert np.array_equal(oracle.e4m3_to_f64(codes) * s[:, None], rows.astype(np.float64))
    codes, s = oracle.quant_rows_e4m3(np.zeros((2, 64), np.float32))
    assert (s == 1.0).all() and (codes == 0).all()
    v = (rs.standard_normal((64, 1000)) * np.exp(rs.uniform(-30, 30, (64, 1)))).astype(np.float32)
    codes, s = oracle.quant_rows_e4m3(v)
    am = np.abs(v).argmax(axis=1)
    assert (np.abs(oracle.e4m3_to_f64(codes[np.arange(64), am])) == 448.0).all()
    ncodes, ns = oracle.quant_rows_e4m3(-v)
    assert np.array_equal(ns, s) and np.array_equal(ncodes, codes ^ 0x80)
    deq = oracle.act_e4m3(v)
    sd = s.astype(np.float64)[:, None]
    bound = np.maximum(np.abs(v) * 2.0 ** -4, sd * 2.0 ** -10) * (1 + 1e-6)
    assert (np.abs(deq - v) <= bound).all()


def test_expert_ffn_act_quant_is_the_quantised_operands():
    """With act_quant the expert sees E4M3 rows of x and of its BF16-stored SwiGLU
    output: an x already on the E4M3 grid with amax 448 (scale 1) goes through unchanged,
    so the first product equals the unquantised one; the output then moves by no more
    than the E4M3 step of a (2^-4 relative per entry) allows."""
    rs = np.random.default_rng(8)
    H, I = 64, 32
    grid = oracle.E4M3_TABLE[:0x7F] / 448.0
    x = rs.choice(grid, size=(5, H)) * rs.choice([-1.0, 1.0], size=(5, H))
    x[:, 0] = 1.0
    x = (x * 448.0).astype(np.float32)                       # amax 448: scale 1
    assert np.array_equal(oracle.act_e4m3(x), x.astype(np.float64))
    w13 = rs.standard_normal((2 * I, H)) / 8 / np.sqrt(H) / 448
    w2 = rs.standard_normal((H, I)) / np.sqrt(I)
    y = oracle.expert_ffn(x.astype(np.float64), w13, w2)
    yq = oracle.expert_ffn(x.astype(np.float64), w13, w2, act_quant=True)
    g = x.astype(np.float64) @ w13[:I].T
    a = oracle.silu(g) * (x.astype(np.float64) @ w13[I:].T)
    bound = (np.abs(a) * (2.0 ** -4 + 2.0 ** -8) + np.abs(a).max(1, keepdims=True) * 2.0 ** -18) @ np.abs(w2.T)
    assert (np.abs(yq - y) <= bound).all()
    assert not np.array_equal(yq, y)


def test_bf16_widening_matches_torch():
    import torch
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    mine = oracle.bf16_to_f32(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    fin = np.isfinite(ref)
    assert np.array_equal(mine[fin].view(np.uint32), ref[fin].view(np.uint32))


# ---------------------------------------------------------------------------
# norms and residual
# ---------------------------------------------------------------------------
def test_prenorm_closed_forms_and_order():
    H = 5120
    c = np.float32(0.75)
    xh, r = oracle.prenorm(np.full((1, H), c, np.float32), None, 1e-6)
    assert abs(float(xh[0, 0]) - 0.75 / math.sqrt(0.5625 + 1e-6)) < 2e-7
    x = normal(0, (77,), (16, H))
    xh, r = oracle.prenorm(x, None, 1e-6)
    ms = np.mean(x.astype(np.float64) ** 2, 1)
    got = np.mean(xh.astype(np.float64) ** 2, 1)
    assert np.allclose(got, ms / (ms + 1e-6), rtol=1e-5)
    # exact-rational check of the fixed order on a short row
    xs = normal(0, (78,), (1, 130))
    p = [0.0] * 64
    for l in range(64):
        for h in range(l, 130, 64):
            p[l] = fma_f32(xs[0, h], xs[0, h], p[l])
    o = 32
    while o >= 1:
        for l in range(o):
            p[l] = round_f32(Fraction(p[l]) + Fraction(p[l + o]))
        o //= 2
    ms32 = round_f32(Fraction(p[0]) / 130)
    rr = round_f32(1 / Fraction(math.sqrt(float(np.float32(ms32 + np.float32(1e-6))))))
    _, r1 = oracle.prenorm(xs, None, 1e-6)
    # r = 1/sqrtf(ms+eps): sqrt correctly rounded, then a correctly rounded reciprocal
    s32 = np.sqrt(np.float32(ms32) + np.float32(1e-6), dtype=np.float32)
    assert r1[0] == np.float32(1.0) / s32
    assert abs(float(r1[0]) - rr) <= 1e-6 * rr


def pin_rmsnorm_constant_vector():
    """RMSNorm of c * 1 is sign(c) |c| / sqrt(c^2 + eps), times the gain (the mean of
    squares of a constant vector is c^2).  eps large enough that its place matters."""
    H, eps = 8, 0.5
    g = np.array([2.0, 0.5, 1.0, 3.0, -1.0, 0.25, 1.5, 4.0])
    for c in (-1.5, 0.75, 3.0):
        got = oracle.rmsnorm64(np.full((1, H), c), g, eps)
        want = np.sign(c) * abs(c) / math.sqrt(c * c + eps) * g
        assert np.allclose(got[0], want, rtol=1e-14, atol=0.0), (c, got, want)


def pin_rmsnorm_known_mean_square_per_row():
    """Rows with hand-computed mean squares, normalised each on its own: [3, 4, 0, 0]
    has mean square 25/4, [1, 1, 1, 1] has 1, [0, 0, 0, 2] has 1; a non-unit gain
    multiplies the normalised value (not the input)."""
    eps = 0.75
    y = np.array([[3.0, 4.0, 0.0, 0.0], [1.0, 1.0, 1.0, 1.0], [0.0, 0.0, 0.0, 2.0]])
    ms = np.array([25.0 / 4.0, 1.0, 1.0])
    g = np.array([1.0, 2.0, -0.5, 3.0])
    got = oracle.rmsnorm64(y, g, eps)
    want = np.empty_like(y)
    for t in range(3):
        for j in range(4):
            want[t, j] = y[t, j] / math.sqrt(ms[t] + eps) * g[j]
    assert np.allclose(got, want, rtol=1e-14, atol=0.0)
    # no gain = unit gain
    assert np.allclose(oracle.rmsnorm64(y, None, eps), want / g, rtol=1e-14, atol=0.0)


def pin_sublayer_impulse_closed_form():
    """A residual stream with one nonzero entry per token, through experts that all hold
    one impulse weight each (so the routing does not matter and the MoE output has one
    nonzero entry): every step of pre-norm -> MoE -> post-norm -> residual has a closed
    form.  h' = sqrt((k-1)/k) h + (1/sqrt k) RMSNorm(y) g_post (Beam overview,
    "Residual stream")."""
    H, I, E, G, Kg, K, alpha = 64, 8, 16, 4, 2, 4, 2.5
    h0, j0, m0 = 5, 3, 41
    a, b, d = 0.25, -0.5, 1.75
    eps = 0.3
    w13 = np.zeros((E, 2 * I, H), np.float32)
    w13[:, j0, h0] = a
    w13[:, I + j0, h0] = b
    w2 = np.zeros((E, H, I), np.float32)
    w2[:, m0, j0] = d
    bank = oracle.ExpertBank(w13, w2, "f32")
    rs = np.random.default_rng(31)
    wr = rs.standard_normal((H, E)).astype(np.float32)
    c_tok = np.array([1.5, -4.0, 0.25], np.float32)        # two tokens' magnitudes differ
    h = np.zeros((3, H), np.float32)
    h[:, h0] = c_tok
    g_post = np.ones(H, np.float32)
    g_post[m0] = 1.5
    for k in (4, 10):
        r = oracle.sublayer_forward(h, None, g_post, k, eps, wr, None, bank, G, Kg, K, alpha)
        c1, c2 = math.sqrt((k - 1) / k), 1.0 / math.sqrt(k)
        for t, c in enumerate(c_tok.astype(np.float64)):
            xh = c / math.sqrt(c * c / H + eps)              # pre-norm of c e_h0 at h0
            y = alpha * d * (a * xh) / (1.0 + math.exp(-a * xh)) * (b * xh)
            yn = y / math.sqrt(y * y / H + eps) * 1.5        # post-norm of y e_m0 at m0
            want = np.zeros(H)
            want[h0] = c1 * c
            want[m0] = c2 * yn
            # FP32 pre-norm and FP32 combine weights: ~1e-6 relative
            assert np.allclose(r["h_new"][t], want, rtol=2e-6, atol=1e-7), (k, t, r["h_new"][t], want)
            assert np.allclose(r["y"][t], np.where(np.arange(H) == m0, y, 0.0), rtol=2e-6, atol=1e-7)


POSTNORM_PINS = (pin_rmsnorm_constant_vector, pin_rmsnorm_known_mean_square_per_row,
                 pin_sublayer_impulse_closed_form)


@pytest.mark.parametrize("pin", POSTNORM_PINS, ids=lambda f: f.__name__)
def test_postnorm_and_sublayer_pins(pin):
    pin()


def _mutant_rmsnorm(kind):
    def f(y, gain, eps):
        if kind == "eps_outside_sqrt":
            r = 1.0 / (np.sqrt(np.mean(y * y, axis=1, keepdims=True)) + eps)
        elif kind == "mean_wrong_axis":
            r = 1.0 / np.sqrt(np.mean(y * y, axis=0, keepdims=True) + eps)
        elif kind == "gain_before_norm":
            y = y * (1.0 if gain is None else gain.astype(np.float64))
            return y / np.sqrt(np.mean(y * y, axis=1, keepdims=True) + eps)
        out = y * r
        return out if gain is None else out * gain.astype(np.float64)
    return f


@pytest.mark.parametrize("mistake", ["eps_outside_sqrt", "mean_wrong_axis", "gain_before_norm",
                                     "c1_c2_swapped"])
def test_postnorm_pins_catch_planted_mistakes(mistake, monkeypatch):
    """Each plausible mistake in the post-norm or the residual, planted in the oracle on
    the CPU, fails at least one of the pins above."""
    if mistake == "c1_c2_swapped":
        good = oracle.residual_coeffs
        monkeypatch.setattr(oracle, "residual_coeffs", lambda k: good(k)[::-1])
    else:
        monkeypatch.setattr(oracle, "rmsnorm64", _mutant_rmsnorm(mistake))
    failed = 0
    for pin in POSTNORM_PINS:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed >= 1, f"no pin caught {mistake}"


def test_residual_constant_scale_and_equal_weights():
    """c1^2 + c2^2 = 1; after steps 2..n the stream is (1/sqrt n) * (embedding + sum
    of outputs): every contribution carries the same weight (pages: 104 additions)."""
    facts = json.load(open(os.path.join(GOLDEN, "beam_page_facts.json")))
    for k in range(2, 200):
        c1, c2 = oracle.residual_coeffs(k)
        assert abs(c1 * c1 + c2 * c2 - 1.0) < 1e-15
    n_add = facts["residual_additions"]
    n = n_add + 1                       # the embedding is step 1
    dim = n
    h = np.zeros((1, dim)); h[0, 0] = 1.0          # embedding = unit vector 0
    for k in range(2, n + 1):
        out = np.zeros((1, dim)); out[0, k - 1] = 1.0
        h = oracle.residual_update(h, out, k)
    assert np.allclose(h, 1 / math.sqrt(n), rtol=1e-12)


def test_page_shape_facts():
    """Param-count identities printed on the pages fix the expert shape."""
    f = json.load(open(os.path.join(GOLDEN, "beam_page_facts.json")))
    w = WORKLOADS["beam_prefill_t4096"]
    assert (w.H, w.I, w.E, w.G, w.Kg, w.K, w.alpha) == (
        f["hidden_size"], f["expert_intermediate"], f["experts_per_layer"], f["groups"],
        f["kept_groups"], f["routed_per_token"], f["routed_scale"])
    assert w.E // w.G == f["group_size"]
    per_expert = 3 * w.H * w.I
    assert abs(per_expert / f["params_per_expert"] - 1) < 0.01
    share = f["moe_layers"] * w.E * per_expert / f["total_params"]
    assert abs(share - f["expert_param_share"]) < 0.001
    # active per token = 49 layers x 8 routed experts + the non-expert parameters
    active = f["moe_layers"] * w.K * per_expert + f["non_expert_params"]
    assert abs(active / f["active_params"] - 1) < 0.02
