"""Pins of the CPU oracle against things other than itself.

Each test ties one oracle function to hand-worked values (tests/golden),
closed forms, brute force on tiny inputs, or a library routine on a special
case, chosen so that a dropped term, a wrong sign or index, or a transposed
operand fails at least one of them.  CPU only.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def bf16_bits(values):
    t = torch.tensor(values, dtype=torch.float32).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def f32_of_bits(b):
    return float(np.array([int(b) << 16], np.uint32).view(np.float32)[0])


# ---------------------------------------------------------------- formats

def exact_bf16_round(v: Fraction) -> Fraction:
    """Round a rational to the nearest bf16 value, ties to even (8 significant
    bits, exponent range of fp32, subnormal spacing 2^-133).  Finite only."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = math.floor(math.log2(a))
    # correct floor(log2) for rationals
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    q = Fraction(2) ** (e - 7)  # spacing of bf16 numbers at this exponent
    n = a / q
    fl = math.floor(n)
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * q


def test_f64_to_bf16_single_rounding(oracle_lib):
    rng = np.random.default_rng(5)
    vals = list(rng.standard_normal(3000) * np.exp(rng.uniform(-40, 40, 3000)))
    # ties and near-ties around 1 and a subnormal region
    vals += [1 + 2 ** -8, 1 + 2 ** -8 + 2 ** -40, 1 + 2 ** -8 - 2 ** -40, 1 + 3 * 2 ** -8,
             -(1 + 2 ** -8), 2.0 ** -130 * 1.5, 2.0 ** -134, 2.0 ** -134 * 1.0000001,
             3 * 2.0 ** -135, 0.0, -0.0, 1.0, -2.5]
    for v in vals:
        want = exact_bf16_round(Fraction(v))
        got = f32_of_bits(oracle_lib.f64_to_bf16(v))
        assert Fraction(got) == want, (v, got, float(want))


def test_f32_to_bf16_matches_torch_rne(oracle_lib):
    # torch's fp32 -> bf16 cast is round-to-nearest-even: a library routine.
    rng = np.random.default_rng(6)
    vals = np.concatenate([rng.standard_normal(2000).astype(np.float32),
                           np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 65504.0, 1e-39, -0.0],
                                    np.float32)])
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for v, r in zip(vals, ref):
        assert oracle_lib.f32_to_bf16(float(v)) == int(r)
    assert oracle_lib.f32_to_bf16(float("inf")) == 0x7F80
    nan_bits = oracle_lib.f32_to_bf16(float("nan"))
    assert (nan_bits & 0x7F80) == 0x7F80 and (nan_bits & 0x7F) != 0


# ---------------------------------------------------------------- router

def test_sigmoid_values(oracle_lib):
    from scipy.special import expit
    assert oracle_lib.sigmoid(0.0) == 0.5
    assert oracle_lib.sigmoid(float("inf")) == 1.0
    assert oracle_lib.sigmoid(float("-inf")) == 0.0
    assert math.isnan(oracle_lib.sigmoid(float("nan")))
    rng = np.random.default_rng(1)
    xs = rng.standard_normal(2000).astype(np.float32) * 8
    mism = 0
    for x in xs:
        ref = np.float32(expit(np.float64(x)))  # scipy's logistic, rounded once to fp32
        got = np.float32(oracle_lib.sigmoid(float(x)))
        if got != ref:
            mism += 1
            assert abs(float(got) - float(ref)) <= 2 ** -24 * abs(float(ref)) * 2
        # symmetry sigma(-x) = 1 - sigma(x)
        assert abs(oracle_lib.sigmoid(float(-x)) + float(got) - 1.0) < 2e-7
    assert mism <= 2


def test_logits_fixed_order_is_ascending_d(oracle_lib):
    # In fp32, 2^24 + 1 rounds back to 2^24.  Ascending order therefore gives
    # 0, while summing the last two terms first gives 1.
    x = bf16_bits([1.0, 1.0, 1.0])[None, :]
    w = np.array([[2.0 ** 24], [1.0], [-(2.0 ** 24)]], np.float32)
    assert oracle_lib.logits(x, w)[0, 0] == 0.0
    # reversed channel order gives the other rounding
    assert oracle_lib.logits(x, w[::-1].copy())[0, 0] == 1.0


def test_logits_within_fp32_error_bound(oracle_lib):
    rng = np.random.default_rng(2)
    T, d, E = 16, 384, 16
    x = bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    w = (rng.standard_normal((d, E)) * 0.02).astype(np.float32)
    got = oracle_lib.logits(x, w).astype(np.float64)
    xf = oracle_lib.bf16_bits_to_f32(x).astype(np.float64)
    exact = xf @ w.astype(np.float64)           # bf16*fp32 products are exact in fp64
    absdot = np.abs(xf) @ np.abs(w.astype(np.float64))
    bound = d * 2.0 ** -24 / (1 - d * 2.0 ** -24) * absdot
    assert np.all(np.abs(got - exact) <= bound)
    # and it is not trivially exact: the chain really rounds in fp32
    assert np.any(got != exact)


def test_hand_route_example(oracle_lib):
    g = gold("hand_route_d2_e3_k2.json")
    x = bf16_bits(g["x"])[None, :]
    w = np.array(g["w_router"], np.float32)
    lg = oracle_lib.logits(x, w)[0]
    assert list(lg) == g["cases"][0]["logits"]
    for case in g["cases"]:
        r = oracle_lib.route(x, w, np.array(case["bias"], np.float32), g["k"], nthreads=1)
        assert list(r["idx"][0]) == case["idx"]
        assert np.allclose(r["gate"][0], case["gate"], atol=1e-7, rtol=0)
        assert abs(float(r["margin"][0]) - case["margin"]) <= 1e-7
    # bias changes the choice but not the gate values
    r0 = oracle_lib.route(x, w, np.array(g["cases"][0]["bias"], np.float32), 2, 1)
    r1 = oracle_lib.route(x, w, np.array(g["cases"][1]["bias"], np.float32), 2, 1)
    assert list(r0["idx"][0]) != list(r1["idx"][0])
    assert np.array_equal(r0["gate"], r1["gate"])


def _brute_topk(keys, k):
    """All C(E,k) subsets: the largest key sum wins; among equal sums the
    lexicographically smallest index tuple (lowest-index tie-break).  NaN
    keys count as -inf.  Slot order: descending key, then ascending index."""
    E = len(keys)
    kk = [(-math.inf if math.isnan(v) else float(v)) for v in keys]
    best = None
    for sub in itertools.combinations(range(E), k):
        s = sum(Fraction(kk[i]) if kk[i] != -math.inf else Fraction(-10 ** 9) for i in sub)
        cand = (s, tuple(-i for i in sub))
        if best is None or cand > best[0]:
            best = (cand, sub)
    sub = best[1]
    return sorted(sub, key=lambda i: (-kk[i] if kk[i] != -math.inf else math.inf, i))


def test_select_matches_brute_force_subsets(oracle_lib):
    rng = np.random.default_rng(3)
    for trial in range(300):
        E = int(rng.integers(2, 8))
        k = int(rng.integers(1, E + 1))
        keys = rng.integers(-3, 4, E).astype(np.float32) / 4  # many ties
        if trial % 5 == 0:
            keys[rng.integers(0, E)] = np.nan
        if trial % 7 == 0:
            keys[rng.integers(0, E)] = -0.0
        got = list(oracle_lib.select(keys[None, :], k)[0])
        assert got == _brute_topk(list(keys), k), (keys, k, got)


def test_select_matches_stable_argsort(oracle_lib):
    rng = np.random.default_rng(4)
    keys = rng.standard_normal((200, 16)).astype(np.float32)
    keys[:, 3] = keys[:, 5]  # exact ties
    got = oracle_lib.select(keys, 4)
    ref = np.argsort(-keys, axis=1, kind="stable")[:, :4]  # library stable sort
    assert np.array_equal(got, ref)


def _rand_layer(T=64, d=128, E=16, k=4, seed=0, bias_range=0.05):
    rng = np.random.default_rng(seed)
    x = bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    w = (rng.standard_normal((d, E)) * 0.05).astype(np.float32)
    b = rng.uniform(-bias_range, bias_range, E).astype(np.float32)
    return x, w, b


def test_zero_bias_selects_topk_of_logits(oracle_lib):
    x, w, _ = _rand_layer(T=256, seed=7)
    r = oracle_lib.route(x, w, np.zeros(16, np.float32), 4)
    lg = oracle_lib.logits(x, w)
    ref = torch.topk(torch.from_numpy(lg), 4, dim=1).indices.numpy()
    ok = r["margin"] >= 1e-6
    assert ok.mean() > 0.9
    assert np.array_equal(np.sort(r["idx"][ok], 1), np.sort(ref[ok], 1))


def test_route_invariants_and_gates(oracle_lib):
    x, w, b = _rand_layer(T=300, seed=8)
    r = oracle_lib.route(x, w, b, 4)
    idx, g, s = r["idx"], r["gate"], r["scores"]
    for t in range(idx.shape[0]):
        assert len(set(idx[t])) == 4
        keys = s[t] + b
        assert all(keys[idx[t, j]] >= keys[idx[t, j + 1]] for j in range(3))
        chosen = s[t, idx[t]]
        # gate is the unbiased score over the fp32 slot-order sum of chosen scores
        tot = np.float32(0)
        for v in chosen:
            tot = np.float32(tot + v)
        assert np.array_equal(g[t], (chosen / tot).astype(np.float32))
    assert np.allclose(g.sum(1), 1.0, atol=1e-6)
    # k = 1: the gate is exactly one
    r1 = oracle_lib.route(x, w, b, 1)
    assert np.all(r1["gate"] == 1.0)


def test_bias_changes_selection_not_gates(oracle_lib):
    x, w, b = _rand_layer(T=400, seed=9)
    r0 = oracle_lib.route(x, w, b, 4)
    b2 = b + np.random.default_rng(10).uniform(-0.02, 0.02, 16).astype(np.float32)
    r1 = oracle_lib.route(x, w, b2, 4)
    same = np.all(r0["idx"] == r1["idx"], axis=1)
    assert same.any() and (~same).any()
    assert np.array_equal(r0["gate"][same], r1["gate"][same])
    # a large bias on a fixed set forces that set; gates stay s / sum(s) over it
    forced = np.zeros(16, np.float32)
    forced[[2, 5, 11, 13]] = 4.0
    rf = oracle_lib.route(x, w, forced, 4)
    assert np.all(np.sort(rf["idx"], 1) == np.array([2, 5, 11, 13]))
    s = rf["scores"]
    for t in range(0, 400, 37):
        chosen = s[t, rf["idx"][t]]
        assert np.allclose(rf["gate"][t], chosen / chosen.sum(), atol=1e-7)


def test_nan_scores_rank_last(oracle_lib):
    x, w, b = _rand_layer(T=8, seed=11)
    w = w.copy()
    w[:, 3] = np.nan  # expert 3's logit is NaN for every token
    r = oracle_lib.route(x, w, b, 4)
    assert not np.any(r["idx"] == 3)
    x2 = x.copy()
    x2[0, 0] = 0x7FC0  # NaN activation: every logit of token 0 is NaN
    r2 = oracle_lib.route(x2, w, b, 4)
    assert list(r2["idx"][0]) == [0, 1, 2, 3]
    assert np.all(np.isnan(r2["gate"][0]))


def test_margin_definition(oracle_lib):
    x, w, b = _rand_layer(T=50, seed=12)
    r = oracle_lib.route(x, w, b, 4)
    keys = (r["scores"] + b).astype(np.float32)
    srt = -np.sort(-keys, axis=1)
    assert np.array_equal(r["margin"], (srt[:, 3] - srt[:, 4]).astype(np.float32))
    rall = oracle_lib.route(x, w, b, 16)
    assert np.all(np.isinf(rall["margin"]))


# ---------------------------------------------------------------- balance statistic

def test_seq_balance_closed_forms(oracle_lib):
    g = gold("seq_balance_closed_form.json")
    for case in g["cases"]:
        L = oracle_lib.seq_balance(np.array(case["scores"], np.float32),
                                   np.array(case["idx"], np.int32), 2, g["alpha"])
        assert L.shape == (1,)
        assert abs(L[0] - case["L"]) <= 1e-18


def test_seq_balance_invariants(oracle_lib):
    x, w, b = _rand_layer(T=512, seed=13)
    r = oracle_lib.route(x, w, b, 4)
    S = 128
    L = oracle_lib.seq_balance(r["scores"], r["idx"], S, 1.0)
    # per sequence: sum_i f_i = E and sum_i P_i = 1, so L/alpha lies in (0, E/k]
    for q in range(4):
        sl = slice(q * S, (q + 1) * S)
        cnt = np.bincount(r["idx"][sl].ravel(), minlength=16)
        f = 16 / (4 * S) * cnt
        P = (r["scores"][sl].astype(np.float64) /
             r["scores"][sl].astype(np.float64).sum(1, keepdims=True)).mean(0)
        assert abs(f.sum() - 16) < 1e-12 and abs(P.sum() - 1) < 1e-12
        assert abs(L[q] - (f * P).sum()) < 1e-12
        assert 0 < L[q] <= 16 / 4
    # alpha scales linearly
    L2 = oracle_lib.seq_balance(r["scores"], r["idx"], S, 1e-4)
    assert np.allclose(L2, L * 1e-4, rtol=1e-15)


# ---------------------------------------------------------------- permutation

def test_permute_invariants(oracle_lib):
    rng = np.random.default_rng(14)
    for T, E, k in ((1, 4, 2), (37, 16, 4), (300, 8, 2), (64, 256, 8)):
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        p = oracle_lib.permute(idx, E)
        assert p["counts"].sum() == T * k
        assert np.array_equal(p["counts"], np.bincount(idx.ravel(), minlength=E))
        assert p["offsets"][0] == 0 and p["offsets"][E] == T * k
        assert np.array_equal(np.diff(p["offsets"]), p["counts"])
        # pos is a bijection onto the rows; each row points back to its token
        assert np.array_equal(np.sort(p["pos"].ravel()), np.arange(T * k))
        for t in range(T):
            for j in range(k):
                row = p["pos"][t, j]
                e = idx[t, j]
                assert p["perm_src"][row] == t
                assert p["offsets"][e] <= row < p["offsets"][e + 1]
        # group contents: the tokens that chose e, ascending
        for e in range(E):
            seg = p["perm_src"][p["offsets"][e]:p["offsets"][e + 1]]
            assert np.array_equal(seg, np.nonzero((idx == e).any(1))[0])


# ---------------------------------------------------------------- expert FFN

def test_ffn_hand_cases(oracle_lib):
    g = gold("hand_ffn_d1_h1.json")
    for c in g["cases"]:
        y = oracle_lib.expert_ffn(bf16_bits([c["x"]]), bf16_bits([[c["w1"]]]),
                                  bf16_bits([[c["w3"]]]), bf16_bits([[c["w2"]]]))
        assert int(y[0]) == int(c["y_bits"], 16)
        # h is recoverable with w2 = 1
        y1 = oracle_lib.expert_ffn(bf16_bits([c["x"]]), bf16_bits([[c["w1"]]]),
                                   bf16_bits([[c["w3"]]]), bf16_bits([[1.0]]))
        assert f32_of_bits(y1[0]) == c["h_bf16"]


def test_ffn_structure_identity_shift_permutation(oracle_lib):
    # W1 = I, W3 = shift (row h reads channel h+1), W2 = permutation P.
    # Then y_o = bf16(silu(x_p) * x_{p+1}) with p = perm[o].  A transposed W3
    # (reading h-1) or W2 (inverse permutation) breaks it.
    d = 8
    rng = np.random.default_rng(15)
    xv = bf16_bits(rng.standard_normal(d).astype(np.float32))
    xf = oracle_lib.bf16_bits_to_f32(xv).astype(np.float64)
    I = np.eye(d, dtype=np.float32)
    shift = np.zeros((d, d), np.float32)
    for h in range(d - 1):
        shift[h, h + 1] = 1.0
    perm = rng.permutation(d)
    P = np.zeros((d, d), np.float32)
    for o in range(d):
        P[o, perm[o]] = 1.0
    y = oracle_lib.expert_ffn(xv, bf16_bits(I), bf16_bits(shift), bf16_bits(P))
    silu = torch.nn.functional.silu(torch.from_numpy(xf)).numpy()  # library SiLU
    hb = np.array([oracle_lib.f64_to_bf16(silu[h] * (xf[h + 1] if h + 1 < d else 0.0))
                   for h in range(d)], np.uint16)
    assert np.array_equal(y, hb[perm])


def test_ffn_matches_fp64_matmul(oracle_lib):
    rng = np.random.default_rng(16)
    d, H = 64, 32
    x = bf16_bits(rng.standard_normal(d).astype(np.float32))
    w1 = bf16_bits((rng.standard_normal((H, d)) * 0.1).astype(np.float32))
    w3 = bf16_bits((rng.standard_normal((H, d)) * 0.1).astype(np.float32))
    w2 = bf16_bits((rng.standard_normal((d, H)) * 0.1).astype(np.float32))
    f = oracle_lib.bf16_bits_to_f32
    xf, W1, W3, W2 = (f(a).astype(np.float64) for a in (x, w1, w3, w2))
    a, b = W1 @ xf, W3 @ xf
    h = np.array([f(np.array([oracle_lib.f64_to_bf16(v)], np.uint16))[0]
                  for v in a / (1 + np.exp(-a)) * b], np.float64)
    ref = np.array([oracle_lib.f64_to_bf16(v) for v in W2 @ h], np.uint16)
    got = oracle_lib.expert_ffn(x, w1, w3, w2)
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------- combine / layer

def _mini_params(d=64, E=8, k=2, H=64, Hs=64, seed=17, T=48):
    rng = np.random.default_rng(seed)
    x = bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    p = {
        "w_router": (rng.standard_normal((d, E)) * 0.1).astype(np.float32),
        "bias": rng.uniform(-0.05, 0.05, E).astype(np.float32),
        "w1": bf16_bits((rng.standard_normal((E, H, d)) * 0.05).astype(np.float32)),
        "w3": bf16_bits((rng.standard_normal((E, H, d)) * 0.05).astype(np.float32)),
        "w2": bf16_bits((rng.standard_normal((E, d, H)) * 0.05).astype(np.float32)),
    }
    if Hs:
        p["ws1"] = bf16_bits((rng.standard_normal((Hs, d)) * 0.05).astype(np.float32))
        p["ws3"] = bf16_bits((rng.standard_normal((Hs, d)) * 0.05).astype(np.float32))
        p["ws2"] = bf16_bits((rng.standard_normal((d, Hs)) * 0.05).astype(np.float32))
    return x, p


@pytest.mark.parametrize("E,k,Hs", [(8, 2, 64), (16, 4, 64), (8, 2, 0), (6, 6, 64)])
def test_dense_masked_equals_sparse(oracle_lib, E, k, Hs):
    """The pages' dense formulation (every expert on every token, unchosen ones
    weighted by zero) gives bit for bit the sparse layer."""
    x, p = _mini_params(E=E, k=k, Hs=Hs)
    res = oracle_lib.bf16_bits_to_f32(x)  # also exercise the residual input
    resb = x
    sp = oracle_lib.layer(x, p, k, residual=resb)
    dn = oracle_lib.dense_masked(x, sp["gate"], sp["idx"], p["w1"], p["w3"], p["w2"],
                                 p.get("ws1"), p.get("ws3"), p.get("ws2"), residual=resb)
    assert np.array_equal(sp["out"], dn)
    assert res.shape == x.shape


def test_combine_closed_forms(oracle_lib):
    # zero expert weights: the layer returns the residual unchanged
    x, p = _mini_params()
    for name in ("w2", "ws2"):
        p[name] = np.zeros_like(p[name])
    out = oracle_lib.layer(x, p, 2, residual=x)["out"]
    assert np.array_equal(out, x)
    # without residual and shared expert, one chosen expert with gate 1 (k = 1)
    # reproduces that expert's output row exactly
    x, p = _mini_params(Hs=0)
    r = oracle_lib.layer(x, p, 1)
    for t in range(x.shape[0]):
        e = r["idx"][t, 0]
        y = oracle_lib.expert_ffn(x[t], p["w1"][e], p["w3"][e], p["w2"][e])
        assert np.array_equal(r["out"][t], y)


def test_small_config_shape(oracle_lib):
    # the pages' small configuration: 8 experts, 2 chosen per token
    x, p = _mini_params(E=8, k=2, T=128)
    r = oracle_lib.layer(x, p, 2, seq_len=64)
    assert r["idx"].shape == (128, 2) and r["counts"].sum() == 256
    assert r["seq_balance"].shape == (2,)


# ---------------------------------------------------------------- bias update

def test_bias_update_closed_form(oracle_lib):
    g = gold("bias_update_closed_form.json")
    b_in = np.array(g["bias_in"], np.float32)
    b = oracle_lib.update_bias(np.array(g["counts"], np.int32), b_in, g["T"], g["k"], g["gamma"])
    gam = np.float32(g["gamma"])
    want = np.array([np.float32(bi + np.float32(gam * np.float32(s)))
                     for bi, s in zip(b_in, g["direction"])], np.float32)
    assert np.array_equal(b, want)
    assert b[1] == b_in[1] and b[3] == b_in[3]
    assert b[0] == -gam and b[2] == np.float32(-0.25 + gam)


def test_bias_update_balanced_is_noop(oracle_lib):
    b = np.linspace(-0.3, 0.3, 16).astype(np.float32)
    out = oracle_lib.update_bias(np.full(16, 128, np.int32), b, 512, 4)
    assert np.array_equal(out, b)


# ---------------------------------------------------------------- RMSNorm

def test_rmsnorm_hand_example(oracle_lib):
    g = gold("hand_rmsnorm_d4.json")
    out = oracle_lib.rmsnorm(bf16_bits([g["x"]]), np.array(g["gain"], np.float32), g["eps"])
    assert out[0].tolist() == g["out_bits"]


def test_rmsnorm_constant_rows_give_the_gain(oracle_lib):
    # a constant row c has rms |c|: each output is sign(c) * g_i exactly
    d = 64
    gain = np.array([0.5, 2.0, -1.0, 1.5] * (d // 4), np.float32)
    x = bf16_bits([[3.0] * d, [-0.25] * d, [1e-3] * d])
    out = oracle_lib.bf16_bits_to_f32(oracle_lib.rmsnorm(x, gain, 0.0))
    assert np.array_equal(out[0], gain)
    assert np.array_equal(out[1], -gain)
    assert np.array_equal(out[2], gain)


def test_rmsnorm_scale_invariance_and_gain_index(oracle_lib):
    rng = np.random.default_rng(7)
    T, d = 9, 384
    xf = rng.standard_normal((T, d)).astype(np.float32)
    x = bf16_bits(xf)
    ones = np.ones(d, np.float32)
    base = oracle_lib.rmsnorm(x, ones, 0.0)
    # scaling a row by a power of two changes nothing (eps = 0)
    x8 = bf16_bits(oracle_lib.bf16_bits_to_f32(x) * 8.0)
    assert np.array_equal(oracle_lib.rmsnorm(x8, ones, 0.0), base)
    # a power-of-two gain per column scales exactly that column
    gain = (2.0 ** (np.arange(d) % 3 - 1)).astype(np.float32)
    scaled = oracle_lib.bf16_bits_to_f32(oracle_lib.rmsnorm(x, gain, 0.0))
    assert np.array_equal(scaled, oracle_lib.bf16_bits_to_f32(base) * gain)
    # rows are independent: permuting rows permutes the outputs
    perm = rng.permutation(T)
    assert np.array_equal(oracle_lib.rmsnorm(x[perm], ones, 0.0), base[perm])
    # the output's mean square is 1 within one bf16 rounding per element
    o = oracle_lib.bf16_bits_to_f32(base).astype(np.float64)
    assert np.all(np.abs((o ** 2).mean(axis=1) - 1.0) < 2 * 2.0 ** -8)


def test_rmsnorm_eps_and_zero_row(oracle_lib):
    d = 128
    x = bf16_bits([[0.0] * d, [1e-4] * d])
    out = oracle_lib.bf16_bits_to_f32(oracle_lib.rmsnorm(x, np.ones(d, np.float32), 1e-6))
    assert np.all(out[0] == 0.0)  # no NaN from 0/0
    # eps enters under the root: 1e-4 / sqrt(1e-8 + 1e-6) = 0.0995037...
    expect = 1e-4 / math.sqrt(1e-8 + 1e-6)
    assert np.all(np.abs(out[1] - expect) <= 2.0 ** -8 * expect)
    assert not np.allclose(out[1], 1.0)  # eps = 0 would give 1


def test_block_with_zero_experts_is_the_residual(oracle_lib):
    """x + MoE(RMSNorm(x)) with every expert weight zero returns x itself: the
    residual is the block's input, not its normalised input."""
    rng = np.random.default_rng(3)
    T, d, E, k, H = 40, 64, 8, 2, 64
    x = bf16_bits(rng.standard_normal((T, d)))
    p = {"norm": (1 + 0.1 * rng.standard_normal(d)).astype(np.float32),
         "w_router": (0.1 * rng.standard_normal((d, E))).astype(np.float32),
         "bias": np.zeros(E, np.float32),
         "w1": np.zeros((E, H, d), np.uint16), "w3": np.zeros((E, H, d), np.uint16),
         "w2": np.zeros((E, d, H), np.uint16), "ws1": np.zeros((H, d), np.uint16),
         "ws3": np.zeros((H, d), np.uint16), "ws2": np.zeros((d, H), np.uint16)}
    r = oracle_lib.block(x, p, k)
    assert np.array_equal(r["out"], x)
    assert np.array_equal(r["xn"], oracle_lib.rmsnorm(x, p["norm"], 1e-6))
    # routing saw the normalised input
    assert np.array_equal(r["idx"], oracle_lib.route(r["xn"], p["w_router"], p["bias"], k)["idx"])


# ---------------------------------------------------------------- backward

def _bwd_case(seed, T=6, d=8, E=4, k=2, H=4, Hs=4, scale=0.5):
    rng = np.random.default_rng(seed)
    p = {"w_router": rng.standard_normal((d, E)) * scale,
         "w1": rng.standard_normal((E, H, d)) * scale, "w3": rng.standard_normal((E, H, d)) * scale,
         "w2": rng.standard_normal((E, d, H)) * scale}
    if Hs:
        p.update({"ws1": rng.standard_normal((Hs, d)) * scale,
                  "ws3": rng.standard_normal((Hs, d)) * scale,
                  "ws2": rng.standard_normal((d, Hs)) * scale})
    x = rng.standard_normal((T, d))
    idx = np.array([rng.permutation(E)[:k] for _ in range(T)], np.int32)
    dout = rng.standard_normal((T, d))
    return p, x, idx, dout


@pytest.mark.parametrize("S,alpha,Hs", [(3, 0.3, 4), (0, 0.0, 4), (6, 1.0, 0)])
def test_backward_matches_finite_differences(oracle_lib, S, alpha, Hs):
    """The exact fp64 gradient against central differences of the fp64 layer
    (choice of experts fixed): every input and weight, with and without the
    balance term and the shared expert."""
    p, x, idx, dout = _bwd_case(11 + S, Hs=Hs)
    g = oracle_lib.layer_backward(x, p, idx, dout, S, alpha, round_storage=False)

    def loss(xx, pp):
        o, lb = oracle_lib.forward_f64(xx, pp, idx, S, alpha)
        return float((dout * o).sum() + lb)

    eps = 1e-6
    for name, key in [("x", "dx"), ("w_router", "dw_router"), ("w1", "dw1"), ("w3", "dw3"),
                      ("w2", "dw2")] + ([("ws1", "dws1"), ("ws3", "dws3"), ("ws2", "dws2")] if Hs else []):
        base = x if name == "x" else p[name]
        num = np.zeros_like(base)
        for ii in np.ndindex(base.shape):
            plus, minus = base.copy(), base.copy()
            plus[ii] += eps
            minus[ii] -= eps
            if name == "x":
                num[ii] = (loss(plus, p) - loss(minus, p)) / (2 * eps)
            else:
                num[ii] = (loss(x, {**p, name: plus}) - loss(x, {**p, name: minus})) / (2 * eps)
        err = np.abs(num - g[key]).max() / max(np.abs(num).max(), 1e-30)
        assert err < 1e-6, (name, err)


def test_backward_unchosen_experts_get_no_gradient(oracle_lib):
    """The pages' dense formulation weights unchosen experts by zero, so their
    weights get exactly zero gradient; chosen ones do not."""
    p, x, idx, dout = _bwd_case(5, T=5, E=6, k=2)
    idx[:] = np.array([0, 3], np.int32)  # experts 1, 2, 4, 5 never chosen
    g = oracle_lib.layer_backward(x, p, idx, dout, 0, 0.0, round_storage=False)
    for key in ("dw1", "dw3", "dw2"):
        for e in (1, 2, 4, 5):
            assert not g[key][e].any(), (key, e)
        for e in (0, 3):
            assert np.abs(g[key][e]).max() > 0, (key, e)


def test_backward_linear_in_dout_and_balance_alone(oracle_lib):
    p, x, idx, dout = _bwd_case(9, T=8, E=4, k=2)
    _, _, _, dout2 = _bwd_case(10, T=8, E=4, k=2)
    a = oracle_lib.layer_backward(x, p, idx, dout, 0, 0.0, round_storage=False)
    b = oracle_lib.layer_backward(x, p, idx, dout2, 0, 0.0, round_storage=False)
    c = oracle_lib.layer_backward(x, p, idx, dout + dout2, 0, 0.0, round_storage=False)
    for key in ("dx", "dw_router", "dw1", "dw2", "dws3"):
        assert np.allclose(c[key], a[key] + b[key], rtol=1e-12, atol=1e-12), key
    # no upstream gradient and no balance term: nothing; with the balance
    # term alone, only the router (and x through it) receives a gradient
    z = oracle_lib.layer_backward(x, p, idx, np.zeros_like(dout), 4, 0.0, round_storage=False)
    assert not any(z[key].any() for key in ("dx", "dw_router", "dw1", "dws2"))
    bal = oracle_lib.layer_backward(x, p, idx, np.zeros_like(dout), 4, 0.5, round_storage=False)
    assert bal["dw_router"].any() and bal["dx"].any()
    assert not any(bal[key].any() for key in ("dw1", "dw3", "dw2", "dws1", "dws3", "dws2"))


def test_backward_forward_f64_is_the_layer(oracle_lib):
    """The fp64 layer the gradient is taken of is the forward oracle without
    its bf16 storage points: on bf16 inputs the two agree within bf16 error."""
    import torch
    rng = np.random.default_rng(21)
    T, d, E, k, H = 64, 64, 8, 2, 64
    xb = bf16_bits(rng.standard_normal((T, d)))
    bf = lambda a: bf16_bits(a)  # noqa: E731
    p = {"w_router": (0.2 * rng.standard_normal((d, E))).astype(np.float32),
         "bias": np.zeros(E, np.float32),
         "w1": bf(0.1 * rng.standard_normal((E, H, d))), "w3": bf(0.1 * rng.standard_normal((E, H, d))),
         "w2": bf(0.1 * rng.standard_normal((E, d, H))), "ws1": bf(0.1 * rng.standard_normal((H, d))),
         "ws3": bf(0.1 * rng.standard_normal((H, d))), "ws2": bf(0.1 * rng.standard_normal((d, H)))}
    ref = oracle_lib.layer(xb, p, k)
    o64, _ = oracle_lib.forward_f64(xb, p, ref["idx"])
    out = oracle_lib.bf16_bits_to_f32(ref["out"]).astype(np.float64)
    assert np.abs(out - o64).max() <= 2e-2 * np.abs(o64).max()
    assert np.linalg.norm(out - o64) / np.linalg.norm(o64) < 1e-2
    # ... and the rounded backward stays within bf16 error of the exact one
    dout = bf16_bits(rng.standard_normal((T, d)))
    g0 = oracle_lib.layer_backward(xb, p, ref["idx"], dout, 0, 0.0, round_storage=False)
    g1 = oracle_lib.layer_backward(xb, p, ref["idx"], dout, 0, 0.0, round_storage=True)
    for key in ("dx", "dw_router", "dw1", "dw2", "dws1"):
        rel = np.linalg.norm(g1[key] - g0[key]) / np.linalg.norm(g0[key])
        assert rel < 2e-2, (key, rel)
