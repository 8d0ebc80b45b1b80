"""Pins of the MLA attention oracle (CPU).  Each is tied to something other
than the oracle's own formula: closed forms of the rotation, torch's
scaled-dot-product attention (a library implementation) on a lossless
latent, a single-token closed form through matrix products, causality, the
decode step continuing a prefill, and the pages' cache figures."""
import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_params(rng, d, nh, dc, dn, dr, dv, scale=0.3):
    return {"w_q": rng.standard_normal((nh * (dn + dr), d)) * scale,
            "w_dkv": rng.standard_normal((dc, d)) * scale,
            "w_kr": rng.standard_normal((dr, d)) * scale,
            "w_uk": rng.standard_normal((nh * dn, dc)) * scale,
            "w_uv": rng.standard_normal((nh * dv, dc)) * scale,
            "w_o": rng.standard_normal((d, nh * dv)) * scale}


def test_cache_numbers_per_token_match_the_pages():
    g = json.load(open(os.path.join(GOLDEN, "mla_cache_size.json")))
    nh, dc, dr = g["heads"], g["latent"], g["rope_key"]
    dn, dv = 32, 32  # the reading: per head a 32 + 16 key and a 32 value
    assert nh * (dn + dr) + nh * dv == g["plain_numbers_per_token"]
    assert dc + dr == g["mla_numbers_per_token"]
    # the oracle's caches hold exactly dc + dr numbers per token
    rng = np.random.default_rng(3)
    p = rand_params(rng, 64, nh, dc, dn, dr, dv, 0.05)
    r = oracle.mla_prefill(rng.standard_normal((2, 64)), p, nh, 1, 2, 2)
    assert r["cache_kv"].shape[-1] + r["cache_kr"].shape[-1] == 144


def test_rope_closed_forms():
    # one pair: the plane rotation by the position (the first angle is 1)
    for pos in (0.0, 1.0, 2.5, 37.0):
        u = oracle.mla_rope([0.3, -1.2], pos)
        c, s = np.cos(pos), np.sin(pos)
        assert np.allclose(u, [0.3 * c + 1.2 * s, 0.3 * s - 1.2 * c], atol=1e-15)
    # pair m turns by pos * 10000^(-2m/16): a hand value for m = 1
    u = oracle.mla_rope([0, 0, 1, 0] + [0] * 12, 1.0)
    ang = 10000.0 ** (-2.0 / 16)
    assert np.allclose(u[2:4], [np.cos(ang), np.sin(ang)], atol=1e-15)
    assert not u[:2].any() and not u[4:].any()
    rng = np.random.default_rng(5)
    a, b = rng.standard_normal(16), rng.standard_normal(16)
    assert np.allclose(oracle.mla_rope(a, 0.0), a, atol=0)               # position 0
    assert np.isclose(np.linalg.norm(oracle.mla_rope(a, 91.0)), np.linalg.norm(a))  # a rotation
    # scores depend on the relative position only
    for m, n in ((7, 3), (200, 196), (4, 0)):
        lhs = oracle.mla_rope(a, m) @ oracle.mla_rope(b, n)
        rhs = oracle.mla_rope(a, m - n) @ b
        assert np.isclose(lhs, rhs, rtol=1e-12, atol=1e-12)


def test_lossless_latent_equals_torch_attention():
    """With the latent as wide as the model and W_dkv = I, MLA is multi-head
    attention with keys [W_uk x, rope(W_kr x)] and values W_uv x, the rotary
    key shared by the heads: torch's scaled_dot_product_attention (causal)
    gives the same output in fp64."""
    rng = np.random.default_rng(7)
    B, S, d, nh, dn, dr, dv = 2, 9, 16, 3, 4, 4, 5
    dc = d
    p = rand_params(rng, d, nh, dc, dn, dr, dv)
    p["w_dkv"] = np.eye(d)
    x = rng.standard_normal((B * S, d))
    res = rng.standard_normal((B * S, d))
    r = oracle.mla_prefill(x, p, nh, B, S, S, residual=res, round_storage=False)
    xs = x.reshape(B, S, d)
    q = np.einsum("bsd,jd->bsj", xs, p["w_q"]).reshape(B, S, nh, dn + dr)
    kr = np.einsum("bsd,jd->bsj", xs, p["w_kr"])
    for b in range(B):
        for s in range(S):
            for h in range(nh):
                q[b, s, h, dn:] = oracle.mla_rope(q[b, s, h, dn:], s)
            kr[b, s] = oracle.mla_rope(kr[b, s], s)
    kn = np.einsum("bsd,jd->bsj", xs, p["w_uk"]).reshape(B, S, nh, dn)
    k = np.concatenate([kn, np.broadcast_to(kr[:, :, None, :], (B, S, nh, dr))], axis=-1)
    v = np.einsum("bsd,jd->bsj", xs, p["w_uv"]).reshape(B, S, nh, dv)
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(a.transpose(0, 2, 1, 3))) for a in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True,
                                                         scale=1.0 / np.sqrt(dn + dr))
    o = o.numpy().transpose(0, 2, 1, 3).reshape(B * S, nh * dv)
    ref = res + o @ p["w_o"].T
    assert np.allclose(r["out"], ref, rtol=1e-10, atol=1e-10)
    # the caches: the latent is x itself, the rotary key rotated
    assert np.allclose(r["cache_kv"].reshape(B * S, d), x, atol=0)
    assert np.allclose(r["cache_kr"].reshape(B * S, dr), kr.reshape(B * S, dr), atol=1e-12)


def test_single_token_attends_to_itself_only():
    """A one-token sequence puts all attention on itself: the output is
    r + W_o W_uv W_dkv x (matrix products), whatever the queries and keys."""
    rng = np.random.default_rng(11)
    d, nh, dc, dn, dr, dv = 24, 3, 8, 4, 4, 6
    p = rand_params(rng, d, nh, dc, dn, dr, dv)
    x = rng.standard_normal((5, d))
    res = rng.standard_normal((5, d))
    r = oracle.mla_prefill(x, p, nh, 5, 1, 1, residual=res, round_storage=False)
    ref = res + x @ p["w_dkv"].T @ p["w_uv"].T @ p["w_o"].T
    assert np.allclose(r["out"], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("round_storage", [False, True])
def test_causal_prefix_and_decode_continue_prefill(round_storage):
    rng = np.random.default_rng(13)
    B, S, L, d, nh, dc, dn, dr, dv = 3, 7, 10, 32, 2, 16, 8, 4, 8
    p = rand_params(rng, d, nh, dc, dn, dr, dv, 0.2)
    if round_storage:
        p = {k: oracle.bf16_bits_to_f32(np.vectorize(oracle.f64_to_bf16)(v).astype(np.uint16))
             for k, v in p.items()}
    x = rng.standard_normal((B * S, d))
    full = oracle.mla_prefill(x, p, nh, B, S, L, round_storage=round_storage)
    # causality: changing the last token changes no earlier output
    x2 = x.copy().reshape(B, S, d)
    x2[:, -1] += 1.0
    alt = oracle.mla_prefill(x2.reshape(B * S, d), p, nh, B, S, L, round_storage=round_storage)
    o1, o2 = full["out"].reshape(B, S, d), alt["out"].reshape(B, S, d)
    assert np.array_equal(o1[:, :-1], o2[:, :-1])
    assert not np.array_equal(o1[:, -1], o2[:, -1])
    # prefill of S-1 tokens, then the last token decoded: the same row and caches
    head = oracle.mla_prefill(x.reshape(B, S, d)[:, :-1].reshape(-1, d), p, nh, B, S - 1, L,
                              round_storage=round_storage)
    dec = oracle.mla_decode(x.reshape(B, S, d)[:, -1], p, nh, np.full(B, S - 1), head["cache_kv"],
                            head["cache_kr"], round_storage=round_storage)
    assert np.array_equal(dec["out"], o1[:, -1])
    assert np.array_equal(dec["cache_kv"], full["cache_kv"])
    assert np.array_equal(dec["cache_kr"], full["cache_kr"])
