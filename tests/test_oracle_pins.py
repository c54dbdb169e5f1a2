"""Pins of the CPU oracle to what the pages and the mathematics fix (no GPU).

Each test checks the oracle against something other than itself: numbers printed on
the pages (tests/golden/k2_page_counts.json), closed forms, brute force on tiny inputs,
library routines (scipy's expit, torch's silu / rms_norm / linear, numpy's stable
argsort and bincount) and invariants stated on the pages.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import expit

import oracle
from oracle import moe_oracle as mo

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "k2_page_counts.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _bf16_round(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def _layer(rng, T=24, d=32, E=12, I=16, Is=16, k=3, bias_scale=0.01, bf16=True):
    x = rng.standard_normal((T, d))
    w_r = rng.standard_normal((E, d)) / math.sqrt(d)
    b = rng.uniform(-bias_scale, bias_scale, E).astype(np.float32)
    w1 = rng.standard_normal((E, I, d)) / math.sqrt(d)
    w3 = rng.standard_normal((E, I, d)) / math.sqrt(d)
    w2 = rng.standard_normal((E, d, I)) / math.sqrt(I)
    ws1 = rng.standard_normal((Is, d)) / math.sqrt(d)
    ws3 = rng.standard_normal((Is, d)) / math.sqrt(d)
    ws2 = rng.standard_normal((d, Is)) / math.sqrt(Is)
    if bf16:
        x, w1, w3, w2, ws1, ws3, ws2 = map(_bf16_round, (x, w1, w3, w2, ws1, ws3, ws2))
    w_r = w_r.astype(np.float32)
    return dict(x=x, w_r=w_r, b=b, w1=w1, w3=w3, w2=w2, ws1=ws1, ws3=ws3, ws2=ws2, top_k=k)


# --------------------------------------------------------------------- page numbers
def test_param_count_matches_k2_page():
    g = _golden()
    cfg = g["k2_config"]["value"]
    n = oracle.moe_param_count(d_model=cfg["hidden_size"], n_experts=cfg["n_routed_experts"],
                               d_expert=cfg["moe_intermediate_size"],
                               d_shared=cfg["moe_intermediate_size"],
                               n_shared=cfg["n_shared_experts"])
    assert n == g["moe_params_per_block"]["value"]
    block = n + 2 * g["moe_block_rmsnorm_params"]["value"] + g["mla_params"]["value"]
    assert block == g["block_params"]["value"]
    assert block * g["n_moe_blocks"]["value"] == g["all_moe_blocks_params"]["value"]


def test_param_count_discriminates_shape_mistakes():
    # a transposed or dropped array would change the count: check a few wrong variants
    good = oracle.moe_param_count(d_model=7168, n_experts=384, d_expert=2048, d_shared=2048)
    assert oracle.moe_param_count(d_model=7168, n_experts=384, d_expert=2048, d_shared=2048,
                                  n_shared=0) != good
    assert oracle.moe_param_count(d_model=7168, n_experts=385, d_expert=2048, d_shared=2048) != good


def test_latent_up_projection_count():
    g = _golden()
    # the latent up-projection is [out=7168, in=3584] as synth/oracle store it
    assert 7168 * 3584 == g["latent_up_proj_params"]["value"]


# --------------------------------------------------------------------- primitives
def test_sigmoid_and_silu_against_library():
    v = np.linspace(-40, 40, 2001)
    np.testing.assert_allclose(oracle.sigmoid(v), expit(v), rtol=1e-15, atol=0)
    t = torch.from_numpy(v)
    np.testing.assert_allclose(oracle.silu(v), torch.nn.functional.silu(t).numpy(), rtol=1e-14, atol=1e-300)
    assert oracle.sigmoid(np.array([0.0]))[0] == 0.5
    assert oracle.silu(np.array([0.0]))[0] == 0.0


def test_rmsnorm_against_torch():
    rng = np.random.default_rng(1)
    u = rng.standard_normal((5, 37))
    ref = torch.nn.functional.rms_norm(torch.from_numpy(u), (37,), eps=1e-6).numpy()
    np.testing.assert_allclose(oracle.rmsnorm(u, 1e-6), ref, rtol=1e-13)


def test_swiglu_is_textbook_mlp():
    rng = np.random.default_rng(2)
    L = _layer(rng)
    x = torch.from_numpy(L["x"])
    F = torch.nn.functional
    ref = F.linear(F.silu(F.linear(x, torch.from_numpy(L["ws1"]))) * F.linear(x, torch.from_numpy(L["ws3"])),
                   torch.from_numpy(L["ws2"])).numpy()
    np.testing.assert_allclose(oracle.swiglu(L["x"], L["ws1"], L["ws3"], L["ws2"]), ref, rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------------------- router
def test_gates_invariants():
    rng = np.random.default_rng(3)
    L = _layer(rng, T=200, E=40, k=8)
    r = oracle.route(L["x"], L["w_r"], L["b"], 8)
    idx, G = r["topk_idx"], r["topk_w"]
    assert idx.shape == (200, 8) and G.shape == (200, 8)
    for t in range(200):
        assert len(set(idx[t].tolist())) == 8             # exactly k distinct experts
    assert np.all(G > 0)
    np.testing.assert_allclose(G.sum(axis=1), 2.827, rtol=0, atol=1e-12)
    Gd = oracle.gate_matrix(idx, G, 40)
    assert np.all((Gd != 0).sum(axis=1) == 8)              # k nonzero gates per token
    # gates are proportional to the unbiased sigmoid of the chosen experts
    s_sel = np.take_along_axis(expit(L["x"] @ L["w_r"].astype(np.float64).T), idx.astype(np.int64), axis=1)
    ratio = G / s_sel
    np.testing.assert_allclose(ratio, ratio[:, :1].repeat(8, axis=1), rtol=1e-12)


def test_topk_brute_force_e16_k2():
    rng = np.random.default_rng(4)
    L = _layer(rng, T=64, d=256, E=16, k=2, bias_scale=0.05)
    r = oracle.route(L["x"], L["w_r"], L["b"], 2)
    sc = r["score"]
    for t in range(64):
        best = max(itertools.combinations(range(16), 2), key=lambda p: (sc[t, p[0]] + sc[t, p[1]], [-p[0], -p[1]]))
        assert set(r["topk_idx"][t].tolist()) == set(best)
        # order: descending score
        a, b_ = r["topk_idx"][t]
        assert sc[t, a] >= sc[t, b_]


def test_topk_brute_force_e10_k3():
    rng = np.random.default_rng(5)
    L = _layer(rng, T=40, d=16, E=10, k=3, bias_scale=0.1)
    r = oracle.route(L["x"], L["w_r"], L["b"], 3)
    sc = r["score"]
    for t in range(40):
        best = max(itertools.combinations(range(10), 3), key=lambda p: sum(sc[t, list(p)]))
        assert set(r["topk_idx"][t].tolist()) == set(best)


def _one_hot_router(zs, b):
    """x = e_0 and W_r[:, 0] = z, so the logits are exactly the given z."""
    E = len(zs)
    x = np.zeros((1, 4))
    x[0, 0] = 1.0
    w_r = np.zeros((E, 4), dtype=np.float32)
    w_r[:, 0] = zs
    return x, w_r, np.asarray(b, dtype=np.float32)


def test_bias_is_added_to_sigmoid_not_logit():
    # sigma(z0) + b0 = 0.5 + 0.3 = 0.8 > sigma(z1) + b1 = 0.622, but z0 + b0 = 0.3 < z1 + b1 = 0.5
    x, w_r, b = _one_hot_router([0.0, 0.5], [0.3, 0.0])
    r = oracle.route(x, w_r, b, 1)
    assert r["topk_idx"][0, 0] == 0


def test_bias_not_in_gates():
    x, w_r, b = _one_hot_router([1.0, -1.0, 0.25, 2.0], [0.0, 5.0, 0.0, 0.0])
    r = oracle.route(x, w_r, b, 2)
    assert set(r["topk_idx"][0].tolist()) == {1, 3}     # expert 1 only through its bias
    s = expit(np.array([1.0, -1.0, 0.25, 2.0]))
    want = {1: 2.827 * s[1] / (s[1] + s[3]), 3: 2.827 * s[3] / (s[1] + s[3])}
    for j in range(2):
        e = int(r["topk_idx"][0, j])
        assert r["topk_w"][0, j] == pytest.approx(want[e], rel=1e-7)
    # with the bias folded in, the gate of expert 1 would be far larger
    assert want[1] < 2.827 * (s[1] + 5.0) / (s[1] + 5.0 + s[3]) - 0.5


def test_tie_break_lower_index():
    x, w_r, b = _one_hot_router([0.1, 0.7, 0.7, 0.2], [0.0, 0.0, 0.0, 0.0])
    r = oracle.route(x, w_r, b, 1)
    assert r["topk_idx"][0, 0] == 1 and r["gap"][0] == 0.0
    r = oracle.route(x, w_r, b, 2)
    assert r["topk_idx"][0].tolist() == [1, 2]


def test_zero_bias_selects_topk_logits():
    rng = np.random.default_rng(6)
    L = _layer(rng, T=50, d=64, E=20, k=4, bias_scale=0.0)
    b = np.zeros(20, dtype=np.float32)
    r = oracle.route(L["x"], L["w_r"], b, 4)
    z = L["x"] @ L["w_r"].astype(np.float64).T
    want = np.argsort(-z, axis=1, kind="stable")[:, :4]
    for t in range(50):
        if r["gap"][t] > 1e-6:
            assert set(r["topk_idx"][t].tolist()) == set(want[t].tolist())


def test_k_equals_e_selects_all():
    rng = np.random.default_rng(7)
    L = _layer(rng, T=10, d=16, E=6, k=6)
    r = oracle.route(L["x"], L["w_r"], L["b"], 6)
    s = expit(L["x"] @ L["w_r"].astype(np.float64).T)
    Gd = oracle.gate_matrix(r["topk_idx"], r["topk_w"], 6)
    np.testing.assert_allclose(Gd, 2.827 * s / s.sum(axis=1, keepdims=True), rtol=1e-13)
    assert np.all(np.isinf(r["gap"]))


# ------------------------------------------------------------------------ permute
def test_permute_against_library_sort():
    rng = np.random.default_rng(8)
    T, k, E = 300, 8, 50
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    counts, offsets, perm, inv = oracle.permute(idx, E)
    flat = idx.reshape(-1)
    np.testing.assert_array_equal(counts, np.bincount(flat, minlength=E))
    np.testing.assert_array_equal(offsets, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
    np.testing.assert_array_equal(perm, np.argsort(flat, kind="stable"))
    assert counts.sum() == T * k and offsets[-1] == T * k
    np.testing.assert_array_equal(perm[inv], np.arange(T * k))       # inv is perm's inverse
    for e in range(E):
        seg = perm[offsets[e]:offsets[e + 1]]
        assert np.all(flat[seg] == e)                                  # segment e holds expert e
        assert np.all(np.diff(seg) > 0)                                 # token ascending


def test_permute_empty_experts_and_single_expert():
    idx = np.array([[3], [3], [3]], dtype=np.int32)
    counts, offsets, perm, inv = oracle.permute(idx, 5)
    assert counts.tolist() == [0, 0, 0, 3, 0]
    assert offsets.tolist() == [0, 0, 0, 0, 3, 3]
    assert perm.tolist() == [0, 1, 2] and inv.tolist() == [0, 1, 2]


# ----------------------------------------------------------------------- forward
def _run(L, fn, **kw):
    args = dict(L)
    args.update(kw)
    k = args.pop("top_k")
    if fn == "dense":
        return oracle.moe_dense(args["x"], args["w_r"], args["b"], args["w1"], args["w3"], args["w2"],
                                args["ws1"], args["ws3"], args["ws2"], k, args.get("alpha", 2.827))
    return oracle.moe_sparse(args["x"], args["w_r"], args["b"], k, args.get("alpha", 2.827),
                             w1=args["w1"], w3=args["w3"], w2=args["w2"],
                             shared=(args["ws1"], args["ws3"], args["ws2"]), tokens=kw.get("tokens"))


def test_dense_equals_sparse():
    rng = np.random.default_rng(9)
    L = _layer(rng, T=64, d=64, E=16, I=32, Is=32, k=2)
    dn = _run(L, "dense")
    sp = _run(L, "sparse")
    np.testing.assert_allclose(sp["y_routed"], dn["y_routed"], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(sp["out"], dn["out"], rtol=1e-12, atol=1e-13)
    assert np.abs(dn["y_routed"]).max() > 0.1


def test_sparse_token_subset_matches_full():
    rng = np.random.default_rng(10)
    L = _layer(rng, T=40, d=32, E=12, k=3)
    full = _run(L, "sparse")
    sub = _run(L, "sparse", tokens=[3, 17, 39])
    np.testing.assert_allclose(sub["out"], full["out"][[3, 17, 39]], rtol=1e-13, atol=1e-14)


def test_shared_only_when_routed_weights_vanish():
    rng = np.random.default_rng(11)
    L = _layer(rng)
    r0 = _run(L, "dense", alpha=0.0)
    assert np.array_equal(r0["out"], r0["y_shared"])
    L2 = dict(L, w2=np.zeros_like(L["w2"]))
    r1 = _run(L2, "sparse")
    assert np.array_equal(r1["out"], r1["y_shared"])


def test_single_expert_closed_form():
    rng = np.random.default_rng(12)
    L = _layer(rng, T=7, d=16, E=1, I=8, Is=8, k=1)
    r = _run(L, "dense")
    np.testing.assert_allclose(r["topk_w"], 2.827, rtol=1e-15)
    F = torch.nn.functional
    x = torch.from_numpy(L["x"])

    def mlp(w1, w3, w2):
        return F.linear(F.silu(F.linear(x, torch.from_numpy(w1))) * F.linear(x, torch.from_numpy(w3)),
                        torch.from_numpy(w2)).numpy()
    want = 2.827 * mlp(L["w1"][0], L["w3"][0], L["w2"][0]) + mlp(L["ws1"], L["ws3"], L["ws2"])
    np.testing.assert_allclose(r["out"], want, rtol=1e-12, atol=1e-13)


def test_scalar_closed_form():
    # d = I = Is = 1, E = 1, k = 1: out = 2.827 * w2 * silu(w1 x) * (w3 x) + shared term
    x = np.array([[0.75]])
    L = dict(x=x, w_r=np.array([[0.3]], dtype=np.float32), b=np.array([0.0], dtype=np.float32),
             w1=np.array([[[1.5]]]), w3=np.array([[[-0.5]]]), w2=np.array([[[2.0]]]),
             ws1=np.array([[0.25]]), ws3=np.array([[4.0]]), ws2=np.array([[-1.0]]), top_k=1)

    def silu(v):
        return v / (1.0 + math.exp(-v))
    want = 2.827 * 2.0 * silu(1.5 * 0.75) * (-0.5 * 0.75) + (-1.0) * silu(0.25 * 0.75) * (4.0 * 0.75)
    for fn in ("dense", "sparse"):
        assert _run(L, fn)["out"][0, 0] == pytest.approx(want, rel=1e-14)


def test_latent_reduces_to_normalised_k2_layer():
    # with W_down = W_up = identity the latent layer is RMSNorm(y_routed) + y_shared
    rng = np.random.default_rng(13)
    L = _layer(rng, T=20, d=32, E=8, I=16, Is=16, k=2)
    eye = np.eye(32)
    lat = oracle.moe_latent(L["x"], L["w_r"], L["b"], eye, L["w1"], L["w3"], L["w2"], eye,
                            L["ws1"], L["ws3"], L["ws2"], 2)
    sp = _run(L, "sparse")
    ref = torch.nn.functional.rms_norm(torch.from_numpy(sp["y_routed"]), (32,), eps=1e-6).numpy()
    np.testing.assert_allclose(lat["y_routed"], ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lat["out"], ref + sp["y_shared"], rtol=1e-12, atol=1e-13)


def _latent_layer(rng, T=12, d=32, Lw=24, E=8, I=16, k=2):
    """A latent layer with non-square, non-orthogonal projections: W_down [Lw, d] and
    W_up [d, Lw] (Lw != d), experts on the latent width, shared expert on the full width."""
    base = _layer(rng, T=T, d=d, E=E, I=I, Is=I, k=k)
    base["w_down"] = _bf16_round(rng.standard_normal((Lw, d)) / math.sqrt(d) * 1.7 + 0.05)
    base["w_up"] = _bf16_round(rng.standard_normal((d, Lw)) / math.sqrt(Lw) * 0.6 - 0.03)
    base["w1"] = _bf16_round(rng.standard_normal((E, I, Lw)) / math.sqrt(Lw))
    base["w3"] = _bf16_round(rng.standard_normal((E, I, Lw)) / math.sqrt(Lw))
    base["w2"] = _bf16_round(rng.standard_normal((E, Lw, I)) / math.sqrt(I))
    return base


def _latent_torch_reference(L, eps=1e-6, alpha=2.827):
    """The latent forward written with torch's functional ops, token by token: the router
    picks on the full-width x; the chosen experts run on l = x W_down^T; their gate-weighted
    sum is RMS-normalised on the latent width FIRST and projected up SECOND; the shared
    expert runs on the full-width x ("Kimi K3 · Latent up-projection", the printed forward:
    the routed-expert norm is applied before the routed-expert up-projection)."""
    F = torch.nn.functional
    t64 = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))  # noqa: E731
    x = t64(L["x"])
    r = oracle.route(L["x"], L["w_r"], L["b"], L["top_k"], alpha)   # routing pinned elsewhere
    lat = F.linear(x, t64(L["w_down"]))
    rows = []
    for t in range(x.shape[0]):
        acc = torch.zeros(lat.shape[1], dtype=torch.float64)
        for j in range(L["top_k"]):
            e = int(r["topk_idx"][t, j])
            h = F.silu(F.linear(lat[t], t64(L["w1"][e]))) * F.linear(lat[t], t64(L["w3"][e]))
            acc = acc + float(r["topk_w"][t, j]) * F.linear(h, t64(L["w2"][e]))
        rows.append(acc)
    y_lat = torch.stack(rows)
    u_hat = F.rms_norm(y_lat, (y_lat.shape[1],), eps=eps)
    shared = F.linear(F.silu(F.linear(x, t64(L["ws1"]))) * F.linear(x, t64(L["ws3"])),
                      t64(L["ws2"]))
    return (F.linear(u_hat, t64(L["w_up"])) + shared).numpy()


def _latent_of(L, fn=None):
    fn = fn or oracle.moe_latent
    return fn(L["x"], L["w_r"], L["b"], L["w_down"], L["w1"], L["w3"], L["w2"], L["w_up"],
              L["ws1"], L["ws3"], L["ws2"], L["top_k"])["out"]


def test_latent_norm_before_up_projection_against_torch():
    """Non-square W_down / W_up: the oracle's latent layer equals the torch composition in
    the page's order (route on x, project down, experts, weighted sum, RMSNorm on the
    latent, project up, add the shared expert on x)."""
    L = _latent_layer(np.random.default_rng(31))
    np.testing.assert_allclose(_latent_of(L), _latent_torch_reference(L), rtol=1e-11, atol=1e-12)


def _latent_norm_after_up(x, w_r, b, w_down, w1, w3, w2, w_up, ws1, ws3, ws2, top_k,
                          alpha=2.827, eps=1e-6):
    """A plausible mistake: the same pieces with the RMSNorm applied after the
    up-projection (on the model width) instead of before it (on the latent width)."""
    r = mo.route(x, w_r, b, top_k, alpha)
    lat = np.asarray(x, dtype=np.float64) @ np.asarray(w_down, dtype=np.float64).T
    sp = mo.moe_sparse(lat, w_r, b, top_k, alpha, w1=w1, w3=w3, w2=w2, shared=None, routing=r)
    y = mo.rmsnorm(sp["y_routed"] @ np.asarray(w_up, dtype=np.float64).T, eps)
    return dict(out=y + mo.swiglu(x, ws1, ws3, ws2))


def test_latent_pin_catches_norm_after_up_projection():
    """The swapped order is caught by the non-square pin above.  With identity
    projections the two orders agree, so the identity pin alone would miss it."""
    L = _latent_layer(np.random.default_rng(31))
    want = _latent_torch_reference(L)
    swapped = _latent_of(L, _latent_norm_after_up)
    assert np.abs(swapped - want).max() > 1e-2 * np.abs(want).max()
    # the same swap on square identity projections is invisible
    Li = _layer(np.random.default_rng(13), T=20, d=32, E=8, I=16, Is=16, k=2)
    Li["w_down"] = Li["w_up"] = np.eye(32)
    np.testing.assert_allclose(_latent_of(Li, _latent_norm_after_up), _latent_of(Li),
                               rtol=1e-12, atol=1e-13)


def test_a_planted_mistake_is_caught(monkeypatch):
    """Plant a mistake in the oracle (on the CPU) and check the pins notice it."""
    rng = np.random.default_rng(14)
    L = _layer(rng, T=16, d=16, E=1, I=8, Is=8, k=1)
    good = _run(L, "dense")["out"]
    monkeypatch.setattr(mo, "silu", lambda v: np.asarray(v, dtype=np.float64) * mo.sigmoid(-np.asarray(v)))
    bad = _run(L, "dense")["out"]
    assert not np.allclose(good, bad)


# ------------------------------------------------- block: pre-MoE norm and residual
def test_rmsnorm_with_gain_against_torch():
    rng = np.random.default_rng(15)
    u = rng.standard_normal((9, 48)) * 3.0
    g = rng.uniform(0.5, 1.5, 48)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(u), (48,), weight=torch.from_numpy(g),
                                       eps=1e-6).numpy()
    np.testing.assert_allclose(oracle.rmsnorm(u, 1e-6, g), ref, rtol=1e-13)


def test_rmsnorm_closed_forms():
    # a constant row c gives c / sqrt(c^2 + eps) times the gain
    g = np.linspace(0.25, 2.0, 16)
    for c in (0.5, -3.0, 1e-4):
        np.testing.assert_allclose(oracle.rmsnorm(np.full((1, 16), c), 1e-6, g)[0],
                                   c / math.sqrt(c * c + 1e-6) * g, rtol=1e-14)
    # eps = 0, unit gain: the output has mean square 1 and ignores a positive scale
    u = np.random.default_rng(16).standard_normal((5, 64))
    v = oracle.rmsnorm(u, 0.0)
    np.testing.assert_allclose(np.mean(v * v, axis=1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(oracle.rmsnorm(7.5 * u, 0.0), v, rtol=1e-14)


def test_round_bf16_against_torch_and_ties():
    rng = np.random.default_rng(17)
    v = (rng.standard_normal(200_000) * np.exp(rng.uniform(-90, 80, 200_000))).astype(np.float32)
    v = np.concatenate([v, np.float32([1e-40, -3e-42, 0.0, -0.0])])      # fp32 subnormals, zeros
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    got = mo.round_bf16(v)
    assert np.array_equal(got, ref)
    # ties go to the even neighbour on the 2^-7 grid at 1.0
    t = mo.round_bf16(np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 1 + 2.0 ** -8 + 2.0 ** -20]))
    assert list(t) == [1.0, 1 + 2.0 ** -6, -1.0, 1 + 2.0 ** -7]
    s = mo.round_bf16(np.array([np.inf, -np.inf, np.nan]))
    assert s[0] == np.inf and s[1] == -np.inf and np.isnan(s[2])


def test_cut_sig16_against_fp32_bit_masking():
    """cut_sig16 on fp32 values equals clearing the 8 lowest stored mantissa bits of the
    fp32 pattern (what a 24-bit float keeps of it), over normal fp32 values of both signs
    and every magnitude; plus hand cases of the grid at 1.0 (spacing 2^-15)."""
    rng = np.random.default_rng(23)
    v = (rng.standard_normal(200_000) * np.exp(rng.uniform(-80, 80, 200_000))).astype(np.float32)
    v = v[np.abs(v) >= np.finfo(np.float32).tiny]
    masked = (v.view(np.uint32) & np.uint32(0xFFFFFF00)).view(np.float32).astype(np.float64)
    assert np.array_equal(mo.cut_sig16(v.astype(np.float64)), masked)
    t = mo.cut_sig16(np.array([1 + 2.0 ** -15, 1 + 2.0 ** -16, 1 + 2.0 ** -15 + 2.0 ** -16,
                               -(1 + 2.0 ** -16), 2 - 2.0 ** -20, 0.0, -0.0]))
    assert list(t) == [1 + 2.0 ** -15, 1.0, 1 + 2.0 ** -15, -1.0, 2 - 2.0 ** -15, 0.0, 0.0]
    s = mo.cut_sig16(np.array([np.inf, -np.inf, np.nan]))
    assert s[0] == np.inf and s[1] == -np.inf and np.isnan(s[2])


def _block(L, x_res, gain, eps=1e-6, **kw):
    args = dict(w1=L["w1"], w3=L["w3"], w2=L["w2"], ws1=L["ws1"], ws3=L["ws3"], ws2=L["ws2"])
    args.update(kw)
    return mo.moe_block(x_res, gain, L["w_r"], L["b"], top_k=L["top_k"], eps=eps, **args)


def test_block_residual_passes_through_when_experts_vanish():
    rng = np.random.default_rng(18)
    L = _layer(rng, T=12, d=32, E=8, I=16, Is=16, k=2)
    g = rng.uniform(0.5, 1.5, 32)
    blk = _block(L, L["x"], g, w2=np.zeros_like(L["w2"]), ws2=np.zeros_like(L["ws2"]))
    assert np.array_equal(blk["out"], L["x"])
    # the experts and the router read the bf16-rounded normalised input
    xf = blk["x_ffn"]
    ref = torch.nn.functional.rms_norm(torch.from_numpy(L["x"]), (32,), weight=torch.from_numpy(g),
                                       eps=1e-6)
    assert np.array_equal(xf, ref.to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy())
    r = mo.route(xf, L["w_r"], L["b"], 2)
    assert np.array_equal(blk["topk_idx"], r["topk_idx"])


def test_block_zero_gain_routes_by_bias_alone():
    # gain 0: x_ffn = 0, every sigmoid is 1/2, the bias alone picks the experts, the
    # gates are alpha/k each and every expert sees a zero input, so the output is x'_n
    rng = np.random.default_rng(19)
    L = _layer(rng, T=6, d=32, E=8, I=16, Is=16, k=3)
    blk = _block(L, L["x"], np.zeros(32))
    want = np.argsort(-L["b"].astype(np.float64), kind="stable")[:3]
    for t in range(6):
        assert sorted(blk["topk_idx"][t]) == sorted(want)
    np.testing.assert_allclose(blk["topk_w"], 2.827 / 3, rtol=1e-15)
    assert np.array_equal(blk["out"], L["x"])


def test_block_delta_ignores_input_scale_and_gain_scales_x_ffn():
    # with eps = 0 the norm output does not change when x'_n is scaled by a power of two,
    # so Delta_ffn does not either and the output moves by exactly the scaled residual
    rng = np.random.default_rng(20)
    L = _layer(rng, T=10, d=32, E=8, I=16, Is=16, k=2)
    g = rng.uniform(0.5, 1.5, 32)
    a = _block(L, L["x"], g, eps=0.0)
    b = _block(L, 4.0 * L["x"], g, eps=0.0)
    assert np.array_equal(a["x_ffn"], b["x_ffn"])
    np.testing.assert_allclose(b["out"] - 4.0 * L["x"], a["delta"], rtol=0, atol=1e-12)
    assert np.abs(a["delta"]).max() > 0.05
    # doubling the gain doubles x_ffn exactly (bf16 rounding commutes with x2)
    c = _block(L, L["x"], 2.0 * g)
    d = _block(L, L["x"], g)
    assert np.array_equal(c["x_ffn"], 2.0 * d["x_ffn"])


def test_block_token_subset_matches_full():
    rng = np.random.default_rng(21)
    L = _layer(rng, T=20, d=32, E=8, I=16, Is=16, k=2)
    g = rng.uniform(0.5, 1.5, 32)
    full = _block(L, L["x"], g)
    sub = _block(L, L["x"], g, tokens=[0, 7, 19])
    np.testing.assert_allclose(sub["out"], full["out"][[0, 7, 19]], rtol=1e-13, atol=1e-14)


# ------------------------------------------------------ FP8 block-scaled weights (f3)
def test_e4m3_table_against_torch_float8():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = mo.E4M3_TABLE
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.isnan(got).sum() == 2 and np.isnan(got[0x7F]) and np.isnan(got[0xFF])


def test_e4m3_landmarks():
    v = mo.e4m3_value
    assert v(0x7E) == 448.0                      # largest finite: 1.75 x 2^8
    assert v(0x08) == 2.0 ** -6                  # smallest normal
    assert v(0x01) == 2.0 ** -9                  # smallest subnormal
    assert v(0x07) == 7 * 2.0 ** -9              # largest subnormal
    assert v(0x38) == 1.0 and v(0xB8) == -1.0 and v(0x3C) == 1.5
    assert v(0x00) == 0.0 and math.copysign(1.0, v(0x80)) == -1.0


def test_block_dequant_indexes_blocks_by_out_then_in():
    # a 2 x 3 grid of blocks (N = 256, K = 384) with a distinct scale per block and every
    # code 1.0: each weight equals its own block's scale (a transposed block index fails)
    q = np.full((256, 384), 0x38, dtype=np.uint8)
    sc = np.array([[1.0, 2.0, 3.0], [5.0, 7.0, 11.0]])
    w = mo.dequant_fp8_blocks(q, sc)
    for bn in range(2):
        for bk in range(3):
            blk = w[bn * 128:(bn + 1) * 128, bk * 128:(bk + 1) * 128]
            assert np.all(blk == sc[bn, bk])
    # codes are decoded per element: a single -1.5 at (130, 200) gives -1.5 x 7
    q2 = q.copy()
    q2[130, 200] = 0xBC
    assert mo.dequant_fp8_blocks(q2, sc)[130, 200] == -10.5
    # leading (expert) dims broadcast
    w3 = mo.dequant_fp8_blocks(np.stack([q, q2]), np.stack([sc, 2 * sc]))
    assert np.array_equal(w3[1], 2 * mo.dequant_fp8_blocks(q2, sc))
