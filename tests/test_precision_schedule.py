"""The oracle's bf16-points diagnostic mode, and what the HIP path's precision schedule can
hold (no GPU).

The HIP layer rounds the SwiGLU hidden row h to bf16 (the down GEMM's MFMA operand),
keeps each expert's output row with 16 significant bits (its 24-bit rows) and rounds the
layer output once; the sums stay fp32.  moe_sparse(..., bf16_points=KERNEL_BF16_POINTS)
replays that schedule in float64.  It is a diagnostic: it attributes
differences between the GPU and the exact oracle, and it never replaces the exact oracle
as the reference.

Pins: the rounding points against torch's own bf16 casts on a small layer.  Limits: the
replay against the exact oracle on seeded inputs of the shapes the GPU tests use, which
records where the schedule with h rounded once stays inside max |err| <= 2e-2 * RMS(out)
and where it does not (few slots per token, narrow experts: the final rounding and the
rounding of h then leave no margin), and that the two-part h the kernels use on exactly
those shapes brings each back inside.
"""
import math

import numpy as np
import pytest
import torch

import synth_inputs as S
from oracle import moe_oracle as mo

F = torch.nn.functional


def _t(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64))


def _bf(t):
    """torch's round trip through bfloat16 (via float32, as a stored activation)."""
    return t.to(torch.float32).to(torch.bfloat16).to(torch.float64)


def _cut16(t):
    """16 significant bits toward zero, with torch's frexp (the rounding itself is pinned
    against fp32 bit masking in tests/test_oracle_pins.py)."""
    m, e = torch.frexp(t)
    return torch.ldexp(torch.trunc(m * 65536.0) / 65536.0, e)


def _layer(seed, T=40, d=64, E=6, I=32, k=2):
    rng = np.random.default_rng(seed)
    r = lambda *s: rng.standard_normal(s)  # noqa: E731
    return dict(x=r(T, d), w_r=(r(E, d) / math.sqrt(d)).astype(np.float32),
                b=rng.uniform(-0.01, 0.01, E).astype(np.float32),
                w1=r(E, I, d) / math.sqrt(d), w3=r(E, I, d) / math.sqrt(d),
                w2=r(E, d, I) / math.sqrt(I), ws1=r(I, d) / math.sqrt(d),
                ws3=r(I, d) / math.sqrt(d), ws2=r(d, I) / math.sqrt(I), k=k)


def _torch_schedule(L, points):
    """The layer with torch ops, rounding through torch's bf16 cast at `points`."""
    r = mo.route(L["x"], L["w_r"], L["b"], L["k"])
    x = _t(L["x"])

    def mlp(w1, w3, w2):
        h = F.silu(F.linear(x, _t(w1))) * F.linear(x, _t(w3))
        if "h" in points:
            h = _bf(h)
        y = F.linear(h, _t(w2))
        return y

    y_r = torch.zeros(x.shape[0], x.shape[1], dtype=torch.float64)
    for e in range(L["w1"].shape[0]):
        ye = mlp(L["w1"][e], L["w3"][e], L["w2"][e])
        if "expert_out" in points:
            ye = _bf(ye)
        elif "y24" in points:
            ye = _cut16(ye)
        g = torch.zeros(x.shape[0], dtype=torch.float64)
        for j in range(L["k"]):
            hit = torch.from_numpy(r["topk_idx"][:, j] == e)
            g[hit] = torch.from_numpy(r["topk_w"][:, j])[hit]
        y_r = y_r + g[:, None] * ye
    y_s = mlp(L["ws1"], L["ws3"], L["ws2"])
    if "y24" in points:
        y_s = _cut16(y_s)
    if "y_routed" in points:
        y_r = _bf(y_r)
    if "y_shared" in points:
        y_s = _bf(y_s)
    out = y_r + y_s
    if "out" in points:
        out = _bf(out)
    return out.numpy()


def _oracle_schedule(L, points):
    return mo.moe_sparse(L["x"], L["w_r"], L["b"], L["k"], w1=L["w1"], w3=L["w3"], w2=L["w2"],
                         shared=(L["ws1"], L["ws3"], L["ws2"]), bf16_points=points)["out"]


@pytest.mark.parametrize("points", [(), mo.KERNEL_BF16_POINTS, mo.PAGE_BF16_POINTS, ("h",),
                                    ("expert_out",), ("y24",), ("y_routed", "y_shared")])
def test_bf16_points_against_torch_casts(points):
    L = _layer(41)
    got = _oracle_schedule(L, points)
    want = _torch_schedule(L, points)
    if "out" in points:
        # both sides round the same float64 sums (up to summation order, ~1e-16), so they
        # agree exactly or, at a rounding boundary, by one bf16 step
        step = np.ldexp(1.0, np.frexp(np.abs(want))[1] - 8)
        assert np.all(np.abs(got - want) <= step)
        assert np.mean(got == want) > 0.999
    else:
        np.testing.assert_allclose(got, want, rtol=1e-9, atol=1e-12)


def test_bf16_points_change_values_by_rounding_only():
    """Each point perturbs the output by about bf16's unit roundoff, never more."""
    L = _layer(42)
    exact = _oracle_schedule(L, ())
    for pts in (("h",), mo.KERNEL_BF16_POINTS, mo.PAGE_BF16_POINTS):
        d = np.abs(_oracle_schedule(L, pts) - exact)
        assert 0 < d.max() < 2.0 ** -6 * np.abs(exact).max()


def _replay_ratio(cfg, seed, bias=None, points=mo.KERNEL_BF16_POINTS):
    """max |schedule replay - exact| / RMS(exact) over the tokens outside the near-tie
    window, on the GPU tests' seeded inputs."""
    inp = S.make_inputs(cfg, "cpu", seed=seed)
    if bias is not None:
        inp["b"] = bias
    f = {k: v.to(torch.float64).numpy() for k, v in inp.items()}
    r = mo.route(f["x"], f["w_r"], inp["b"].numpy(), cfg["top_k"], cfg["routed_scale"])
    kw = dict(w1=f["w1"], w3=f["w3"], w2=f["w2"], shared=(f["ws1"], f["ws3"], f["ws2"]),
              routing=r)
    exact = mo.moe_sparse(f["x"], None, None, cfg["top_k"], cfg["routed_scale"], **kw)["out"]
    replay = mo.moe_sparse(f["x"], None, None, cfg["top_k"], cfg["routed_scale"],
                           bf16_points=points, **kw)["out"]
    keep = r["gap"] >= 1e-6
    return np.abs(replay - exact)[keep].max() / np.sqrt(np.mean(exact[keep] ** 2))


def _same_experts_bias(n, top):
    b = torch.zeros(n)
    b[:top] = 10.0
    return b


SHAPES = {
    # name: (config, seed, bias, ratio range of the replay with h rounded once to bf16)
    "tiny (64 tokens, k 2)": (S.CONFIGS["tiny"], 0, None, (0.010, 0.020)),
    "tiny, 300 tokens all on experts 0-1 (k 2)": (
        S.with_overrides("tiny", tokens=300), 6, _same_experts_bias(16, 2), (0.020, 0.030)),
    "tiny, 300 tokens all on experts 0-7 (k 8)": (
        S.with_overrides("tiny", tokens=300, top_k=8), 6, _same_experts_bias(16, 8), (0.010, 0.020)),
    "d 128, E 7, I 64, 600 tokens, k 2": (
        dict(tokens=600, d_model=128, n_experts=7, top_k=2, d_expert=64, d_shared=64,
             routed_scale=2.827, bias="uniform"), 27, None, (0.020, 0.030)),
    "d 128, E 7, I 64, 600 tokens, k 3": (
        dict(tokens=600, d_model=128, n_experts=7, top_k=3, d_expert=64, d_shared=64,
             routed_scale=2.827, bias="uniform"), 27, None, (0.010, 0.020)),
    "d 128, E 7, I 64, 600 tokens, k 1": (
        dict(tokens=600, d_model=128, n_experts=7, top_k=1, d_expert=64, d_shared=64,
             routed_scale=2.827, bias="uniform"), 27, None, (0.020, 0.030)),
    "d 128, E 1024, I 64, 4096 tokens, k 8": (
        dict(tokens=4096, d_model=128, n_experts=1024, top_k=8, d_expert=64, d_shared=64,
             routed_scale=2.827, bias="uniform"), 0, None, (0.020, 0.030)),
    "d 128, E 1024, I 128, 4096 tokens, k 8": (
        dict(tokens=4096, d_model=128, n_experts=1024, top_k=8, d_expert=128, d_shared=128,
             routed_scale=2.827, bias="uniform"), 0, None, (0.020, 0.030)),
    "d 128, E 1024, I 256, 4096 tokens, k 8": (
        dict(tokens=4096, d_model=128, n_experts=1024, top_k=8, d_expert=256, d_shared=256,
             routed_scale=2.827, bias="uniform"), 0, None, (0.010, 0.020)),
}


@pytest.mark.parametrize("name", list(SHAPES))
def test_kernel_schedule_limits(name):
    """Where the bf16-h schedule holds the 2e-2 * RMS bar on its own and where it cannot:
    a range above 0.02 marks a shape no implementation of this schedule passes."""
    cfg, seed, bias, (lo, hi) = SHAPES[name]
    ratio = _replay_ratio(cfg, seed, bias)
    print(f"{name}: schedule replay max|err| / RMS = {ratio:.4f}")
    assert lo <= ratio < hi, ratio


def _two_part(cfg):
    """The kernels' rule for h in two bf16 parts (the binding's h_width)."""
    return cfg["top_k"] <= 2 or cfg["d_expert"] <= 128


def test_two_part_rule_matches_the_binding():
    from mixture_experts_transformer_sigmoid_amd import binding as B
    for cfg, *_ in SHAPES.values():
        dims = B.dims_for(cfg)
        assert B.h_width(dims) == (2 if _two_part(cfg) else 1) * cfg["d_expert"]


@pytest.mark.parametrize("name", [n for n in SHAPES if _two_part(SHAPES[n][0])])
def test_two_part_h_holds_the_bar(name):
    """With at most two slots per token, or experts at most 128 wide, the kernels keep h
    in two bf16 parts (16 significant bits); the replay of that schedule is inside the bar
    on every such shape, also where the single rounding is not."""
    cfg, seed, bias, _ = SHAPES[name]
    ratio = _replay_ratio(cfg, seed, bias, mo.KERNEL_BF16_POINTS_TWO_PART)
    print(f"{name}: two-part-h replay max|err| / RMS = {ratio:.4f}")
    assert ratio < 0.0185, ratio


def test_no_shape_left_outside_the_bar():
    """Every shape whose single-rounding replay misses the bar is one where the kernels
    use two parts."""
    for name, (cfg, _, _, (lo, _)) in SHAPES.items():
        assert lo < 0.020 or _two_part(cfg), name


def test_two_part_h_replay_against_torch():
    """The "h2" point: torch's bf16 cast of h plus the cast of its remainder."""
    L = _layer(43)
    r = mo.route(L["x"], L["w_r"], L["b"], L["k"])
    x = _t(L["x"])
    got = mo.moe_sparse(L["x"], L["w_r"], L["b"], L["k"], w1=L["w1"], w3=L["w3"], w2=L["w2"],
                        shared=None, routing=r, bf16_points=("h2",))["y_routed"]
    want = torch.zeros(x.shape[0], x.shape[1], dtype=torch.float64)
    for t in range(x.shape[0]):
        for j in range(L["k"]):
            e = int(r["topk_idx"][t, j])
            h = F.silu(F.linear(x[t], _t(L["w1"][e]))) * F.linear(x[t], _t(L["w3"][e]))
            hi = _bf(h)
            want[t] += float(r["topk_w"][t, j]) * F.linear(hi + _bf(h - hi), _t(L["w2"][e]))
    np.testing.assert_allclose(got, want.numpy(), rtol=1e-9, atol=1e-12)
