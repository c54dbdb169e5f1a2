"""Parity of the FP8 block-scaled expert path (moe_*_fp8) against the CPU oracle.

The weights are E4M3 codes with one fp32 scale per 128 x 128 block; the oracle
dequantises them exactly (code value x scale, float64) and runs the same layer.  The
contract is the bf16 path's: routing exact outside the near-tie window (the router is
unchanged), max |out - oracle| <= 2e-2 * RMS(oracle); and the step-by-step checks of h
and Y against the exactly dequantised weights, since the kernels dequantise without
rounding (fp32 accumulation error only).  The split entry points and moe_forward_fp8
must agree bit for bit.
"""
import numpy as np
import pytest
import torch

import mixture_experts_transformer_sigmoid_amd as M
import synth_inputs as S
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

DEV = "cuda"
GAP = 1e-6
TOL = 2e-2


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def say(msg):
    print(msg, flush=True)


def bf16r(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def fp8_inputs(cfg, seed=0, weights=None):
    inp = dict(weights) if weights is not None else {
        k: v.to(DEV) for k, v in S.make_fp8_weights(cfg, "cpu", seed, shared=cfg["d_shared"] > 0).items()}
    inp.update({k: v.to(DEV) for k, v in S.make_activations(cfg, "cpu", seed).items()})
    return inp


def dq(inp, name, e=None):
    q = inp[name] if e is None else inp[name][e]
    s = inp[name + "_scale"] if e is None else inp[name + "_scale"][e]
    return O.dequant_fp8_blocks(q.cpu().numpy(), s.cpu().numpy())


def run_split(cfg, inp):
    dims = M.dims_for(cfg)
    T, E, k, d, I = cfg["tokens"], cfg["n_experts"], cfg["top_k"], cfg["d_model"], cfg["d_expert"]
    ws = M.workspace(dims)
    w = M.fp8_weights(inp)
    idx = torch.empty(T, k, dtype=torch.int32, device=DEV)
    gw = torch.empty(T, k, dtype=torch.float32, device=DEV)
    M.moe_route(dims, inp["x"], inp["w_r"], inp["b"], idx, gw, None, ws)
    counts = torch.empty(E, dtype=torch.int32, device=DEV)
    offs = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    perm = torch.empty(T * k, dtype=torch.int32, device=DEV)
    inv = torch.empty(T * k, dtype=torch.int32, device=DEV)
    M.moe_permute(dims, idx, counts, offs, perm, inv, ws)
    rows = T * k + (T if cfg["d_shared"] else 0)
    h = torch.full((rows, I), float("nan"), dtype=torch.bfloat16, device=DEV)
    M.moe_expert_gate_up_fp8(dims, inp["x"], perm, offs, w, h, ws)
    y = torch.full((T * k, d), float("nan"), dtype=torch.float32, device=DEV)
    ys = torch.full((T, d), float("nan"), dtype=torch.float32, device=DEV) if cfg["d_shared"] else None
    M.moe_expert_down_fp8(dims, h, offs, w, y, ys, ws)
    out = torch.full((T, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    M.moe_combine(dims, y, inv, gw, ys, out)
    # the layer keeps its expert rows as 24-bit floats (the low 8 mantissa bits cleared):
    # the same combine over those values is what moe_forward_fp8 must return
    out24 = torch.full((T, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    y24 = (y.view(torch.int32) & -256).view(torch.float32)
    ys24 = (ys.view(torch.int32) & -256).view(torch.float32) if ys is not None else None
    M.moe_combine(dims, y24, inv, gw, ys24, out24)
    fw = torch.full((T, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    M.moe_forward_fp8(dims, inp["x"], inp["w_r"], inp["b"], w, fw, ws)
    torch.cuda.synchronize()
    return dict(idx=idx, w=gw, counts=counts, offs=offs, perm=perm, inv=inv, h=h, y=y, ys=ys,
                out=out, out24=out24, fw=fw)


def check_bound(got, want, lim, what):
    got = np.asarray(got, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    worst = (np.abs(got - want) / lim).max()
    say(f"  {what}: max|err| {np.abs(got - want).max():.3e}, worst err/bound {worst:.3f}")
    assert worst <= 1.0, (what, worst)


def full_check(cfg, inp, sample=None, seed=0, intermediates=True, inter_tokens=2,
               per_row_bar=False):
    T, k = cfg["tokens"], cfg["top_k"]
    say(f"fp8 case T={T} d={cfg['d_model']} E={cfg['n_experts']} k={k} I={cfg['d_expert']} "
        f"Is={cfg['d_shared']}")
    g = run_split(cfg, inp)
    # every output element was written (each was pre-filled with NaN): no row tile or
    # n-block of the device-built work list was missed
    for name in ("h", "y", "ys", "out", "fw"):
        if g[name] is not None:
            assert bool(torch.isfinite(g[name].float()).all()), f"{name}: elements never written"
    assert torch.equal(g["fw"].view(torch.int16), g["out24"].view(torch.int16)), \
        "forward != split with 24-bit expert rows"
    again = run_split(cfg, inp)
    assert torch.equal(again["out"].view(torch.int16), g["out"].view(torch.int16)), "not deterministic"
    x = f64(inp["x"])
    ref = O.route(x, f64(inp["w_r"]), inp["b"].cpu().numpy(), k, cfg["routed_scale"])
    keep = ref["gap"] >= GAP
    gi = np.sort(g["idx"].cpu().numpy(), axis=1)
    bad = np.nonzero(np.any(gi != np.sort(ref["topk_idx"], axis=1), axis=1) & keep)[0]
    assert bad.size == 0, f"routing differs on {bad.size} tokens"
    toks = np.arange(T) if sample is None else np.sort(
        np.random.default_rng(seed).choice(T, size=min(sample, T), replace=False))
    toks = toks[keep[toks]]
    get = lambda e: (dq(inp, "w1", e), dq(inp, "w3", e), dq(inp, "w2", e))  # noqa: E731
    shared = (dq(inp, "ws1"), dq(inp, "ws3"), dq(inp, "ws2")) if cfg["d_shared"] else None
    o = O.moe_sparse(x, None, None, k, cfg["routed_scale"], get_expert=get, shared=shared,
                     tokens=toks, routing=ref)
    got = f64(g["out"])[toks]
    err = np.abs(got - o["out"])
    rms = np.sqrt(np.mean(o["out"] ** 2))
    say(f"  out: max|err| {err.max():.3e}  tol {TOL * rms:.3e}  (rms {rms:.3e}); "
        f"near-tie tokens excluded {int((~keep).sum())}")
    if per_row_bar:
        # rows of very different magnitude: the bar per token, on that token's RMS
        row_rms = np.sqrt(np.mean(o["out"] ** 2, axis=1, keepdims=True))
        worst = (err / (TOL * row_rms)).max()
        say(f"  out, per-row bar: worst err/bound {worst:.3f}")
        assert worst <= 1.0
    else:
        assert err.max() <= TOL * rms
    if intermediates:
        # h rows and expert outputs of a few tokens against the exactly dequantised weights
        inv = g["inv"].cpu().numpy()
        idx = g["idx"].cpu().numpy()
        h_all = g["h"]
        pick = toks[:inter_tokens] if np.isscalar(inter_tokens) else [t for t in toks if t in inter_tokens]
        for t in pick:
            for j in range(k):
                e = int(idx[t, j])
                w1, w3, w2 = get(e)
                row = int(inv[t * k + j])
                gg, uu = x[t] @ w1.T, x[t] @ w3.T
                exact = O.silu(gg) * uu
                lim = 2.0 ** -7 * np.abs(bf16r(exact)) + 1e-5 * (np.abs(gg) + 1) * (np.abs(uu) + 1)
                hr = f64(h_all[row])
                check_bound(hr, bf16r(exact), lim, f"h (token {t}, expert {e})")
                yr = f64(g["y"][row])
                check_bound(yr, hr @ w2.T, 2.0 ** -12 * (np.abs(hr) @ np.abs(w2).T) + 1e-30,
                            f"y (token {t}, expert {e})")
    return g


def test_fp8_tiny_skinny():
    cfg = S.CONFIGS["tiny"]
    full_check(cfg, fp8_inputs(cfg))


@pytest.mark.parametrize("T", [1, 37, 300])
def test_fp8_ragged(T):
    # T = 300 puts 1200 rows on 25 groups (48 per group): the 256-row kernel, with K = 512
    # (eight 64-k chunks: one pass of its six-chunk loop and a tail of two) and K = 256 (four
    # chunks: the tail alone)
    cfg = S.with_overrides("tiny", tokens=T, d_model=512, n_experts=24, top_k=3, d_expert=256,
                           d_shared=256)
    full_check(cfg, fp8_inputs(cfg, seed=T))


def test_fp8_wide_kernel_no_shared():
    # top-8 of 16 as at K2: without the shared expert the output RMS is small and with
    # two or three large gates the bf16 rounding of h and of the output sit at the edge of
    # the 2e-2 * RMS bar (1.01 of it at k = 3, with h and Y exact); eight gates of ~0.35
    # average that rounding down, as they do at the K2 shape (d = 512: the 256-row kernel
    # needs a reduction of at least 512)
    cfg = S.with_overrides("tiny", tokens=600, d_model=512, n_experts=16, top_k=8, d_shared=0)
    full_check(cfg, fp8_inputs(cfg, seed=3))


def test_fp8_zero_and_extreme_scales():
    # one all-zero block (scale 0) and scales 2^-20 / 2^10 elsewhere: the kernels stay exact
    # (h and Y against the exactly dequantised weights for every token that uses experts
    # 0, 1 or 2); outputs then span four orders of magnitude, so the output bar is per row
    cfg = S.with_overrides("tiny", tokens=40)
    inp = fp8_inputs(cfg, seed=4)
    inp["w1_scale"][0, 0, 0] = 0.0
    inp["w3_scale"][1] *= 2.0 ** -20
    inp["w2_scale"][2] *= 2.0 ** 10
    idx = None
    dims = M.dims_for(cfg)
    ws = M.workspace(dims)
    ti = torch.empty(40, cfg["top_k"], dtype=torch.int32, device=DEV)
    tw = torch.empty(40, cfg["top_k"], dtype=torch.float32, device=DEV)
    M.moe_route(dims, inp["x"], inp["w_r"], inp["b"], ti, tw, None, ws)
    idx = ti.cpu().numpy()
    touch = [t for t in range(40) if np.isin(idx[t], [0, 1, 2]).any()]
    assert touch
    full_check(cfg, inp, inter_tokens=touch, per_row_bar=True)


def test_fp8_zero_and_extreme_scales_wide():
    # the same scale edits on the 256-row kernel (600 tokens, top-8 of 16: ~300 rows per
    # expert, one full row tile and one partial one; d = 512, four 128-k blocks): its
    # per-128-k-block partial sums must keep the zero block and the extreme scales exact too
    cfg = S.with_overrides("tiny", tokens=600, d_model=512, n_experts=16, top_k=8)
    inp = fp8_inputs(cfg, seed=5)
    inp["w1_scale"][0, 0, 1] = 0.0
    inp["w3_scale"][1] *= 2.0 ** -20
    inp["w2_scale"][2] *= 2.0 ** 10
    dims = M.dims_for(cfg)
    ws = M.workspace(dims)
    T, k = cfg["tokens"], cfg["top_k"]
    ti = torch.empty(T, k, dtype=torch.int32, device=DEV)
    tw = torch.empty(T, k, dtype=torch.float32, device=DEV)
    M.moe_route(dims, inp["x"], inp["w_r"], inp["b"], ti, tw, None, ws)
    idx = ti.cpu().numpy()
    touch = [t for t in range(T) if np.isin(idx[t], [0, 1, 2]).any()][:24]
    assert touch
    full_check(cfg, inp, inter_tokens=touch, per_row_bar=True)


def test_fp8_wide_kernel_main_loop_every_token():
    # K = 1024 (gate/up) and 512 (down): 16 and 8 chunks of 64, so the 256-row kernel runs
    # its six-chunk loop twice and once, then tails of four and two chunks; experts of
    # ~240 rows fill one row tile, the shared expert's 1024 rows four.  Every token is
    # compared, and 16 tokens' h and Y.  (Over these 1M outputs the kernels' schedule, h and
    # the output in bf16, replayed on the host reaches 0.92 of the bar; the GPU matches it.)
    cfg = S.with_overrides("tiny", tokens=1024, d_model=1024, n_experts=16, top_k=4,
                           d_expert=512, d_shared=512)
    full_check(cfg, fp8_inputs(cfg, seed=6), inter_tokens=16)


@pytest.mark.parametrize("T", [33, 2048])
def test_fp8_max_experts_1024(T):
    # the largest E (16 experts per lane in the selection), top-8, at d = 128 (the skinny
    # kernels), every token compared.  Larger batches put a larger output in play where the
    # bf16 output step alone (half an ulp, 0.0156 from 4 up) is most of the bar: the
    # kernels' schedule replayed on the host (h and the output in bf16), which the GPU
    # matches, reaches 1.08 of the bar at 4096 tokens; at 2048 it stays at 0.82.  The
    # 256-row kernel would need more than 16 rows per group at d >= 512, i.e. at least
    # 1,823 tokens: the same replay then reaches 0.95-1.27 of the bar (2048 tokens, seeds
    # 0-2), so no every-token case there can hold it.  The tile list of 1,025 groups on the
    # 256-row kernels is covered by the bf16 case at d = 512, the FP8 256-row kernel on
    # tiles of a few rows by test_fp8_wide_kernel_small_tiles.
    cfg = S.with_overrides("tiny", tokens=T, d_model=128, n_experts=1024, top_k=8,
                           d_expert=256, d_shared=256)
    full_check(cfg, fp8_inputs(cfg, seed=7 + T), inter_tokens=4)


def test_fp8_wide_kernel_small_tiles():
    # 128 experts, top-8, 300 tokens at d = 512: 21 rows per group, just past the FP8
    # switch to the 256-row kernel, so most row tiles hold a few to a few dozen rows of
    # 256.  Every token compared (schedule replay: 0.82 of the bar).
    cfg = S.with_overrides("tiny", tokens=300, d_model=512, n_experts=128, top_k=8,
                           d_expert=256, d_shared=256)
    full_check(cfg, fp8_inputs(cfg, seed=8), inter_tokens=4)


@pytest.fixture(scope="module")
def k2_fp8_weights():
    say("generating K2-shape FP8 weights on the GPU (384 experts, d 7168, I 2048)")
    w = S.make_fp8_weights("k2_decode", DEV)
    torch.cuda.synchronize()
    yield w
    del w
    torch.cuda.empty_cache()


def test_fp8_k2_decode_128(k2_fp8_weights):
    cfg = S.CONFIGS["k2_decode"]
    full_check(cfg, fp8_inputs(cfg, weights=k2_fp8_weights), sample=32)


def test_fp8_k2_prefill_8192(k2_fp8_weights):
    cfg = S.CONFIGS["k2_prefill"]
    full_check(cfg, fp8_inputs(cfg, weights=k2_fp8_weights), sample=32)
