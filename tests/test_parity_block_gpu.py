"""Parity of the fused block entry point (moe_forward_block) against the CPU oracle.

moe_forward_block takes the residual stream x'_n, applies the pre-MoE RMSNorm (learned
gain, eps), runs the layer on the normalised input and adds the residual before the one
bf16 rounding of the output.  Contract:
  x_ffn   the normalised bf16 input the call leaves in the workspace, bit-exact against
          the oracle's norm (fp64, rounded to fp32 then bf16) on every token
  routing as in moe_forward (exact outside the near-tie window; near ties excluded)
  out     |out - (x'_n + Delta)| <= 2e-2 * RMS(Delta) + half a bf16 ulp of the value,
          per element: the layer's error bar on Delta plus the final rounding
"""
import numpy as np
import pytest
import torch

import mixture_experts_transformer_sigmoid_amd as M
import synth_inputs as S
from oracle import moe_oracle as O
from test_parity_gpu import check_permute, check_routing

pytestmark = pytest.mark.gpu

DEV = "cuda"
GAP = 1e-6
TOL = 2e-2
EPS = 1e-6


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def say(msg):
    print(msg, flush=True)


def block_inputs(cfg, seed=0, weights=None):
    inp = dict(weights) if weights is not None else {
        k: v.to(DEV) for k, v in S.make_weights(cfg, "cpu", seed, shared=cfg["d_shared"] > 0).items()}
    inp.update({k: v.to(DEV) for k, v in S.make_block_activations(cfg, "cpu", seed).items()})
    return inp


def run_block(cfg, inp, eps=EPS):
    dims = M.dims_for(cfg)
    T, d = cfg["tokens"], cfg["d_model"]
    ws = M.block_workspace(dims)
    out = torch.full((T, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    M.moe_forward_block(dims, inp["x_res"], inp["norm_w"], eps, inp["w_r"], inp["b"], inp["w1"],
                        inp["w3"], inp["w2"], inp.get("ws1"), inp.get("ws3"), inp.get("ws2"), out,
                        ws)
    torch.cuda.synchronize()
    base = M.moe_workspace_bytes(dims)
    x_ffn = ws[base: base + T * d * 2].view(torch.bfloat16).view(T, d).clone()
    run_block.ws = ws
    return out, x_ffn


def half_ulp_bf16(v):
    """Half the bf16 spacing at |v| (8 significant bits): 2^(floor(log2|v|) - 8)."""
    _, e = np.frexp(np.abs(v))
    return np.ldexp(1.0, e - 9)


def check_block(cfg, inp, eps=EPS, sample=None, seed=0):
    T = cfg["tokens"]
    say(f"block case T={T} d={cfg['d_model']} E={cfg['n_experts']} k={cfg['top_k']} "
        f"I={cfg['d_expert']} Is={cfg['d_shared']} eps={eps}")
    out, x_ffn = run_block(cfg, inp, eps)
    rw = M.routing_in_workspace(M.dims_for(cfg), run_block.ws)
    g = {"idx": rw["topk_idx"].clone(), "w": rw["topk_w"].clone(), "counts": rw["counts"].clone(),
         "offsets": rw["offsets"].clone(), "perm": rw["perm_rows"].clone(),
         "inv": rw["inv_perm"].clone()}
    again, _ = run_block(cfg, inp, eps)
    assert torch.equal(out.view(torch.int16), again.view(torch.int16)), "not deterministic"
    x_res = f64(inp["x_res"])
    gain = f64(inp["norm_w"])
    # the normalised input, every token, in row chunks
    g_ffn = f64(x_ffn)
    for a in range(0, T, 1024):
        want = O.round_bf16(O.rmsnorm(x_res[a:a + 1024], eps, gain))
        bad = np.argwhere(g_ffn[a:a + 1024] != want)
        assert bad.size == 0, f"x_ffn differs at {bad[:4] + [a, 0]}"
    say("  x_ffn bit-exact")
    # the call's own routing (on its x_ffn) and permutation, left at the front of the workspace
    dims = M.dims_for(cfg)
    r_all = O.route(g_ffn, f64(inp["w_r"]), inp["b"].cpu().numpy(), cfg["top_k"],
                    cfg["routed_scale"])
    n_ex = check_routing(g, r_all, dims)
    check_permute(g, dims)
    say(f"  routing and permutation exact ({n_ex} near-tie tokens excluded)")
    toks = np.arange(T) if sample is None else np.sort(
        np.random.default_rng(seed).choice(T, size=min(sample, T), replace=False))
    get = lambda e: (f64(inp["w1"][e]), f64(inp["w3"][e]), f64(inp["w2"][e]))  # noqa: E731
    sh = (f64(inp["ws1"]), f64(inp["ws3"]), f64(inp["ws2"])) if cfg["d_shared"] else (None,) * 3
    ref = O.moe_block(x_res, gain, f64(inp["w_r"]), inp["b"].cpu().numpy(), None, None, None,
                      *sh, top_k=cfg["top_k"], alpha=cfg["routed_scale"], eps=eps,
                      get_expert=get, tokens=toks)
    keep = ref["gap"] >= GAP
    got = f64(out)[toks][keep]
    want = ref["out"][keep]
    assert np.all(np.isfinite(got))
    rms = np.sqrt(np.mean(ref["delta"][keep] ** 2)) if keep.any() else 0.0
    lim = TOL * rms + half_ulp_bf16(np.maximum(np.abs(got), np.abs(want)))
    worst = (np.abs(got - want) / lim).max() if keep.any() else 0.0
    say(f"  out: max|err| {np.abs(got - want).max() if keep.any() else 0:.3e}, worst err/bound "
        f"{worst:.3f} (rms Delta {rms:.3e}); near-tie tokens excluded {int((~keep).sum())}")
    assert worst <= 1.0
    return out, x_ffn


def test_block_tiny():
    cfg = S.CONFIGS["tiny"]
    check_block(cfg, block_inputs(cfg))


@pytest.mark.parametrize("T", [1, 37, 300, 600])
def test_block_ragged(T):
    # up to 512 tokens the router kernel normalises the residual stream itself; 600 takes
    # the norm kernel and the GEMM router
    cfg = S.with_overrides("tiny", tokens=T, d_model=320, n_experts=24, top_k=3, d_expert=192,
                           d_shared=192)
    check_block(cfg, block_inputs(cfg, seed=T))


def test_block_no_shared_eps_zero():
    cfg = S.with_overrides("tiny", tokens=50, d_shared=0)
    check_block(cfg, block_inputs(cfg, seed=5), eps=0.0)


def test_block_zero_gain_returns_residual():
    # gain 0: x_ffn = 0, every expert sees a zero input, Delta = 0: out is x'_n bit for bit
    cfg = S.CONFIGS["tiny"]
    inp = block_inputs(cfg, seed=6)
    inp["norm_w"] = torch.zeros_like(inp["norm_w"])
    out, x_ffn = run_block(cfg, inp)
    assert torch.count_nonzero(x_ffn.float()) == 0
    assert torch.equal(out.view(torch.int16), inp["x_res"].view(torch.int16))


def test_block_w2_zero_returns_residual():
    cfg = S.CONFIGS["tiny"]
    inp = block_inputs(cfg, seed=7)
    inp["w2"] = torch.zeros_like(inp["w2"])
    inp["ws2"] = torch.zeros_like(inp["ws2"])
    out, _ = run_block(cfg, inp)
    assert torch.equal(out.view(torch.int16), inp["x_res"].view(torch.int16))


def test_block_k2_decode_128(k2_weights):
    cfg = S.CONFIGS["k2_decode"]
    check_block(cfg, block_inputs(cfg, weights=k2_weights), sample=64)


def test_block_k2_prefill_8192(k2_weights):
    cfg = S.CONFIGS["k2_prefill"]
    check_block(cfg, block_inputs(cfg, weights=k2_weights), sample=64)
