"""Parity of the latent mixture of experts (moe_forward_latent) against the CPU oracle.

Routing uses x itself (width d).  The routed experts work on x W_down^T (width L), the
gate-weighted sum of their outputs goes through an RMSNorm and W_up back to width d, and
the shared expert works on x.  Same bar as the K2 layer: routing exact outside the
near-tie window, max |out - oracle| <= 2e-2 * RMS(oracle).
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


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def say(msg):
    print(msg, flush=True)


def run_latent(cfg, inp):
    dims = M.dims_for(cfg)
    L = cfg["d_latent"]
    ws = M.latent_workspace(dims, L)
    out = torch.full((cfg["tokens"], cfg["d_model"]), float("nan"), dtype=torch.bfloat16, device=DEV)
    M.moe_forward_latent(dims, L, inp["x"], inp["w_r"], inp["b"], inp["w_down"], inp["w1"],
                         inp["w3"], inp["w2"], inp["w_up"], inp.get("ws1"), inp.get("ws3"),
                         inp.get("ws2"), out, ws)
    torch.cuda.synchronize()
    return out, ws


def check(cfg, inp, sample=None, seed=0):
    T = cfg["tokens"]
    say(f"latent case T={T} d={cfg['d_model']} L={cfg['d_latent']} E={cfg['n_experts']} k={cfg['top_k']}")
    out, ws = run_latent(cfg, inp)
    dims = M.dims_for(cfg)
    rw = M.routing_in_workspace(dims, ws)
    g = {"idx": rw["topk_idx"], "w": rw["topk_w"], "counts": rw["counts"],
         "offsets": rw["offsets"], "perm": rw["perm_rows"], "inv": rw["inv_perm"]}
    again, _ = run_latent(cfg, inp)
    assert torch.equal(out.view(torch.int16), again.view(torch.int16)), "not deterministic"
    r = O.route(f64(inp["x"]), f64(inp["w_r"]), inp["b"].cpu().numpy(), cfg["top_k"],
                cfg["routed_scale"])
    # the latent call's own routing (on the full-width x) and permutation
    n_ex = check_routing(g, r, dims)
    check_permute(g, dims)
    say(f"  routing and permutation exact ({n_ex} near-tie tokens excluded)")
    keep = r["gap"] >= GAP
    toks = np.arange(T) if sample is None else np.sort(
        np.random.default_rng(seed).choice(T, size=min(sample, T), replace=False))
    toks = toks[keep[toks]]
    get = lambda e: (f64(inp["w1"][e]), f64(inp["w3"][e]), f64(inp["w2"][e]))  # noqa: E731
    ref = O.moe_latent(f64(inp["x"]), f64(inp["w_r"]), inp["b"].cpu().numpy(), f64(inp["w_down"]),
                       None, None, None, f64(inp["w_up"]), f64(inp["ws1"]), f64(inp["ws3"]),
                       f64(inp["ws2"]), cfg["top_k"], cfg["routed_scale"], tokens=toks,
                       get_expert=get)
    got = f64(out)[toks]
    assert np.all(np.isfinite(got))
    err = np.abs(got - ref["out"])
    rms = np.sqrt(np.mean(ref["out"] ** 2))
    say(f"  out: max|err| {err.max():.3e}  tol {TOL * rms:.3e}  (rms {rms:.3e}); "
        f"near-tie tokens excluded {int((~keep).sum())}")
    assert err.max() <= TOL * rms


def test_latent_tiny():
    cfg = S.CONFIGS["tiny_latent"]
    check(cfg, {k: v.to(DEV) for k, v in S.make_inputs(cfg, "cpu").items()})


@pytest.mark.parametrize("T", [1, 45])
def test_latent_ragged(T):
    cfg = S.with_overrides("tiny_latent", tokens=T, d_latent=192)
    check(cfg, {k: v.to(DEV) for k, v in S.make_inputs(cfg, "cpu", seed=T).items()})


def test_latent_routed_experts_on_the_wide_kernel():
    """The routed experts reduce over the latent width L: from L = 512 on they take the
    256-row kernels (here 75 rows per expert), below it the skinny ones, as the smaller
    latent cases do.  Every token is compared.  The kernels' schedule (latent input, h and
    the output in bf16, the normalised latent in two parts) replayed on the host reaches
    0.88 of the bar on these inputs."""
    cfg = S.with_overrides("tiny_latent", tokens=300, d_model=1024, d_latent=512, n_experts=16,
                           top_k=4, d_expert=256, d_shared=256)
    check(cfg, {k: v.to(DEV) for k, v in S.make_inputs(cfg, "cpu", seed=71).items()})


def test_latent_router_over_several_expert_tiles():
    """64 experts: each 16-token block of the router spans four expert tiles, and the last
    of them to finish takes the block's top-k (an arrival count per block).  The latent
    entry point's own routing and permutation, and every token's output (the kernels'
    schedule replayed on the host reaches 0.68 of the bar on these inputs)."""
    cfg = S.with_overrides("tiny_latent", tokens=100, n_experts=64, top_k=8, d_expert=256,
                           d_shared=256)
    check(cfg, {k: v.to(DEV) for k, v in S.make_inputs(cfg, "cpu", seed=71).items()})


@pytest.mark.parametrize("T", [12, 600])
def test_latent_shared_expert_kernel_choice(T):
    """The shared expert runs as a launch of its own (one group of T rows): the skinny
    kernel up to 512 rows, the 256-row kernel above."""
    cfg = S.with_overrides("tiny_latent", tokens=T, d_model=512, d_latent=256, d_expert=256,
                           d_shared=256)
    check(cfg, {k: v.to(DEV) for k, v in S.make_inputs(cfg, "cpu", seed=50 + T).items()})


def test_latent_k2_shape_4096():
    cfg = S.CONFIGS["latent"]
    say("generating latent-MoE weights on the GPU (384 experts on a 3584-wide latent)")
    inp = S.make_inputs(cfg, DEV)
    torch.cuda.synchronize()
    check(cfg, inp, sample=64)
    del inp
    torch.cuda.empty_cache()
