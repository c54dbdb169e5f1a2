"""moe_forward_noalloc against moe_forward, through the C ABI.

The no-allocation entry point runs moe_forward's kernels on the library's fixed device
scratch instead of a caller's workspace, so its output must equal moe_forward's bit for
bit.  Each case makes two calls in a row, the second with fewer tokens: the scratch keeps
the first call's contents, and nothing of them may leak into the second result.  The entry
point is also captured in a HIP graph and replayed (it allocates nothing and launches no
memset): every replay must reproduce the eager result, with an eager call on other inputs
through the same scratch between replays.
"""
import numpy as np
import pytest
import torch

import mixture_experts_transformer_sigmoid_amd as M
import synth_inputs as S

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(msg):
    print(msg, flush=True)


def _args(inp, T):
    return (inp["x"][:T], inp["w_r"], inp["b"], inp["w1"], inp["w3"], inp["w2"], inp.get("ws1"),
            inp.get("ws3"), inp.get("ws2"))


def _forward(dims, inp):
    out = torch.full((dims.tokens, dims.d_model), float("nan"), dtype=torch.bfloat16, device=DEV)
    M.moe_forward(dims, *_args(inp, dims.tokens), out, M.workspace(dims))
    return out


def _noalloc(dims, inp):
    out = torch.full((dims.tokens, dims.d_model), float("nan"), dtype=torch.bfloat16, device=DEV)
    M.moe_forward_noalloc(dims, *_args(inp, dims.tokens), out)
    return out


def _two_calls(cfg, inp, sizes):
    for T in sizes:
        dims = M.dims_for(cfg, tokens=T)
        assert M.moe_workspace_bytes(dims) <= M.NOALLOC_SCRATCH_BYTES
        say(f"  noalloc T={T} d={dims.d_model} E={dims.n_experts} k={dims.top_k} "
            f"I={dims.d_expert} (scratch use {M.moe_workspace_bytes(dims)} bytes)")
        got = _noalloc(dims, inp)
        want = _forward(dims, inp)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(got.float()).all()), "unwritten output elements"
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), \
            f"T={T}: {int((got != want).sum())} elements differ from moe_forward"


def test_noalloc_small_then_smaller():
    cfg = S.CONFIGS["tiny"]
    inp = {k: v.to(DEV) for k, v in S.make_inputs(cfg, "cpu", seed=21).items()}
    _two_calls(cfg, inp, [64, 20])


def test_noalloc_wide_kernels_then_skinny():
    # 600 tokens: the router's GEMM path and the 256-row expert GEMMs; then 37 tokens:
    # the small-batch router and the skinny GEMMs on the same scratch
    cfg = dict(tokens=600, d_model=1024, n_experts=16, top_k=4, d_expert=512, d_shared=512,
               routed_scale=2.827, bias="uniform")
    inp = {k: v.to(DEV) for k, v in S.make_inputs(cfg, "cpu", seed=22).items()}
    _two_calls(cfg, inp, [600, 37])


def test_noalloc_k2_decode(k2_weights):
    cfg = S.CONFIGS["k2_decode"]
    inp = dict(k2_weights)
    inp.update(S.make_activations(cfg, DEV))
    _two_calls(cfg, inp, [128, 64])


def test_noalloc_rejects_beyond_scratch():
    cfg = S.CONFIGS["k2_decode"]
    dims = M.dims_for(cfg, tokens=513)
    x = torch.empty((8, 16), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(M.MoeError) as ei:
        M.moe_forward_noalloc(dims, x, x, x, x, x, x, x, x, x, x)
    assert ei.value.status == M.MOE_ESCRATCH


def _call(dims, inp, out):
    M.moe_forward_noalloc(dims, inp["x"], inp["w_r"], inp["b"], inp["w1"], inp["w3"], inp["w2"],
                          inp["ws1"], inp["ws3"], inp["ws2"], out)


@pytest.mark.parametrize("name,tokens", [("tiny", 64), ("wide", 600)])
def test_noalloc_graph_replays_match_eager(name, tokens):
    cfg = S.CONFIGS["tiny"] if name == "tiny" else dict(
        tokens=tokens, d_model=1024, n_experts=16, top_k=4, d_expert=512, d_shared=512,
        routed_scale=2.827, bias="uniform")
    inp = {k: v.to(DEV) for k, v in S.make_inputs(cfg, "cpu", seed=61).items()}
    other = {k: v.to(DEV) for k, v in S.make_inputs(cfg, "cpu", seed=62).items()}
    dims = M.dims_for(cfg)
    want = torch.empty(cfg["tokens"], cfg["d_model"], dtype=torch.bfloat16, device=DEV)
    M.moe_forward(dims, inp["x"], inp["w_r"], inp["b"], inp["w1"], inp["w3"], inp["w2"],
                  inp["ws1"], inp["ws3"], inp["ws2"], want, M.workspace(dims))
    out = torch.empty_like(want)
    scratch_user = torch.empty_like(want)
    _call(dims, inp, out)                  # first call on the device: scratch address lookup
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _call(dims, inp, out)
    torch.cuda.synchronize()
    for i in range(4):
        out.fill_(float("nan"))
        _call(dims, other, scratch_user)   # eager work through the same scratch
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"replay {i}: equal {torch.equal(out.view(torch.int16), want.view(torch.int16))}",
              flush=True)
        assert torch.equal(out.view(torch.int16), want.view(torch.int16)), f"replay {i}"
