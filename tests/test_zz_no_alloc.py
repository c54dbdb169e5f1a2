"""moe_forward_noalloc against moe_forward, through the C ABI.

The no-allocation entry point runs moe_forward's kernels on the library's fixed device
scratch instead of a caller's workspace, so its output must equal moe_forward's bit for
bit.  Each case makes two calls in a row, the second with fewer tokens: the scratch keeps
the first call's contents, and nothing of them may leak into the second result.
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
    dims = M.dims_for(cfg, tokens=451)
    x = torch.empty((8, 16), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(M.MoeError) as ei:
        M.moe_forward_noalloc(dims, x, x, x, x, x, x, x, x, x, x)
    assert ei.value.status == M.MOE_ESCRATCH
