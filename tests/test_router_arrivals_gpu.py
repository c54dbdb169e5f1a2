"""The small-batch router's arrival counts, through the C ABI, against the CPU oracle.

Up to 512 tokens and above 16 experts, each 16-token block of the router is spread over
one workgroup per 16 experts; the last of them to finish (it counts arrivals in a device
counter kept per workspace, which it puts back to zero) takes the block's top-k and gates.
These tests check that the counts start from zero on every call: many calls in a row on
one workspace with changing shapes, calls on two streams at once with their own
workspaces, and a call captured in a HIP graph and replayed between eager calls.  Routing
is compared with the oracle as in test_parity_gpu.py (bit-exact sets outside the near-tie
window, gates within 1e-5), or bit for bit with an eager call on the same input.
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


def say(msg):
    print(msg, flush=True)


def _cfg(T, E, k=8):
    return dict(tokens=T, d_model=256, n_experts=E, top_k=k, d_expert=128, d_shared=128,
                routed_scale=2.827, bias="uniform")


def _route(dims, inp, ws, stream=None):
    T, k = dims.tokens, dims.top_k
    idx = torch.full((T, k), -7, dtype=torch.int32, device=DEV)
    w = torch.full((T, k), float("nan"), dtype=torch.float32, device=DEV)
    M.moe_route(dims, inp["x"][:T], inp["w_r"], inp["b"], idx, w, None, ws, stream=stream)
    return idx, w


def _check(idx, w, inp, dims, what):
    x = inp["x"][:dims.tokens].to("cpu", torch.float64).numpy()
    ref = O.route(x, inp["w_r"].to("cpu", torch.float64).numpy(), inp["b"].cpu().numpy(),
                  dims.top_k, dims.routed_scale)
    keep = ref["gap"] >= GAP
    gi = np.sort(idx.cpu().numpy(), axis=1)
    oi = np.sort(ref["topk_idx"], axis=1)
    bad = np.nonzero(np.any(gi != oi, axis=1) & keep)[0]
    assert bad.size == 0, f"{what}: routing differs on {bad.size} tokens, e.g. {bad[:5]}"
    gw = w.cpu().numpy().astype(np.float64)
    order = np.argsort(idx.cpu().numpy(), axis=1)
    og = np.take_along_axis(ref["topk_w"], np.argsort(ref["topk_idx"], axis=1), axis=1)
    dg = np.abs(np.take_along_axis(gw, order, axis=1) - og)[keep]
    assert dg.size == 0 or dg.max() <= 1e-5, (what, dg.max())
    return int((~keep).sum())


def test_one_workspace_many_shapes():
    """One workspace, calls of changing expert and token counts back to back (ragged last
    blocks, 2 to 64 expert tiles, 1 to 32 token blocks), each compared with the oracle."""
    seq = [(128, 384), (45, 17), (512, 1024), (1, 65), (300, 384), (16, 64), (17, 200),
           (128, 384)]
    need = max(M.moe_workspace_bytes(M.dims_for(_cfg(T, E))) for T, E in seq)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    inputs = {}
    results = []
    for i, (T, E) in enumerate(seq):
        if E not in inputs:
            inputs[E] = {k: v.to(DEV) for k, v in
                         S.make_inputs(_cfg(512, E), "cpu", seed=70 + E).items()}
        dims = M.dims_for(_cfg(512, E), tokens=T)
        say(f"  call {i}: T={T} E={E}")
        results.append((dims, E, _route(dims, inputs[E], ws)))
    torch.cuda.synchronize()
    for i, (dims, E, (idx, w)) in enumerate(results):
        n = _check(idx, w, inputs[E], dims, f"call {i} (T={dims.tokens}, E={E})")
        say(f"  call {i}: routing equal, {n} near-tie tokens excluded")


def test_two_streams_own_workspaces():
    """Two streams, each with its own workspace and input, 12 routing calls each, queued
    alternately with no synchronisation between them (the launches may run at the same
    time); every call's result is compared with the oracle."""
    cfg = _cfg(128, 384)
    dims = M.dims_for(cfg)
    a = {k: v.to(DEV) for k, v in S.make_inputs(cfg, "cpu", seed=81).items()}
    b = dict(a)
    b["x"] = S.make_inputs(cfg, "cpu", seed=82)["x"].to(DEV)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    wss = [M.workspace(dims), M.workspace(dims)]
    torch.cuda.synchronize()
    outs = [[], []]
    for _ in range(12):
        for j, inp in enumerate((a, b)):
            with torch.cuda.stream(streams[j]):
                outs[j].append(_route(dims, inp, wss[j], stream=streams[j]))
    torch.cuda.synchronize()
    for j, inp in enumerate((a, b)):
        for i, (idx, w) in enumerate(outs[j]):
            _check(idx, w, inp, dims, f"stream {j} call {i}")
    say("  24 calls on two streams: routing equal")


def test_many_calls_in_a_row_agree():
    """400 routing calls back to back on one workspace at the K2 decode shape of the router
    (128 tokens, 384 experts: 24 workgroups per token block meet at each count), each into
    its own output: every call equals the first bit for bit, and the first equals the
    oracle.  A handoff between workgroups that read a score before it was out would show as
    a call that differs."""
    cfg = dict(tokens=128, d_model=7168, n_experts=384, top_k=8, d_expert=64, d_shared=64,
               routed_scale=2.827, bias="uniform")
    dims = M.dims_for(cfg)
    g = torch.Generator(device=DEV)
    g.manual_seed(3)
    inp = {"x": torch.randn(128, 7168, generator=g, device=DEV).to(torch.bfloat16),
           "w_r": torch.randn(384, 7168, generator=g, device=DEV) / 7168 ** 0.5,
           "b": torch.rand(384, generator=g, device=DEV) * 0.02 - 0.01}
    ws = M.workspace(dims)
    n = 400
    idx = torch.full((n, 128, 8), -7, dtype=torch.int32, device=DEV)
    w = torch.full((n, 128, 8), float("nan"), dtype=torch.float32, device=DEV)
    for i in range(n):
        M.moe_route(dims, inp["x"], inp["w_r"], inp["b"], idx[i], w[i], None, ws)
    torch.cuda.synchronize()
    _check(idx[0], w[0], inp, dims, "first call")
    same_idx = (idx == idx[0]).all(dim=2).all(dim=1)
    same_w = (w.view(torch.int32) == w[0].view(torch.int32)).all(dim=2).all(dim=1)
    bad = torch.nonzero(~(same_idx & same_w)).flatten().tolist()
    say(f"  {n} calls: {len(bad)} differ from the first")
    assert not bad, bad[:10]


def test_layer_on_two_streams_own_workspaces():
    """The whole layer (moe_forward, 128 tokens, 64 experts) on two streams at once, each
    with its own workspace and input, 8 calls each queued alternately: every call's output
    equals the one the same input gives alone, bit for bit."""
    cfg = _cfg(128, 64)
    dims = M.dims_for(cfg)
    base = {k: v.to(DEV) for k, v in S.make_inputs(cfg, "cpu", seed=85).items()}
    xs = [base["x"], S.make_inputs(cfg, "cpu", seed=86)["x"].to(DEV)]

    def forward(x, out, ws, stream=None):
        M.moe_forward(dims, x, base["w_r"], base["b"], base["w1"], base["w3"], base["w2"],
                      base["ws1"], base["ws3"], base["ws2"], out, ws, stream=stream)

    want = []
    for x in xs:
        o = torch.empty(dims.tokens, dims.d_model, dtype=torch.bfloat16, device=DEV)
        forward(x, o, M.workspace(dims))
        want.append(o)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    wss = [M.workspace(dims), M.workspace(dims)]
    outs = [[], []]
    for _ in range(8):
        for j in range(2):
            o = torch.empty(dims.tokens, dims.d_model, dtype=torch.bfloat16, device=DEV)
            with torch.cuda.stream(streams[j]):
                forward(xs[j], o, wss[j], stream=streams[j])
            outs[j].append(o)
    torch.cuda.synchronize()
    for j in range(2):
        for i, o in enumerate(outs[j]):
            assert torch.equal(o.view(torch.int16), want[j].view(torch.int16)), (j, i)
    say("  16 layer calls on two streams: outputs equal")


def test_graph_replays_between_eager_calls():
    """moe_forward (T = 100, 64 experts: four expert tiles per token block) captured in a
    HIP graph on its workspace, then replayed four times with a new input copied in before
    each replay, and eager calls on another workspace (and on the graph's own, after the
    replay) in between: every replay's output and routing must equal an eager call's on the
    same input, bit for bit."""
    cfg = _cfg(100, 64)
    dims = M.dims_for(cfg)
    inps = [{k: v.to(DEV) for k, v in S.make_inputs(cfg, "cpu", seed=90 + i).items()}
            for i in range(3)]
    base = inps[0]

    def forward(x, out, ws):
        M.moe_forward(dims, x, base["w_r"], base["b"], base["w1"], base["w3"], base["w2"],
                      base["ws1"], base["ws3"], base["ws2"], out, ws)

    want = []
    for inp in inps:
        o = torch.empty(dims.tokens, dims.d_model, dtype=torch.bfloat16, device=DEV)
        ws = M.workspace(dims)
        forward(inp["x"], o, ws)
        torch.cuda.synchronize()
        want.append((o, M.routing_in_workspace(dims, ws)))
    x = base["x"].clone()
    out = torch.empty(dims.tokens, dims.d_model, dtype=torch.bfloat16, device=DEV)
    ws_graph = M.workspace(dims)
    ws_other = M.workspace(dims)
    other = torch.empty_like(out)
    forward(x, out, ws_graph)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        forward(x, out, ws_graph)
    torch.cuda.synchronize()
    for i in range(4):
        j = (i + 1) % 3
        forward(inps[(j + 1) % 3]["x"], other, ws_other)   # eager, another workspace
        x.copy_(inps[j]["x"])
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = M.routing_in_workspace(dims, ws_graph)
        same = torch.equal(out.view(torch.int16), want[j][0].view(torch.int16))
        say(f"  replay {i} (input {j}): output equal {same}")
        assert same, f"replay {i}"
        for key in ("topk_idx", "topk_w"):
            assert torch.equal(got[key], want[j][1][key]), (i, key)
        forward(inps[j]["x"], other, ws_graph)               # eager, the graph's workspace
        torch.cuda.synchronize()
        assert torch.equal(other.view(torch.int16), want[j][0].view(torch.int16)), f"eager {i}"


def test_released_workspace_and_graph():
    """A call captured in a graph pins its workspace's slot; after the graph is destroyed
    and the workspace released (moe_workspace_release), calls on other workspaces and on
    the released one (which takes a slot again) still route as the oracle does."""
    cfg = _cfg(100, 64)
    dims = M.dims_for(cfg)
    inp = {k: v.to(DEV) for k, v in S.make_inputs(cfg, "cpu", seed=95).items()}
    ws = M.workspace(dims)
    idx = torch.empty(100, 8, dtype=torch.int32, device=DEV)
    w = torch.empty(100, 8, dtype=torch.float32, device=DEV)
    M.moe_route(dims, inp["x"], inp["w_r"], inp["b"], idx, w, None, ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        M.moe_route(dims, inp["x"], inp["w_r"], inp["b"], idx, w, None, ws)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    _check(idx, w, inp, dims, "graph replay")
    del g
    M.moe_workspace_release(ws)
    M.moe_workspace_release(ws)          # a second release is ignored
    for j, space in enumerate((M.workspace(dims), ws, M.workspace(dims))):
        i2, w2 = _route(dims, inp, space)
        torch.cuda.synchronize()
        _check(i2, w2, inp, dims, f"after release, call {j}")
