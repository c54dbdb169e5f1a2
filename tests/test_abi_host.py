"""Host-side checks of libmoe's C ABI (no GPU): the library loads, exports every entry
point include/moe.h declares, and rejects bad arguments before launching anything.

Every call here is built to fail a host-side check, so no kernel is ever queued."""
import ctypes
import os
import re

import pytest

import mixture_experts_transformer_sigmoid_amd as M
from mixture_experts_transformer_sigmoid_amd import binding as B

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moe.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_\w+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = M.lib()
    names = _declared()
    assert "moe_forward" in names and "moe_route" in names and len(names) >= 9
    for n in names:
        assert hasattr(L, n), n
    assert sorted(B.EXPORTS) == names


def _header_params():
    """Parameter types of every moe_status function in include/moe.h, in order."""
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    out = {}
    for name, params in re.findall(r"moe_status\s+(moe_\w+)\s*\(([^)]*)\)\s*;", src):
        out[name] = [re.sub(r"\w+$", "", p.strip()).strip() for p in params.split(",")]
    return out


def _ctype_of(c):
    """The ctypes class the binding should declare for one C parameter type."""
    c = c.replace("const ", "").replace(" ", "")
    if c.startswith("moe_dims*"):
        return ctypes.POINTER(B.MoeDims)
    if c.startswith("moe_fp8_weights*"):
        return ctypes.POINTER(B.MoeFp8Weights)
    if c.startswith("size_t*"):
        return ctypes.POINTER(ctypes.c_size_t)
    if c.endswith("*"):
        return ctypes.c_void_p
    return {"size_t": ctypes.c_size_t, "float": ctypes.c_float, "int32_t": ctypes.c_int32}[c]


def test_binding_argtypes_follow_header():
    """Each entry point's argtypes match the header's parameter list one for one, so a
    missing or misplaced argument fails here rather than as a ctypes error on the GPU."""
    L = M.lib()
    decl = _header_params()
    assert len(decl) == len(B.EXPORTS) - 1          # every export but moe_status_str
    for name, params in decl.items():
        want = [_ctype_of(c) for c in params]
        got = list(getattr(L, name).argtypes)
        assert got == want, (name, params)


def test_status_strings():
    for code in range(6):
        assert M.status_str(code).startswith("MOE_")
    assert "unknown" in M.status_str(99)


def test_struct_layout_matches_header():
    assert ctypes.sizeof(B.MoeDims) == 32
    assert B.MoeDims.routed_scale.offset == 28


def _k2(T=128):
    return M.moe_dims(T, 7168, 384, 8, 2048, 2048, 2.827)


def test_workspace_bytes_grow_with_tokens():
    a = M.moe_workspace_bytes(_k2(128))
    b = M.moe_workspace_bytes(_k2(8192))
    assert 0 < a < b
    # holds at least the h and y buffers of the grouped rows
    assert b >= 8192 * 9 * (2048 + 7168) * 2
    assert M.moe_workspace_bytes(_k2(0)) > 0


@pytest.mark.parametrize("bad,code", [
    (dict(top_k=9), M.MOE_EUNSUPPORTED),
    (dict(top_k=0), M.MOE_EINVAL),
    (dict(n_experts=4, top_k=8), M.MOE_EINVAL),
    (dict(d_model=7000), M.MOE_EUNSUPPORTED),
    (dict(d_expert=100), M.MOE_EUNSUPPORTED),
    (dict(d_shared=1024), M.MOE_EUNSUPPORTED),
    (dict(n_experts=2000), M.MOE_EUNSUPPORTED),
    (dict(tokens=-1), M.MOE_EINVAL),
    (dict(routed_scale=float("nan")), M.MOE_EINVAL),
    (dict(tokens=1 << 40), M.MOE_EUNSUPPORTED),
    (dict(tokens=150_000), M.MOE_EUNSUPPORTED),          # x would need 2 GiB or more
    (dict(d_model=1 << 16, d_expert=1 << 14, d_shared=1 << 14),
     M.MOE_EUNSUPPORTED),                                  # one weight matrix near 2 GiB
    (dict(tokens=(1 << 23) + 1, d_model=64, d_expert=64, d_shared=64, top_k=1),
     M.MOE_EUNSUPPORTED),                                  # per-token grids above 2^32 items
])
def test_bad_dims_rejected(bad, code):
    kw = dict(tokens=128, d_model=7168, n_experts=384, top_k=8, d_expert=2048, d_shared=2048,
              routed_scale=2.827)
    kw.update(bad)
    d = M.moe_dims(**kw)
    n = ctypes.c_size_t(0)
    assert M.lib().moe_workspace_bytes(ctypes.byref(d), ctypes.byref(n)) == code


def test_largest_x_accepted():
    # x just under 2 GiB at d = 7168 (149,796 tokens) is addressable
    d = M.moe_dims(149_796, 7168, 384, 8, 2048, 2048)
    n = ctypes.c_size_t(0)
    assert M.lib().moe_workspace_bytes(ctypes.byref(d), ctypes.byref(n)) == M.MOE_OK


def _fake(addr):
    return ctypes.c_void_p(addr)


def test_null_and_misaligned_pointers_rejected():
    L = M.lib()
    d = _k2()
    P = _fake(0x100000)          # 16-byte aligned, never dereferenced: every call fails first
    Q = _fake(0x100002)          # misaligned
    ws_need = M.moe_workspace_bytes(d)
    # null x
    assert L.moe_forward(ctypes.byref(d), None, P, P, P, P, P, P, P, P, P, P, ws_need, None) == M.MOE_EINVAL
    # misaligned weight
    assert L.moe_forward(ctypes.byref(d), P, P, P, Q, P, P, P, P, P, P, P, ws_need, None) == M.MOE_EINVAL
    # workspace too small
    assert L.moe_forward(ctypes.byref(d), P, P, P, P, P, P, P, P, P, P, P, ws_need - 1, None) == M.MOE_EWORKSPACE
    # workspace misaligned
    assert L.moe_forward(ctypes.byref(d), P, P, P, P, P, P, P, P, P, P, _fake(0x100010), ws_need, None) == M.MOE_EINVAL
    # shared expert declared but missing
    assert L.moe_expert_down(ctypes.byref(d), P, P, P, None, P, P, P, ws_need, None) == M.MOE_EINVAL
    # route without logits needs the workspace
    assert L.moe_route(ctypes.byref(d), P, P, P, P, P, None, None, 0, None) == M.MOE_EINVAL
    assert L.moe_route(ctypes.byref(d), P, P, P, P, P, None, P, 16, None) == M.MOE_EWORKSPACE
    # null dims
    assert L.moe_combine(None, P, P, P, P, P, None) == M.MOE_EINVAL


def test_zero_tokens_is_a_noop():
    L = M.lib()
    d = _k2(0)
    assert L.moe_forward(ctypes.byref(d), None, None, None, None, None, None, None, None, None,
                         None, None, 0, None) == M.MOE_OK
    assert L.moe_combine(ctypes.byref(d), None, None, None, None, None, None) == M.MOE_OK


def test_binding_raises_on_error():
    with pytest.raises(M.MoeError) as ei:
        M.moe_workspace_bytes(M.moe_dims(1, 7168, 384, 9, 2048, 2048))
    assert ei.value.status == M.MOE_EUNSUPPORTED


def test_binding_refuses_host_tensors():
    """A host tensor never reaches the library (a kernel would fault on its address)."""
    import torch
    d = M.moe_dims(4, 64, 4, 2, 64, 64)
    y = torch.zeros(8, 64)
    with pytest.raises(ValueError, match="device tensors"):
        M.moe_combine(d, y, torch.zeros(8, dtype=torch.int32), torch.zeros(8), None,
                      torch.zeros(4, 64, dtype=torch.bfloat16))


def test_latent_dims_checked():
    n = ctypes.c_size_t(0)
    L = M.lib()
    d = _k2(4096)
    assert L.moe_latent_workspace_bytes(ctypes.byref(d), 3584, ctypes.byref(n)) == M.MOE_OK
    assert n.value > M.moe_workspace_bytes(_k2(0))
    assert L.moe_latent_workspace_bytes(ctypes.byref(d), 100, ctypes.byref(n)) == M.MOE_EUNSUPPORTED
    assert L.moe_latent_workspace_bytes(ctypes.byref(d), 0, ctypes.byref(n)) == M.MOE_EINVAL
    assert L.moe_latent_workspace_bytes(ctypes.byref(d), 16384, ctypes.byref(n)) == M.MOE_EUNSUPPORTED
    P = _fake(0x100000)
    assert L.moe_forward_latent(ctypes.byref(d), 3584, None, P, P, P, P, P, P, P, P, P, P, P, P,
                                n.value, None) == M.MOE_EINVAL
    assert L.moe_forward_latent(ctypes.byref(d), 3584, P, P, P, P, P, P, P, P, P, P, P, P, P,
                                n.value - 1, None) == M.MOE_EWORKSPACE


def test_block_arguments_checked():
    L = M.lib()
    d = _k2(128)
    P = _fake(0x100000)
    Q = _fake(0x10000000)        # [T, d] bf16 is 1.8 MB: far from P
    base = M.moe_workspace_bytes(d)
    need = M.moe_block_workspace_bytes(d)
    assert need == base + 128 * 7168 * 2
    args = lambda x, g, eps, out, n: (ctypes.byref(d), x, g, ctypes.c_float(eps), P, P, P, P, P,  # noqa: E731
                                      P, P, P, out, P, n, None)
    # the x_ffn buffer is part of the workspace
    assert L.moe_forward_block(*args(P, P, 1e-6, Q, base)) == M.MOE_EWORKSPACE
    assert L.moe_forward_block(*args(P, P, 1e-6, Q, need - 1)) == M.MOE_EWORKSPACE
    # output aliasing the residual, or overlapping it by one row, null gain, bad eps
    assert L.moe_forward_block(*args(P, P, 1e-6, P, need)) == M.MOE_EINVAL
    assert L.moe_forward_block(*args(P, P, 1e-6, _fake(0x100000 + 7168 * 2), need)) == M.MOE_EINVAL
    assert L.moe_forward_block(*args(_fake(0x100000 + 7168 * 2), P, 1e-6, P, need)) == M.MOE_EINVAL
    assert L.moe_forward_block(*args(P, None, 1e-6, Q, need)) == M.MOE_EINVAL
    assert L.moe_forward_block(*args(P, P, -1.0, Q, need)) == M.MOE_EINVAL
    assert L.moe_forward_block(*args(P, P, float("nan"), Q, need)) == M.MOE_EINVAL
    z = _k2(0)
    assert L.moe_forward_block(ctypes.byref(z), None, None, ctypes.c_float(1e-6), None, None, None,
                               None, None, None, None, None, None, None, 0, None) == M.MOE_OK


def test_fp8_arguments_checked():
    L = M.lib()
    P = _fake(0x100000)
    ws_need = M.moe_workspace_bytes(_k2(128))
    good = B.MoeFp8Weights(*([0x100000] * 12))
    d = _k2(128)
    args = lambda dims, w, n: (ctypes.byref(dims), P, P, P, w, P, P, n, None)  # noqa: E731
    # null weight struct, misaligned codes, scales only need 4 bytes
    assert L.moe_forward_fp8(ctypes.byref(d), P, P, P, None, P, P, ws_need, None) == M.MOE_EINVAL
    bad = B.MoeFp8Weights(*([0x100000] * 12))
    bad.w2 = 0x100004
    assert L.moe_forward_fp8(*args(d, ctypes.byref(bad), ws_need)) == M.MOE_EINVAL
    sc4 = B.MoeFp8Weights(*([0x100000] * 12))
    sc4.w1_scale = 0x100004
    assert L.moe_forward_fp8(*args(d, ctypes.byref(sc4), ws_need - 1)) == M.MOE_EWORKSPACE
    # widths must be multiples of 128 (the scale blocks) and at most 16384
    d192 = M.moe_dims(128, 7168, 384, 8, 192, 192)
    assert L.moe_forward_fp8(*args(d192, ctypes.byref(good), ws_need)) == M.MOE_EUNSUPPORTED
    d_big = M.moe_dims(16, 16512, 8, 2, 128, 128)
    n = ctypes.c_size_t(0)
    assert L.moe_workspace_bytes(ctypes.byref(d_big), ctypes.byref(n)) == M.MOE_OK
    assert L.moe_forward_fp8(ctypes.byref(d_big), P, P, P, ctypes.byref(good), P, P, n.value,
                             None) == M.MOE_EUNSUPPORTED
    # the shared expert's pointers are checked only when there is one
    ns = M.moe_dims(128, 7168, 384, 8, 2048, 0)
    noshared = B.MoeFp8Weights(*([0x100000] * 6 + [0] * 6))
    assert L.moe_expert_gate_up_fp8(ctypes.byref(ns), P, P, P, ctypes.byref(noshared), P, P, 0,
                                    None) == M.MOE_EWORKSPACE
    assert L.moe_expert_gate_up_fp8(ctypes.byref(d), P, P, P, ctypes.byref(noshared), P, P,
                                    ws_need, None) == M.MOE_EINVAL
    # T = 0: nothing to do, nothing dereferenced
    z = _k2(0)
    assert L.moe_forward_fp8(ctypes.byref(z), None, None, None, ctypes.byref(good), None, None, 0,
                             None) == M.MOE_OK
    assert L.moe_expert_down_fp8(ctypes.byref(z), None, None, ctypes.byref(good), None, None,
                                 None, 0, None) == M.MOE_OK


def test_noalloc_host_checks():
    """moe_forward_noalloc rejects, before touching the GPU, null or misaligned pointers and
    dims whose intermediates exceed its fixed scratch (MOE_ESCRATCH, with a message naming
    the limit); T = 0 is a no-op."""
    L = M.lib()
    P = _fake(0x100000)
    Q = _fake(0x100002)
    assert B.NOALLOC_SCRATCH_BYTES == 128 << 20
    d = _k2(128)
    assert M.moe_workspace_bytes(d) <= B.NOALLOC_SCRATCH_BYTES
    assert L.moe_forward_noalloc(ctypes.byref(d), None, P, P, P, P, P, P, P, P, P, None) == M.MOE_EINVAL
    assert L.moe_forward_noalloc(ctypes.byref(d), P, P, P, Q, P, P, P, P, P, P, None) == M.MOE_EINVAL
    # the largest K2 batch that fits, and the first that does not
    assert M.moe_workspace_bytes(_k2(512)) <= B.NOALLOC_SCRATCH_BYTES < M.moe_workspace_bytes(_k2(513))
    big = _k2(513)
    assert L.moe_forward_noalloc(ctypes.byref(big), P, P, P, P, P, P, P, P, P, P, None) == M.MOE_ESCRATCH
    assert "MOE_NOALLOC_SCRATCH_BYTES" in M.status_str(M.MOE_ESCRATCH)
    z = _k2(0)
    assert L.moe_forward_noalloc(ctypes.byref(z), None, None, None, None, None, None, None, None,
                                 None, None, None) == M.MOE_OK
    assert L.moe_forward_noalloc(None, P, P, P, P, P, P, P, P, P, P, None) == M.MOE_EINVAL
