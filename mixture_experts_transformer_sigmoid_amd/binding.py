"""Thin ctypes binding of libmoe (include/moe.h): argument marshalling only.

Every function has the C entry point's name and argument order; tensors are passed as
device pointers, the stream defaults to torch's current stream.  All arithmetic runs
in the library's HIP kernels; there is no fallback: a missing library raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# MOE_LIB names another build of the same library (the host-sanitizer build of build.py)
LIB_PATH = os.environ.get("MOE_LIB") or os.path.join(_PKG, "libmoe.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP, MOE_ESCRATCH = range(6)
# moe.h's MOE_NOALLOC_SCRATCH_BYTES: the fixed device scratch of moe_forward_noalloc
NOALLOC_SCRATCH_BYTES = 128 << 20
# moe.h's MOE_HSPLIT_MAX_TOP_K and MOE_HSPLIT_MAX_D_EXPERT: up to this top_k, or up to this
# expert width, the bf16 entry points keep h in two bf16 parts, rows of 2I
HSPLIT_MAX_TOP_K = 2
HSPLIT_MAX_D_EXPERT = 128


def h_width(dims) -> int:
    """Columns per row of h for the bf16 entry points (moe_expert_gate_up / _down)."""
    two = int(dims.top_k) <= HSPLIT_MAX_TOP_K or int(dims.d_expert) <= HSPLIT_MAX_D_EXPERT
    return (2 if two else 1) * int(dims.d_expert)

# every exported symbol of include/moe.h
EXPORTS = ("moe_status_str", "moe_workspace_bytes", "moe_route", "moe_permute",
           "moe_expert_gate_up", "moe_expert_down", "moe_expert_ffn", "moe_combine",
           "moe_forward", "moe_latent_workspace_bytes", "moe_forward_latent",
           "moe_block_workspace_bytes", "moe_forward_block", "moe_expert_gate_up_fp8",
           "moe_expert_down_fp8", "moe_forward_fp8", "moe_forward_noalloc",
           "moe_workspace_release")


class MoeDims(ctypes.Structure):
    _fields_ = [("tokens", ctypes.c_int64), ("d_model", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("d_expert", ctypes.c_int32), ("d_shared", ctypes.c_int32),
                ("routed_scale", ctypes.c_float)]


class MoeFp8Weights(ctypes.Structure):
    """moe_fp8_weights: device pointers of the E4M3 codes and their block scales."""
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "w1", "w3", "w2", "w1_scale", "w3_scale", "w2_scale",
        "ws1", "ws3", "ws2", "ws1_scale", "ws3_scale", "ws2_scale")]


def fp8_weights(t: dict) -> MoeFp8Weights:
    """MoeFp8Weights from a dict of device tensors keyed by the field names (the shared
    expert's entries may be missing)."""
    return MoeFp8Weights(*[t[n].data_ptr() if t.get(n) is not None else None
                           for n, _ in MoeFp8Weights._fields_])


class MoeError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(msg)
        self.status = status


_lib = None
_P = ctypes.c_void_p
_S = ctypes.c_size_t


def lib():
    """Load libmoe.so (after torch, so both share one HIP runtime).  Raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libmoe.so not built ({LIB_PATH}); run __graft_entry__.build()")
    L = ctypes.CDLL(LIB_PATH)
    st = ctypes.c_int
    D = ctypes.POINTER(MoeDims)
    L.moe_status_str.restype = ctypes.c_char_p
    L.moe_status_str.argtypes = [ctypes.c_int]
    sig = {
        "moe_workspace_bytes": [D, ctypes.POINTER(ctypes.c_size_t)],
        "moe_route": [D, _P, _P, _P, _P, _P, _P, _P, _S, _P],
        "moe_permute": [D, _P, _P, _P, _P, _P, _P, _S, _P],
        "moe_expert_gate_up": [D, _P, _P, _P, _P, _P, _P, _P, _P, _P, _S, _P],
        "moe_expert_down": [D, _P, _P, _P, _P, _P, _P, _P, _S, _P],
        "moe_expert_ffn": [D, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _S, _P],
        "moe_combine": [D, _P, _P, _P, _P, _P, _P],
        "moe_forward": [D, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _S, _P],
        "moe_forward_noalloc": [D, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
        "moe_workspace_release": [_P],
        "moe_block_workspace_bytes": [D, ctypes.POINTER(ctypes.c_size_t)],
        "moe_forward_block": [D, _P, _P, ctypes.c_float, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                              _S, _P],
        "moe_expert_gate_up_fp8": [D, _P, _P, _P, ctypes.POINTER(MoeFp8Weights), _P, _P, _S, _P],
        "moe_expert_down_fp8": [D, _P, _P, ctypes.POINTER(MoeFp8Weights), _P, _P, _P, _S, _P],
        "moe_forward_fp8": [D, _P, _P, _P, ctypes.POINTER(MoeFp8Weights), _P, _P, _S, _P],
        "moe_latent_workspace_bytes": [D, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)],
        "moe_forward_latent": [D, ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                               _P, _S, _P],
    }
    for name, args in sig.items():
        fn = getattr(L, name)
        fn.restype = st
        fn.argtypes = args
    _lib = L
    return L


def status_str(status: int) -> str:
    return lib().moe_status_str(int(status)).decode()


def _check(rc):
    if rc != MOE_OK:
        raise MoeError(rc, status_str(rc))


def moe_dims(tokens, d_model, n_experts, top_k, d_expert, d_shared, routed_scale=2.827):
    return MoeDims(int(tokens), int(d_model), int(n_experts), int(top_k), int(d_expert),
                   int(d_shared), float(routed_scale))


def dims_for(cfg: dict, tokens=None) -> MoeDims:
    """moe_dims from a config dict (keys as in synth_inputs.CONFIGS)."""
    return moe_dims(cfg["tokens"] if tokens is None else tokens, cfg["d_model"], cfg["n_experts"],
                    cfg["top_k"], cfg["d_expert"], cfg["d_shared"], cfg.get("routed_scale", 2.827))


def _ptr(t):
    """A tensor's device address.  Host tensors and strided views are refused: the library
    cannot tell a host address from a device one (a kernel reading it faults), and it reads
    every array densely in the layout moe.h gives."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"libmoe takes device tensors; got one on {t.device}")
    if not t.is_contiguous():
        raise ValueError("libmoe takes contiguous tensors; got a strided view")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def moe_workspace_bytes(dims: MoeDims) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_workspace_bytes(ctypes.byref(dims), ctypes.byref(n)))
    return n.value


def workspace(dims: MoeDims, device="cuda") -> torch.Tensor:
    """A device buffer of moe_workspace_bytes(dims) bytes (torch owns the memory)."""
    return torch.empty(max(moe_workspace_bytes(dims), 256), dtype=torch.uint8, device=device)


def routing_in_workspace(dims: MoeDims, ws: torch.Tensor) -> dict:
    """Views of the routing and permutation arrays a layer entry point leaves at the start
    of its workspace (moe.h, moe_workspace_bytes): topk_idx, topk_w, counts, offsets,
    perm_rows, inv_perm."""
    T, E, k = int(dims.tokens), int(dims.n_experts), int(dims.top_k)
    out, off = {}, 0
    for name, n, dt, shape in (("topk_idx", T * k, torch.int32, (T, k)),
                               ("topk_w", T * k, torch.float32, (T, k)),
                               ("counts", E, torch.int32, (E,)),
                               ("offsets", E + 1, torch.int32, (E + 1,)),
                               ("perm_rows", T * k, torch.int32, (T * k,)),
                               ("inv_perm", T * k, torch.int32, (T * k,))):
        out[name] = ws[off:off + 4 * n].view(dt).view(shape)
        off += (4 * n + 255) // 256 * 256
    return out


def _ws(ws):
    return (None, 0) if ws is None else (_ptr(ws), ws.numel() * ws.element_size())


def moe_route(dims, x, w_router, bias, topk_idx, topk_w, logits=None, ws=None, stream=None):
    wp, wn = _ws(ws)
    _check(lib().moe_route(ctypes.byref(dims), _ptr(x), _ptr(w_router), _ptr(bias), _ptr(topk_idx),
                           _ptr(topk_w), _ptr(logits), wp, wn, _stream(stream)))


def moe_permute(dims, topk_idx, counts, offsets, perm_rows, inv_perm, ws, stream=None):
    wp, wn = _ws(ws)
    _check(lib().moe_permute(ctypes.byref(dims), _ptr(topk_idx), _ptr(counts), _ptr(offsets),
                             _ptr(perm_rows), _ptr(inv_perm), wp, wn, _stream(stream)))


def moe_expert_gate_up(dims, x, perm_rows, offsets, w1, w3, ws1, ws3, h, ws, stream=None):
    wp, wn = _ws(ws)
    _check(lib().moe_expert_gate_up(ctypes.byref(dims), _ptr(x), _ptr(perm_rows), _ptr(offsets),
                                    _ptr(w1), _ptr(w3), _ptr(ws1), _ptr(ws3), _ptr(h), wp, wn,
                                    _stream(stream)))


def moe_expert_down(dims, h, offsets, w2, ws2, y_routed, y_shared, ws, stream=None):
    wp, wn = _ws(ws)
    _check(lib().moe_expert_down(ctypes.byref(dims), _ptr(h), _ptr(offsets), _ptr(w2), _ptr(ws2),
                                 _ptr(y_routed), _ptr(y_shared), wp, wn, _stream(stream)))


def moe_expert_ffn(dims, x, perm_rows, offsets, w1, w3, w2, ws1, ws3, ws2, y_routed, y_shared, ws,
                   stream=None):
    wp, wn = _ws(ws)
    _check(lib().moe_expert_ffn(ctypes.byref(dims), _ptr(x), _ptr(perm_rows), _ptr(offsets),
                                _ptr(w1), _ptr(w3), _ptr(w2), _ptr(ws1), _ptr(ws3), _ptr(ws2),
                                _ptr(y_routed), _ptr(y_shared), wp, wn, _stream(stream)))


def moe_combine(dims, y_routed, inv_perm, topk_w, y_shared, out, stream=None):
    _check(lib().moe_combine(ctypes.byref(dims), _ptr(y_routed), _ptr(inv_perm), _ptr(topk_w),
                             _ptr(y_shared), _ptr(out), _stream(stream)))


def moe_forward(dims, x, w_router, bias, w1, w3, w2, ws1, ws3, ws2, out, ws, stream=None):
    wp, wn = _ws(ws)
    _check(lib().moe_forward(ctypes.byref(dims), _ptr(x), _ptr(w_router), _ptr(bias), _ptr(w1),
                             _ptr(w3), _ptr(w2), _ptr(ws1), _ptr(ws3), _ptr(ws2), _ptr(out), wp,
                             wn, _stream(stream)))


def moe_workspace_release(ws):
    """The workspace will not be used again: its slot of the router's arrival counts may go
    to another workspace (moe.h, moe_workspace_release)."""
    _check(lib().moe_workspace_release(_ptr(ws)))


def moe_forward_noalloc(dims, x, w_router, bias, w1, w3, w2, ws1, ws3, ws2, out, stream=None):
    """moe_forward without a workspace: the library's fixed device scratch holds the
    intermediates (raises MoeError MOE_ESCRATCH when the dims need more)."""
    _check(lib().moe_forward_noalloc(ctypes.byref(dims), _ptr(x), _ptr(w_router), _ptr(bias),
                                     _ptr(w1), _ptr(w3), _ptr(w2), _ptr(ws1), _ptr(ws3),
                                     _ptr(ws2), _ptr(out), _stream(stream)))


def moe_block_workspace_bytes(dims: MoeDims) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_block_workspace_bytes(ctypes.byref(dims), ctypes.byref(n)))
    return n.value


def block_workspace(dims: MoeDims, device="cuda") -> torch.Tensor:
    return torch.empty(max(moe_block_workspace_bytes(dims), 256), dtype=torch.uint8, device=device)


def moe_forward_block(dims, x_res, norm_w, norm_eps, w_router, bias, w1, w3, w2, ws1, ws3, ws2,
                      out, ws, stream=None):
    wp, wn = _ws(ws)
    _check(lib().moe_forward_block(ctypes.byref(dims), _ptr(x_res), _ptr(norm_w),
                                   float(norm_eps), _ptr(w_router), _ptr(bias), _ptr(w1),
                                   _ptr(w3), _ptr(w2), _ptr(ws1), _ptr(ws3), _ptr(ws2), _ptr(out),
                                   wp, wn, _stream(stream)))


def moe_expert_gate_up_fp8(dims, x, perm_rows, offsets, w: MoeFp8Weights, h, ws, stream=None):
    wp, wn = _ws(ws)
    _check(lib().moe_expert_gate_up_fp8(ctypes.byref(dims), _ptr(x), _ptr(perm_rows),
                                        _ptr(offsets), ctypes.byref(w), _ptr(h), wp, wn,
                                        _stream(stream)))


def moe_expert_down_fp8(dims, h, offsets, w: MoeFp8Weights, y_routed, y_shared, ws, stream=None):
    wp, wn = _ws(ws)
    _check(lib().moe_expert_down_fp8(ctypes.byref(dims), _ptr(h), _ptr(offsets), ctypes.byref(w),
                                     _ptr(y_routed), _ptr(y_shared), wp, wn, _stream(stream)))


def moe_forward_fp8(dims, x, w_router, bias, w: MoeFp8Weights, out, ws, stream=None):
    wp, wn = _ws(ws)
    _check(lib().moe_forward_fp8(ctypes.byref(dims), _ptr(x), _ptr(w_router), _ptr(bias),
                                 ctypes.byref(w), _ptr(out), wp, wn, _stream(stream)))


def moe_latent_workspace_bytes(dims: MoeDims, d_latent: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_latent_workspace_bytes(ctypes.byref(dims), int(d_latent), ctypes.byref(n)))
    return n.value


def latent_workspace(dims: MoeDims, d_latent: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(moe_latent_workspace_bytes(dims, d_latent), 256), dtype=torch.uint8,
                       device=device)


def moe_forward_latent(dims, d_latent, x, w_router, bias, w_down, w1, w3, w2, w_up, ws1, ws3, ws2,
                       out, ws, stream=None):
    wp, wn = _ws(ws)
    _check(lib().moe_forward_latent(ctypes.byref(dims), int(d_latent), _ptr(x), _ptr(w_router),
                                    _ptr(bias), _ptr(w_down), _ptr(w1), _ptr(w3), _ptr(w2),
                                    _ptr(w_up), _ptr(ws1), _ptr(ws3), _ptr(ws2), _ptr(out), wp,
                                    wn, _stream(stream)))
