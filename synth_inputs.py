"""Seeded synthetic inputs for the MoE FFN layer (shared by tests, smoke and bench).

This module only draws random numbers: it holds none of the method's arithmetic.  Both
the HIP path and the CPU oracle are fed the very same tensors it returns (the oracle
gets host copies).

Recipe (per tensor; "fan_in" is the width the matrix reads):
  x    ~ N(0, 1)                   [T, d]       bf16
  W_r  ~ N(0, 1/d)                 [E, d]       fp32   (router, [out, in])
  b    ~ U(-0.01, 0.01)            [E]          fp32   (selection bias)
  W1, W3 ~ N(0, 1/d)               [E, I, d]    bf16
  W2   ~ N(0, 1/I)                 [E, d, I]    bf16
  Ws1, Ws3 ~ N(0, 1/d), Ws2 ~ N(0, 1/Is)        bf16   (shared expert)
Skewed routing: b_e = -0.5 * ln(rank_e) with rank a seeded permutation of 1..E, so a
few experts take most tokens and many take none.
Latent variant: W_down ~ N(0, 1/d) [L, d], experts on the latent width L, W_up ~
N(0, 1/L) [d, L].
FP8 weights: the same N(0, 1/fan_in) draws stored as E4M3 codes with one fp32 scale
per 128 x 128 block (block max |w| / 448), as a block-scaled checkpoint holds them.
Block (pre-MoE norm + residual): the residual stream x'_n = N(0, 1) * c_j with a
per-channel scale c_j ~ U(0.25, 4) (so the norm has real work), bf16; the norm gain
gamma ~ U(0.5, 1.5) rounded to bf16 (a checkpoint's gain is bf16), passed as fp32.

Every tensor (and every expert slice of the stacked weights) has its own seed derived
from (seed, tensor id, slice), so one expert can be regenerated alone.  Values are drawn
in fp32 with torch's generator on the requested device, then rounded to nearest-even
bf16 where the layer stores bf16.
"""
from __future__ import annotations

import math

import torch

# tensor ids (stable: they enter the per-tensor seeds)
TID = {"x": 0, "w_r": 1, "b": 2, "w1": 3, "w3": 4, "w2": 5, "ws1": 6, "ws3": 7, "ws2": 8,
       "w_down": 9, "w_up": 10, "rank": 11, "x_res": 12, "norm_w": 13, "chan": 14}

CONFIGS = {
    # small case the oracle finishes in well under a second
    "tiny": dict(tokens=64, d_model=256, n_experts=16, top_k=2, d_expert=128, d_shared=128,
                 routed_scale=2.827, bias="uniform"),
    # K2 shape, decode-sized batch
    "k2_decode": dict(tokens=128, d_model=7168, n_experts=384, top_k=8, d_expert=2048,
                      d_shared=2048, routed_scale=2.827, bias="uniform"),
    # K2 shape, prefill (4 sequences x 2048 positions, flattened: the layer is per token)
    "k2_prefill": dict(tokens=8192, d_model=7168, n_experts=384, top_k=8, d_expert=2048,
                       d_shared=2048, routed_scale=2.827, bias="uniform"),
    # K2 shape, skewed routing
    "k2_skew": dict(tokens=4096, d_model=7168, n_experts=384, top_k=8, d_expert=2048,
                    d_shared=2048, routed_scale=2.827, bias="zipf"),
    # small latent MoE case the oracle finishes in well under a second
    "tiny_latent": dict(tokens=64, d_model=256, n_experts=16, top_k=2, d_expert=128, d_shared=128,
                        routed_scale=2.827, bias="uniform", d_latent=128),
    # latent MoE: experts on a 3584-wide latent
    "latent": dict(tokens=4096, d_model=7168, n_experts=384, top_k=8, d_expert=2048,
                   d_shared=2048, routed_scale=2.827, bias="uniform", d_latent=3584),
}


def _seed(seed: int, tid: int, part: int = 0) -> int:
    return ((seed * 1_000_003 + tid) * 1_000_003 + part) % (2 ** 62)


def _gen(device, seed, tid, part=0):
    g = torch.Generator(device=device)
    g.manual_seed(_seed(seed, tid, part))
    return g


def normal(shape, std, dtype, device, seed, tid, part=0):
    g = _gen(device, seed, tid, part)
    v = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        v.mul_(std)
    return v.to(dtype)


def _stacked(n, shape, std, device, seed, tid):
    out = torch.empty((n,) + tuple(shape), dtype=torch.bfloat16, device=device)
    for e in range(n):
        out[e] = normal(shape, std, torch.bfloat16, device, seed, tid, e + 1)
    return out


def bias(cfg, device, seed=0):
    E = cfg["n_experts"]
    kind = cfg.get("bias", "uniform")
    if kind == "uniform":
        g = _gen(device, seed, TID["b"])
        return (torch.rand(E, generator=g, device=device, dtype=torch.float32) * 0.02 - 0.01)
    if kind == "zipf":
        g = _gen("cpu", seed, TID["rank"])
        rank = torch.randperm(E, generator=g).to(torch.float64) + 1.0
        return (-0.5 * torch.log(rank)).to(torch.float32).to(device)
    if kind == "zero":
        return torch.zeros(E, dtype=torch.float32, device=device)
    raise ValueError(kind)


def make_weights(cfg, device="cpu", seed=0, shared=True):
    """The layer's learned arrays (router, bias excluded) for a config dict or name."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    d, E = cfg["d_model"], cfg["n_experts"]
    I, Is = cfg["d_expert"], cfg["d_shared"]
    L = cfg.get("d_latent")
    w = L if L else d                       # the width the routed experts read
    out = {
        "w_r": normal((E, d), 1.0 / math.sqrt(d), torch.float32, device, seed, TID["w_r"]),
        "w1": _stacked(E, (I, w), 1.0 / math.sqrt(w), device, seed, TID["w1"]),
        "w3": _stacked(E, (I, w), 1.0 / math.sqrt(w), device, seed, TID["w3"]),
        "w2": _stacked(E, (w, I), 1.0 / math.sqrt(I), device, seed, TID["w2"]),
    }
    if shared and Is:
        out["ws1"] = normal((Is, d), 1.0 / math.sqrt(d), torch.bfloat16, device, seed, TID["ws1"])
        out["ws3"] = normal((Is, d), 1.0 / math.sqrt(d), torch.bfloat16, device, seed, TID["ws3"])
        out["ws2"] = normal((d, Is), 1.0 / math.sqrt(Is), torch.bfloat16, device, seed, TID["ws2"])
    if L:
        out["w_down"] = normal((L, d), 1.0 / math.sqrt(d), torch.bfloat16, device, seed, TID["w_down"])
        out["w_up"] = normal((d, L), 1.0 / math.sqrt(L), torch.bfloat16, device, seed, TID["w_up"])
    return out


FP8_BLOCK = 128
FP8_MAX = 448.0


def _fp8_blocks(w):
    """Store an fp32 [N, K] matrix the way an FP8 block-scaled checkpoint does: one fp32
    scale per 128 x 128 block (the block's largest magnitude over 448, the largest E4M3
    value; 1 for an all-zero block) and E4M3 bytes of w / scale (torch's float8_e4m3fn
    cast, nearest even).  Returns (uint8 [N, K], float32 [N/128, K/128])."""
    N, K = w.shape
    blk = w.reshape(N // FP8_BLOCK, FP8_BLOCK, K // FP8_BLOCK, FP8_BLOCK)
    amax = blk.abs().amax(dim=(1, 3))
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
    q = (blk / scale[:, None, :, None]).reshape(N, K).to(torch.float8_e4m3fn)
    return q.view(torch.uint8), scale.to(torch.float32)


def _stacked_fp8(n, shape, std, device, seed, tid):
    q = torch.empty((n,) + tuple(shape), dtype=torch.uint8, device=device)
    sc = torch.empty((n, shape[0] // FP8_BLOCK, shape[1] // FP8_BLOCK), dtype=torch.float32,
                     device=device)
    for e in range(n):
        q[e], sc[e] = _fp8_blocks(normal(shape, std, torch.float32, device, seed, tid, e + 1))
    return q, sc


def make_fp8_weights(cfg, device="cpu", seed=0, shared=True):
    """Expert weights in FP8 block-scaled form: for each of w1, w3, w2 (and ws1, ws3, ws2)
    a uint8 array of E4M3 codes with the bf16 layout, plus "<name>_scale" [.., N/128,
    K/128] fp32.  The same normal draws as make_weights, before any rounding; the router
    stays fp32."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    d, E = cfg["d_model"], cfg["n_experts"]
    I, Is = cfg["d_expert"], cfg["d_shared"]
    out = {"w_r": normal((E, d), 1.0 / math.sqrt(d), torch.float32, device, seed, TID["w_r"])}
    out["w1"], out["w1_scale"] = _stacked_fp8(E, (I, d), 1.0 / math.sqrt(d), device, seed, TID["w1"])
    out["w3"], out["w3_scale"] = _stacked_fp8(E, (I, d), 1.0 / math.sqrt(d), device, seed, TID["w3"])
    out["w2"], out["w2_scale"] = _stacked_fp8(E, (d, I), 1.0 / math.sqrt(I), device, seed, TID["w2"])
    if shared and Is:
        for name, shape, fan in (("ws1", (Is, d), d), ("ws3", (Is, d), d), ("ws2", (d, Is), Is)):
            out[name], out[name + "_scale"] = _fp8_blocks(
                normal(shape, 1.0 / math.sqrt(fan), torch.float32, device, seed, TID[name]))
    return out


def make_activations(cfg, device="cpu", seed=0):
    """The token batch x and the selection bias b for a config dict or name."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    return {"x": normal((cfg["tokens"], cfg["d_model"]), 1.0, torch.bfloat16, device, seed, TID["x"]),
            "b": bias(cfg, device, seed)}


def make_block_activations(cfg, device="cpu", seed=0):
    """Residual stream x'_n [T, d] bf16, norm gain [d] fp32 and the selection bias."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    d = cfg["d_model"]
    g = _gen(device, seed, TID["chan"])
    chan = torch.rand(d, generator=g, device=device, dtype=torch.float32) * 3.75 + 0.25
    x = normal((cfg["tokens"], d), 1.0, torch.float32, device, seed, TID["x_res"])
    g = _gen(device, seed, TID["norm_w"])
    gain = torch.rand(d, generator=g, device=device, dtype=torch.float32) + 0.5
    return {"x_res": (x * chan).to(torch.bfloat16),
            "norm_w": gain.to(torch.bfloat16).to(torch.float32),
            "b": bias(cfg, device, seed)}


def make_inputs(cfg, device="cpu", seed=0, shared=True):
    """All inputs of the layer for a config dict (or a CONFIGS name)."""
    out = make_weights(cfg, device, seed, shared)
    out.update(make_activations(cfg, device, seed))
    return out


def with_overrides(name, **kw):
    cfg = dict(CONFIGS[name])
    cfg.update(kw)
    return cfg
