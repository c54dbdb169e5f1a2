"""Plain CPU oracle of the sigmoid-routed mixture-of-experts FFN (Kimi K2 / DeepSeek-V3 style).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or run this
module: only the tests, the smoke check in ``__graft_entry__`` and the CPU-baseline leg
of ``bench.py`` use it.  It shares no code with the HIP library and imports nothing
from it; it takes plain numpy arrays (any float dtype) and computes in float64.

Sources (the pages this follows; cited by page title and the part of the page):

* "Kimi K2 · Transformer blocks" (atlas.klimoza.dev, MoE transformer block), the
  mixture-of-experts equations:
      z = x_ffn W_r ;  s = sigma(z) ;  E_sel_i = [ i in top_8(s + b) ] ;
      G_i = 2.827 s_i E_sel_i / sum_j s_j E_sel_j ;
      g = x W1 ; u = x W3 ; a = g sigma(g) ; h = a (.) u ; E_i = h W2 ;
      y_routed = sum_{i=1..384} G_i E_i ; y_shared = same SwiGLU with the shared
      expert's weights ; Delta_ffn = y_routed + y_shared,
  and the table "Exact per-instance accounting" (MoE parameters 16,958,226,816).
* "nnterp encyclopedia · kimi_k2", section "The mixture of experts" (experts selected on
  sigmoid + bias, all 384 eligible, each gate the selected expert's sigmoid score with
  the bias left out, renormalised and multiplied by 2.827) and section
  "Config" (384 experts, 8 per token, moe_intermediate_size 2048, one shared expert,
  routed_scaling_factor 2.827, norm_topk_prob true, n_group = topk_group = 1).
* "Kimi K3 · Latent up-projection", the printed moe_infer: count tokens per expert,
  group the (token, slot) pairs by expert, run each expert on its group, put the
  outputs back in slot order and take the weighted sum over the k slots in fp32.

Readings where the pages are silent:

* Weights are stored [out, in] (the K3 page states this for its projection); so
  ``w_r`` is [E, d], ``w1``/``w3`` are [E, I, d], ``w2`` is [E, d, I].
* Top-k tie-break: the lower expert index wins.
* The selection compares the stored fp32 activations: z rounded to fp32, s = sigma(z)
  rounded to fp32, then the biased score s + b taken exactly (float64) and compared.
  Tokens whose k-th and (k+1)-th scores lie within 1e-6 are near ties that any fp32
  implementation may order either way.  All values (gates, FFN, sums) are float64.
* The bias enters only the selection, added to sigma(z), never to z and never to G.
* No epsilon in the renormalising denominator (the denominator is > 0).
* RMSNorm: u / sqrt(mean(u^2) + eps) times the gain (the pre-MoE norm; the latent
  variant's norm has unit gain).  The normalised block input x_ffn is a bf16 activation:
  it is rounded to fp32, then to bf16 (nearest-even both times) before use.
* The residual x'_n is added to Delta_ffn in full precision (the kernel adds it in fp32
  and rounds the sum to bf16 once).
* FP8 expert weights: OCP E4M3 values with one fp32 scale per 128 x 128 block of each
  [out, in] matrix; the weight is value x scale, exactly (dequant_fp8_blocks).

Parity pins: tests/test_oracle_pins.py pins every function here against something other
than itself: library routines (scipy, torch), brute force on tiny inputs, closed forms,
invariants and discriminating special cases, the page's parameter count, and a planted
mistake that a pin must catch.  The pages print no worked example of output values, so no
pin is a page-printed output.
"""
from __future__ import annotations

import math

import numpy as np

ALPHA_K2 = 2.827


# ----------------------------------------------------------------------------- shapes
def moe_param_shapes(d_model, n_experts, d_expert, d_shared, n_shared=1):
    """Shapes of every learned array one MoE block holds, [out, in] storage.

    "Kimi K2 · Transformer blocks", parameter table: the mixture of experts counts the
    384 routed SwiGLU experts, the shared expert, the router matrix and the selection
    bias (one value per expert).  Nothing else (no router bias term)."""
    shapes = {
        "w_r": (n_experts, d_model),
        "b": (n_experts,),
        "w1": (n_experts, d_expert, d_model),
        "w3": (n_experts, d_expert, d_model),
        "w2": (n_experts, d_model, d_expert),
    }
    if n_shared:
        i_s = d_shared * n_shared
        shapes.update({"ws1": (i_s, d_model), "ws3": (i_s, d_model), "ws2": (d_model, i_s)})
    return shapes


def moe_param_count(**kw):
    return int(sum(math.prod(s) for s in moe_param_shapes(**kw).values()))


# ------------------------------------------------------------------------ primitives
def sigmoid(v):
    """sigma(v) = 1 / (1 + exp(-v)), float64; the K2 page's s = sigma(z) and a = g sigma(g)."""
    v = np.asarray(v, dtype=np.float64)
    out = np.empty_like(v)
    pos = v >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-v[pos]))
    e = np.exp(v[~pos])            # stable form for negative arguments
    out[~pos] = e / (1.0 + e)
    return out


def silu(v):
    """a = g sigma(g) (K2 page, expert equations; the config's hidden_act 'silu')."""
    v = np.asarray(v, dtype=np.float64)
    return v * sigmoid(v)


def rmsnorm(u, eps=1e-6, gain=None):
    """RMSNorm: u / sqrt(mean(u^2) + eps) per row, times the gain when one is given.

    "Kimi K2 · Transformer blocks": x_ffn = RMSNorm(x'_n) before the mixture of experts,
    with a learned gain of d_model values ("MoE RMSNorm" row of the parameter table) and
    rms_norm_eps 1e-6 in the config; the latent variant's norm has unit gain."""
    u = np.asarray(u, dtype=np.float64)
    v = u / np.sqrt(np.mean(u * u, axis=-1, keepdims=True) + eps)
    return v if gain is None else v * np.asarray(gain, dtype=np.float64)


def round_bf16(v):
    """Round to bfloat16 the way a stored activation is: to fp32 first, then to the
    8-significant-bit bfloat16 grid, both round-to-nearest-even; returned as float64.

    bfloat16 keeps fp32's sign and 8-bit exponent and the top 7 of its 23 stored
    mantissa bits; rounding to nearest-even on the 16 dropped bits adds 0x7fff plus the
    lowest kept bit before truncating.  NaN stays NaN, infinities stay infinite."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    bits = f.view(np.uint32).astype(np.uint64)
    keep_lsb = (bits >> 16) & 1
    r = ((bits + 0x7FFF + keep_lsb) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32).astype(np.float64)
    return np.where(np.isnan(f), np.nan, out)


def _f64(a):
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------- FP8 block-scaled weights
# "nnterp encyclopedia · kimi_k2" (loading a K2 checkpoint) and "Kimi K2 · Transformer
# blocks" (parameter accounting, which leaves out "FP8 block scales"): K2's expert weights
# are stored as FP8 values in blocks, each block with its own scale.  The pages give
# neither the FP8 encoding nor the block size; the reading taken here is the OCP FP8
# E4M3 encoding (1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, no
# infinities, exponent and mantissa all ones = NaN) and square 128 x 128 blocks of the
# [out, in] matrix, one fp32 scale each, the stored weight being value x scale.
FP8_BLOCK = 128


def e4m3_value(code):
    """The real number an OCP E4M3 byte encodes (float64; NaN for the two NaN codes)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 0xF, code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6          # subnormal: 0.m x 2^(1 - 7)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def dequant_fp8_blocks(q, scale, block=FP8_BLOCK):
    """w[n, k] = value(q[n, k]) * scale[n // block, k // block], float64.

    q: uint8 [N, K] (or [..., N, K]); scale: [ceil(N / block), ceil(K / block)] (same
    leading dims)."""
    q = np.asarray(q, dtype=np.uint8)
    sc = _f64(scale)
    v = E4M3_TABLE[q]
    rows = np.arange(q.shape[-2]) // block
    cols = np.arange(q.shape[-1]) // block
    return v * sc[..., rows[:, None], cols[None, :]]


# ---------------------------------------------------------------------------- router
def route(x, w_r, b, top_k, alpha=ALPHA_K2):
    """Router: z = x W_r^T, s = sigma(z), top-k of (s + b), gates alpha * s / sum(s).

    "Kimi K2 · Transformer blocks", MoE equations z, s, E_sel, G_i;
    "nnterp encyclopedia · kimi_k2", "The mixture of experts" (bias only in the choice,
    all 384 experts candidates since n_group = 1).

    Returns a dict:
      z        [T, E] float64 logits
      s        [T, E] float64 sigmoid scores
      score    [T, E] float64 decision scores fl32(sigma(fl32(z))) + b, exact
      score32  [T, E] float32 the same rounded to fp32 (the slot order a fp32 kernel sees)
      topk_idx [T, k] int32   selected experts, descending score, ties to lower index
      topk_w   [T, k] float64 gates G (same order)
      gap      [T]    float64 score of the k-th pick minus that of the (k+1)-th
                      (+inf when k == E): tokens with a tiny gap can flip under rounding
    """
    x = _f64(x)
    w_r = _f64(w_r)
    b = np.asarray(b, dtype=np.float32)
    T = x.shape[0]
    E = w_r.shape[0]
    if not (1 <= top_k <= E):
        raise ValueError("top_k must be in [1, E]")
    z = x @ w_r.T                                  # library matmul as the GEMM step
    s = sigmoid(z)
    # the stored activations are fp32: z and s = sigma(z) rounded to fp32; the biased
    # score is then compared exactly
    z32 = z.astype(np.float32)
    s32 = sigmoid(z32.astype(np.float64)).astype(np.float32)
    score = s32.astype(np.float64) + b.astype(np.float64)
    # order experts by (score descending, index ascending)
    idx = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((idx, -score), axis=-1)
    sel = order[:, :top_k].astype(np.int32)
    if top_k < E:
        kth = np.take_along_axis(score, order[:, top_k - 1:top_k], axis=1)[:, 0]
        nxt = np.take_along_axis(score, order[:, top_k:top_k + 1], axis=1)[:, 0]
        gap = kth - nxt
    else:
        gap = np.full(T, np.inf)
    s_sel = np.take_along_axis(s, sel, axis=1)
    den = s_sel.sum(axis=1, keepdims=True)
    assert np.all(den > 0.0), "renormalising denominator must be positive"
    gates = alpha * s_sel / den
    return {"z": z, "s": s, "score": score, "score32": score.astype(np.float32), "topk_idx": sel,
            "topk_w": gates, "gap": gap}


def gate_matrix(topk_idx, topk_w, n_experts):
    """Dense G [T, E]: G_i on the selected experts, 0 elsewhere (the K2 page's G_i)."""
    T = topk_idx.shape[0]
    G = np.zeros((T, n_experts), dtype=np.float64)
    np.put_along_axis(G, np.asarray(topk_idx, dtype=np.int64), _f64(topk_w), axis=1)
    return G


# --------------------------------------------------------------------------- permute
def permute(topk_idx, n_experts):
    """Group the T*k (token, slot) pairs by expert.

    "Kimi K3 · Latent up-projection", moe_infer: tokens per expert, the flat slots sorted
    by expert, each expert's rows a contiguous segment starting at the running sum.
    Order inside a segment is not fixed by the page; the oracle's is token ascending.

    Returns counts [E], offsets [E+1] (exclusive scan), perm [T*k] (perm[p] = t*k + slot
    of the p-th grouped row) and inv [T*k] (inv[t*k + slot] = its grouped row).
    """
    flat = np.asarray(topk_idx, dtype=np.int64).reshape(-1)
    counts = np.zeros(n_experts, dtype=np.int64)
    for e in flat:                                 # plain histogram
        counts[e] += 1
    offsets = np.zeros(n_experts + 1, dtype=np.int64)
    for e in range(n_experts):                     # exclusive scan
        offsets[e + 1] = offsets[e] + counts[e]
    fill = offsets[:-1].copy()
    perm = np.empty(flat.size, dtype=np.int64)
    inv = np.empty(flat.size, dtype=np.int64)
    for j, e in enumerate(flat):                   # stable scatter, token ascending
        perm[fill[e]] = j
        inv[j] = fill[e]
        fill[e] += 1
    return (counts.astype(np.int32), offsets.astype(np.int32),
            perm.astype(np.int32), inv.astype(np.int32))


def cut_sig16(v):
    """Keep 16 significant bits of each value and drop the rest (rounding toward zero), as
    a 24-bit float row holds an fp32 result: sign, 8-bit exponent and the top 15 stored
    mantissa bits.  From the definition, in float64: with |v| = m 2^e, m in [0.5, 1), the
    kept value is trunc(m 2^16) 2^(e - 16).  Zero, NaN and infinities pass unchanged."""
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)
    out = np.ldexp(np.trunc(m * 65536.0) / 65536.0, e)
    return np.where(np.isfinite(v), out, v)


# ------------------------------------------------------------------------------- FFN
def swiglu(x_rows, w1, w3, w2, bf16_points=()):
    """One SwiGLU expert on a set of rows: g = x W1, u = x W3, a = g sigma(g), h = a u,
    E = h W2 ("Kimi K2 · Transformer blocks", expert and shared-expert equations).
    Weights [out, in]; float64 throughout, except that "h" in bf16_points rounds h to
    bf16 (the diagnostic mode below)."""
    x_rows = _f64(x_rows)
    g = x_rows @ _f64(w1).T
    u = x_rows @ _f64(w3).T
    h = silu(g) * u
    if "h" in bf16_points:
        h = round_bf16(h)
    elif "h2" in bf16_points:
        hi = round_bf16(h)
        h = hi + round_bf16(h - hi)
    return h @ _f64(w2).T


# ------------------------------------------------------- diagnostic: bf16 points
# DIAGNOSTIC ONLY, never a pass/fail reference: moe_sparse(..., bf16_points=...) rounds
# chosen intermediates to bf16 (round_bf16: to fp32, then to bf16, nearest-even) so that
# a difference between the HIP path and the exact oracle can be attributed to a precision
# schedule rather than to a mistake.  The points:
#   "h"           the SwiGLU hidden row, before the down projection
#   "h2"          the same row kept as two bf16 parts, bf16(h) + bf16(h - bf16(h))
#   "expert_out"  each expert's output row E_i
#   "y24"         each expert's output row and the shared expert's output cut to 16
#                 significant bits toward zero (cut_sig16; the 24-bit rows of the layer)
#   "y_routed"    the gate-weighted sum over the k slots
#   "y_shared"    the shared expert's output
#   "out"         the layer output
# PAGE_BF16_POINTS: where a bf16 copy of the module rounds ("Kimi K3 · Latent
# up-projection", moe_infer: expert outputs in the module dtype, weighted sum taken in
# fp32 and cast back; the shared output added in the module dtype).
# KERNEL_BF16_POINTS: the HIP layer's schedule (h is the down GEMM's bf16 operand; expert
# outputs and the shared output kept with 16 significant bits; the weighted sum in fp32;
# one final rounding), and KERNEL_BF16_POINTS_TWO_PART the same with h in two bf16 parts
# (top_k <= 2 or I <= 128).
PAGE_BF16_POINTS = ("h", "expert_out", "y_routed", "y_shared", "out")
KERNEL_BF16_POINTS = ("h", "y24", "out")
KERNEL_BF16_POINTS_TWO_PART = ("h2", "y24", "out")


def _expert_getter(w1, w3, w2):
    return lambda e: (w1[e], w3[e], w2[e])


def moe_dense(x, w_r, b, w1, w3, w2, ws1, ws3, ws2, top_k, alpha=ALPHA_K2):
    """Delta_ffn by the page's dense definition: every expert runs on every token and
    y_routed = sum over all E experts (ascending) of G_i E_i; small inputs only.
    Returns dict with route outputs, y_routed, y_shared, out (all float64)."""
    r = route(x, w_r, b, top_k, alpha)
    E = _f64(w_r).shape[0]
    G = gate_matrix(r["topk_idx"], r["topk_w"], E)
    y_r = np.zeros((x.shape[0], np.shape(w2)[1]), dtype=np.float64)
    for e in range(E):
        y_r = y_r + G[:, e:e + 1] * swiglu(x, w1[e], w3[e], w2[e])
    y_s = swiglu(x, ws1, ws3, ws2) if ws1 is not None else np.zeros_like(y_r)
    return dict(r, y_routed=y_r, y_shared=y_s, out=y_r + y_s)


def moe_sparse(x, w_r, b, top_k, alpha=ALPHA_K2, *, get_expert=None, w1=None, w3=None,
               w2=None, shared=None, tokens=None, routing=None, bf16_points=()):
    """Delta_ffn computed only through the k selected experts of each token.

    Follows the grouping of the K3 page's moe_infer (rows grouped by expert, each
    expert run once on its rows, outputs put back per slot) and the K2 page's sum
    y_routed = sum_i G_i E_i taken over the selected experts in ascending expert order.

    get_expert(e) -> (w1_e, w3_e, w2_e) lets a caller hand over one expert at a time
    (large shapes); shared = (ws1, ws3, ws2) or None.  tokens: optional list of token
    rows to evaluate (sampled check); routing: a precomputed route() result.
    bf16_points: the diagnostic rounding points above (empty: exact, the reference).
    """
    if get_expert is None:
        get_expert = _expert_getter(w1, w3, w2)
    r = routing if routing is not None else route(x, w_r, b, top_k, alpha)
    x = np.asarray(x)
    T = x.shape[0]
    rows = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    sel = r["topk_idx"][rows]
    gates = r["topk_w"][rows]
    # group the (row, slot) pairs by expert
    by_expert: dict[int, list[tuple[int, int]]] = {}
    for i in range(rows.size):
        for j in range(sel.shape[1]):
            by_expert.setdefault(int(sel[i, j]), []).append((i, j))
    per_slot: dict[tuple[int, int], np.ndarray] = {}
    for e in sorted(by_expert):
        pairs = by_expert[e]
        w1e, w3e, w2e = get_expert(e)
        out_e = swiglu(x[rows[[i for i, _ in pairs]]], w1e, w3e, w2e, bf16_points)
        if "expert_out" in bf16_points:
            out_e = round_bf16(out_e)
        elif "y24" in bf16_points:
            out_e = cut_sig16(out_e)
        for n, pr in enumerate(pairs):
            per_slot[pr] = out_e[n]
    d = next(iter(per_slot.values())).shape[0] if per_slot else _f64(w_r).shape[1]
    y_r = np.zeros((rows.size, d), dtype=np.float64)
    for i in range(rows.size):
        for j in np.argsort(sel[i], kind="stable"):          # ascending expert index
            y_r[i] = y_r[i] + gates[i, j] * per_slot[(i, int(j))]
    if shared is not None:
        y_s = swiglu(x[rows], *shared, bf16_points)
        if "y24" in bf16_points:
            y_s = cut_sig16(y_s)
    else:
        y_s = np.zeros_like(y_r)
    if "y_routed" in bf16_points:
        y_r = round_bf16(y_r)
    if "y_shared" in bf16_points:
        y_s = round_bf16(y_s)
    out = y_r + y_s
    if "out" in bf16_points:
        out = round_bf16(out)
    return dict(r, rows=rows, y_routed=y_r, y_shared=y_s, out=out)


# ------------------------------------------------------------------ latent variant
def moe_latent(x, w_r, b, w_down, w1, w3, w2, w_up, ws1, ws3, ws2, top_k,
               alpha=ALPHA_K2, eps=1e-6, tokens=None, get_expert=None):
    """Latent mixture of experts ("Kimi K3 · Latent up-projection", the module's forward):

        z, s, sel, G = route(x)               on the full width d
        l = x W_down^T                        [T, L]
        u = sum_{i in sel} G_i E_i(l)         experts of width L
        u_hat = RMSNorm(u)                    unit gain, on the latent width
        out = u_hat W_up^T + y_shared(x)      shared expert on the full width

    The norm comes before the up-projection, in the order the page's forward applies its
    routed-expert norm and routed-expert up-projection."""
    r = route(x, w_r, b, top_k, alpha)
    x64 = _f64(x)
    rows = np.arange(x64.shape[0]) if tokens is None else np.asarray(tokens, dtype=np.int64)
    lat = x64[rows] @ _f64(w_down).T
    if get_expert is None:
        get_expert = _expert_getter(w1, w3, w2)
    sub = {k: v[rows] for k, v in r.items() if isinstance(v, np.ndarray) and v.shape[:1] == (x64.shape[0],)}
    sparse = moe_sparse(lat, w_r, b, top_k, alpha, get_expert=get_expert, shared=None,
                        routing=sub)
    u_hat = rmsnorm(sparse["y_routed"], eps)
    y_r = u_hat @ _f64(w_up).T
    y_s = swiglu(x64[rows], ws1, ws3, ws2)
    return dict(r, rows=rows, latent=lat, y_latent=sparse["y_routed"], y_routed=y_r,
                y_shared=y_s, out=y_r + y_s)


# ----------------------------------------------------------- block: norm + residual
def moe_block(x_res, gain, w_r, b, w1=None, w3=None, w2=None, ws1=None, ws3=None, ws2=None,
              top_k=8, alpha=ALPHA_K2, eps=1e-6, *, get_expert=None, tokens=None):
    """The MoE half of a transformer block ("Kimi K2 · Transformer blocks", MoE block
    equations; the DeepseekV3DecoderLayer forward printed on that page):

        x_ffn = RMSNorm(x'_n)  (gain, eps)  ->  Delta_ffn = MoE(x_ffn)
        x_{n+1} = x'_n + Delta_ffn

    x_ffn is an activation of the bf16 model, so it is rounded to bf16 (via fp32) before
    the router and the experts read it; everything else is float64.  tokens: optional
    rows to evaluate (the norm and the routing are per token)."""
    x_res = _f64(x_res)
    rows = np.arange(x_res.shape[0]) if tokens is None else np.asarray(tokens, dtype=np.int64)
    x_ffn = round_bf16(rmsnorm(x_res[rows], eps, gain))
    shared = None if ws1 is None else (ws1, ws3, ws2)
    m = moe_sparse(x_ffn, w_r, b, top_k, alpha, get_expert=get_expert, w1=w1, w3=w3, w2=w2,
                   shared=shared)
    return dict(m, rows=rows, x_ffn=x_ffn, delta=m["out"], out=x_res[rows] + m["out"])
