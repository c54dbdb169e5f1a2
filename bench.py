"""Throughput of the K2-shape MoE FFN layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload k2_decode|k2_prefill]

A step is one moe_forward over the batch: router, top-k and gates, permutation,
gate/up GEMM with SwiGLU, down GEMM, combine with the shared expert.  Inputs (seeded,
synthetic, K2 shape: d 7168, 384 experts, top-8, I 2048, one shared expert, bf16
weights, fp32 router) are resident in HBM before the timed region.  Prints one JSON
line: whole-layer tokens/s for the main workload (128-token decode by default), the
roofline of the dominant kernel (the gate/up grouped GEMM) timed with HIP events on
the stream it runs on, the 8192-token prefill figure, the 4096-token skewed-routing figure,
the block, FP8-weight and latent variants, measured ceilings (read-only stream, copy,
vendor GEMM), the committed rocprofv3 counter summaries for the measured kernels (HBM bytes,
MFMA utilisation) while the kernel sources match them, and the CPU oracle timed on a
bounded sample on the host cores.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "K2 MoE-layer tokens/s (128 & 8192 tok, bf16); % of HBM / MFMA peak"
# the gate/up kernel each workload runs (decode: a few rows per expert; prefill: many)
GATEUP_KERNEL = {"k2_decode": "ffn_skinny_kernel<1, 16, 0, false>", "k2_prefill": "ffn_lds_kernel<0>"}
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s


TRAFFIC_JSON = os.path.join(ROOT, "profiles", "hbm_traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "mixture_experts_transformer_sigmoid_amd", "csrc", f)
                  for f in ("ffn.hip", "grouped.h", "tiles.h", "common.h")]
COPY_BYTES = 1 << 30
SETTLE_S = 2.0                  # idle pause between input generation and timing
READ_BYTES = 4 << 30


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def write_traffic(fetch_csv, write_csv):
    """Turn two rocprofv3 --pmc counter CSVs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch) of a
    --copy-calibration run into profiles/hbm_traffic.json: bytes per launch per kernel and
    launch grid (one kernel can serve several workloads), each counter scaled by what it
    reads for the 1 GiB calibration copy."""
    import csv
    import collections
    out = {"source_sha256": kernel_source_hash(), "kernels": {}, "scale": {}}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        copy = max(float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"])
        scale = (COPY_BYTES / 1024) / copy
        out["scale"][counter] = scale
        per = collections.defaultdict(list)
        for r in rows:
            if "copyBuffer" in r["Kernel_Name"]:
                continue
            per[(r["Kernel_Name"], r["Grid_Size"])].append(float(r["Counter_Value"]) * 1024 * scale)
        key = "read_bytes" if counter == "FETCH_SIZE" else "write_bytes"
        for (name, grid), v in per.items():
            g = out["kernels"].setdefault(name, {}).setdefault(grid, {})
            g[key] = sum(v) / len(v)
            g["launches"] = len(v)
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
    print(json.dumps(out, indent=1))


MFMA_JSON = os.path.join(ROOT, "profiles", "mfma_util.json")
XCDS = 8          # MI355X: 8 accelerator complex dies (GRBM_GUI_ACTIVE is summed over them)
SIMDS = 1024      # 256 CUs x 4 SIMDs
MFMA_FLOP_PER_SIMD_CYCLE = 1024   # dense bf16: 2.5 PFLOP/s = 1024 SIMDs x 2.4 GHz x 1024


def write_mfma(csv_path):
    """Turn a rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE
    SQ_INSTS_VALU_MFMA_MOPS_BF16 counter CSV into profiles/mfma_util.json: per kernel and
    grid, the MFMA-busy fraction of the active cycles (busy cycles summed over the SIMDs
    / (active cycles per XCD x SIMDs)), the bf16 MFMA flops the hardware counted (MOPS x
    512), the kernel time and the clock that the active cycles imply."""
    import csv
    import collections
    per = collections.defaultdict(dict)
    for r in csv.DictReader(open(csv_path)):
        key = (r["Kernel_Name"], r["Grid_Size"], r["Dispatch_Id"])
        per[key][r["Counter_Name"]] = float(r["Counter_Value"])
        per[key]["_s"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    groups = collections.defaultdict(list)
    for (name, grid, _), v in per.items():
        if v.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) > 0 and "GRBM_GUI_ACTIVE" in v:
            groups[(name, grid)].append(v)
    out = {"source_sha256": kernel_source_hash(), "kernels": {}}
    for (name, grid), vs in groups.items():
        n = len(vs)
        sec = sum(v["_s"] for v in vs) / n
        active = sum(v["GRBM_GUI_ACTIVE"] for v in vs) / n / XCDS
        busy = sum(v["SQ_VALU_MFMA_BUSY_CYCLES"] for v in vs) / n
        flops = sum(v.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) for v in vs) / n * 512
        out["kernels"].setdefault(name, {})[grid] = {
            "launches": n, "ms": sec * 1e3, "clock_ghz": active / sec / 1e9,
            "mfma_busy_frac": busy / (active * SIMDS), "mfma_flops": flops,
            "mfma_tflops": flops / sec / 1e12}
    with open(MFMA_JSON, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
    print(json.dumps(out, indent=1))


def mfma_for(kernel_substr, grid):
    """The committed MFMA counters of one kernel launch shape, or None when missing or the
    kernel sources changed since they were taken."""
    try:
        with open(MFMA_JSON) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != kernel_source_hash():
        return None
    for name, grids in t["kernels"].items():
        if kernel_substr in name and str(grid) in grids:
            return grids[str(grid)]
    return None


def traffic_for(kernel_substr, algorithmic_bytes):
    """HBM bytes per launch of a kernel from the committed counter summary, or None when it
    is missing or the kernel sources changed since the counters were taken.  One kernel can
    serve several workloads (the decode gate/up kernel also runs the tiny config), each with
    its own launch grid: the entry taken is the one whose bytes are nearest the launch's
    algorithmic bytes, and only if within a factor of 2 of them."""
    try:
        with open(TRAFFIC_JSON) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != kernel_source_hash():
        return None
    best = None
    for name, grids in t["kernels"].items():
        if kernel_substr not in name:
            continue
        for v in grids.values():
            if "read_bytes" not in v or "write_bytes" not in v:
                continue
            b = v["read_bytes"] + v["write_bytes"]
            if best is None or abs(math.log(b / algorithmic_bytes)) < abs(math.log(best / algorithmic_bytes)):
                best = b
    if best is None or abs(math.log(best / algorithmic_bytes)) > math.log(2.0):
        return None
    return best


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="k2_decode", choices=["k2_decode", "k2_prefill"])
    ap.add_argument("--no-prefill", action="store_true", help="skip the 8192-token figure")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-latent", action="store_true", help="skip the latent-MoE figure")
    ap.add_argument("--no-skew", action="store_true", help="skip the skewed-routing figure")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8-weight figures")
    ap.add_argument("--no-block", action="store_true",
                    help="skip the fused norm + residual block figure")
    ap.add_argument("--cpu-sample", type=int, default=128,
                    help="tokens in the oracle sample (default: all 128 of the decode batch)")
    ap.add_argument("--no-power", action="store_true",
                    help="skip sampling socket power / clock during the prefill loop")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the measured HBM-copy and vendor-GEMM peaks")
    ap.add_argument("--write-mfma", metavar="COUNTER_CSV",
                    help="write profiles/mfma_util.json from a --pmc SQ_VALU_MFMA_BUSY_CYCLES "
                         "GRBM_GUI_ACTIVE SQ_INSTS_VALU_MFMA_MOPS_BF16 counter CSV and exit")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/hbm_traffic.json from two --pmc counter CSVs and exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one 1 GiB device-to-device copy (a plain copy kernel of known size "
                         "for scaling HBM byte counters)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def algorithmic(cfg, active, T):
    """Bytes and flops of one layer pass and of one gate/up launch (each weight of an
    active expert counted once; activations read/written once)."""
    d, I, Is, E, k = cfg["d_model"], cfg["d_expert"], cfg["d_shared"], cfg["n_experts"], cfg["top_k"]
    expert_w = 3 * d * I * 2                      # bytes of one expert's W1, W3, W2 (bf16)
    rows = T * k + (T if Is else 0)
    layer_bytes = (active * expert_w + (3 * d * Is * 2 if Is else 0) + E * d * 4 + E * 4
                   + T * d * 2 + T * d * 2)
    layer_flops = 2 * 3 * d * I * T * k + (2 * 3 * d * Is * T if Is else 0)
    gateup_units = active + (1 if Is else 0)        # experts whose W1, W3 stream through
    gateup_bytes = gateup_units * 2 * d * I * 2 + T * d * 2 + rows * I * 2
    gateup_flops = 2 * 2 * d * I * rows
    return dict(layer_bytes=layer_bytes, layer_flops=layer_flops, gateup_bytes=gateup_bytes,
                gateup_flops=gateup_flops, gateup_units=gateup_units)


def time_forward(M, torch, dims, inp, out, ws, steps, warmup, per_step=None):
    """Mean ms per moe_forward over `steps` back-to-back calls (HIP events on the launch
    stream around all of them).  With per_step a list, an event between consecutive calls
    also gives each call's own time (appended to it)."""
    for _ in range(warmup):
        M.moe_forward(dims, inp["x"], inp["w_r"], inp["b"], inp["w1"], inp["w3"], inp["w2"],
                      inp["ws1"], inp["ws3"], inp["ws2"], out, ws)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    wall = time.perf_counter()
    ev[0].record()
    for i in range(steps):
        M.moe_forward(dims, inp["x"], inp["w_r"], inp["b"], inp["w1"], inp["w3"], inp["w2"],
                      inp["ws1"], inp["ws3"], inp["ws2"], out, ws)
        if per_step is not None or i == steps - 1:
            ev[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall
    if per_step is not None:
        per_step.extend(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    return ev[0].elapsed_time(ev[steps]) / steps, wall


def time_block(M, torch, S, cfg, weights, steps, warmup):
    """moe_forward_block (pre-MoE RMSNorm + layer + residual add) on the same weights."""
    dev = weights["w1"].device
    act = S.make_block_activations(cfg, dev)
    dims = M.dims_for(cfg)
    ws = M.block_workspace(dims, dev)
    out = torch.empty(cfg["tokens"], cfg["d_model"], dtype=torch.bfloat16, device=dev)

    def call():
        M.moe_forward_block(dims, act["x_res"], act["norm_w"], 1e-6, weights["w_r"], act["b"],
                            weights["w1"], weights["w3"], weights["w2"], weights["ws1"],
                            weights["ws3"], weights["ws2"], out, ws)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        call()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def time_fp8(M, torch, S, dev, act, steps, warmup, prefill):
    """The layer with FP8 block-scaled expert weights (moe_forward_fp8) at decode (and
    prefill), plus its decode gate/up launch for the roofline."""
    cfg = S.CONFIGS["k2_decode"]
    w = S.make_fp8_weights(cfg, dev)
    fw = M.fp8_weights(w)
    dims = M.dims_for(cfg)
    T, d, I = cfg["tokens"], cfg["d_model"], cfg["d_expert"]
    ws = M.workspace(dims, dev)
    out = torch.empty(T, d, dtype=torch.bfloat16, device=dev)

    def timed(fn, n, w_):
        for _ in range(w_):
            fn()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(n):
            fn()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / n

    ms = timed(lambda: M.moe_forward_fp8(dims, act["x"], w["w_r"], act["b"], fw, out, ws), steps,
               warmup)
    st = split_state(M, torch, dims, {"x": act["x"], "w_r": w["w_r"], "b": act["b"]}, ws)
    active = int((st["counts"] > 0).sum())
    h = torch.empty(T * 9, I, dtype=torch.bfloat16, device=dev)
    gu = timed(lambda: M.moe_expert_gate_up_fp8(dims, act["x"], st["perm"], st["offsets"], fw, h,
                                                ws), steps, warmup)
    units = active + 1
    gu_bytes = units * 2 * I * d + units * 2 * (I // 128) * (d // 128) * 4 + T * d * 2 + T * 9 * I * 2
    layer_bytes = (units * 3 * I * d + units * 3 * (I // 128) * (d // 128) * 4
                   + cfg["n_experts"] * d * 4 + 2 * T * d * 2)
    res = {"entry": "moe_forward_fp8 (E4M3 expert weights, one fp32 scale per 128x128 block)",
           "decode_ms_per_step": ms, "decode_tokens_per_s": T / (ms * 1e-3),
           "decode_layer_hbm_gbs": layer_bytes / (ms * 1e-3) / 1e9,
           "gate_up": {"kernel": "ffn_skinny_fp8_kernel<4, 1, 0>", "ms_per_launch": gu,
                       "bytes_per_launch": gu_bytes, "achieved_gbs": gu_bytes / (gu * 1e-3) / 1e9,
                       "frac": gu_bytes / (gu * 1e-3) / 1e9 / HBM_PEAK_GBS},
           "active_experts": active}
    if prefill:
        pcfg = S.CONFIGS["k2_prefill"]
        pact = S.make_activations(pcfg, dev)
        pdims = M.dims_for(pcfg)
        del ws, h
        pws = M.workspace(pdims, dev)
        pout = torch.empty(pcfg["tokens"], d, dtype=torch.bfloat16, device=dev)
        pms = timed(lambda: M.moe_forward_fp8(pdims, pact["x"], w["w_r"], pact["b"], fw, pout, pws),
                    max(3, min(steps, 10)), 1)
        flops = 2 * 3 * d * I * pcfg["tokens"] * (pcfg["top_k"] + 1)
        res.update({"prefill_ms_per_step": pms, "prefill_tokens_per_s": pcfg["tokens"] / (pms * 1e-3),
                    "prefill_mfma_tflops": flops / (pms * 1e-3) / 1e12})
    return res


def split_state(M, torch, dims, inp, ws):
    """Route and permute once: the gate/up GEMM's inputs."""
    T, E, k = dims.tokens, dims.n_experts, dims.top_k
    dev = inp["x"].device
    idx = torch.empty(T, k, dtype=torch.int32, device=dev)
    w = torch.empty(T, k, dtype=torch.float32, device=dev)
    M.moe_route(dims, inp["x"], inp["w_r"], inp["b"], idx, w, None, ws)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(T * k, dtype=torch.int32, device=dev)
    inv = torch.empty(T * k, dtype=torch.int32, device=dev)
    M.moe_permute(dims, idx, counts, offsets, perm, inv, ws)
    torch.cuda.synchronize()
    return dict(idx=idx, w=w, counts=counts, offsets=offsets, perm=perm, inv=inv)


def time_gate_up(M, torch, dims, inp, st, ws, steps, warmup):
    """Average duration of one moe_expert_gate_up call (tile-list kernel + GEMM kernel),
    HIP events on the current stream, which is the stream the kernels run on."""
    T, k = dims.tokens, dims.top_k
    h = torch.empty(T * k + T, dims.d_expert, dtype=torch.bfloat16, device=inp["x"].device)

    def call():
        M.moe_expert_gate_up(dims, inp["x"], st["perm"], st["offsets"], inp["w1"], inp["w3"],
                             inp["ws1"], inp["ws3"], h, ws)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        call()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def time_latent(M, torch, S, dev, steps):
    """moe_forward_latent at the latent-MoE shape: T=4096, d=7168, L=3584, 384 experts."""
    cfg = S.CONFIGS["latent"]
    inp = S.make_inputs(cfg, dev)
    dims = M.dims_for(cfg)
    L, T, d, I, Is, E, k = (cfg["d_latent"], cfg["tokens"], cfg["d_model"], cfg["d_expert"],
                            cfg["d_shared"], cfg["n_experts"], cfg["top_k"])
    ws = M.latent_workspace(dims, L, dev)
    out = torch.empty(T, d, dtype=torch.bfloat16, device=dev)

    def call():
        M.moe_forward_latent(dims, L, inp["x"], inp["w_r"], inp["b"], inp["w_down"], inp["w1"],
                             inp["w3"], inp["w2"], inp["w_up"], inp["ws1"], inp["ws3"], inp["ws2"],
                             out, ws)
    call()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        call()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    # every routed expert is active at this batch (checked by the parity test's counts)
    byts = (E * 3 * L * I * 2 + 2 * d * L * 2 + 3 * d * Is * 2 + E * d * 4 + E * 4
            + T * d * 2 + T * d * 2)
    flops = 2 * T * d * L * 2 + 2 * 3 * L * I * T * k + 2 * 3 * d * Is * T
    del inp, ws
    torch.cuda.empty_cache()
    return {"workload": "latent MoE: T=4096, d=7168, latent 3584, 384 experts top-8, I=2048, "
                        "RMSNorm, up-projection, shared expert on 7168",
            "steps": steps, "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3),
            "hbm_gbs": byts / (ms * 1e-3) / 1e9, "hbm_frac": byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "mfma_tflops": flops / (ms * 1e-3) / 1e12,
            "mfma_frac": flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS}


def measure_ceilings(torch, dev):
    """Achievable peaks on this GPU, next to the published ones: a 1 GiB device copy (read +
    write) for HBM, and the vendor GEMM (torch.matmul -> hipBLASLt) on an 8192^3 bf16
    product with N(0, 1) operands and with all-zero operands.  bf16 MFMA throughput on this
    part depends on the data: random operands toggle the datapath and the chip lowers its
    clock to stay in its power budget."""
    def timed(fn, n):
        fn()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(n):
            fn()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / n
    src = torch.full((COPY_BYTES,), 7, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    copy_ms = timed(lambda: dst.copy_(src), 5)
    del src, dst
    # read-only stream over a 4 GiB array: the faster of two torch reductions (row sums of
    # 65,536 rows of 64 KiB as fp32, and the int64 total), the fastest two on this part; a
    # lower bound on what a read stream can reach (a tuned kernel can beat it by a few %)
    rd = torch.full((READ_BYTES // 4,), 1.0, dtype=torch.float32, device=dev)
    read_ms = min(timed(lambda: rd.view(65536, -1).sum(dim=1), 10),
                  timed(lambda: rd.view(torch.int64).sum(), 10))
    del rd
    n = 8192
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    a = torch.randn(n, n, device=dev, generator=g).to(torch.bfloat16)
    b = torch.randn(n, n, device=dev, generator=g).to(torch.bfloat16)
    rand_ms = timed(lambda: torch.matmul(a, b), 5)
    a.zero_()
    b.zero_()
    zero_ms = timed(lambda: torch.matmul(a, b), 5)
    del a, b
    torch.cuda.empty_cache()
    flops = 2.0 * n ** 3
    return {"hbm_copy_gbs": 2 * COPY_BYTES / (copy_ms * 1e-3) / 1e9,
            "hbm_read_gbs": READ_BYTES / (read_ms * 1e-3) / 1e9,
            "mfma_bf16_random_tflops": flops / (rand_ms * 1e-3) / 1e12,
            "mfma_bf16_zeros_tflops": flops / (zero_ms * 1e-3) / 1e12,
            "how": "1 GiB device-to-device copy (bytes read + written); a read-only pass over "
                   "a 4 GiB array (bytes read; the faster of fp32 row sums and an int64 total); "
                   "torch.matmul "
                   "(hipBLASLt) 8192x8192x8192 bf16, N(0,1) operands and all-zero operands"}


def sample_power(M, torch, dims, inp, out, ws, seconds=6.0):
    """Socket power and graphics clock while the layer runs back to back: amd-smi is
    sampled from a thread while the main thread keeps the GPU busy.  Returns None when
    amd-smi is not available."""
    import re
    import shutil
    import subprocess
    import threading
    smi = shutil.which("amd-smi") or ("/opt/rocm/bin/amd-smi" if os.path.exists("/opt/rocm/bin/amd-smi") else None)
    if smi is None:
        return None
    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            try:
                txt = subprocess.run([smi, "metric", "-p", "-c"], capture_output=True, text=True,
                                     timeout=10).stdout
            except (OSError, subprocess.SubprocessError):
                return
            w = re.findall(r"SOCKET_POWER:\s*([0-9.]+)\s*W", txt)
            clk, section = [], ""
            for line in txt.splitlines():
                head = re.match(r"^\s*([A-Z]+_?\d*):\s*$", line)
                if head:
                    section = head.group(1)
                    continue
                m = re.match(r"^\s*CLK:\s*([0-9.]+)\s*MHz", line)
                if m and section.startswith("GFX"):  # graphics clock of each XCD
                    clk.append(float(m.group(1)))
            if w:
                samples.append((float(w[0]), sum(clk) / len(clk) if clk else None))
            stop.wait(0.5)

    def call():
        M.moe_forward(dims, inp["x"], inp["w_r"], inp["b"], inp["w1"], inp["w3"], inp["w2"],
                      inp["ws1"], inp["ws3"], inp["ws2"], out, ws)
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    th = threading.Thread(target=sampler, daemon=True)
    t_end = time.perf_counter() + seconds
    th.start()
    n = 0
    while time.perf_counter() < t_end:
        for _ in range(10):
            call()
        torch.cuda.synchronize()
        n += 10
    stop.set()
    th.join(timeout=15)
    if not samples:
        return None
    ws_ = [p for p, _ in samples]
    cs = [c for _, c in samples if c is not None]
    return {"socket_power_w": sum(ws_) / len(ws_), "socket_power_w_max": max(ws_),
            "gfx_clock_mhz": (sum(cs) / len(cs)) if cs else None, "samples": len(samples),
            "layer_passes": n, "how": "amd-smi metric -p -c every 0.5 s while moe_forward runs "
                                      "back to back (k2_prefill)"}


def cpu_baseline(torch, S, cfg, inp, n_tok):
    """The oracle as it stands on a bounded sample: route + sparse FFN for n_tok tokens of
    the batch (all of them by default), timed on the host cores.  The weights are staged on
    the host as bf16 beforehand; their conversion to float64, which the oracle's expert
    getter does one expert at a time, is timed separately and left out of the figure."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import moe_oracle as O
    T = cfg["tokens"]
    toks = np.sort(np.random.default_rng(0).choice(T, size=min(n_tok, T), replace=False))
    x = inp["x"][toks].to("cpu", torch.float64).numpy()
    w_r = inp["w_r"].to("cpu", torch.float64).numpy()
    b = inp["b"].cpu().numpy()
    r = O.route(x, w_r, b, cfg["top_k"], cfg["routed_scale"])
    need = sorted(set(int(e) for e in r["topk_idx"].reshape(-1)))
    host = {e: (inp["w1"][e].cpu(), inp["w3"][e].cpu(), inp["w2"][e].cpu()) for e in need}
    shared = tuple(t.cpu().to(torch.float64).numpy() for t in (inp["ws1"], inp["ws3"], inp["ws2"]))
    conv = [0.0]

    def get(e):
        c = time.perf_counter()
        out = tuple(t.to(torch.float64).numpy() for t in host[e])
        conv[0] += time.perf_counter() - c
        return out
    t = time.perf_counter()
    r = O.route(x, w_r, b, cfg["top_k"], cfg["routed_scale"])
    O.moe_sparse(x, w_r, b, cfg["top_k"], cfg["routed_scale"], get_expert=get, shared=shared,
                 routing=r)
    el = time.perf_counter() - t - conv[0]
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [torch.get_num_threads()])
    return {"value": len(toks) / el, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{len(toks)} of the {T} tokens (route + {len(need)} experts + shared, "
                      f"float64 numpy, {el:.1f} s; the bf16 -> float64 weight conversion, "
                      f"{conv[0]:.1f} s, left out)"}


def near_ties(M, torch, dims, x, w_r, b, ws):
    """Tokens whose k-th and (k+1)-th biased scores are within 1e-6: the ones a parity check
    leaves out of the bit-exact routing comparison.  Scores from the layer's own logits
    (moe_route), fl32(sigmoid(z)) + b in fp32."""
    T, E, k = int(dims.tokens), int(dims.n_experts), int(dims.top_k)
    dev = x.device
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    z = torch.empty((T, E), dtype=torch.float32, device=dev)
    M.moe_route(dims, x, w_r, b, idx, w, z, ws)
    sc = torch.sigmoid(z) + b.float()
    top = torch.topk(sc, min(k + 1, E), dim=1).values
    if k >= E:
        return 0
    return int(((top[:, k - 1] - top[:, k]) < 1e-6).sum())


def time_tiny(M, torch, S, dev, calls=200):
    """The tiny config (64 tokens, d 256, 16 experts, top-2): a latency-bound call.  Reports
    the mean per call over back-to-back calls (HIP events) and the median wall time of one
    call followed by a synchronisation."""
    cfg = S.CONFIGS["tiny"]
    inp = {k: v.to(dev) for k, v in S.make_inputs(cfg, "cpu").items()}
    dims = M.dims_for(cfg)
    ws = M.workspace(dims, dev)
    out = torch.empty(cfg["tokens"], cfg["d_model"], dtype=torch.bfloat16, device=dev)

    def call():
        M.moe_forward(dims, inp["x"], inp["w_r"], inp["b"], inp["w1"], inp["w3"], inp["w2"],
                      inp["ws1"], inp["ws3"], inp["ws2"], out, ws)
    for _ in range(10):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(calls):
        call()
    e1.record()
    torch.cuda.synchronize()
    walls = []
    for _ in range(50):
        t = time.perf_counter()
        call()
        torch.cuda.synchronize()
        walls.append(time.perf_counter() - t)
    walls.sort()
    per = e0.elapsed_time(e1) / calls
    res = {"workload": "tiny: T=64, d=256, 16 experts top-2 (x2.827), I=Is=128, bf16 kernels",
           "us_per_call_pipelined": per * 1e3, "us_per_call_synchronised": walls[len(walls) // 2] * 1e6,
           "tokens_per_s": cfg["tokens"] / (per * 1e-3), "graph": None}
    eager = out.clone()
    # the same call captured once into a HIP graph and replayed (the library allocates
    # nothing and launches no memset, so the five launches capture as they are); a figure
    # of its own, left out if the capture fails on this software stack
    try:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            call()
        torch.cuda.synchronize()
    except Exception as exc:  # noqa: BLE001
        log(f"tiny: graph capture failed ({exc}); graph figure left out")
        torch.cuda.synchronize()
        return res
    out.fill_(float("nan"))
    g.replay()
    torch.cuda.synchronize()
    same = bool(torch.equal(out.view(torch.int16), eager.view(torch.int16)))
    e0.record()
    for _ in range(calls):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    gper = e0.elapsed_time(e1) / calls
    gwalls = []
    for _ in range(50):
        t = time.perf_counter()
        g.replay()
        torch.cuda.synchronize()
        gwalls.append(time.perf_counter() - t)
    gwalls.sort()
    res["graph"] = {"us_per_replay_pipelined": gper * 1e3,
                    "us_per_replay_synchronised": gwalls[len(gwalls) // 2] * 1e6,
                    "output_equals_eager": same}
    return res


def main():
    args = parse()
    if args.write_traffic:
        write_traffic(*args.write_traffic)
        return
    if args.write_mfma:
        write_mfma(args.write_mfma)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported "
              "(the layer is measured on one GPU's share; across GPUs it would shard by expert "
              "parallelism, which is not built)",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import mixture_experts_transformer_sigmoid_amd as M
    import synth_inputs as S

    dev = torch.device("cuda:0")
    cfg = S.CONFIGS[args.workload]
    log("generating K2-shape weights on the GPU")
    weights = S.make_weights(cfg, dev)
    inp = dict(weights)
    inp.update(S.make_activations(cfg, dev))
    dims = M.dims_for(cfg)
    T = cfg["tokens"]
    ws = M.workspace(dims, dev)
    out = torch.empty(T, cfg["d_model"], dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    # let the device go quiet before the first timed leg: right after another process
    # released tens of GB (a test run, a previous bench), the first 20-step decode leg
    # came out up to 3% slow in some runs, and never after a pause
    time.sleep(SETTLE_S)

    log(f"timing moe_forward, {args.workload}, T={T}")
    steps_ms = []
    ms, wall = time_forward(M, torch, dims, inp, out, ws, args.steps, args.warmup, steps_ms)
    st = split_state(M, torch, dims, inp, ws)
    active = int((st["counts"] > 0).sum())
    alg = algorithmic(cfg, active, T)
    if args.copy_calibration:
        src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: {1 << 30} bytes read, {1 << 30} bytes written")
        del src, dst
    gu_ms = time_gate_up(M, torch, dims, inp, st, ws, args.steps, args.warmup)
    gu_gbs = alg["gateup_bytes"] / (gu_ms * 1e-3) / 1e9
    layer_gbs = alg["layer_bytes"] / (ms * 1e-3) / 1e9
    layer_tfs = alg["layer_flops"] / (ms * 1e-3) / 1e12
    res = {
        "metric": METRIC, "value": T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: one MoE FFN layer, T={T} tokens, d=7168, "
                               "384 experts top-8 (x2.827), I=2048, 1 shared expert, bf16 "
                               "weights/activations, fp32 router and accumulation",
                   "tokens": T, "active_experts": active},
        "roofline": {"bound": "hbm", "achieved": gu_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gu_gbs / HBM_PEAK_GBS, "traffic": traffic_for(GATEUP_KERNEL[args.workload], alg["gateup_bytes"]),
                     "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                     "kernel": GATEUP_KERNEL[args.workload] + " (+ its tile-list launch)",
                     "ms_per_launch": gu_ms, "bytes_per_launch": alg["gateup_bytes"]},
        "step_ms": {"median": sorted(steps_ms)[len(steps_ms) // 2], "min": min(steps_ms),
                    "max": max(steps_ms)},
        "layer": {"hbm_gbs": layer_gbs, "hbm_frac": layer_gbs / HBM_PEAK_GBS,
                  "mfma_tflops": layer_tfs, "mfma_frac": layer_tfs / MFMA_BF16_PEAK_TFLOPS,
                  "algorithmic_bytes": alg["layer_bytes"], "algorithmic_flops": alg["layer_flops"]},
    }
    res["config"]["near_tie_tokens"] = near_ties(M, torch, dims, inp["x"], inp["w_r"], inp["b"], ws)
    log(f"{args.workload}: {ms:.3f} ms/step, {res['value']:.0f} tok/s, layer {layer_gbs:.0f} GB/s, "
        f"gate/up {gu_ms:.3f} ms = {gu_gbs:.0f} GB/s, "
        f"{res['config']['near_tie_tokens']} near-tie tokens")
    if not args.no_block:
        del ws
        bms = time_block(M, torch, S, cfg, weights, args.steps, args.warmup)
        res["block"] = {"entry": "moe_forward_block (pre-MoE RMSNorm, layer, residual add)",
                        "tokens": T, "ms_per_step": bms, "tokens_per_s": T / (bms * 1e-3),
                        "added_us_vs_layer": (bms - ms) * 1e3}
        log(f"block ({args.workload}): {bms:.3f} ms/step ({(bms - ms) * 1e3:+.1f} us vs the layer)")
        ws = M.workspace(dims, dev)

    if not args.no_prefill and args.workload != "k2_prefill":
        pcfg = S.CONFIGS["k2_prefill"]
        pin = dict(weights)
        pin.update(S.make_activations(pcfg, dev))
        pdims = M.dims_for(pcfg)
        del ws
        pws = M.workspace(pdims, dev)
        pout = torch.empty(pcfg["tokens"], pcfg["d_model"], dtype=torch.bfloat16, device=dev)
        log("timing moe_forward, k2_prefill, T=8192")
        psteps = max(3, min(args.steps, 10))
        psteps_ms = []
        pms, _ = time_forward(M, torch, pdims, pin, pout, pws, psteps, 1, psteps_ms)
        pst = split_state(M, torch, pdims, pin, pws)
        pact = int((pst["counts"] > 0).sum())
        palg = algorithmic(pcfg, pact, pcfg["tokens"])
        ptf = palg["layer_flops"] / (pms * 1e-3) / 1e12
        pgb = palg["layer_bytes"] / (pms * 1e-3) / 1e9
        power = None if args.no_power else sample_power(M, torch, pdims, pin, pout, pws)
        pties = near_ties(M, torch, pdims, pin["x"], pin["w_r"], pin["b"], pws)
        res["prefill"] = {"workload": "k2_prefill: T=8192 (4 x 2048), same layer", "steps": psteps,
                          "near_tie_tokens": pties,
                          "ms_per_step": pms, "tokens_per_s": pcfg["tokens"] / (pms * 1e-3),
                          "step_ms": {"median": sorted(psteps_ms)[len(psteps_ms) // 2],
                                      "min": min(psteps_ms), "max": max(psteps_ms)},
                          "mfma_tflops": ptf, "mfma_frac": ptf / MFMA_BF16_PEAK_TFLOPS,
                          "hbm_gbs": pgb, "hbm_frac": pgb / HBM_PEAK_GBS, "active_experts": pact}
        if not args.no_block:
            del pws
            pbms = time_block(M, torch, S, pcfg, weights, psteps, 1)
            pws = None
        # MFMA counters of the prefill GEMMs (committed rocprofv3 --pmc summary, taken on
        # the current kernel sources): busy fraction of the active cycles, implied clock
        ctr = {role: mfma_for("ffn_lds_kernel<%d>" % epi, grid) for role, epi, grid in
               (("gate_up", 0, 2756608), ("down", 1, 4825088))}
        if all(ctr.values()):
            res["prefill"]["mfma_counters"] = {
                role: {"busy_frac": c["mfma_busy_frac"], "clock_ghz": c["clock_ghz"],
                       "counted_tflops": c["mfma_tflops"]} for role, c in ctr.items()}
        if power is not None:
            res["prefill"]["power"] = power
            log(f"prefill power: {power['socket_power_w']:.0f} W socket, "
                f"graphics clock {power['gfx_clock_mhz'] or 0:.0f} MHz")
        if not args.no_block:
            res["prefill"]["block_ms_per_step"] = pbms
            log(f"block (k2_prefill): {pbms:.3f} ms/step ({(pbms - pms) * 1e3:+.1f} us vs the layer)")
        log(f"prefill: {pms:.3f} ms/step, {res['prefill']['tokens_per_s']:.0f} tok/s, "
            f"{ptf:.0f} TFLOP/s ({100 * ptf / MFMA_BF16_PEAK_TFLOPS:.1f}% MFMA)")
        del pws, pin

    if not args.no_skew and args.workload != "k2_skew":
        scfg = S.CONFIGS["k2_skew"]
        sin = dict(weights)
        sin.update(S.make_activations(scfg, dev))
        sdims = M.dims_for(scfg)
        sws = M.workspace(sdims, dev)
        sout = torch.empty(scfg["tokens"], scfg["d_model"], dtype=torch.bfloat16, device=dev)
        log("timing moe_forward, k2_skew, T=4096")
        ssteps = max(3, min(args.steps, 10))
        sms, _ = time_forward(M, torch, sdims, sin, sout, sws, ssteps, 1)
        sst = split_state(M, torch, sdims, sin, sws)
        cnt = sst["counts"].to("cpu")
        sact = int((cnt > 0).sum())
        salg = algorithmic(scfg, sact, scfg["tokens"])
        stf = salg["layer_flops"] / (sms * 1e-3) / 1e12
        res["skew"] = {"workload": "k2_skew: T=4096, same layer, selection bias -0.5 ln(rank) over a "
                                   "seeded ranking of the experts (most tokens on ~20 experts)",
                       "steps": ssteps, "ms_per_step": sms, "tokens_per_s": scfg["tokens"] / (sms * 1e-3),
                       "mfma_tflops": stf, "mfma_frac": stf / MFMA_BF16_PEAK_TFLOPS,
                       "active_experts": sact, "max_rows_per_expert": int(cnt.max()),
                       "near_tie_tokens": near_ties(M, torch, sdims, sin["x"], sin["w_r"], sin["b"], sws),
                       "hbm_gbs": salg["layer_bytes"] / (sms * 1e-3) / 1e9}
        log(f"skew: {sms:.3f} ms/step, {res['skew']['tokens_per_s']:.0f} tok/s, {stf:.0f} TFLOP/s, "
            f"{sact} active experts, up to {int(cnt.max())} rows")
        del sws, sin, sout

    if not args.no_fp8:
        log("timing moe_forward_fp8 (FP8 block-scaled expert weights)")
        fres = time_fp8(M, torch, S, dev, {"x": inp["x"], "b": inp["b"]}, args.steps,
                        args.warmup, not args.no_prefill)
        res["fp8"] = fres
        log(f"fp8: decode {fres['decode_ms_per_step']:.3f} ms/step "
            f"({fres['decode_tokens_per_s']:.0f} tok/s), gate/up {fres['gate_up']['ms_per_launch']:.3f} ms"
            f" = {fres['gate_up']['achieved_gbs']:.0f} GB/s"
            + (f"; prefill {fres['prefill_ms_per_step']:.3f} ms" if "prefill_ms_per_step" in fres else ""))
        torch.cuda.empty_cache()
    tiny = time_tiny(M, torch, S, dev)
    res["tiny"] = tiny
    gr = tiny["graph"]
    log(f"tiny: {tiny['us_per_call_pipelined']:.1f} us per call back to back, "
        f"{tiny['us_per_call_synchronised']:.1f} us with a synchronisation"
        + ("" if gr is None else
           f"; from a HIP graph {gr['us_per_replay_pipelined']:.1f} and "
           f"{gr['us_per_replay_synchronised']:.1f} us (output equal to eager: "
           f"{gr['output_equals_eager']})"))
    if not args.no_cpu_baseline:
        log(f"timing the CPU oracle on {args.cpu_sample} tokens")
        res["cpu_baseline"] = cpu_baseline(torch, S, cfg, inp, args.cpu_sample)
        log(f"cpu oracle: {res['cpu_baseline']['value']:.2f} tok/s on {res['cpu_baseline']['cores']} threads")
    if not args.no_ceilings:
        ceil = measure_ceilings(torch, dev)
        res["ceilings"] = ceil
        rt = ceil["mfma_bf16_random_tflops"]
        res["roofline"]["frac_of_measured_read"] = res["roofline"]["achieved"] / ceil["hbm_read_gbs"]
        for leg in ("prefill", "skew"):
            if leg in res:
                res[leg]["mfma_frac_of_measured_random"] = res[leg]["mfma_tflops"] / rt
        log(f"ceilings: copy {ceil['hbm_copy_gbs']:.0f} GB/s, read {ceil['hbm_read_gbs']:.0f} GB/s; vendor GEMM bf16 {rt:.0f} TFLOP/s "
            f"(random), {ceil['mfma_bf16_zeros_tflops']:.0f} TFLOP/s (zeros)")
    if not args.no_latent:
        # latent variant (experts on a 3584-wide latent), 4096 tokens; its own weights
        del weights
        for key in list(inp):
            del inp[key]
        torch.cuda.empty_cache()
        lres = time_latent(M, torch, S, dev, max(3, min(args.steps, 10)))
        if "ceilings" in res:
            lres["mfma_frac_of_measured_random"] = (lres["mfma_tflops"]
                                                    / res["ceilings"]["mfma_bf16_random_tflops"])
        res["latent"] = lres
        log(f"latent: {lres['ms_per_step']:.3f} ms/step, {lres['tokens_per_s']:.0f} tok/s, "
            f"{lres['hbm_gbs']:.0f} GB/s, {lres['mfma_tflops']:.0f} TFLOP/s")
        inp = None

    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
