"""Benchmark: W4A16 MoE decode layer (and dense GEMV) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]

Prints ONE JSON line.  A step is one full pass of the hot path over one batch of
synthetic input: for the default workload, one token through the whole MoE layer
of the Qwen 3.6 35B-A3B shape (router GEMV, softmax/top-8/renormalise, grouped
W13 + SiLU over 8 routed + 1 shared expert, down projection + weighted combine).
Inputs are resident in HBM before the timed region.  To keep the 256 MB
Infinity Cache from serving the weights, steps rotate over layer replicas and a
pool of tokens (distinct expert sets), so a step streams cold weights as a real
40-layer decode would.

The K timed steps are captured once in a HIP graph (removing host launch cost)
and replayed; W eager warm-up steps and one untimed replay precede the timed
replay.  The library's measurement entry point records HIP events between its
launches on the stream they run on, giving each kernel's average duration over
the timed region; the dominant one is reported in `roofline`.

`cpu_baseline` times the CPU oracle on a bounded sample of the same workload
(a few tokens, weights pre-quantised untimed, dequantisation on the fly).
"""

import argparse
import ctypes as C
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth
# MI355X published dense matrix peaks (TFLOP/s): the exact-split E2M1 path runs
# bf16 MFMA; the MX path's fp4 x fp8 scaled MFMA is priced at the fp8 rate
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}
METRIC = "MoE-layer µs/token and achieved HBM GB/s (% of peak), W4A16 decode"


# ----------------------------------------------------------------------------- HIP events


class HipEvents:
    """Raw hipEvent_t handles from the HIP runtime torch has loaded."""

    def __init__(self):
        path = None
        for ln in open("/proc/self/maps"):
            if "libamdhip64" in ln:
                path = ln.split()[-1]
                break
        self.hip = C.CDLL(path or "libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.hip.hipEventDestroy.argtypes = [C.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = C.c_void_p()
            if self.hip.hipEventCreate(C.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(e.value)
        return out

    def elapsed_ms(self, a, b):
        ms = C.c_float()
        if self.hip.hipEventElapsedTime(C.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(e)


# ----------------------------------------------------------------------------- helpers


def source_digest():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "bit_block_scaled_router_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel, workload):
    """HBM bytes per dispatch from committed rocprofv3 counter runs, if still current."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        db = json.load(f)
    rec = db.get(workload, {}).get(kernel)
    if not rec or rec.get("source_digest") != source_digest():
        return None
    return rec.get("hbm_bytes_per_dispatch")


COPY_KIB = 256 * 1024  # the --calibrate-copy kernel reads and writes 256 MiB


def ingest_counters(paths, workload):
    """Per-kernel means of rocprofv3 --pmc CSV files (counter_collection.csv).

    Prints one line per (kernel, counter).  When FETCH_SIZE and WRITE_SIZE are
    both present, each is scaled by what it reads for the plain 256 MiB copy of
    --calibrate-copy (the first three copyBuffer dispatches) and the HBM bytes
    per dispatch are stored in profiles/traffic.json under `workload` with the
    current kernel source digest."""
    import csv
    import re
    vals = {}  # (kernel, counter) -> list
    calib = {}
    for path in paths:
        with open(path, newline="") as f:
            for row in csv.DictReader(f):
                name, ctr, v = row["Kernel_Name"], row["Counter_Name"], float(row["Counter_Value"])
                if "copyBuffer" in name:
                    calib.setdefault(ctr, []).append(v)
                    continue
                m = re.search(r"w4k::(k_\w+)", name)
                if m:
                    vals.setdefault((m.group(1), ctr), []).append(v)
    out = {}
    for (k, c), v in sorted(vals.items()):
        print(f"{k:20s} {c:28s} dispatches={len(v):5d} mean={sum(v) / len(v):.3f}")
        out.setdefault(k, {})[c] = sum(v) / len(v)
        out[k]["dispatches"] = len(v)
    factors = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        if c in calib and len(calib[c]) >= 3:
            factors[c] = COPY_KIB / (sum(calib[c][:3]) / 3)
            print(f"calibration {c}: {sum(calib[c][:3]) / 3:.1f} KiB per 256 MiB copy -> factor {factors[c]:.5f}")
    if len(factors) == 2:
        path = os.path.join(ROOT, "profiles", "traffic.json")
        db = json.load(open(path)) if os.path.exists(path) else {}
        rec = db.setdefault(workload, {})
        for k, d in out.items():
            if "FETCH_SIZE" in d and "WRITE_SIZE" in d:
                b = (d["FETCH_SIZE"] * factors["FETCH_SIZE"] + d["WRITE_SIZE"] * factors["WRITE_SIZE"]) * 1024
                rec[k] = {"hbm_bytes_per_dispatch": round(b), "fetch_kib": round(d["FETCH_SIZE"], 3),
                          "write_kib": round(d["WRITE_SIZE"], 3), "fetch_factor": round(factors["FETCH_SIZE"], 5),
                          "write_factor": round(factors["WRITE_SIZE"], 5), "source_digest": source_digest()}
                print(f"{k:20s} HBM bytes per dispatch {b:,.0f}")
        with open(path, "w") as f:
            json.dump(db, f, indent=1)
            f.write("\n")


def clone_layer(w4, layer):
    """A deep copy of a device MoE layer (new addresses, same contents)."""
    def cq(q):
        g = q.global_scales.clone() if q.global_scales is not None else None
        sc = q.scales.clone() if q.scales is not None else None
        return w4.QMatrix(q.fmt, q.groups, q.n, q.k, q.codes.clone(), sc, g)

    kw = {}
    if layer.has_shared:
        kw = dict(shared_w13=cq(layer.shared_w13), shared_w2=cq(layer.shared_w2),
                  shared_gate_w=layer.shared_gate_w.clone())
    rb = layer.router_bias.clone() if layer.router_bias is not None else None
    return w4.MoELayer(layer.hidden, layer.inter, layer.num_experts, layer.top_k, layer.router_w.clone(),
                       cq(layer.w13), cq(layer.w2), router_bias=rb, **kw)


def weight_bytes(fmt, n, k):
    """Bytes of one quantised [n][k] matrix: codes, block scales (FP16 per 16 or per
    128; NVFP4: one UE4M3 byte per 16 plus a 4-byte global scale; MXFP4: one
    E8M0 byte per 32)."""
    if fmt == "nvfp4":
        return n * k // 2 + n * k // 16 + 4
    if fmt == "mxfp4":
        return n * k // 2 + n * k // 32
    if fmt == "bf16":
        return n * k * 2
    return n * k // 2 + n * k // (128 if fmt == "int4" else 16) * 2


def moe_bytes(shape, distinct):
    """Algorithmic HBM bytes of one MoE step: every byte the method must move once.

    router bf16 [E][H]; for each distinct selected expert and the shared expert,
    W13 and W2 codes (half a byte per element) and block scales; shared-gate
    bf16 [H]; x and y bf16 [T][H]."""
    H, I, E, T = shape.hidden, shape.inter, shape.num_experts, shape.tokens
    per_expert = weight_bytes(shape.fmt, 2 * I, H) + weight_bytes(shape.fmt, H, I)
    sfmt = shape.shared_fmt or shape.fmt
    b = E * H * 2 + distinct * per_expert + 2 * T * H * 2
    if shape.has_shared:
        b += weight_bytes(sfmt, 2 * I, H) + weight_bytes(sfmt, H, I) + H * 2
    return b


def stage_bytes(shape, distinct, n_stages=3):
    """Algorithmic bytes per launch of each MoE kernel (T = shape.tokens).

    Single-token path (3 kernels): router, W13 + SiLU over all (token, slot),
    down + combine.  Batched path (5 kernels): router, top-k + grouping, W13 per
    expert group, W2 per expert group, ordered combine.  Weights count once per
    distinct expert (the batched path reads each active expert once)."""
    H, I, E, T, K = shape.hidden, shape.inter, shape.num_experts, shape.tokens, shape.top_k
    S = K + (1 if shape.has_shared else 0)
    w13 = weight_bytes(shape.fmt, 2 * I, H)
    w2 = weight_bytes(shape.fmt, H, I)
    sfmt = shape.shared_fmt or shape.fmt
    sh = 1 if shape.has_shared else 0
    # the shared expert's matrices replace one routed expert's in the sums below
    dw13, dw2 = sh * (weight_bytes(sfmt, 2 * I, H) - w13), sh * (weight_bytes(sfmt, H, I) - w2)
    nexp = distinct + sh
    router = E * H * 2 + (H * 2 if shape.has_shared else 0) + T * H * 2 + T * (E + 1) * 4
    if n_stages == 3:
        return {
            "k_router": router,
            "k_moe_w13": nexp * w13 + dw13 + T * H * 2 + T * E * 4 + T * S * I * 4,
            "k_moe_down": nexp * w2 + dw2 + T * S * I * 4 + T * K * 8 + T * H * 2,
        }
    rows = T * K + T  # routed pairs + shared rows
    if n_stages in (7, 8):  # grouping over three launches (large batches)
        b = stage_bytes(shape, distinct, n_stages - 2)
        b.pop("k_moe_route_group")
        nblk = (T + 15) // 16
        b["k_route_topk"] = T * E * 4 + T * K * 12 + nblk * E * 4
        b["k_route_scan"] = 2 * nblk * E * 4 + E * 4 + (1 + 3 * min(E, T * K)) * 4
        b["k_route_scatter"] = T * K * 4 + nblk * E * 4 + E * 4 + rows * 4
        return b
    if n_stages == 6:  # MX: x and h travel as MXFP8 (a byte per element + a scale byte per 32)
        return {
            "k_router": router,
            "k_mx_quant": T * H * 2 + T * H * 33 // 32,
            "k_moe_route_group": T * E * 4 + T * K * 8 + rows * 4,
            "k_moe_mx13": nexp * w13 + T * H * 33 // 32 + rows * I * 33 // 32,
            "k_moe_mx2": nexp * w2 + rows * I * 33 // 32 + rows * H * 4,
            "k_moe_gcombine": rows * H * 4 + T * K * 8 + T * H * 2,
        }
    return {
        "k_router": router,
        "k_moe_route_group": T * E * 4 + T * K * 8 + rows * 4,
        "k_moe_gw13": nexp * w13 + dw13 + T * H * 2 + rows * I * 4,
        "k_moe_gw2": nexp * w2 + dw2 + rows * I * 4 + rows * H * 4,
        "k_moe_gcombine": rows * H * 4 + T * K * 8 + T * H * 2,
    }


ROUTER_MFMA_MIN_T = 64  # the library runs the router as an MFMA GEMM from this batch size


LARGE_BATCH_PAIRS = 4096  # past this many (token, slot) pairs the grouped GEMM kernels run


def stage_names(n_stages, T, K, mx):
    """Kernel names in launch order for the library's stage count at T tokens."""
    router = "k_router_mfma" if T >= ROUTER_MFMA_MIN_T else "k_router"
    if n_stages == 3:
        return [router, "k_moe_w13", "k_moe_down"]
    grouping = ["k_moe_route_group"] if n_stages in (5, 6) else ["k_route_topk", "k_route_scan", "k_route_scatter"]
    experts = ["k_mx_quant"] if mx else []
    large = T * K > LARGE_BATCH_PAIRS
    if mx:
        proj = ["k_moe_pfmx13", "k_moe_pfmx2"] if large else ["k_moe_mx13", "k_moe_mx2"]
    else:
        proj = ["k_moe_pf13", "k_moe_pf2"] if large else ["k_moe_gw13", "k_moe_gw2"]
    return [router] + experts + grouping + proj + ["k_moe_gcombine"]


def launch_bytes(shape, distinct, n_stages):
    """stage_bytes keyed by the kernel names stage_names gives for the same call."""
    sb = stage_bytes(shape, distinct, n_stages)
    if shape.tokens >= ROUTER_MFMA_MIN_T:
        sb["k_router_mfma"] = sb.pop("k_router")
    if shape.tokens * shape.top_k > LARGE_BATCH_PAIRS:  # the grouped GEMM kernels move the same algorithmic bytes
        for a, b in (("k_moe_gw13", "k_moe_pf13"), ("k_moe_gw2", "k_moe_pf2"), ("k_moe_mx13", "k_moe_pfmx13"),
                     ("k_moe_mx2", "k_moe_pfmx2")):
            if a in sb:
                sb[b] = sb.pop(a)
    return sb


def stage_flops(shape):
    """Algorithmic flops per launch of the grouped projections (2 per multiply-add:
    every routed pair and every shared row through W13 and W2)."""
    rows = shape.tokens * shape.top_k + (shape.tokens if shape.has_shared else 0)
    w13 = 2 * rows * 2 * shape.inter * shape.hidden
    w2 = 2 * rows * shape.hidden * shape.inter
    return {"k_moe_gw13": w13, "k_moe_gw2": w2, "k_moe_mx13": w13, "k_moe_mx2": w2, "k_moe_pf13": w13,
            "k_moe_pf2": w2, "k_moe_pfmx13": w13, "k_moe_pfmx2": w2}


# ----------------------------------------------------------------------------- CPU baseline


def cpu_baseline_moe(shape, tokens, reps):
    """Oracle forward per token (float64, dequantisation on the fly), bounded sample."""
    import oracle
    from oracle import ops
    from bit_block_scaled_router_amd import synth

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - optional
        blas_threads = 1
    rw = synth.router_weight(shape)
    xs = np.stack([synth.x_row(shape.seed, shape.hidden, t) for t in range(tokens)])
    bias = synth.router_bias(shape)
    need = set()
    for t in range(tokens):
        ids, _ = ops.route(ops.router_logits(rw, xs[t], bias), shape.top_k)
        need.update(int(e) for e in ids)
    ofmts = {"e2m1": oracle.FMT_E2M1, "int4": oracle.FMT_INT4, "nvfp4": oracle.FMT_NVFP4, "bf16": oracle.FMT_BF16,
             "mxfp4": oracle.FMT_MXFP4}
    fmt = ofmts[shape.fmt]
    sfmt = ofmts[shape.shared_fmt] if shape.shared_fmt else fmt
    q13 = {e: oracle.quantize(fmt, synth.expert_w13(shape, e)) for e in need}
    q2 = {e: oracle.quantize(fmt, synth.expert_w2(shape, e)) for e in need}
    kw = {}
    if shape.has_shared:
        kw = dict(shared_w13=oracle.quantize(sfmt, synth.shared_w13(shape)),
                  shared_w2=oracle.quantize(sfmt, synth.shared_w2(shape)),
                  shared_gate_w=synth.shared_gate_weight(shape), shared_fmt=sfmt)
    times = []
    for _ in range(reps):
        layer = ops.MoELayer(fmt, shape.hidden, shape.inter, shape.num_experts, shape.top_k, rw,
                             lambda e: q13[e], lambda e: q2[e], router_bias=bias, **kw)
        t0 = time.perf_counter()
        ops.moe_forward(layer, xs)
        times.append(time.perf_counter() - t0)
    per_token_us = float(np.median(times)) / tokens * 1e6
    return {
        "value": per_token_us,
        "unit": "us/layer-token",
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": f"{tokens} token(s) of the same layer shape, float64 oracle forward with on-the-fly "
                  f"dequantisation, weights pre-quantised untimed; median of {reps} runs",
        "host_cores_available": len(os.sched_getaffinity(0)),
    }


def cpu_baseline_gemv(shape, reps, max_rows=8192):
    """Oracle GEMV on the workload, or on its first `max_rows` rows scaled to the
    full row count (the oracle is a row-by-row definition, so time is linear in rows)."""
    import oracle
    from bit_block_scaled_router_amd import synth

    ofmt = {"e2m1": oracle.FMT_E2M1, "int4": oracle.FMT_INT4, "nvfp4": oracle.FMT_NVFP4}[shape.fmt]
    rows = min(shape.n, max_rows)
    w = synth.normal_f32((rows, shape.k), synth.SIGMA_W, shape.seed, 9) if rows < shape.n else synth.dense_weight(shape)
    q = oracle.quantize(ofmt, w)
    x = synth.dense_x(shape)
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        oracle.gemv(ofmt, q[0], q[1], x, *q[2:])
        times.append(time.perf_counter() - t0)
    scale = shape.n / rows
    sample = (f"the full {shape.n}x{shape.k} GEMV" if rows == shape.n else
              f"the first {rows} of {shape.n} rows, time scaled by {scale:.2f}") + f", median of {reps} runs"
    return {"value": float(np.median(times)) * 1e6 * scale, "unit": "us/call", "cores": 1, "kind": "oracle",
            "sample": sample, "host_cores_available": len(os.sched_getaffinity(0))}


# ----------------------------------------------------------------------------- GPU runs


def workload_shapes(synth):
    """bench workload name -> synth shape."""
    return {"qwen-t1": synth.QWEN_MOE_T1, "qwen-t32": synth.QWEN_MOE_T32, "tiny": synth.TINY_MOE,
            "gemv-e2m1": synth.GEMV_E2M1, "gemv-int4": synth.GEMV_INT4,
            "qwen-t1-nvfp4": synth.QWEN_MOE_T1_NVFP4, "gemv-nvfp4": synth.GEMV_NVFP4,
            "gemv-lmhead": synth.GEMV_LMHEAD, "qwen-t1-bf16shared": synth.QWEN_MOE_T1_BF16SH,
            "qwen-t1-mxfp4": synth.QWEN_MOE_T1_MX, "qwen-t32-mxfp4": synth.QWEN_MOE_T32_MX,
            "qwen-prefill": synth.QWEN_MOE_PREFILL, "qwen-prefill-mxfp4": synth.QWEN_MOE_PREFILL_MX,
            "qwen-t32-nvfp4": synth.QWEN_MOE_T32_NVFP4, "qwen-t32-bf16shared": synth.QWEN_MOE_T32_BF16SH,
            "qwen-t32-int4": synth.QWEN_MOE_T32_INT4}


WORKLOADS = ["qwen-t1", "qwen-t32", "tiny", "gemv-e2m1", "gemv-int4", "qwen-t1-nvfp4", "gemv-nvfp4", "gemv-lmhead",
             "qwen-t1-bf16shared", "qwen-t1-mxfp4", "qwen-t32-mxfp4", "qwen-prefill", "qwen-prefill-mxfp4",
             "qwen-t32-nvfp4", "qwen-t32-bf16shared", "qwen-t32-int4"]


def run_moe(args, torch, w4, wl, synth):
    shape = workload_shapes(synth)[args.workload]
    T = shape.tokens
    print(f"[bench] building {shape.name} ({args.replicas} replicas)", file=sys.stderr, flush=True)
    base = wl.build_moe_layer(shape, device="cuda")
    layers = [base] + [clone_layer(w4, base) for _ in range(args.replicas - 1)]
    pool = np.stack([np.stack([synth.x_row(shape.seed, shape.hidden, p * T + t) for t in range(T)])
                     for p in range(args.pool)])
    xs = wl.bf16_tensor(pool, "cuda")  # [P][T][H]
    y = torch.empty((T, shape.hidden), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((T, shape.top_k), dtype=torch.int32, device="cuda")
    ws = w4.alloc_workspace(base, T)
    # distinct routed experts per step (for the algorithmic byte count)
    distinct = []
    for p in range(args.pool):
        w4.moe_w4a16_forward(base, xs[p], y=y, topk_ids=ids, ws=ws)
        distinct.append(len(set(ids.cpu().numpy().ravel().tolist())))
    torch.cuda.synchronize()
    n_steps = args.steps
    R, P = len(layers), args.pool
    for i in range(args.warmup):
        w4.moe_w4a16_forward(layers[i % R], xs[i % P], y=y, ws=ws)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(n_steps):
                w4.moe_w4a16_forward(layers[i % R], xs[i % P], y=y, ws=ws)
    torch.cuda.synchronize()
    g.replay()  # untimed warm replay
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record()
    g.replay()
    end.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_total = start.elapsed_time(end)

    # per-kernel durations: the same K steps launched eagerly through the
    # measurement entry point, whose kernels carry start/stop HIP events
    n_stages = w4.moe_w4a16_stage_count(base, T)
    names = stage_names(n_stages, T, shape.top_k, shape.fmt == "mxfp4")
    hip = HipEvents()
    ne = 2 * n_stages
    evs = hip.create(ne * n_steps)
    for i in range(n_steps):
        w4.moe_w4a16_forward_timed(layers[i % R], xs[i % P], y, ws, evs[ne * i:ne * i + ne])
    torch.cuda.synchronize()
    stage = {k: [] for k in names}
    for i in range(n_steps):
        e = evs[ne * i:ne * i + ne]
        for si, k in enumerate(names):
            stage[k].append(hip.elapsed_ms(e[2 * si], e[2 * si + 1]))
    hip.destroy(evs)
    stage_us = {k: float(np.mean(v)) * 1e3 for k, v in stage.items()}

    # eager (no graph) rate for context
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(min(n_steps, 200)):
        w4.moe_w4a16_forward(layers[i % R], xs[i % P], y=y, ws=ws)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) / min(n_steps, 200) * 1e3

    d_mean = float(np.mean(distinct))
    ms_step = ms_total / n_steps
    us_token = ms_step * 1e3 / T
    step_bytes = moe_bytes(shape, d_mean)
    sb = launch_bytes(shape, d_mean, n_stages)
    dom = max(stage_us, key=stage_us.get)
    achieved = sb[dom] / (stage_us[dom] * 1e-6) / 1e9
    traffic = load_traffic(dom, shape.name)
    # the dominant kernel's bound: HBM bytes or MFMA flops, whichever takes longer
    # at the published peaks
    fl = stage_flops(shape).get(dom)
    mfma_peak = MFMA_PEAK_TFLOPS["fp8" if shape.fmt == "mxfp4" else "bf16"]
    roof = {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS}
    if fl is not None:
        tflops = fl / (stage_us[dom] * 1e-6) / 1e12
        roof["mfma_tflops"] = tflops
        roof["mfma_frac"] = tflops / mfma_peak
        roof["mfma_peak"] = mfma_peak
        roof["algorithmic_flops_per_launch"] = fl
        if fl / (mfma_peak * 1e12) > sb[dom] / (HBM_PEAK_GBS * 1e9):
            roof.update({"bound": "mfma", "achieved": tflops, "peak": mfma_peak, "unit": "TFLOP/s",
                         "frac": tflops / mfma_peak, "hbm_gbps": achieved})
    res = {
        "metric": METRIC,
        "value": us_token,
        "unit": "us/layer-token",
        "n_gpus": 1,
        "steps": n_steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": shape.name, "hidden": shape.hidden, "experts": shape.num_experts,
            "top_k": shape.top_k, "inter": shape.inter, "shared_inter": shape.shared_inter,
            "tokens_per_step": T, "zipf_s": shape.zipf_s, "weights": {"e2m1": "E2M1 codes + FP16 scale per 16",
                        "nvfp4": "E2M1 codes + UE4M3 scale per 16 + fp32 scale per matrix",
                        "int4": "int4 codes + FP16 scale per 128",
                        "mxfp4": "E2M1 codes + E8M0 scale per 32"}[shape.fmt]
                       + (", shared expert bf16" if shape.shared_fmt == "bf16" else ""),
            "activations": ("bf16; MXFP8 (E4M3 + E8M0 per 32) inside the experts" if shape.fmt == "mxfp4"
                            else "bf16"), "accumulate": "fp32", "layer_replicas": R, "token_pool": P,
            "mean_distinct_experts": d_mean, "timing": "HIP graph replay of the K steps",
        },
        "hbm_gbps": step_bytes / (ms_step * 1e-3) / 1e9,
        "pct_hbm_peak": 100.0 * step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "algorithmic_bytes_per_step": step_bytes,
        "stage_us": stage_us,
        "eager_ms_per_step": eager_ms,
        "wall_s_timed": t_wall,
        "roofline": {
            **roof,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": sb[dom], "avg_launch_us": stage_us[dom],
            "note": "avg launch duration from start/stop HIP events the runtime records around each "
                    "kernel (hipExtLaunchKernel) over K eager steps of the same workload",
        },
    }
    return res, shape


def run_gemv(args, torch, w4, wl, synth):
    shape = workload_shapes(synth)[args.workload]
    print(f"[bench] building {shape.name} ({args.replicas} replicas)", file=sys.stderr, flush=True)
    base = wl.build_dense(shape, "cuda")
    reps = [base] + [w4.QMatrix(base.fmt, 1, base.n, base.k, base.codes.clone(), base.scales.clone(),
                                base.global_scales.clone() if base.global_scales is not None else None)
                     for _ in range(args.replicas - 1)]
    x = wl.bf16_tensor(synth.dense_x(shape), "cuda")
    y = torch.empty(shape.n, dtype=torch.bfloat16, device="cuda")
    R = len(reps)
    for i in range(args.warmup):
        w4.w4a16_gemv(reps[i % R], x, y=y)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(args.steps):
                w4.w4a16_gemv(reps[i % R], x, y=y)
    g.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    g.replay()
    end.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / args.steps
    g_bytes = weight_bytes(shape.fmt, shape.n, shape.k) + shape.k * 2 + shape.n * 2
    gbs = g_bytes / (ms_step * 1e-3) / 1e9
    res = {
        "metric": METRIC, "value": ms_step * 1e3, "unit": "us/call", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": shape.name, "n": shape.n, "k": shape.k, "format": shape.fmt,
                   "replicas": R, "timing": "HIP graph replay of the K steps"},
        "hbm_gbps": gbs, "pct_hbm_peak": 100 * gbs / HBM_PEAK_GBS, "algorithmic_bytes_per_step": g_bytes,
        "roofline": {"bound": "hbm", "kernel": "k_gemv", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": load_traffic("k_gemv", shape.name),
                     "algorithmic_bytes_per_launch": g_bytes, "avg_launch_us": ms_step * 1e3,
                     "note": "graph replay time per launch (one kernel per step)"},
    }
    return res, shape


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="qwen-t1",
                    choices=WORKLOADS)
    ap.add_argument("--replicas", type=int, default=0, help="weight replicas (0 = workload default)")
    ap.add_argument("--pool", type=int, default=64, help="token pool (MoE workloads)")
    ap.add_argument("--cpu-tokens", type=int, default=1)
    ap.add_argument("--cpu-reps", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first copy 256 MiB device-to-device 3 times (a plain copy of known size for counter runs)")
    ap.add_argument("--ingest-counters", nargs="+", metavar="CSV",
                    help="summarise rocprofv3 --pmc CSV files of a run of this workload (no GPU needed)")
    args = ap.parse_args()
    if args.ingest_counters:
        from bit_block_scaled_router_amd import synth
        ingest_counters(args.ingest_counters, workload_shapes(synth)[args.workload].name)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    if args.replicas <= 0:  # enough weight bytes that the 256 MB Infinity Cache cannot hold them
        args.replicas = 4 if args.workload in ("gemv-lmhead",) or not args.workload.startswith("gemv") else 128
    if args.workload.startswith("qwen-t32"):
        args.pool = min(args.pool, 8)
    if args.workload.startswith("qwen-prefill"):  # 2048 tokens per step
        args.pool = min(args.pool, 2)

    import torch

    import bit_block_scaled_router_amd as w4
    from bit_block_scaled_router_amd import synth, workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    w4.lib()
    if args.calibrate_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.workload.startswith("gemv"):
        res, shape = run_gemv(args, torch, w4, wl, synth)
        cpu = None if args.no_cpu_baseline else cpu_baseline_gemv(shape, args.cpu_reps)
    else:
        res, shape = run_moe(args, torch, w4, wl, synth)
        cpu = None if args.no_cpu_baseline else cpu_baseline_moe(
            shape, args.cpu_tokens if shape.tokens == 1 else 4, args.cpu_reps if shape.tokens == 1 else 2)
    res["cpu_baseline"] = cpu
    res["device"] = torch.cuda.get_device_name(0)
    res["source_digest"] = source_digest()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
