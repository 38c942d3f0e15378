"""Benchmark: W4A16 MoE decode layer (and dense GEMV) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]

Prints ONE JSON line.  A step is one full pass of the hot path over one batch of
synthetic input: for the default workload, one token through the whole MoE layer
of the Qwen 3.6 35B-A3B shape (router GEMV, softmax/top-8/renormalise, grouped
W13 + SiLU over 8 routed + 1 shared expert, down projection + weighted combine).
Inputs are resident in HBM before the timed region.  To keep the 256 MB
Infinity Cache from serving weights, steps rotate over 4 replicas of the routed
experts (4 x 483 MiB), over enough copies of the routing-independent tensors
(router, shared-gate weight, shared expert: at least 288 MB of copies) and over a
pool of tokens (distinct expert sets), so each step streams cold weights as a
real 40-layer decode would.

The K timed steps are captured once in a HIP graph (removing host launch cost)
and replayed after W eager warm-up steps and one untimed replay.  Each kernel's
duration is measured the way a kernel trace sees it, in isolation: the captured
graph's kernel nodes of one stage (the same K launches, same arguments, same
order) are copied into a graph of their own, which is replayed and timed; the
per-launch average is `stage_us`, and the stage with the largest one is the
dominant kernel of `roofline`.  Every step has its own workspace slot (one per
token of the pool), so a stage replayed alone reads the intermediates its own
step wrote.

`ceiling` times the library's streaming-read probe on a buffer the size of the
dominant kernel's algorithmic bytes (rotated over >= 1.3 GB) and on 4 GiB: the
box's practical read rate, a second denominator beside the 8 TB/s peak.
`cpu_baseline` times the CPU oracle on a bounded sample of the same workload;
`variants` holds it single-threaded and on all cores, with dequantisation on the
fly and cached.
"""

import argparse
import ctypes as C
import hashlib
import json
import os
import shutil
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


class Dim3(C.Structure):
    _fields_ = [("x", C.c_uint32), ("y", C.c_uint32), ("z", C.c_uint32)]


class KernelNodeParams(C.Structure):  # hipKernelNodeParams
    _fields_ = [("blockDim", Dim3), ("extra", C.c_void_p), ("func", C.c_void_p), ("gridDim", Dim3),
                ("kernelParams", C.c_void_p), ("sharedMemBytes", C.c_uint)]


class HipRuntime:
    """The HIP runtime torch has loaded: raw events, graph surgery and versions."""

    def __init__(self):
        path = None
        for ln in open("/proc/self/maps"):
            if "libamdhip64" in ln:
                path = ln.split()[-1]
                break
        self.hip = h = C.CDLL(path or "libamdhip64.so")
        P, SZ = C.c_void_p, C.c_size_t
        h.hipEventCreate.argtypes = [C.POINTER(P)]
        h.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), P, P]
        h.hipEventDestroy.argtypes = [P]
        h.hipEventRecord.argtypes = [P, P]
        h.hipEventSynchronize.argtypes = [P]
        h.hipGraphGetRootNodes.argtypes = [P, C.POINTER(P), C.POINTER(SZ)]
        h.hipGraphNodeGetDependentNodes.argtypes = [P, C.POINTER(P), C.POINTER(SZ)]
        h.hipGraphNodeGetType.argtypes = [P, C.POINTER(C.c_int)]
        h.hipGraphKernelNodeGetParams.argtypes = [P, C.POINTER(KernelNodeParams)]
        h.hipGraphCreate.argtypes = [C.POINTER(P), C.c_uint]
        h.hipGraphAddKernelNode.argtypes = [C.POINTER(P), P, C.POINTER(P), SZ, C.POINTER(KernelNodeParams)]
        h.hipGraphInstantiate.argtypes = [C.POINTER(P), P, P, C.c_char_p, SZ]
        h.hipGraphLaunch.argtypes = [P, P]
        h.hipGraphExecDestroy.argtypes = [P]
        h.hipGraphDestroy.argtypes = [P]
        h.hipStreamSynchronize.argtypes = [P]
        h.hipRuntimeGetVersion.argtypes = [C.POINTER(C.c_int)]
        h.hipDriverGetVersion.argtypes = [C.POINTER(C.c_int)]

    def _ok(self, st, what):
        if st != 0:
            raise RuntimeError(f"{what} failed ({st})")

    def create(self, n):
        out = []
        for _ in range(n):
            e = C.c_void_p()
            self._ok(self.hip.hipEventCreate(C.byref(e)), "hipEventCreate")
            out.append(e.value)
        return out

    def elapsed_ms(self, a, b):
        ms = C.c_float()
        self._ok(self.hip.hipEventElapsedTime(C.byref(ms), a, b), "hipEventElapsedTime")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(e)

    def versions(self):
        rt, dr = C.c_int(0), C.c_int(0)
        self.hip.hipRuntimeGetVersion(C.byref(rt))
        self.hip.hipDriverGetVersion(C.byref(dr))
        return {"hip_runtime": rt.value, "hip_driver": dr.value, "library": self.hip._name}

    def kernel_chain(self, graph):
        """Kernel nodes of a captured single-stream graph in launch order."""
        h = self.hip
        n = C.c_size_t(0)
        self._ok(h.hipGraphGetRootNodes(graph, None, C.byref(n)), "hipGraphGetRootNodes")
        if n.value != 1:
            raise RuntimeError(f"expected one root node, got {n.value}")
        roots = (C.c_void_p * 1)()
        self._ok(h.hipGraphGetRootNodes(graph, roots, C.byref(n)), "hipGraphGetRootNodes")
        chain, node = [], roots[0]
        while node:
            t = C.c_int(-1)
            self._ok(h.hipGraphNodeGetType(node, C.byref(t)), "hipGraphNodeGetType")
            if t.value == 0:  # hipGraphNodeTypeKernel
                chain.append(node)
            m = C.c_size_t(0)
            self._ok(h.hipGraphNodeGetDependentNodes(node, None, C.byref(m)), "hipGraphNodeGetDependentNodes")
            if m.value > 1:
                raise RuntimeError("the captured graph is not a single chain")
            if m.value == 0:
                break
            nxt = (C.c_void_p * 1)()
            self._ok(h.hipGraphNodeGetDependentNodes(node, nxt, C.byref(m)), "hipGraphNodeGetDependentNodes")
            node = nxt[0]
        return chain

    def replay_nodes_us(self, nodes, stream, reps=2, spin=None):
        """Copy the kernel nodes (in order, one chain) into a graph of their own,
        replay it and return the average microseconds per launch (best of reps)."""
        h = self.hip
        g = C.c_void_p()
        self._ok(h.hipGraphCreate(C.byref(g), 0), "hipGraphCreate")
        prev = None
        for node in nodes:
            p = KernelNodeParams()
            self._ok(h.hipGraphKernelNodeGetParams(node, C.byref(p)), "hipGraphKernelNodeGetParams")
            new = C.c_void_p()
            deps = (C.c_void_p * 1)(prev) if prev is not None else None
            self._ok(h.hipGraphAddKernelNode(C.byref(new), g, deps, 1 if prev is not None else 0, C.byref(p)),
                     "hipGraphAddKernelNode")
            prev = new.value
        ex = C.c_void_p()
        self._ok(h.hipGraphInstantiate(C.byref(ex), g, None, None, 0), "hipGraphInstantiate")
        e0, e1 = self.create(2)
        try:
            self._ok(h.hipGraphLaunch(ex, stream), "hipGraphLaunch")  # warm
            self._ok(h.hipStreamSynchronize(stream), "hipStreamSynchronize")
            best = None
            for _ in range(reps):
                if spin is not None:  # keep the GPU busy while the host submits the graph
                    spin()
                self._ok(h.hipEventRecord(e0, stream), "hipEventRecord")
                self._ok(h.hipGraphLaunch(ex, stream), "hipGraphLaunch")
                self._ok(h.hipEventRecord(e1, stream), "hipEventRecord")
                self._ok(h.hipEventSynchronize(e1), "hipEventSynchronize")
                us = self.elapsed_ms(e0, e1) * 1e3 / len(nodes)
                best = us if best is None else min(best, us)
        finally:
            self.destroy([e0, e1])
            h.hipGraphExecDestroy(ex)
            h.hipGraphDestroy(g)
        return best


def machine_info(hip):
    """Device, ROCm/HIP versions and clocks (rocm-smi, when it answers)."""
    import subprocess
    import torch

    props = torch.cuda.get_device_properties(0)
    info = {"device": torch.cuda.get_device_name(0), "arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count, "torch": torch.__version__, "torch_hip": torch.version.hip}
    info.update(hip.versions())
    try:
        with open("/opt/rocm/.info/version") as f:
            info["rocm"] = f.read().strip()
    except OSError:
        info["rocm"] = None
    # Under a profiler the child would inherit the profiler's preloaded library,
    # which opens the GPU before rocm-smi's "#!/usr/bin/env python3" line execs
    # the interpreter: such a run does not sample the clocks.  Otherwise the
    # script runs under this interpreter directly (no exec hop inside the child).
    if any(k.startswith("ROCPROF") for k in os.environ) or "rocprof" in os.environ.get("LD_PRELOAD", ""):
        info["clocks"] = "not sampled under a profiler"
        return info
    try:
        smi = shutil.which("rocm-smi")
        if smi is None:
            raise FileNotFoundError("rocm-smi")
        with open(smi, "rb") as f:
            python_script = b"python" in f.readline()
        cmd = ([sys.executable, smi] if python_script else [smi]) + ["--showclocks", "--json"]
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=30)
        clk = json.loads(r.stdout) if r.returncode == 0 else None
        if isinstance(clk, dict) and clk:
            card = clk[sorted(clk)[0]]
            info["clocks"] = {k: v for k, v in card.items() if "clock" in k.lower() or k.lower().startswith(("sclk", "mclk", "fclk", "socclk"))}
            info["clocks_note"] = "rocm-smi's current levels when sampled after the run (idle), not the clock under load"
        else:
            info["clocks"] = None
    except Exception as e:  # rocm-smi missing or refused: say so
        info["clocks"] = f"unavailable: {type(e).__name__}"
    return info


def stream_ceiling(torch, w4, nbytes, min_total=1300 << 20, steps=200):
    """GB/s of the streaming-read probe on buffers of nbytes (rotated over enough
    copies to exceed min_total), as graph replay."""
    nbytes = max(16, nbytes // 16 * 16)
    copies = max(1, -(-min_total // nbytes)) if nbytes < min_total else 1
    bufs = [torch.ones(nbytes, dtype=torch.uint8, device="cuda") for _ in range(copies)]
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    n = max(steps, copies) if nbytes < min_total else 5
    for b in bufs[:4]:
        w4.w4_bench_stream_read(b, sink)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(n):
                w4.w4_bench_stream_read(bufs[i % copies], sink)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    us = timed_replay_ms(torch, g) * 1e3 / n
    del g, bufs
    torch.cuda.empty_cache()
    return {"bytes": nbytes, "us_per_launch": us, "gbps": nbytes / (us * 1e-6) / 1e9, "copies": copies}


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


def _clone_q(w4, q):
    g = q.global_scales.clone() if q.global_scales is not None else None
    sc = q.scales.clone() if q.scales is not None else None
    return w4.QMatrix(q.fmt, q.groups, q.n, q.k, q.codes.clone(), sc, g, layout=q.layout)


def make_layers(w4, base, routed_replicas, copies):
    """`copies` layer descriptors over the same weights' values at distinct
    addresses: layer i takes the routed experts of replica i % routed_replicas
    and its own copy of the router, router bias, shared-gate weight and shared
    expert (layer 0 is `base` itself)."""
    routed = [(base.w13, base.w2)] + [(_clone_q(w4, base.w13), _clone_q(w4, base.w2))
                                      for _ in range(routed_replicas - 1)]
    layers = [base]
    for i in range(1, copies):
        kw = {}
        if base.has_shared:
            kw = dict(shared_w13=_clone_q(w4, base.shared_w13), shared_w2=_clone_q(w4, base.shared_w2),
                      shared_gate_w=base.shared_gate_w.clone())
        rb = base.router_bias.clone() if base.router_bias is not None else None
        w13, w2 = routed[i % routed_replicas]
        layers.append(w4.MoELayer(base.hidden, base.inter, base.num_experts, base.top_k, base.router_w.clone(),
                                  w13, w2, router_bias=rb, **kw))
    return layers


def shared_copy_bytes(layer):
    """Bytes of one copy of the routing-independent tensors of a device layer."""
    def qb(q):
        return q.codes.numel() * q.codes.element_size() + (
            q.scales.numel() * q.scales.element_size() if q.scales is not None else 0)
    b = layer.router_w.numel() * 2
    if layer.has_shared:
        b += qb(layer.shared_w13) + qb(layer.shared_w2) + layer.shared_gate_w.numel() * 2
    return b


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


def stage_bytes(shape, distinct, n_stages=3, decode=False):
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
    if decode:  # router; W13 rows + K tiles of W2 per (token, slot, tile); ordered combine of the tiles
        part = T * S * (I // 16) * H * 4  # fp32 tile contributions (scratch: not counted for the expert launch)
        return {
            "k_router": router,
            "k_moe_dec": nexp * (w13 + w2) + dw13 + dw2 + T * H * 2 + T * E * 4,
            "k_moe_dec_combine": part + T * K * 4 + T * H * 2,
        }
    if n_stages == 3:
        return {
            "k_router": router,
            "k_moe_w13": nexp * w13 + dw13 + T * H * 2 + T * E * 4 + T * S * I * 4,
            "k_moe_down": nexp * w2 + dw2 + T * S * I * 4 + T * K * 8 + T * H * 2,
        }
    rows = T * K + T  # routed pairs + shared rows
    if n_stages in (7, 8):  # grouping over three launches (large batches)
        b = stage_bytes(shape, distinct, n_stages - 2)
        b.pop("k_moe_rank_group")
        nblk = (T + 15) // 16
        b["k_route_topk"] = T * E * 4 + T * K * 12 + nblk * E * 4
        b["k_route_scan"] = 2 * nblk * E * 4 + E * 4 + (1 + 3 * min(E, T * K)) * 4
        b["k_route_scatter"] = T * K * 4 + nblk * E * 4 + E * 4 + rows * 4
        return b
    if n_stages == 6:  # MX: x and h travel as MXFP8 (a byte per element + a scale byte per 32)
        return {
            "k_router": router,
            "k_mx_quant": T * H * 2 + T * H * 33 // 32,
            "k_moe_rank_group": T * E * 4 + T * K * 8 + rows * 4,
            "k_moe_mx13": nexp * w13 + T * H * 33 // 32 + rows * I * 33 // 32,
            "k_moe_mx2": nexp * w2 + rows * I * 33 // 32 + rows * H * 4,
            "k_moe_gcombine": rows * H * 4 + T * K * 8 + T * H * 2,
        }
    return {
        "k_router": router,
        "k_moe_rank_group": T * E * 4 + T * K * 8 + rows * 4,
        "k_moe_gw13": nexp * w13 + dw13 + T * H * 2 + rows * I * 4,
        "k_moe_gw2": nexp * w2 + dw2 + rows * I * 4 + rows * H * 4,
        "k_moe_gcombine": rows * H * 4 + T * K * 8 + T * H * 2,
    }


# weight layouts in HBM: (gate/up and dense matrices, down projections); tags of
# W4_LAYOUT_CANONICAL = 0, W4_LAYOUT_GFX950_V1 = 1 (row records),
# W4_LAYOUT_GFX950_KT16 = 2 (K-tiled down projections: the decode kernels)
LAYOUTS = {"canonical": (0, 0), "gfx950": (1, 1), "decode": (1, 2)}


DECODE_DEFAULT = ()  # workloads measured with K-tiled down projections by default


CANONICAL_DEFAULT = ("qwen-prefill", "qwen-prefill-mxfp4")  # measured faster in the canonical layout


def default_layout(workload):
    """The layout each workload is measured in unless --layout says otherwise."""
    if workload in DECODE_DEFAULT:
        return "decode"
    return "canonical" if workload in CANONICAL_DEFAULT else "gfx950"

ROUTER_MFMA_MIN_T = 160  # the library runs the router as an MFMA GEMM from this batch size


LARGE_BATCH_PAIRS = 1024  # past this many (token, slot) pairs the grouped GEMM kernels run (not for int4)


def stage_names(n_stages, T, K, mx, decode=False, int4=False):
    """Kernel names in launch order for the library's stage count at T tokens
    (int4 experts keep the per-group projection kernels past LARGE_BATCH_PAIRS)."""
    router = "k_router_mfma" if T >= ROUTER_MFMA_MIN_T else "k_router"
    if decode:
        return [router, "k_moe_dec", "k_moe_dec_combine"]
    if n_stages == 3:
        return [router, "k_moe_w13", "k_moe_down"]
    grouping = ["k_moe_rank_group"] if n_stages in (5, 6) else ["k_route_topk", "k_route_scan", "k_route_scatter"]
    experts = ["k_mx_quant"] if mx else []
    large = T * K > LARGE_BATCH_PAIRS and not int4
    if mx:
        proj = ["k_moe_pfmx13", "k_moe_pfmx2"] if large else ["k_moe_mx13", "k_moe_mx2"]
    else:
        proj = ["k_moe_pf13", "k_moe_pf2"] if large else ["k_moe_gw13", "k_moe_gw2"]
    return [router] + experts + grouping + proj + ["k_moe_gcombine"]


def launch_bytes(shape, distinct, n_stages, decode=False):
    """stage_bytes keyed by the kernel names stage_names gives for the same call."""
    sb = stage_bytes(shape, distinct, n_stages, decode)
    if shape.tokens >= ROUTER_MFMA_MIN_T:
        sb["k_router_mfma"] = sb.pop("k_router")
    if shape.tokens * shape.top_k > LARGE_BATCH_PAIRS and shape.fmt != "int4":  # the grouped GEMM kernels move the same algorithmic bytes
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


def _blas_info():
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        return ([f"{p.get('internal_api')} {p.get('version')} ({p.get('threading_layer', '')})" for p in info
                 if p.get("user_api") == "blas"], max([p.get("num_threads", 1) for p in info] or [1]))
    except Exception:  # pragma: no cover - optional
        return [], 1


def _timed(fn, reps):
    fn()  # warm-up (first touch, BLAS thread start)
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
    return float(np.median(times))


def _thread_settings():
    """(label, thread count) pairs: one thread and every core the process may use."""
    n = len(os.sched_getaffinity(0))
    return [("1 thread", 1), (f"{n} threads", n)]


def _limits(n):
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(limits=n)
    except Exception:  # pragma: no cover - optional
        import contextlib
        return contextlib.nullcontext()


def cpu_baseline_moe(shape, tokens, reps):
    """Oracle forward per token (float64), bounded sample: single-threaded and on
    all cores, with dequantisation on the fly (a fresh layer per run) and cached
    (the layer's dequantised experts kept across runs)."""
    import oracle
    from oracle import ops
    from bit_block_scaled_router_amd import synth

    blas, _ = _blas_info()
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

    def new_layer():
        return ops.MoELayer(fmt, shape.hidden, shape.inter, shape.num_experts, shape.top_k, rw,
                            lambda e: q13[e], lambda e: q2[e], router_bias=bias, **kw)

    variants = []
    for label, n in _thread_settings():
        with _limits(n):
            fly = _timed(lambda: ops.moe_forward(new_layer(), xs), reps)
            cached_layer = new_layer()
            cached = _timed(lambda: ops.moe_forward(cached_layer, xs), reps)
        for kind, t in (("dequantisation on the fly", fly), ("dequantised experts cached", cached)):
            variants.append({"threads": n, "dequant": kind, "us_per_layer_token": t / tokens * 1e6,
                             "algorithmic_gbps": moe_bytes(shape, len(need)) / shape.tokens * tokens / t / 1e9})
    head = [v for v in variants if v["threads"] == _thread_settings()[-1][1] and "fly" in v["dequant"]][0]
    return {
        "value": head["us_per_layer_token"],
        "unit": "us/layer-token",
        "cores": head["threads"],
        "kind": "oracle",
        "sample": f"{tokens} token(s) of the same layer shape, float64 oracle forward with on-the-fly "
                  f"dequantisation, weights pre-quantised untimed; median of {reps} runs after one warm-up "
                  f"(value: all cores; `variants`: 1 thread and all cores, dequantisation on the fly and cached)",
        "host_cores_available": len(os.sched_getaffinity(0)),
        "blas": blas,
        "variants": variants,
    }


def cpu_baseline_gemv(shape, reps, max_rows=8192):
    """Oracle GEMV on the workload, or on its first `max_rows` rows scaled to the
    full row count (the oracle is a row-by-row definition, so time is linear in
    rows): single-threaded and on all cores, dequantising on the fly and with the
    dequantised matrix cached."""
    import oracle
    from oracle import ops
    from bit_block_scaled_router_amd import synth

    blas, _ = _blas_info()
    ofmt = {"e2m1": oracle.FMT_E2M1, "int4": oracle.FMT_INT4, "nvfp4": oracle.FMT_NVFP4}[shape.fmt]
    rows = min(shape.n, max_rows)
    w = synth.normal_f32((rows, shape.k), synth.SIGMA_W, shape.seed, 9) if rows < shape.n else synth.dense_weight(shape)
    q = oracle.quantize(ofmt, w)
    x = synth.dense_x(shape)
    scale = shape.n / rows
    wdeq = oracle.dequant(ofmt, *q)
    xv = oracle.bf16_bits_to_f64(x)
    variants = []
    for label, n in _thread_settings():
        with _limits(n):
            fly = _timed(lambda: oracle.gemv(ofmt, q[0], q[1], x, *q[2:]), reps)
            cached = _timed(lambda: np.asarray(wdeq, dtype=np.float64) @ xv, reps)
        for kind, t in (("dequantisation on the fly", fly), ("dequantised matrix cached", cached)):
            variants.append({"threads": n, "dequant": kind, "us_per_call": t * 1e6 * scale})
    head = [v for v in variants if v["threads"] == 1 and "fly" in v["dequant"]][0]
    sample = (f"the full {shape.n}x{shape.k} GEMV" if rows == shape.n else
              f"the first {rows} of {shape.n} rows, time scaled by {scale:.2f}") + \
        f", median of {reps} runs after one warm-up (value: 1 thread, dequantisation on the fly)"
    return {"value": head["us_per_call"], "unit": "us/call", "cores": 1, "kind": "oracle", "sample": sample,
            "host_cores_available": len(os.sched_getaffinity(0)), "blas": blas, "variants": variants}


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


def run_moe(args, torch, w4, wl, synth, hip):
    shape = workload_shapes(synth)[args.workload]
    if args.tokens:  # the same layer at another batch size (sweeps; not a reported workload)
        import dataclasses
        shape = dataclasses.replace(shape, tokens=args.tokens, name=f"{shape.name}@T{args.tokens}")
    if args.seed is not None:  # other synthetic weights and tokens of the same shape
        import dataclasses
        shape = dataclasses.replace(shape, seed=args.seed)
    T = shape.tokens
    l13, l2 = LAYOUTS[args.layout]
    base = wl.build_moe_layer(shape, device="cuda", layout=l13, w2_layout=l2)
    # copies of the routing-independent tensors: at least 288 MB of them, so that
    # a copy comes back only after more than the Infinity Cache has streamed by
    per_copy = shared_copy_bytes(base)
    ncopies = max(args.replicas, min(128, -(-(288 << 20) // per_copy)))
    print(f"[bench] {shape.name}: {args.replicas} routed replicas, {ncopies} copies of the router and shared "
          f"expert ({ncopies * per_copy / 2**20:.0f} MiB)", file=sys.stderr, flush=True)
    layers = make_layers(w4, base, args.replicas, ncopies)
    pool = np.stack([np.stack([synth.x_row(shape.seed, shape.hidden, p * T + t) for t in range(T)])
                     for p in range(args.pool)])
    xs = wl.bf16_tensor(pool, "cuda")  # [P][T][H]
    y = torch.empty((T, shape.hidden), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((T, shape.top_k), dtype=torch.int32, device="cuda")
    ws_bytes = w4.moe_w4a16_workspace_bytes(base, T)
    wsz = (ws_bytes + 255) // 256 * 256
    ws_all = torch.empty(wsz * args.pool, dtype=torch.uint8, device="cuda")
    wss = [ws_all[p * wsz:p * wsz + ws_bytes] for p in range(args.pool)]  # one slot per pool token
    # distinct routed experts per step (for the algorithmic byte count)
    distinct = []
    for p in range(args.pool):
        w4.moe_w4a16_forward(base, xs[p], y=y, topk_ids=ids, ws=wss[p])
        distinct.append(len(set(ids.cpu().numpy().ravel().tolist())))
    torch.cuda.synchronize()
    n_steps = args.steps
    NL, P = len(layers), args.pool

    def step(i):
        w4.moe_w4a16_forward(layers[i % NL], xs[i % P], y=y, ws=wss[i % P])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph(keep_graph=True)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(n_steps):
                step(i)
    g.instantiate()
    torch.cuda.synchronize()
    g.replay()  # untimed warm replay
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    ms_total = timed_replay_ms(torch, g)
    t_wall = time.perf_counter() - t_wall

    # per-kernel durations: each stage's K launches replayed alone, in a graph of
    # their own copied from the captured one (same kernels, arguments and order)
    n_stages = w4.moe_w4a16_stage_count(base, T)
    decode = l2 == 2
    names = stage_names(n_stages, T, shape.top_k, shape.fmt == "mxfp4", decode, shape.fmt == "int4")
    stage_us, timing_note = {}, ("avg launch duration: the stage's K launches copied out of the captured graph "
                                 "and replayed alone (graph replay time / K), on the stream the kernels run on")
    try:
        chain = hip.kernel_chain(g.raw_cuda_graph())
        if len(chain) != n_stages * n_steps:
            raise RuntimeError(f"captured {len(chain)} kernels, expected {n_stages} x {n_steps}")
        cur = torch.cuda.current_stream().cuda_stream
        for si, k in enumerate(names):
            stage_us[k] = hip.replay_nodes_us(chain[si::n_stages], cur, spin=lambda: torch.cuda._sleep(2_000_000))
    except Exception as e:  # report, and fall back to the event timings below
        print(f"[bench] isolated stage replay failed: {e}", file=sys.stderr, flush=True)
        stage_us, timing_note = {}, f"isolated stage replay failed ({e}); medians of per-kernel start/stop events"
    # the same launches with start/stop events around each kernel (eager; reported beside it)
    ne = 2 * n_stages
    n_ev = max(n_steps, 300)
    evs = hip.create(ne * n_ev)
    for i in range(n_ev):
        w4.moe_w4a16_forward_timed(layers[i % NL], xs[i % P], y, wss[i % P], evs[ne * i:ne * i + ne])
    torch.cuda.synchronize()
    stage_ev = {k: [] for k in names}
    for i in range(n_ev):
        e = evs[ne * i:ne * i + ne]
        for si, k in enumerate(names):
            stage_ev[k].append(hip.elapsed_ms(e[2 * si], e[2 * si + 1]))
    hip.destroy(evs)
    stage_us_events = {k: float(np.median(v)) * 1e3 for k, v in stage_ev.items()}
    if not stage_us:
        stage_us = dict(stage_us_events)

    # eager (no graph) rate for context
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(min(n_steps, 200)):
        step(i)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) / min(n_steps, 200) * 1e3
    del g
    torch.cuda.synchronize()

    d_mean = float(np.mean(distinct))
    ms_step = ms_total / n_steps
    us_token = ms_step * 1e3 / T
    step_bytes = moe_bytes(shape, d_mean)
    sb = launch_bytes(shape, d_mean, n_stages, decode)
    dom = max(stage_us, key=stage_us.get)
    achieved = sb[dom] / (stage_us[dom] * 1e-6) / 1e9
    traffic = load_traffic(dom, shape.name)
    ceil_same = stream_ceiling(torch, w4, int(sb[dom]))
    ceil_big = stream_ceiling(torch, w4, 4 << 30)
    # the dominant kernel's bound: HBM bytes or MFMA flops, whichever takes longer
    # at the published peaks
    fl = stage_flops(shape).get(dom)
    mfma_peak = MFMA_PEAK_TFLOPS["fp8" if shape.fmt == "mxfp4" else "bf16"]
    roof = {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "frac_of_same_size_read": achieved / ceil_same["gbps"]}
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
            "tokens_per_step": T, "zipf_s": shape.zipf_s, "seed": shape.seed, "weights": {"e2m1": "E2M1 codes + FP16 scale per 16",
                        "nvfp4": "E2M1 codes + UE4M3 scale per 16 + fp32 scale per matrix",
                        "int4": "int4 codes + FP16 scale per 128",
                        "mxfp4": "E2M1 codes + E8M0 scale per 32"}[shape.fmt]
                       + (", shared expert bf16" if shape.shared_fmt == "bf16" else ""),
            "activations": ("bf16; MXFP8 (E4M3 + E8M0 per 32) inside the experts" if shape.fmt == "mxfp4"
                            else "bf16"), "accumulate": "fp32", "routed_expert_replicas": args.replicas,
            "router_shared_copies": NL, "token_pool": P, "weight_layout": args.layout,
            "mean_distinct_experts": d_mean, "timing": "HIP graph replay of the K steps",
        },
        "hbm_gbps": step_bytes / (ms_step * 1e-3) / 1e9,
        "pct_hbm_peak": 100.0 * step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "algorithmic_bytes_per_step": step_bytes,
        "stage_us": stage_us,
        "stage_us_events": stage_us_events,
        "eager_ms_per_step": eager_ms,
        "wall_s_timed": t_wall,
        "ceiling": {"same_size_read": ceil_same, "read_4gib": ceil_big,
                    "step_frac_of_4gib_read": step_bytes / (ms_step * 1e-3) / 1e9 / ceil_big["gbps"]},
        "roofline": {
            **roof,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": sb[dom], "avg_launch_us": stage_us[dom],
            "note": timing_note,
        },
    }
    return res, shape


def timed_replay_ms(torch, g):
    """One replay of graph g between two events on the current stream.  A short
    spin kernel runs first, so the host has submitted the whole graph before the
    start event is reached: the interval holds the graph's kernels only."""
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    torch.cuda._sleep(2_000_000)
    start.record()
    g.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end)


def run_gemv(args, torch, w4, wl, synth, hip):
    shape = workload_shapes(synth)[args.workload]
    if args.seed is not None:
        import dataclasses
        shape = dataclasses.replace(shape, seed=args.seed)
    print(f"[bench] building {shape.name} ({args.replicas} replicas)", file=sys.stderr, flush=True)
    if args.layout == "decode":
        raise SystemExit("the dense GEMV reads row layouts (canonical or gfx950)")
    base = wl.build_dense(shape, "cuda", layout=LAYOUTS[args.layout][0])
    reps = [base] + [_clone_q(w4, base) for _ in range(args.replicas - 1)]
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
    t_wall = time.perf_counter()
    ms_step = timed_replay_ms(torch, g) / args.steps
    t_wall = time.perf_counter() - t_wall
    g_bytes = weight_bytes(shape.fmt, shape.n, shape.k) + shape.k * 2 + shape.n * 2
    gbs = g_bytes / (ms_step * 1e-3) / 1e9
    del g, reps
    torch.cuda.empty_cache()
    ceil_same = stream_ceiling(torch, w4, g_bytes)
    ceil_big = stream_ceiling(torch, w4, 4 << 30)
    res = {
        "metric": METRIC, "value": ms_step * 1e3, "unit": "us/call", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": shape.name, "n": shape.n, "k": shape.k, "format": shape.fmt, "seed": shape.seed,
                   "replicas": R, "weight_layout": args.layout, "timing": "HIP graph replay of the K steps"},
        "hbm_gbps": gbs, "pct_hbm_peak": 100 * gbs / HBM_PEAK_GBS, "algorithmic_bytes_per_step": g_bytes,
        "wall_s_timed": t_wall,
        "ceiling": {"same_size_read": ceil_same, "read_4gib": ceil_big},
        "roofline": {"bound": "hbm", "kernel": "k_gemv", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "frac_of_same_size_read": gbs / ceil_same["gbps"],
                     "traffic": load_traffic("k_gemv", shape.name),
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
    ap.add_argument("--layout", default=None, choices=sorted(LAYOUTS),
                    help="weight layout in HBM: row records (gfx950), row records with K-tiled down "
                         "projections (decode), or the canonical arrays; default per workload")
    ap.add_argument("--pool", type=int, default=64, help="token pool (MoE workloads)")
    ap.add_argument("--cpu-tokens", type=int, default=1)
    ap.add_argument("--tokens", type=int, default=0, help="MoE workloads: tokens per step instead of the workload's")
    ap.add_argument("--seed", type=int, default=None, help="seed of the synthetic weights and inputs (default: the workload's)")
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
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    if args.layout is None:
        args.layout = default_layout(args.workload)
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
    hip = HipRuntime()
    if args.calibrate_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.workload.startswith("gemv"):
        res, shape = run_gemv(args, torch, w4, wl, synth, hip)
        cpu = None if args.no_cpu_baseline else cpu_baseline_gemv(shape, args.cpu_reps)
    else:
        res, shape = run_moe(args, torch, w4, wl, synth, hip)
        cpu = None if args.no_cpu_baseline else cpu_baseline_moe(
            shape, args.cpu_tokens if shape.tokens == 1 else 4, args.cpu_reps if shape.tokens == 1 else 2)
    res["cpu_baseline"] = cpu
    res["machine"] = machine_info(hip)
    res["device"] = res["machine"]["device"]
    res["source_digest"] = source_digest()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
