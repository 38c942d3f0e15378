"""Host-side checks of bench.py's bookkeeping (no GPU): for every MoE workload
the stage names match the library's stage count and every named kernel has an
algorithmic byte count; the flop counts cover the projections; a multi-GPU
request exits with a message; the HBM traffic bookkeeping scales counters by
the copy calibration and goes stale with the kernel sources."""

import subprocess
import sys
import ctypes as C

import pytest

import bench
import bit_block_scaled_router_amd as w4
from bit_block_scaled_router_amd import synth
from conftest import ROOT


def _desc(shape):
    """A layer descriptor with fake device pointers (planning only, nothing launched)."""
    fmt = w4.FORMATS[shape.fmt]
    H, I, E = shape.hidden, shape.inter, shape.num_experts
    sfmt = w4.FORMATS[shape.shared_fmt] if shape.shared_fmt else fmt
    g = w4.GROUP.get(fmt, 1)

    def mat(f, groups, n, k):
        return w4.W4Matrix(f, 0, groups, n, k, 1 << 20, None if f == w4.W4_FMT_BF16 else 1 << 21,
                           (1 << 22) if f == w4.W4_FMT_NVFP4_E4M3S16 else None)

    return w4.MoELayerDesc(H, I, E, shape.top_k, shape.shared_inter or I, 1 << 16, None,
                           mat(fmt, E, 2 * I, H), mat(fmt, E, H, I), 1 if shape.has_shared else 0,
                           mat(sfmt, 1, 2 * I, H), mat(sfmt, 1, H, I), 1 << 17)


MOE = [w for w in bench.WORKLOADS if not w.startswith("gemv")]


@pytest.mark.parametrize("name", MOE)
def test_stage_names_and_bytes(name):
    shape = bench.workload_shapes(synth)[name]
    T = shape.tokens
    n = w4.lib().moe_w4a16_stage_count(C.byref(_desc(shape)), T)
    assert n in (3, 5, 6, 7, 8), n
    names = bench.stage_names(n, T, shape.top_k, shape.fmt == "mxfp4", int4=shape.fmt == "int4")
    assert len(names) == n
    sb = bench.launch_bytes(shape, 8.0, n)
    assert set(sb) == set(names), (sorted(sb), names)
    assert all(v > 0 for v in sb.values())
    fl = bench.stage_flops(shape)
    proj = [k for k in names if k in fl]
    assert len(proj) == (0 if n == 3 else 2)


def test_multi_gpu_request_exits_with_message():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_traffic_ingest_scaling_and_invalidation(tmp_path, monkeypatch, capsys):
    """ingest_counters scales each counter by what it reads for the 256 MiB copy
    (mean of the first three copy dispatches), stores HBM bytes per dispatch with
    the kernel source digest, and load_traffic drops the record once a kernel
    source changes."""
    csrc = tmp_path / "bit_block_scaled_router_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "k.hip").write_text("// v1\n")
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))

    def csv(path, counter, copy_kib, kern_vals):
        rows = ["Kernel_Name,Counter_Name,Counter_Value"]
        rows += [f"__amd_rocclr_copyBuffer,{counter},{v}" for v in copy_kib]
        rows += [f"void w4k::k_moe_w13<1>(w4k::Args),{counter},{v}" for v in kern_vals]
        path.write_text("\n".join(rows) + "\n")
        return str(path)

    # FETCH_SIZE reads half the copied bytes (factor 2), WRITE_SIZE all of them;
    # a fourth copy dispatch is ignored
    f = csv(tmp_path / "f.csv", "FETCH_SIZE", [131072, 131072, 131072, 1], [100.0, 300.0])
    w = csv(tmp_path / "w.csv", "WRITE_SIZE", [262144, 262144, 262144], [10.0, 30.0])
    bench.ingest_counters([f, w], "wl")
    capsys.readouterr()
    want = (200.0 * 2 + 20.0 * 1) * 1024
    assert bench.load_traffic("k_moe_w13", "wl") == round(want)
    assert bench.load_traffic("k_moe_w13", "other") is None
    assert bench.load_traffic("k_moe_w2", "wl") is None
    (csrc / "k.hip").write_text("// v2\n")
    assert bench.load_traffic("k_moe_w13", "wl") is None


@pytest.mark.parametrize("name", ["qwen-t1", "qwen-t1-nvfp4", "tiny"])
def test_decode_stage_names_and_bytes(name):
    shape = bench.workload_shapes(synth)[name]
    names = bench.stage_names(3, shape.tokens, shape.top_k, False, decode=True)
    sb = bench.launch_bytes(shape, float(shape.top_k), 3, decode=True)
    assert set(sb) == set(names) and all(v > 0 for v in sb.values())
    # the expert launch moves every selected expert's W13 and W2 once (and the shared expert's)
    assert sb["k_moe_dec"] >= shape.top_k * (bench.weight_bytes(shape.fmt, 2 * shape.inter, shape.hidden)
                                            + bench.weight_bytes(shape.fmt, shape.hidden, shape.inter))
    assert bench.default_layout(name) in ("decode", "gfx950", "canonical")


@pytest.mark.parametrize("T", [4, 32, 128, 129, 159, 160, 512, 2048])
def test_stage_names_follow_the_library_thresholds(T):
    """bench.py names each stage from its copies of the library's thresholds
    (large-batch kernels past 1024 pairs, MFMA router from 160 tokens); the
    library's own stage count must agree with them at every batch size."""
    import dataclasses
    shape = dataclasses.replace(synth.QWEN_MOE_T32, tokens=T)
    n = w4.lib().moe_w4a16_stage_count(C.byref(_desc(shape)), T)
    names = bench.stage_names(n, T, shape.top_k, False)
    assert len(names) == n == (7 if T * shape.top_k > bench.LARGE_BATCH_PAIRS else 5)
    assert ("k_moe_pf13" in names) == (T * shape.top_k > 1024)
    assert names[0] == ("k_router_mfma" if T >= 160 else "k_router")
    assert set(bench.launch_bytes(shape, 8.0, n)) == set(names)


@pytest.mark.parametrize("T", [32, 256, 512, 1024])
def test_stage_names_int4_batches(T):
    """int4 experts run the per-group projection kernels up to the one-block
    grouping limit and the single-token kernels beyond it, never the
    large-batch GEMM kernels: the bench's names follow the library's count."""
    import dataclasses
    shape = dataclasses.replace(synth.QWEN_MOE_T32, tokens=T, fmt="int4", name=f"int4@{T}")
    n = w4.lib().moe_w4a16_stage_count(C.byref(_desc(shape)), T)
    names = bench.stage_names(n, T, shape.top_k, False, int4=True)
    assert len(names) == n
    assert "k_moe_pf13" not in names and "k_moe_pf2" not in names
    if T * shape.top_k <= 4096:
        assert n == 5 and names[2:4] == ["k_moe_gw13", "k_moe_gw2"]
    else:
        assert n == 3 and names[1:] == ["k_moe_w13", "k_moe_down"]
    assert set(bench.launch_bytes(shape, 8.0, n)) == set(names)
