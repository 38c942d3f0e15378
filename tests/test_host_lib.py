"""Host-side checks of the C-ABI library (no GPU needed).

The library must load without a GPU, export every function include/w4moe.h
declares, and its host quantiser/packer must agree bit for bit with the oracle.
Every invalid argument must return its documented status before any launch.
"""

import ctypes as C
import os
import re

import numpy as np
import pytest

import oracle
from oracle import formats as F
import bit_block_scaled_router_amd as w4
from bit_block_scaled_router_amd import synth
from conftest import ROOT, read_golden_blocks

FMTS = [(w4.W4_FMT_E2M1_F16S16, F.FMT_E2M1), (w4.W4_FMT_INT4_F16S128, F.FMT_INT4)]


def _header_functions():
    text = open(os.path.join(ROOT, "include", "w4moe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    names = _header_functions()
    assert len(names) >= 12
    assert sorted(names) == sorted(w4.EXPORTS)
    L = C.CDLL(os.path.join(ROOT, "bit_block_scaled_router_amd", "libw4moe.so"))
    for n in names:
        assert hasattr(L, n), n


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    """Without the built library the binding raises instead of falling back to
    anything else (there is no CPU path in the package)."""
    from bit_block_scaled_router_amd import _lib
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "libw4moe.so"))
    with pytest.raises(ImportError, match="is missing"):
        _lib.lib()


def test_status_strings_and_version():
    assert w4.w4_status_string(0) == "W4_OK"
    assert w4.w4_status_string(w4.W4_ERR_LAYOUT) == "W4_ERR_LAYOUT"
    assert "gfx950" in w4.w4_version()


def test_sizes_match_stage_p1_and_oracle():
    assert w4.w4_codes_bytes(w4.W4_FMT_E2M1_F16S16, 1, 8192, 2048) == 8_388_608
    assert w4.w4_scales_bytes(w4.W4_FMT_E2M1_F16S16, 1, 8192, 2048) == 2_097_152
    assert w4.w4_scales_bytes(w4.W4_FMT_INT4_F16S128, 1, 8192, 2048) == 262_144
    for fmt, ofmt in FMTS:
        for g, n, k in [(1, 8, 256), (256, 1024, 2048), (3, 5, 512)]:
            assert w4.w4_codes_bytes(fmt, g, n, k) == oracle.codes_bytes(ofmt, g, n, k)
            assert w4.w4_scales_bytes(fmt, g, n, k) == oracle.scales_bytes(ofmt, g, n, k)
    assert w4.w4_codes_bytes(7, 1, 8, 256) == 0  # unknown format
    assert w4.w4_codes_bytes(w4.W4_FMT_E2M1_F16S16, 1, 8, 48) == 0  # k % 32
    assert w4.w4_codes_bytes(w4.W4_FMT_E2M1_F16S16, 1, 8, 256, layout=3) == 0


@pytest.mark.parametrize("fmt,ofmt", FMTS)
def test_quantizer_bit_exact_vs_oracle(fmt, ofmt):
    rng = np.random.default_rng(21)
    g = F.group_size(ofmt)
    w = np.concatenate([
        (rng.standard_normal((64, 8 * g)) * 0.02).astype(np.float32),
        (rng.standard_normal((4, 8 * g)) * 1e-6).astype(np.float32),      # subnormal fp16 scales
        (rng.standard_normal((4, 8 * g)) * 1e3).astype(np.float32),
        np.zeros((1, 8 * g), dtype=np.float32),
        # ratios on every midpoint, and one ulp around
        np.repeat(np.array([[0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] * g], dtype=np.float32), 1, 0)[:, :8 * g],
    ])
    near = w[-1].copy()
    w = np.concatenate([w, np.nextafter(near, np.float32(np.inf))[None], np.nextafter(near, np.float32(0))[None],
                        -near[None]])
    c_lib, s_lib = w4.w4_quantize(fmt, w)
    c_or, s_or = oracle.quantize(ofmt, w)
    assert np.array_equal(s_lib, s_or)
    assert np.array_equal(c_lib, c_or)


def test_quantizer_golden_blocks():
    for name, scale_bits, wv, codes in read_golden_blocks("e2m1_blocks.txt"):
        c, s = w4.w4_quantize(w4.W4_FMT_E2M1_F16S16, np.array([wv + [0.0] * 16], dtype=np.float32))
        assert int(s[0, 0]) == scale_bits, name
        assert w4.w4_unpack_nibbles(c)[0, :16].tolist() == codes, name


def test_quantizer_expert_weights_match_oracle():
    shape = synth.QWEN_MOE_T1
    for e in (0, 255):
        w = synth.expert_w2(shape, e)
        assert all(np.array_equal(a, b) for a, b in zip(w4.w4_quantize(w4.W4_FMT_E2M1_F16S16, w),
                                                          oracle.quantize(F.FMT_E2M1, w)))


def test_quantizer_errors():
    bad = np.zeros((2, 32), dtype=np.float32)
    bad[1, 3] = np.nan
    with pytest.raises(w4.W4Error) as e:
        w4.w4_quantize(w4.W4_FMT_E2M1_F16S16, bad)
    assert e.value.status == w4.W4_ERR_NONFINITE
    with pytest.raises(w4.W4Error) as e:
        w4.w4_quantize(w4.W4_FMT_E2M1_F16S16, np.full((1, 32), 1e6, dtype=np.float32))
    assert e.value.status == w4.W4_ERR_RANGE
    with pytest.raises(w4.W4Error) as e:
        w4.w4_quantize(w4.W4_FMT_INT4_F16S128, np.zeros((1, 64), dtype=np.float32))
    assert e.value.status == w4.W4_ERR_INVALID_ARG
    with pytest.raises(w4.W4Error) as e:
        w4.w4_quantize(9, np.zeros((1, 64), dtype=np.float32))
    assert e.value.status == w4.W4_ERR_LAYOUT


def test_quantizer_nvfp4_matches_oracle():
    rng = np.random.default_rng(22)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] * 2, dtype=np.float32)
    cases = [
        (rng.standard_normal((64, 256)) * 0.02).astype(np.float32),
        # blocks far below the matrix maximum: subnormal and zero UE4M3 scales
        np.concatenate([(rng.standard_normal((4, 64)) * s).astype(np.float32) for s in (1.0, 1e-3, 1e-5, 1e-9)]),
        np.zeros((3, 32), dtype=np.float32),
        # g = 1 (absmax 2688) and a block whose scale is exactly 1.0: ratios on every
        # E2M1 midpoint, and one ulp around them
        np.stack([np.concatenate([np.full(16, 2688, np.float32), mids]),
                  np.concatenate([np.full(16, 2688, np.float32), np.nextafter(mids, np.float32(np.inf))]),
                  np.concatenate([np.full(16, 2688, np.float32), -np.nextafter(mids, np.float32(0))])]),
        synth.expert_w13(synth.QWEN_MOE_T1, 3),
    ]
    for w in cases:
        c_lib, s_lib, g_lib = w4.w4_quantize(w4.W4_FMT_NVFP4_E4M3S16, w)
        c_or, s_or, g_or = oracle.quantize(F.FMT_NVFP4, w)
        assert g_lib == g_or
        assert np.array_equal(s_lib, s_or)
        assert np.array_equal(c_lib, c_or)


def test_quantizer_nvfp4_golden_and_sizes():
    import test_oracle_nvfp4 as T
    for m in T._golden_matrices():
        c, s, g = w4.w4_quantize(w4.W4_FMT_NVFP4_E4M3S16, m["w"][None])
        assert float(g) == m["g"] and np.array_equal(s[0], m["scales"]), m["name"]
        assert np.array_equal(w4.w4_unpack_nibbles(c)[0], m["codes"]), m["name"]
    fmt = w4.W4_FMT_NVFP4_E4M3S16
    assert w4.w4_codes_bytes(fmt, 1, 8192, 2048) + w4.w4_scales_bytes(fmt, 1, 8192, 2048) == 9 * 2 ** 20
    assert w4.w4_scales_bytes(fmt, 2, 3, 64) == oracle.scales_bytes(F.FMT_NVFP4, 2, 3, 64) == 24
    # the global scale output is required for NVFP4
    w = np.ones((1, 32), np.float32)
    c = np.empty((1, 16), np.uint8)
    sb = np.empty((1, 2), np.uint8)
    st = w4.lib().w4_quantize(fmt, w.ctypes.data, 1, 32, c.ctypes.data, sb.ctypes.data, None)
    assert st == w4.W4_ERR_INVALID_ARG


def test_quantizer_mxfp4_matches_oracle():
    import test_oracle_mx as T
    rng = np.random.default_rng(24)
    cases = [
        (rng.standard_normal((64, 256)) * 0.02 * np.exp2(rng.integers(-8, 8, (64, 1)))).astype(np.float32),
        np.concatenate([(rng.standard_normal((4, 64)) * s).astype(np.float32) for s in (1.0, 1e-3, 1e-30, 1e-40)]),
        np.zeros((3, 64), dtype=np.float32),
        synth.expert_w13(synth.QWEN_MOE_T1, 5),
    ]
    fmt = w4.W4_FMT_MXFP4_E8M0S32
    for w in cases:
        c_lib, s_lib = w4.w4_quantize(fmt, w)
        c_or, s_or = oracle.quantize(F.FMT_MXFP4, w)
        assert s_lib.dtype == np.uint8 and np.array_equal(s_lib, s_or)
        assert np.array_equal(c_lib, c_or)
    for b in T._blocks():
        c, s = w4.w4_quantize(fmt, b["w"][None])
        assert int(s[0, 0]) == b["scale"] and np.array_equal(w4.w4_unpack_nibbles(c)[0], b["codes"]), b["name"]
    assert w4.w4_scales_bytes(fmt, 2, 3, 64) == oracle.scales_bytes(F.FMT_MXFP4, 2, 3, 64) == 12
    with pytest.raises(w4.W4Error) as e:
        w4.w4_quantize(fmt, np.zeros((1, 48), dtype=np.float32))  # k must be a multiple of 32
    assert e.value.status == w4.W4_ERR_INVALID_ARG


def test_mxfp4_layer_plan_and_validation():
    mx = w4.W4_FMT_MXFP4_E8M0S32
    H, I, E = 256, 128, 8

    def mxl(**over):
        d = dict(w13=_mat(fmt=mx, groups=E, n=2 * I, k=H), w2=_mat(fmt=mx, groups=E, n=H, k=I),
                 shared_w13=_mat(fmt=mx, groups=1, n=2 * I, k=H), shared_w2=_mat(fmt=mx, groups=1, n=H, k=I))
        d.update(over)
        return _layer(**d)

    L = mxl()
    # 1-3 tokens: the single-token kernels (router, W13 with x quantised per
    # lane, down with h quantised per lane); from 4 tokens the grouped MX path:
    # router, x -> MXFP8, grouping, W13, W2, combine
    assert [w4.lib().moe_w4a16_stage_count(C.byref(L), T) for T in (1, 2, 3, 4, 64)] == [3, 3, 3, 6, 6]
    assert w4.lib().moe_w4a16_workspace_bytes(C.byref(L), 1) > 0
    # more than 1024 pairs group over three launches: 2 more stages
    assert w4.lib().moe_w4a16_stage_count(C.byref(L), 512) == 6
    assert w4.lib().moe_w4a16_stage_count(C.byref(L), 513) == 8
    # at most 65536 pairs per call, at most 16384 tokens
    L8 = mxl(top_k=8)
    assert w4.lib().moe_w4a16_workspace_bytes(C.byref(L8), 8192) > 0
    assert w4.lib().moe_w4a16_workspace_bytes(C.byref(L8), 8193) == 0
    assert _fwd(L8, T=8193, ws_bytes=1 << 40) == w4.W4_ERR_UNSUPPORTED
    assert _fwd(L, T=16385, ws_bytes=1 << 40) == w4.W4_ERR_INVALID_ARG
    # inter off the 128 grid, a bf16 shared expert, mixed formats
    bad_i = _layer(inter=96, shared_inter=96, w13=_mat(fmt=mx, groups=E, n=192, k=H), w2=_mat(fmt=mx, groups=E, n=H, k=96),
                   has_shared=0)
    assert _fwd(bad_i, ws_bytes=1 << 30) == w4.W4_ERR_UNSUPPORTED
    bf = w4.W4_FMT_BF16
    assert _fwd(mxl(shared_w13=_mat(fmt=bf, groups=1, n=2 * I, k=H, scales=None),
                    shared_w2=_mat(fmt=bf, groups=1, n=H, k=I, scales=None)), ws_bytes=1 << 30) == w4.W4_ERR_UNSUPPORTED
    assert _fwd(mxl(w2=_mat(groups=E, n=H, k=I)), ws_bytes=1 << 30) == w4.W4_ERR_LAYOUT
    # E2M1: batched path from T = 4, three grouping launches past 1024 pairs;
    # past 65536 pairs the single-token path
    E2 = _layer(top_k=8)
    assert [w4.lib().moe_w4a16_stage_count(C.byref(E2), T) for T in (3, 4, 128, 129, 8192, 8193)] == [3, 5, 5, 7, 7, 3]
    # the timed entry point wants 12 events on the grouped MX path
    ev = (C.c_void_p * 10)(*([1] * 10))
    st = w4.lib().moe_w4a16_forward_timed(C.byref(L), 1 << 20, 4, 1 << 21, None, None, 1 << 24,
                                          w4.lib().moe_w4a16_workspace_bytes(C.byref(L), 4), 0, ev, 10)
    assert st == w4.W4_ERR_INVALID_ARG


def test_bf16_shared_expert_plan():
    """A bf16 shared expert joins the grouped path (its rows are MFMA operands
    there), past 1024 (token, slot) pairs with the three-launch grouping."""
    bf = w4.W4_FMT_BF16
    for fmt in (w4.W4_FMT_E2M1_F16S16, w4.W4_FMT_NVFP4_E4M3S16):
        g = 1 << 22 if fmt == w4.W4_FMT_NVFP4_E4M3S16 else None
        L = _layer(w13=_mat(fmt=fmt, groups=8, n=256, k=256, gsc=g), w2=_mat(fmt=fmt, groups=8, n=256, k=128, gsc=g),
                   shared_w13=_mat(fmt=bf, groups=1, n=256, k=256, scales=None),
                   shared_w2=_mat(fmt=bf, groups=1, n=256, k=128, scales=None))
        got = [w4.lib().moe_w4a16_stage_count(C.byref(L), T) for T in (1, 3, 4, 512, 513, 16384)]
        assert got == [3, 3, 5, 5, 7, 7], (fmt, got)


def test_int4_layer_plan():
    """int4 experts take the grouped path from T = 4 up to 4096 (token, slot)
    pairs, the single-token path beyond."""
    i4 = w4.W4_FMT_INT4_F16S128
    L = _layer(w13=_mat(fmt=i4, groups=8, n=256, k=256), w2=_mat(fmt=i4, groups=8, n=256, k=128),
               shared_w13=_mat(fmt=i4, groups=1, n=256, k=256), shared_w2=_mat(fmt=i4, groups=1, n=256, k=128))
    assert [w4.lib().moe_w4a16_stage_count(C.byref(L), T) for T in (1, 3, 4, 2048, 2049)] == [3, 3, 5, 5, 3]


def test_bf16_format_quantiser_sizes_and_rules():
    rng = np.random.default_rng(23)
    w = (rng.standard_normal((5, 64)) * 0.02).astype(np.float32)
    w[0, :4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -0.0, 3.0e38]  # ties and extremes
    (bits,) = w4.w4_quantize(w4.W4_FMT_BF16, w)
    (ref,) = oracle.quantize(F.FMT_BF16, w)
    assert np.array_equal(bits, ref)
    fmt = w4.W4_FMT_BF16
    assert w4.w4_codes_bytes(fmt, 2, 3, 64) == 2 * 3 * 64 * 2 and w4.w4_scales_bytes(fmt, 2, 3, 64) == 0
    # the GEMV rejects bf16 matrices; a bf16 routed expert stack is unsupported
    assert w4.lib().w4a16_gemv(C.byref(_mat(fmt=fmt, scales=None)), 1 << 20, 1, 1 << 21, 0) == w4.W4_ERR_UNSUPPORTED
    H, I, E = 256, 128, 8
    L = _layer(shared_w13=_mat(fmt=fmt, groups=1, n=2 * I, k=H, scales=None),
               shared_w2=_mat(fmt=fmt, groups=1, n=H, k=I, scales=None))
    assert w4.lib().moe_w4a16_workspace_bytes(C.byref(L), 1) > 0
    assert w4.lib().moe_w4a16_stage_count(C.byref(L), 8) == 5  # batches run grouped (see the plan test)
    assert _fwd(_layer(w13=_mat(fmt=fmt, groups=E, n=2 * I, k=H, scales=None),
                       w2=_mat(fmt=fmt, groups=E, n=H, k=I, scales=None))) == w4.W4_ERR_UNSUPPORTED
    assert _fwd(_layer(shared_w13=_mat(fmt=fmt, groups=1, n=2 * I, k=H, scales=None))) == w4.W4_ERR_LAYOUT


def test_pack_unpack_all_bytes_and_oracle():
    b = np.arange(256, dtype=np.uint8).reshape(4, 64)
    nib = w4.w4_unpack_nibbles(b)
    assert np.array_equal(nib, oracle.unpack_nibbles(b))
    assert np.array_equal(w4.w4_pack_nibbles(nib), b)
    with pytest.raises(w4.W4Error):
        w4.w4_pack_nibbles(np.full((1, 4), 16, dtype=np.uint8))


# ---------------------------------------------------------------- device entry validation


def _mat(fmt=w4.W4_FMT_E2M1_F16S16, layout=0, groups=1, n=64, k=256, codes=4096, scales=8192, gsc=None):
    return w4.W4Matrix(fmt, layout, groups, n, k, codes, scales, gsc)


def _gemv(W, x=1 << 20, m=1, y=1 << 21):
    return w4.lib().w4a16_gemv(C.byref(W), x, m, y, 0)


def test_gemv_validation_returns_before_launch():
    assert _gemv(_mat(fmt=9)) == w4.W4_ERR_LAYOUT
    assert _gemv(_mat(fmt=w4.W4_FMT_MXFP4_E8M0S32)) == w4.W4_ERR_UNSUPPORTED  # MX serves the MoE layer
    assert _gemv(_mat(layout=7)) == w4.W4_ERR_LAYOUT
    assert _gemv(_mat(k=48)) == w4.W4_ERR_INVALID_ARG
    assert _gemv(_mat(fmt=w4.W4_FMT_INT4_F16S128, k=64)) == w4.W4_ERR_INVALID_ARG
    assert _gemv(_mat(codes=4100)) == w4.W4_ERR_ALIGNMENT
    assert _gemv(_mat(scales=8194)) == w4.W4_ERR_ALIGNMENT
    assert _gemv(_mat(codes=0)) == w4.W4_ERR_INVALID_ARG
    assert _gemv(_mat(groups=2)) == w4.W4_ERR_INVALID_ARG
    assert _gemv(_mat(), m=0) == w4.W4_ERR_UNSUPPORTED
    assert _gemv(_mat(), m=65) == w4.W4_ERR_UNSUPPORTED
    assert _gemv(_mat(), x=(1 << 20) + 2) == w4.W4_ERR_ALIGNMENT
    assert _gemv(_mat(), x=0) == w4.W4_ERR_INVALID_ARG
    assert "x not 16-byte aligned" in w4.w4_last_error() or True
    assert w4.lib().w4a16_gemv(None, 1 << 20, 1, 1 << 21, 0) == w4.W4_ERR_INVALID_ARG
    nv = w4.W4_FMT_NVFP4_E4M3S16
    assert _gemv(_mat(fmt=nv)) == w4.W4_ERR_INVALID_ARG          # NVFP4 without global scales
    assert _gemv(_mat(fmt=nv, gsc=(1 << 23) + 2)) == w4.W4_ERR_ALIGNMENT
    assert _gemv(_mat(fmt=nv, k=48, gsc=1 << 23)) == w4.W4_ERR_INVALID_ARG
    assert w4.lib().w4_dequant_device(C.byref(_mat()), 0, 0) == w4.W4_ERR_INVALID_ARG


def _layer(**over):
    H, I, E, K = 256, 128, 8, 2
    d = dict(hidden=H, inter=I, num_experts=E, top_k=K, shared_inter=I, router_w=1 << 16, router_bias=None,
             w13=_mat(groups=E, n=2 * I, k=H), w2=_mat(groups=E, n=H, k=I), has_shared=1,
             shared_w13=_mat(groups=1, n=2 * I, k=H), shared_w2=_mat(groups=1, n=H, k=I), shared_gate_w=1 << 17)
    d.update(over)
    return w4.MoELayerDesc(*[d[f] for f, _ in w4.MoELayerDesc._fields_])


def _fwd(L, T=1, ws_bytes=None, ws=1 << 24, x=1 << 20, y=1 << 21):
    if ws_bytes is None:
        ws_bytes = w4.lib().moe_w4a16_workspace_bytes(C.byref(L), T) if T >= 1 else 0
    return w4.lib().moe_w4a16_forward(C.byref(L), x, T, y, None, None, ws, ws_bytes, 0)


def test_moe_workspace_size_and_validation():
    L = _layer()
    ws = w4.lib().moe_w4a16_workspace_bytes(C.byref(L), 1)
    assert ws > 0 and ws % 256 == 0
    assert w4.lib().moe_w4a16_workspace_bytes(C.byref(L), 32) > ws
    assert w4.lib().moe_w4a16_workspace_bytes(C.byref(_layer(top_k=9)), 1) == 0
    assert _fwd(_layer(top_k=0)) == w4.W4_ERR_INVALID_ARG
    assert _fwd(_layer(top_k=9)) == w4.W4_ERR_INVALID_ARG
    assert _fwd(_layer(hidden=200)) == w4.W4_ERR_UNSUPPORTED
    assert _fwd(_layer(num_experts=2000)) == w4.W4_ERR_UNSUPPORTED
    assert _fwd(_layer(w13=_mat(groups=8, n=2 * 128, k=512))) == w4.W4_ERR_INVALID_ARG
    assert _fwd(_layer(w2=_mat(fmt=w4.W4_FMT_INT4_F16S128, groups=8, n=256, k=128))) == w4.W4_ERR_LAYOUT
    assert _fwd(_layer(shared_inter=256)) == w4.W4_ERR_UNSUPPORTED
    assert _fwd(_layer(has_shared=2)) == w4.W4_ERR_INVALID_ARG
    assert _fwd(_layer(shared_gate_w=None)) == w4.W4_ERR_INVALID_ARG
    assert _fwd(_layer(router_w=(1 << 16) + 8)) == w4.W4_ERR_ALIGNMENT
    assert _fwd(L, T=0) == w4.W4_ERR_INVALID_ARG
    assert _fwd(L, ws_bytes=ws - 1) == w4.W4_ERR_WORKSPACE
    assert _fwd(L, ws=0) == w4.W4_ERR_WORKSPACE
    assert _fwd(L, ws=(1 << 24) + 64) == w4.W4_ERR_ALIGNMENT
    assert _fwd(L, x=(1 << 20) + 8) == w4.W4_ERR_ALIGNMENT
    assert w4.lib().moe_w4a16_experts(C.byref(L), 1 << 20, 1, None, None, 1 << 21, 1 << 24, ws, 0) \
        == w4.W4_ERR_INVALID_ARG
    assert w4.lib().moe_w4a16_experts(C.byref(L), 1 << 20, 1, 1 << 22, None, 1 << 21, 1 << 24, ws, 0) \
        == w4.W4_ERR_INVALID_ARG


def test_noalloc_refuses_batches_beyond_its_scratch_before_any_hip_call():
    """A batch whose workspace exceeds the no-allocation entry point's scratch is
    refused during validation (fake device pointers: nothing is touched)."""
    L = _layer()
    T = 4096
    need = w4.lib().moe_w4a16_workspace_bytes(C.byref(L), T)
    assert need > 8 << 20
    st = w4.lib().moe_w4a16_forward_noalloc(C.byref(L), 1 << 20, T, 1 << 21, None, None, 0)
    assert st == w4.W4_ERR_WORKSPACE
    assert "scratch" in w4.w4_last_error()
    assert w4.lib().moe_w4a16_forward_noalloc(C.byref(_layer(top_k=9)), 1 << 20, 1, 1 << 21, None, None, 0) \
        == w4.W4_ERR_INVALID_ARG


def test_k_tiled_down_projection_plan_and_validation():
    """A layer whose down projections are K-tiled runs the three decode launches
    for every T (up to 1024); mixing K-tiled and row layouts for the two down
    projections, other formats, or a K-tiled gate/up matrix is refused."""
    KT, V1 = w4.W4_LAYOUT_GFX950_KT16, w4.W4_LAYOUT_GFX950_V1
    H, I, E = 256, 128, 8
    L = _layer(w13=_mat(groups=E, n=2 * I, k=H, layout=V1), w2=_mat(groups=E, n=H, k=I, layout=KT, scales=None),
               shared_w13=_mat(groups=1, n=2 * I, k=H, layout=V1),
               shared_w2=_mat(groups=1, n=H, k=I, layout=KT, scales=None))
    for T in (1, 4, 32, 1024):
        assert w4.lib().moe_w4a16_stage_count(C.byref(L), T) == 3
    assert w4.lib().moe_w4a16_stage_count(C.byref(L), 1025) == 0
    ws1 = w4.lib().moe_w4a16_workspace_bytes(C.byref(L), 1)
    # logits, ids, weights and the fp32 contribution of every (slot, 16-value tile) to every output row
    assert ws1 >= 3 * (I // 16) * H * 4
    mixed = _layer(w2=_mat(groups=E, n=H, k=I, layout=KT, scales=None))
    assert _fwd(mixed) == w4.W4_ERR_UNSUPPORTED
    kt13 = _layer(w13=_mat(groups=E, n=2 * I, k=H, layout=KT, scales=None))
    assert _fwd(kt13) == w4.W4_ERR_UNSUPPORTED
    int4 = _layer(w2=_mat(fmt=w4.W4_FMT_INT4_F16S128, groups=E, n=H, k=I, layout=KT))
    assert _fwd(int4) == w4.W4_ERR_UNSUPPORTED
