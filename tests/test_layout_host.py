"""Host checks of the device weight layout (W4_LAYOUT_GFX950_V1) and of
w4_pack / w4_unpack: the record of every row is its canonical code bytes, then
its block scales in K order, then zero padding to a multiple of 16 bytes (built
here independently with numpy); pack and unpack are exact inverses for every
format; sizes; unknown tags fail loudly."""

import numpy as np
import pytest

import bit_block_scaled_router_amd as w4

FMTS = {
    "e2m1": (w4.W4_FMT_E2M1_F16S16, 16, np.uint16),
    "int4": (w4.W4_FMT_INT4_F16S128, 128, np.uint16),
    "nvfp4": (w4.W4_FMT_NVFP4_E4M3S16, 16, np.uint8),
    "mxfp4": (w4.W4_FMT_MXFP4_E8M0S32, 32, np.uint8),
}


def _random(fmt_name, groups, n, k, seed):
    fmt, g, sdt = FMTS[fmt_name]
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, size=(groups, n, k // 2), dtype=np.uint8)
    scales = rng.integers(0, np.iinfo(sdt).max + 1, size=(groups, n, k // g), dtype=np.int64).astype(sdt)
    return fmt, codes, scales


def _records(codes, scales):
    """Independent construction of the V1 rows: codes, scale bytes, zero padding."""
    G, n, _ = codes.shape
    rows = []
    for c, s in zip(codes.reshape(G * n, -1), scales.reshape(G * n, -1)):
        b = np.concatenate([c, s.view(np.uint8)])
        pad = (-len(b)) % 16
        rows.append(np.concatenate([b, np.zeros(pad, dtype=np.uint8)]))
    return np.stack(rows).reshape(G, n, -1)


@pytest.mark.parametrize("fmt_name", list(FMTS))
@pytest.mark.parametrize("groups,n,k", [(1, 1, 128), (3, 5, 384), (2, 7, 2048), (1, 16, 512)])
def test_pack_matches_record_definition_and_round_trips(fmt_name, groups, n, k):
    fmt, codes, scales = _random(fmt_name, groups, n, k, groups * 1000 + n * 10 + k)
    rec, none = w4.w4_pack(fmt, codes, scales)
    assert none is None
    want = _records(codes, scales)
    assert rec.shape == want.shape and np.array_equal(rec, want)
    assert rec.shape[2] % 16 == 0
    assert rec.size == w4.w4_codes_bytes(fmt, groups, n, k, w4.W4_LAYOUT_GFX950_V1)
    assert w4.w4_scales_bytes(fmt, groups, n, k, w4.W4_LAYOUT_GFX950_V1) == 0
    c2, s2 = w4.w4_unpack(fmt, groups, n, k, rec)
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)
    # canonical -> canonical is a copy
    c3, s3 = w4.w4_pack(fmt, codes, scales, layout=w4.W4_LAYOUT_CANONICAL)
    assert np.array_equal(c3, codes) and np.array_equal(s3, scales)


def test_unpack_ignores_padding():
    fmt, codes, scales = _random("int4", 2, 3, 512, 5)  # 256 + 8 B -> records of 272 B
    rec, _ = w4.w4_pack(fmt, codes, scales)
    assert rec.shape[2] == 272
    rec = rec.copy()
    rec[:, :, 264:] = 0xAB
    c2, s2 = w4.w4_unpack(fmt, 2, 3, 512, rec)
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)


def test_bf16_layouts_coincide():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 65536, size=(1, 4, 64), dtype=np.int64).astype(np.uint16)
    rec, _ = w4.w4_pack(w4.W4_FMT_BF16, bits, None)
    assert np.array_equal(rec.reshape(-1), bits.reshape(-1).view(np.uint8))
    c2, s2 = w4.w4_unpack(w4.W4_FMT_BF16, 1, 4, 64, rec)
    assert s2 is None and np.array_equal(c2, bits)


def test_sizes_of_the_device_layout():
    # 8192 x 2048: E2M1 rows are 1024 + 256 = 1280 B (already a multiple of 16),
    # so the device layout holds exactly the 10.00 MiB of codes + scales
    V1 = w4.W4_LAYOUT_GFX950_V1
    assert w4.w4_codes_bytes(w4.W4_FMT_E2M1_F16S16, 1, 8192, 2048, V1) == 8192 * 1280 == 10 * 2 ** 20
    assert w4.w4_codes_bytes(w4.W4_FMT_INT4_F16S128, 1, 8192, 2048, V1) == 8192 * 1056
    assert w4.w4_codes_bytes(w4.W4_FMT_NVFP4_E4M3S16, 1, 8192, 2048, V1) == 8192 * 1152
    assert w4.w4_codes_bytes(w4.W4_FMT_MXFP4_E8M0S32, 1, 8192, 2048, V1) == 8192 * 1088
    # an expert's W2 (2048 x 512) in int4: 256 + 8 B padded to 272
    assert w4.w4_codes_bytes(w4.W4_FMT_INT4_F16S128, 1, 2048, 512, V1) == 2048 * 272


def test_unknown_layout_fails_loudly():
    fmt, codes, scales = _random("e2m1", 1, 2, 64, 1)
    with pytest.raises(w4.W4Error) as e:
        w4.w4_pack(fmt, codes, scales, layout=7)
    assert e.value.status == w4.W4_ERR_LAYOUT
    assert w4.w4_codes_bytes(fmt, 1, 2, 64, 7) == 0
    with pytest.raises(w4.W4Error) as e:
        w4.w4_unpack(fmt, 1, 2, 64, np.zeros(160, np.uint8), layout=9)
    assert e.value.status == w4.W4_ERR_LAYOUT


def _kt16_records(codes, scales):
    """Independent construction of the K-tiled records: per tile, every row's 8
    code bytes, then every row's scale of the tile, zero padding to 16."""
    G, n, kh = codes.shape
    out = []
    for g in range(G):
        tiles = []
        for t in range(kh // 8):
            b = np.concatenate([codes[g, :, 8 * t:8 * t + 8].reshape(-1), scales[g, :, t].copy().view(np.uint8)])
            tiles.append(np.concatenate([b, np.zeros((-len(b)) % 16, dtype=np.uint8)]))
        out.append(np.stack(tiles))
    return np.stack(out)


@pytest.mark.parametrize("fmt_name", ["e2m1", "nvfp4"])
@pytest.mark.parametrize("groups,n,k", [(1, 1, 32), (3, 5, 64), (2, 2048, 512), (1, 7, 256)])
def test_kt16_matches_record_definition_and_round_trips(fmt_name, groups, n, k):
    fmt, codes, scales = _random(fmt_name, groups, n, k, groups * 7 + n * 3 + k)
    KT = w4.W4_LAYOUT_GFX950_KT16
    rec, none = w4.w4_pack(fmt, codes, scales, layout=KT)
    assert none is None
    want = _kt16_records(codes, scales)
    assert rec.shape == want.shape and np.array_equal(rec, want)
    assert rec.size == w4.w4_codes_bytes(fmt, groups, n, k, KT)
    assert w4.w4_scales_bytes(fmt, groups, n, k, KT) == 0
    c2, s2 = w4.w4_unpack(fmt, groups, n, k, rec, layout=KT)
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)


def test_kt16_sizes_and_formats():
    KT = w4.W4_LAYOUT_GFX950_KT16
    # an expert's down projection 2048 x 512 (E2M1): 32 tiles of 2048 x (8 + 2) B
    assert w4.w4_codes_bytes(w4.W4_FMT_E2M1_F16S16, 1, 2048, 512, KT) == 32 * 20480
    assert w4.w4_codes_bytes(w4.W4_FMT_NVFP4_E4M3S16, 1, 2048, 512, KT) == 32 * 2048 * 9
    # formats whose scale block is not 16 wide are refused
    for fmt in (w4.W4_FMT_INT4_F16S128, w4.W4_FMT_MXFP4_E8M0S32, w4.W4_FMT_BF16):
        assert w4.w4_codes_bytes(fmt, 1, 64, 256, KT) == 0
