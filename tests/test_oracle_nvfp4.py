"""Pins of the oracle's NVFP4 variant (E2M1 codes, UE4M3 per-16 scales, fp32
global scale per matrix) against values fixed outside the oracle: the OCP E4M3
definition (typed table), torch's float8_e4m3fn conversion (an independent
implementation of the same format), hand-worked blocks, brute force and the
9.00 MiB size of the 8192x2048 matrix."""

import numpy as np
import pytest
import torch

import oracle as O
from conftest import read_golden_lines


def test_e4m3_typed_table():
    for line in read_golden_lines("e4m3_values.txt"):
        code, val = line.split()
        v = O.e4m3_value(int(code, 16))
        if val == "nan":
            assert np.isnan(v), code
        else:
            assert v == float(val) and np.signbit(v) == val.startswith("-"), (code, v, val)


def test_e4m3_all_bytes_match_torch():
    b = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.e4m3_value(b)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(got[ok]))


def _torch_e4m3(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_ue4m3_rounding_matches_torch():
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.uniform(0, 448, 30000), 2.0 ** rng.uniform(-14, 8.8, 30000), [0.0, 448.0]])
    x = x.astype(np.float32)
    x = x[x <= 448]
    assert np.array_equal(O.f32_to_ue4m3(x), _torch_e4m3(x))


def test_ue4m3_midpoints_and_neighbours():
    vals = O.e4m3_value(np.arange(0x7F))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)  # exact in fp32
    assert np.array_equal(mids.astype(np.float64), (vals[:-1] + vals[1:]) / 2)
    got = O.f32_to_ue4m3(mids)
    lo = np.arange(0x7E)
    # ties go to the even code
    assert np.array_equal(got, np.where(lo % 2 == 0, lo, lo + 1))
    assert np.array_equal(got, _torch_e4m3(mids))
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    assert np.array_equal(O.f32_to_ue4m3(up), lo + 1)
    assert np.array_equal(O.f32_to_ue4m3(dn), lo)


def test_ue4m3_saturates():
    assert np.all(O.f32_to_ue4m3(np.float32([448, 460, 1e6])) == 0x7E)
    with pytest.raises(ValueError):
        O.f32_to_ue4m3(np.float32([-1.0]))


def _golden_matrices():
    lines = read_golden_lines("nvfp4_blocks.txt")
    out, cur = [], None
    for line in lines:
        key, _, rest = line.partition(" ") if line.startswith("matrix") else line.partition(":")
        if line.startswith("matrix"):
            cur = {"name": rest.strip()}
            out.append(cur)
        elif key == "g":
            cur["g"] = float(rest)
        elif key == "w":
            cur["w"] = np.array([float(v) for v in rest.split()], dtype=np.float32)
        elif key == "scales":
            cur["scales"] = np.array([int(v, 16) for v in rest.split()], dtype=np.uint8)
        elif key == "codes":
            cur["codes"] = np.array([int(v, 16) for v in rest.split()], dtype=np.uint8)
    return out


@pytest.mark.parametrize("m", _golden_matrices(), ids=lambda m: m["name"])
def test_nvfp4_golden(m):
    codes, sb, g = O.quantize_nvfp4(m["w"][None])
    assert float(g) == m["g"]
    assert np.array_equal(sb[0], m["scales"])
    assert np.array_equal(codes[0], m["codes"])


def _rand_matrix(rng, n, k):
    w = rng.normal(0, 0.02, (n, k)).astype(np.float32)
    # rows with small blocks (subnormal UE4M3 scales) and zero blocks
    w[1] *= np.float32(1e-4)
    w[2, :16] = 0
    w[3, 16:48] *= np.float32(1e-6)
    return w


def test_nvfp4_brute_force_codes():
    rng = np.random.default_rng(5)
    w = _rand_matrix(rng, 16, 128)
    codes, sb, g = O.quantize_nvfp4(w)
    assert g == np.float32(np.abs(w).max()) / np.float32(2688)
    d = (O.e4m3_value(sb).astype(np.float32) * g).astype(np.float32)
    vals = O.e2m1_value(np.arange(16))
    for r in range(w.shape[0]):
        for kk in range(w.shape[1]):
            db = d[r, kk // 16]
            q = np.float64(w[r, kk] / db) if db != 0 else 0.0
            err = np.abs(vals - q)
            best = err.min()
            c = codes[r, kk]
            assert err[c] == best, (r, kk, c, q)  # a nearest value
            if vals[c] == 0:
                assert c == 0  # -0 never emitted
            if len({vals[x] for x in range(16) if err[x] == best}) > 1:
                assert (c & 7) % 2 == 0  # a tie goes to the even magnitude code
    # block scales: nearest UE4M3 to the target quotient
    a = np.abs(w.reshape(16, 8, 16)).max(axis=2)
    u = (a / np.float32(6)) / g
    ue = O.e4m3_value(np.arange(0x7F))
    for (r, b), ub in np.ndenumerate(u):
        assert np.abs(ue[sb[r, b]] - ub) == np.abs(ue - ub).min()


def test_nvfp4_block_max_code():
    # a block with a normal UE4M3 scale holds a code of magnitude 6 (its largest
    # element / d lies within 6 (1 +- 2**-4))
    rng = np.random.default_rng(6)
    w = rng.normal(0, 1, (64, 256)).astype(np.float32) * np.float32(2.0) ** rng.integers(-8, 8, (64, 1)).astype(np.float32)
    codes, sb, g = O.quantize_nvfp4(w)
    normal = sb >= 0x08
    mag = (codes & 7).reshape(64, 16, 16).max(axis=2)
    assert normal.sum() > 500
    assert np.all(mag[normal] == 7)


def test_nvfp4_dequant_single_rounding_and_error_bound():
    rng = np.random.default_rng(7)
    w = _rand_matrix(rng, 8, 64)
    codes, sb, g = O.quantize_nvfp4(w)
    deq = O.dequant(O.FMT_NVFP4, O.pack_nibbles(codes), sb, g)
    exact = O.e2m1_value(codes) * np.repeat(O.e4m3_value(sb), 16, axis=1) * np.float64(g)
    assert np.array_equal(deq, exact.astype(np.float32))
    # |deq - w| <= half the largest grid step (2, between 4 and 6) * d where |w| <= 6d;
    # beyond 6d (a block whose scale rounded down, e.g. a subnormal UE4M3 scale)
    # the value saturates at 6d
    d = np.repeat((O.e4m3_value(sb) * np.float64(g)), 16, axis=1)
    w64 = w.astype(np.float64)
    bound = np.maximum(d, np.abs(w64) - 6 * d) + np.abs(w64) * 2.0 ** -20 + 1e-30
    assert np.all(np.abs(deq.astype(np.float64) - w64) <= bound)
    assert np.any(np.abs(w64) > 6 * d)  # the saturating case is exercised


def test_nvfp4_zero_and_sizes():
    c, sb, g = O.quantize_nvfp4(np.zeros((4, 32), np.float32))
    assert g == 0 and not c.any() and not sb.any()
    # 8192 x 2048: 8 MiB codes + 1 MiB UE4M3 scales = 9.00 MiB (plus one fp32)
    assert O.codes_bytes(O.FMT_NVFP4, 1, 8192, 2048) + O.scales_bytes(O.FMT_NVFP4, 1, 8192, 2048) == 9 * 2 ** 20


def test_nvfp4_gemv_one_hot_column():
    rng = np.random.default_rng(8)
    w = rng.normal(0, 0.02, (24, 96)).astype(np.float32)
    packed, sb, g = O.quantize(O.FMT_NVFP4, w)
    deq = O.dequant(O.FMT_NVFP4, packed, sb, g)
    for j in (0, 17, 95):
        x = np.zeros(96, np.uint16)
        x[j] = 0x3F80  # bf16 1.0
        y = O.gemv(O.FMT_NVFP4, packed, sb, x, g)
        assert np.array_equal(y, deq[:, j].astype(np.float64))


def test_nvfp4_power_of_two_covariance():
    # scaling W by 2**j scales g by 2**j and leaves scales and codes unchanged
    rng = np.random.default_rng(9)
    w = rng.normal(0, 0.02, (8, 64)).astype(np.float32)
    c0, s0, g0 = O.quantize_nvfp4(w)
    for j in (-5, 3):
        c1, s1, g1 = O.quantize_nvfp4(w * np.float32(2.0 ** j))
        assert np.array_equal(c0, c1) and np.array_equal(s0, s1) and g1 == g0 * np.float32(2.0 ** j)
