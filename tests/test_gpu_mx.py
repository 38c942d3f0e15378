"""GPU parity of the MX variant (MXFP4 experts: E2M1 codes with an E8M0 scale
per 32; activations and h quantised to MXFP8 per the OCP Microscaling
conversion) through the C ABI against the CPU oracle.  Batches of 4 or more
tokens run every product on the scaled FP4 MFMA (the model below); 1-3 tokens
run the single-token VALU kernels (exact products, fp32 sums; last section).

Bit-exact: dequantised weights, routing ids, x as MXFP8 (codes and scales).

The scaled MFMA does not round an exact dot product once: within each
32-element K block (one shared scale pair) it aligns the products to the
largest and drops low-order bits of the small ones.  Measured on gfx950 with
directed and random operands, a block's sum loses at most about 2**-10.6 of its
largest product; EPS_BLOCK = 2**-9 bounds it with margin, and sums across
blocks and K chunks carry an fp32 allowance of 2**-23 per add (truncation
included).  Propagated through silu(g) * u and the down projection, this gives
a bound on every h element and every output element.

h as MXFP8 is an integer decided by floating point: where the oracle's fp64 h
lies within the bound of an E4M3 rounding midpoint, both neighbours are correct
roundings (likewise both shared exponents where a block's absmax lies within
the bound of a power of two).  Every h element the device stores must be the
oracle's rounding or such an alternative, and such elements must stay rare;
the layer output is then compared with the oracle's down projection and
combine of exactly those h values, within the parity bounds and, per element,
one bf16 rounding plus the derived MFMA allowance.  The plain oracle output
(its own roundings throughout) is reported beside it.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import formats as F
from oracle import ops
import bit_block_scaled_router_amd as w4
from bit_block_scaled_router_amd import synth, workloads as wl
from moe_cases import MAX_REL, MEAN_MIN, MEAN_REL, assert_bf16_close, oracle_layer, tie_free_tokens

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda"
MX = w4.W4_FMT_MXFP4_E8M0S32
EPS_BLOCK = 2.0 ** -9
EPS_ADD = 2.0 ** -23
MAX_FLIP_FRAC = 5e-3


@pytest.mark.parametrize("n,k", [(8, 256), (37, 384), (5, 2176)])
def test_mxfp4_dequant_bit_exact(n, k):
    print(f"mxfp4 dequant n={n} k={k}", flush=True)
    rng = np.random.default_rng(n * 37 + k)
    codes = rng.integers(0, 256, size=(2, n, k // 2), dtype=np.uint8)
    codes[0].reshape(-1)[:256] = np.arange(256, dtype=np.uint8)
    scales = rng.integers(100, 150, size=(2, n, k // 32), dtype=np.uint8)
    m = min(scales[0].size, 251)
    scales[0].reshape(-1)[:m] = np.arange(m, dtype=np.uint8)  # E8M0 bytes 0 .. 250
    W = w4.QMatrix.upload(MX, codes, scales, DEV)
    got = w4.w4_dequant_device(W).cpu().numpy()
    want = np.stack([oracle.dequant(F.FMT_MXFP4, codes[g], scales[g]) for g in range(2)])
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def _ws_layout(shape, T):
    """Byte offsets of the MX path's intermediates in the layer workspace, in
    the library's order (each region 256-byte aligned): logits [T][ceil64(E+1)]
    fp32, ids and weights [T][k], group table, the ranking's arrival counter,
    pair list, h (codes [P+T][I] then
    E8M0 scales [P+T][I/32]), expert outputs fp32 [P+T][H], x codes [T][H] then
    scales [T][H/32], and past 1024 pairs the multi-launch grouping's arrays."""
    def up(v):
        return (v + 255) // 256 * 256
    H, I, E, K = shape.hidden, shape.inter, shape.num_experts, shape.top_k
    P = T * K
    rows = P + T
    off = up(T * ((E + 1 + 63) // 64 * 64) * 4)
    off = up(off + T * K * 4)
    off = up(off + T * K * 4)
    off = up(off + (2 + 3 * min(E, P)) * 4)
    off = up(off + 4)
    off = up(off + rows * 4)
    off_h = off
    off = up(off + rows * I * 4)
    off = up(off + rows * H * 4)
    total = up(off + T * H + T * (H // 32))
    if P > 1024:  # three-launch grouping: pair experts, list starts, block histograms, column tiles, block bases
        tpb = 4 if T <= 256 else 16  # tokens per grouping block
        total = up(total + (P + E + 2 * ((T + tpb - 1) // tpb) * E + 2 * (min(E, P) + P // 64 + 1)) * 4)
    return off_h, off, total


def _e4m3(codes):
    """E4M3 bytes -> float64 (torch's float8_e4m3fn decode)."""
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double().numpy()


def _e4m3_codes(v):
    """Values exactly representable in E4M3 (float64) -> bytes."""
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _dot_bound(w, v):
    """Bound on the device's error in w @ v (scaled MFMA over 32-element blocks,
    fp32 across blocks): per row, EPS_BLOCK * sum over blocks of the block's
    largest |w_k v_k|, plus EPS_ADD * (number of blocks) * sum |w_k v_k|."""
    p = np.abs(w) * np.abs(v)[None, :]
    blocks = p.reshape(p.shape[0], -1, 32)
    return EPS_BLOCK * blocks.max(axis=2).sum(axis=1) + EPS_ADD * blocks.shape[1] * p.sum(axis=1)


def _h_and_bound(w13, x):
    """Oracle h = silu(g) * u (fp64) and a bound on the device's error in it."""
    I = w13.shape[0] // 2
    g, u = w13[:I] @ x, w13[I:] @ x
    e = _dot_bound(w13, x)
    eg, eu = e[:I], e[I:]
    sig = 1.0 / (1.0 + np.exp(-g))
    dsilu = sig * (1.0 + g * (1.0 - sig))
    h = ops.silu(g) * u
    # first-order terms, their product, and a few fp32 ulps for exp, divide, multiply
    err = (np.abs(dsilu) + eg) * eg * (np.abs(u) + eu) + np.abs(ops.silu(g)) * eu + 8 * 2.0 ** -24 * np.abs(h)
    return h, err


def _validate_h(h, err, hq_dev, X_dev):
    """Device h (E4M3 bytes [I], exponents [I/32]) against the oracle's fp64
    pre-quantisation h [I] with the device error bound err [I]; returns (device
    h as float64, flipped elements, blocks with the other exponent, the largest
    |h - midpoint| / err over the flips).  Fails on anything else."""
    ho, Xo = F.mx_e4m3(h)
    nb = len(Xo)
    hb, eb = np.abs(h.reshape(nb, 32)), err.reshape(nb, 32)
    amax = hb.max(axis=1)
    other = X_dev != Xo
    if other.any():
        # only where the absmax may sit on either side of the power of two between them
        edge = np.exp2(np.maximum(X_dev, Xo)[other] + 8.0)
        near = np.abs(hb[other] - edge[:, None]) <= eb[other]
        assert np.all(np.abs(X_dev - Xo)[other] == 1), (X_dev, Xo)
        assert np.all(near.any(axis=1)), (amax[other], edge)
        ho = F.mx_e4m3(h, X_dev)[0]
    sc = np.exp2(np.repeat(X_dev, 32).astype(np.float64))
    hd = _e4m3(hq_dev) * sc
    d = hd != ho
    worst = 0.0
    if d.any():
        a, b = _e4m3_codes(hd[d] / sc[d]).astype(np.int64), _e4m3_codes(ho[d] / sc[d]).astype(np.int64)
        assert np.all((a >> 7) == (b >> 7)) and np.all(np.abs(a - b) == 1), ("not adjacent codes", a, b)
        dist = np.abs(h[d] - (hd[d] + ho[d]) / 2)
        assert np.all(dist <= err[d]), ("flip farther from a midpoint than the error bound", h[d], dist, err[d])
        worst = float(np.max(dist / err[d]))
    return hd, int(d.sum()), int(other.sum()), worst


def _mx_case(shape, dev_layer, or_layer, xb, what, tokens=None, ids=None, w=None, xfail_on_flips=False):
    T = xb.shape[0]
    H, I, K = shape.hidden, shape.inter, shape.top_k
    P = T * K
    ws = w4.alloc_workspace(dev_layer, T)
    off_h, off_x, total = _ws_layout(shape, T)
    assert ws.numel() == total
    if ids is None:
        ids_t = torch.full((T, K), -7, dtype=torch.int32, device=DEV)
        w_t = torch.zeros((T, K), dtype=torch.float32, device=DEV)
        y = w4.moe_w4a16_forward(dev_layer, wl.bf16_tensor(xb), topk_ids=ids_t, topk_w=w_t, ws=ws)
    else:
        ids_t, w_t = torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV)
        y = w4.moe_w4a16_experts(dev_layer, wl.bf16_tensor(xb), ids_t, w_t, ws=ws)
    torch.cuda.synchronize()
    wsb = ws.cpu().numpy()
    ydev = wl.bf16_bits(y)
    ids_dev, w_dev = ids_t.cpu().numpy(), w_t.cpu().numpy()
    # x as MXFP8: bit-exact
    xq = wsb[off_x:off_x + T * H].reshape(T, H)
    xs = wsb[off_x + T * H:off_x + T * H + T * H // 32].reshape(T, H // 32).astype(np.int64) - 127
    xo, Xo = F.mx_e4m3(oracle.bf16_bits_to_f64(xb))
    assert np.array_equal(xs, Xo), what
    assert np.array_equal(_e4m3(xq), xo / np.exp2(np.repeat(Xo, 32, axis=1))), what
    hq = wsb[off_h:off_h + (P + T) * I].reshape(P + T, I)
    hs = wsb[off_h + (P + T) * I:off_h + (P + T) * I * 33 // 32].reshape(P + T, I // 32).astype(np.int64) - 127
    rows = list(range(T)) if tokens is None else list(tokens)
    want, plain, allows = [], [], []
    flips = blocks = 0
    worst = 0.0
    for t in rows:
        if ids is None:
            rids, rw = ops.route(ops.router_logits(or_layer.router_w, xb[t], or_layer.router_bias), K)
            assert np.array_equal(ids_dev[t], rids), (what, t)
            np.testing.assert_allclose(w_dev[t], rw, rtol=2e-6, atol=1e-7)
        else:
            rids, rw = ids[t], w[t].astype(np.float64)
        slots = [(or_layer.expert(int(rids[j])), rw[j], t * K + j) for j in range(K)]
        if or_layer.has_shared:
            slots.append((or_layer.shared(), ops.shared_gate(or_layer.shared_gate_w, xb[t]), P + t))
        acc, allow, mag = np.zeros(H), np.zeros(H), np.zeros(H)
        for (w13, w2), coef, p in slots:
            h, err = _h_and_bound(w13, xo[t])
            hd, nf, nb, wr = _validate_h(h, err, hq[p], hs[p])
            flips, blocks, worst = flips + nf, blocks + nb, max(worst, wr)
            yp = w2 @ hd
            acc += coef * yp
            allow += abs(coef) * _dot_bound(w2, hd)
            mag += np.abs(coef * yp)
        want.append(acc)
        # the combine's fp32 sum over the slots
        allows.append(allow + EPS_ADD * len(slots) * mag)
        plain.append(ops.moe_experts(or_layer, xb[t:t + 1], rids[None], np.asarray(rw)[None])[0])
    want, plain, allows = np.array(want), np.array(plain), np.array(allows)
    rep = assert_bf16_close(ydev[rows], want, what, elem_abs=0.0, elem_allow=allows)
    rep_plain = oracle.error_report(oracle.bf16_bits_to_f64(ydev[rows]), plain)
    n_h = len(rows) * (K + (1 if or_layer.has_shared else 0)) * I
    print(f"{what}: {rep}; h elements on the other side of a midpoint {flips} of {n_h}, blocks with the other "
          f"exponent {blocks}, largest |h - midpoint| / bound {worst:.3g}; vs the oracle's own roundings {rep_plain}",
          flush=True)
    assert flips <= max(4, MAX_FLIP_FRAC * n_h), what
    _plain_bar(rep_plain, ydev[rows].size, what, flips, xfail_on_flips)
    return rep


def _plain_bar(rep_plain, size, what, flips, xfail_on_flips=False):
    """The parity bar against the plain oracle (its own h roundings throughout).

    xfail_on_flips: the case's outputs are few enough that a single h element on
    the other side of an MXFP8 midpoint (caused by the scaled MFMA's per-block
    truncation, within the error model checked above) moves the mean error past
    the bar; such a case is an expected failure when, and only when, the checks
    above show that flips are the whole difference."""
    ok = rep_plain["max_abs"] <= MAX_REL * rep_plain["max_ref"] and (size < MEAN_MIN or rep_plain["rel_l1"] <= MEAN_REL)
    if ok:
        return
    if xfail_on_flips and flips > 0 and rep_plain["max_abs"] <= MAX_REL * rep_plain["max_ref"]:
        pytest.xfail(f"{what}: {flips} h element(s) rounded to the neighbouring MXFP8 value by the scaled MFMA's "
                     f"per-block truncation; relative L1 against the plain oracle {rep_plain['rel_l1']:.3g}")
    raise AssertionError((what, "plain oracle", rep_plain))


@pytest.fixture(scope="module")
def tiny_mx():
    shape = synth.TINY_MOE_MX
    return shape, wl.build_moe_layer(shape, device=DEV), oracle_layer(shape)


@pytest.mark.parametrize("T", [4, 7, 40, 300])
def test_mx_tiny_batches(tiny_mx, T):
    # 8 experts, top-2: groups from 1 row (a partial 16-column tile) to ~75 rows
    shape, dev_layer, or_layer = tiny_mx
    print(f"mx tiny T={T}", flush=True)
    _mx_case(shape, dev_layer, or_layer, tie_free_tokens(shape, or_layer, T, first=100), f"mx tiny T={T}")


def test_mx_tiny_experts_entry(tiny_mx):
    shape, dev_layer, or_layer = tiny_mx
    xb = tie_free_tokens(shape, or_layer, 4, first=20)
    ids = np.array([[1, 6], [6, 1], [3, 3], [0, 7]], dtype=np.int32)
    w = np.array([[0.7, 0.3], [0.5, 0.5], [1.0, 0.25], [0.125, -0.5]], dtype=np.float32)
    # four tokens (1,024 outputs): one h flip moves the mean error by ~4e-4
    _mx_case(shape, dev_layer, or_layer, xb, "mx experts", ids=ids, w=w, xfail_on_flips=True)


@pytest.fixture(scope="module")
def full_mx():
    shape = synth.QWEN_MOE_T32_MX
    print("building the 35B-A3B-shaped MXFP4 layer", flush=True)
    return shape, wl.build_moe_layer(shape, device=DEV), oracle_layer(shape)


def test_mx_full_t32_sampled(full_mx):
    # the whole batch runs on the device; the oracle checks every third token
    shape, dev_layer, or_layer = full_mx
    print("mx full T=32", flush=True)
    xb = tie_free_tokens(shape, or_layer, 32, first=50)
    _mx_case(shape, dev_layer, or_layer, xb, "mx full T=32", tokens=range(0, 32, 3))


def test_mx_full_t512_sampled(full_mx):
    # 512 tokens x top-8 = 4096 pairs (three-launch grouping, large-batch kernels); 8 tokens checked
    shape, dev_layer, or_layer = full_mx
    print("mx full T=512 (sampled)", flush=True)
    xb = tie_free_tokens(shape, or_layer, 512, first=1000)
    _mx_case(shape, dev_layer, or_layer, xb, "mx full T=512", tokens=range(5, 512, 64))


def test_mx_prefill_sampled():
    """T = 2048 (16,384 pairs, ~64 per expert): MFMA router, grouping over three
    launches, MX expert kernels with several column passes per group."""
    shape = synth.QWEN_MOE_PREFILL_MX
    dev_layer = wl.build_moe_layer(shape, device=DEV)
    assert w4.moe_w4a16_stage_count(dev_layer, shape.tokens) == 8
    or_layer = oracle_layer(shape)
    print("mx prefill T=2048 (sampled)", flush=True)
    xb = tie_free_tokens(shape, or_layer, shape.tokens)
    _mx_case(shape, dev_layer, or_layer, xb, "mx prefill T=2048", tokens=[0, 1, 700, 1300, 2046, 2047])


# ------------------------------------------------------------------ 1-3 tokens
#
# The single-token kernels quantise in registers: each lane's 32 activations of
# x (W13) and of h (down) are one MXFP8 block.  E2M1 x E4M3 products are exact
# in fp32; a lane's 32-element sum, its scaling by both shared exponents (exact)
# and the wave reduction add at most 32 + 1 + 6 fp32 roundings (W13, 64 lanes)
# or 32 + 1 + 4 + 1 (down, 16 lanes, times the routing weight), each within
# 2**-24 of the partial sum, itself at most sum |w_k v_k|: EPS_VALU = 64 * 2**-24
# per unit of that sum bounds both.  h is stored in fp32 before the down kernel
# quantises it, so the stored h is checked against the oracle's fp64 h, and its
# MXFP8 rounding (the oracle's quantiser applied to the device h: the kernel's
# conversion is bit-exact) may differ from the oracle's own only across a
# midpoint within that bound.

EPS_VALU = 64 * 2.0 ** -24


def _lanes(k):
    need, L = (k + 31) // 32, 1
    while L < need and L < 64:
        L *= 2
    return L


def _ws_layout_single(shape, T):
    """Offset of h in the single-token path's workspace: logits [T][ceil64(E+1)]
    fp32, ids and weights [T][k], then h [T][S][hstride] fp32 in the down
    kernel's lane order; returns (offset, hstride, lanes per row of the down
    kernel, total bytes)."""
    def up(v):
        return (v + 255) // 256 * 256
    H, I, E, K = shape.hidden, shape.inter, shape.num_experts, shape.top_k
    S = K + (1 if shape.has_shared else 0)
    L2 = _lanes(I)
    hstride = (I + 32 * L2 - 1) // (32 * L2) * 32 * L2
    off = up(T * ((E + 1 + 63) // 64 * 64) * 4)
    off = up(off + T * K * 4)
    off_h = up(off + T * K * 4)
    return off_h, hstride, L2, up(off_h + T * S * hstride * 4)


def _h_order(I, L2):
    """Position of h element i in the down kernel's lane order: lane lk of step s
    holds elements 32 (L2 s + lk) .. +31 as 8 float4."""
    i = np.arange(I)
    span = 32 * L2
    st, rem = i // span, i % span
    return st * span + ((rem & 31) // 4 * L2 + rem // 32) * 4 + (i & 3)


def _valu_bound(w, v):
    return EPS_VALU * (np.abs(w) * np.abs(v)[None, :]).sum(axis=1)


def _mx_case_single(shape, dev_layer, or_layer, xb, what, ids=None, w=None):
    T = xb.shape[0]
    H, I, K = shape.hidden, shape.inter, shape.top_k
    S = K + (1 if shape.has_shared else 0)
    assert w4.moe_w4a16_stage_count(dev_layer, T) == 3
    ws = w4.alloc_workspace(dev_layer, T)
    off_h, hstride, L2, total = _ws_layout_single(shape, T)
    assert ws.numel() == total
    if ids is None:
        ids_t = torch.full((T, K), -7, dtype=torch.int32, device=DEV)
        w_t = torch.zeros((T, K), dtype=torch.float32, device=DEV)
        y = w4.moe_w4a16_forward(dev_layer, wl.bf16_tensor(xb), topk_ids=ids_t, topk_w=w_t, ws=ws)
    else:
        ids_t, w_t = torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV)
        y = w4.moe_w4a16_experts(dev_layer, wl.bf16_tensor(xb), ids_t, w_t, ws=ws)
    torch.cuda.synchronize()
    hws = ws.cpu().numpy()[off_h:off_h + T * S * hstride * 4].view(np.float32).reshape(T, S, hstride)
    hdev = hws[:, :, _h_order(I, L2)].astype(np.float64)
    ydev = wl.bf16_bits(y)
    ids_dev, w_dev = ids_t.cpu().numpy(), w_t.cpu().numpy()
    xo = F.mx_e4m3(oracle.bf16_bits_to_f64(xb))[0]
    want, plain, allows = [], [], []
    flips = blocks = 0
    worst = 0.0
    for t in range(T):
        if ids is None:
            rids, rw = ops.route(ops.router_logits(or_layer.router_w, xb[t], or_layer.router_bias), K)
            assert np.array_equal(ids_dev[t], rids), (what, t)
            np.testing.assert_allclose(w_dev[t], rw, rtol=2e-6, atol=1e-7)
        else:
            rids, rw = ids[t], w[t].astype(np.float64)
        slots = [(or_layer.expert(int(rids[j])), rw[j]) for j in range(K)]
        if or_layer.has_shared:
            slots.append((or_layer.shared(), ops.shared_gate(or_layer.shared_gate_w, xb[t])))
        acc, allow, mag = np.zeros(H), np.zeros(H), np.zeros(H)
        for j, ((w13, w2), coef) in enumerate(slots):
            g, u = w13[:I] @ xo[t], w13[I:] @ xo[t]
            e = _valu_bound(w13, xo[t])
            eg, eu = e[:I], e[I:]
            sig = 1.0 / (1.0 + np.exp(-g))
            dsilu = sig * (1.0 + g * (1.0 - sig))
            h = ops.silu(g) * u
            err = (np.abs(dsilu) + eg) * eg * (np.abs(u) + eu) + np.abs(ops.silu(g)) * eu + 8 * 2.0 ** -24 * np.abs(h)
            hd = hdev[t, j]
            bad = np.abs(hd - h) > err
            assert not bad.any(), (what, t, j, int(bad.sum()), np.max(np.abs(hd - h) / err))
            # the down kernel's MXFP8 rounding of the stored h (bit-exact), against the oracle's own
            hq, Xd = F.mx_e4m3(hd)
            codes = _e4m3_codes(hq / np.exp2(np.repeat(Xd, 32).astype(np.float64)))
            hq2, nf, nb, wr = _validate_h(h, err, codes, Xd)
            assert np.array_equal(hq2, hq)
            flips, blocks, worst = flips + nf, blocks + nb, max(worst, wr)
            yp = w2 @ hq
            acc += coef * yp
            allow += abs(coef) * _valu_bound(w2, hq)
            mag += np.abs(coef * yp)
        want.append(acc)
        allows.append(allow + EPS_ADD * len(slots) * mag)
        plain.append(ops.moe_experts(or_layer, xb[t:t + 1], rids[None], np.asarray(rw)[None])[0])
    want, plain, allows = np.array(want), np.array(plain), np.array(allows)
    rep = assert_bf16_close(ydev, want, what, elem_abs=0.0, elem_allow=allows)
    rep_plain = oracle.error_report(oracle.bf16_bits_to_f64(ydev), plain)
    n_h = T * S * I
    print(f"{what}: {rep}; h elements on the other side of a midpoint {flips} of {n_h}, blocks with the other "
          f"exponent {blocks}, largest |h - midpoint| / bound {worst:.3g}; vs the oracle's own roundings {rep_plain}",
          flush=True)
    assert flips <= max(4, MAX_FLIP_FRAC * n_h), what
    # the plain oracle output (its own h roundings) within the parity bar
    _plain_bar(rep_plain, ydev.size, what, flips)
    return rep


@pytest.mark.parametrize("T", [1, 2, 3])
def test_mx_tiny_single_tokens(tiny_mx, T):
    shape, dev_layer, or_layer = tiny_mx
    for first in range(0, 3 * T, T):
        print(f"mx tiny single-token path T={T} first={first}", flush=True)
        _mx_case_single(shape, dev_layer, or_layer, tie_free_tokens(shape, or_layer, T, first=first),
                        f"mx tiny T={T} first={first}")


def test_mx_tiny_single_tokens_experts_entry(tiny_mx):
    # supplied routing: a repeated expert, a negative weight, an id out of range
    # (its slot reads nothing and the token's output is NaN)
    shape, dev_layer, or_layer = tiny_mx
    xb = tie_free_tokens(shape, or_layer, 3, first=30)
    ids = np.array([[1, 6], [3, 3], [0, 7]], dtype=np.int32)
    w = np.array([[0.7, 0.3], [1.0, 0.25], [0.125, -0.5]], dtype=np.float32)
    _mx_case_single(shape, dev_layer, or_layer, xb, "mx single experts", ids=ids, w=w)
    ids_bad = ids.copy()
    ids_bad[1, 0] = 8
    y = w4.moe_w4a16_experts(dev_layer, wl.bf16_tensor(xb), torch.from_numpy(ids_bad).to(DEV),
                             torch.from_numpy(w).to(DEV))
    yb = oracle.bf16_bits_to_f64(wl.bf16_bits(y))
    assert np.all(np.isnan(yb[1])) and np.all(np.isfinite(yb[[0, 2]]))


def test_mx_full_t1(full_mx):
    shape, dev_layer, or_layer = full_mx
    for t in range(2):
        print(f"mx full token {t}", flush=True)
        _mx_case_single(shape, dev_layer, or_layer, tie_free_tokens(shape, or_layer, 1, first=t), f"mx full t={t}")


def test_mx_full_t3(full_mx):
    shape, dev_layer, or_layer = full_mx
    print("mx full T=3", flush=True)
    _mx_case_single(shape, dev_layer, or_layer, tie_free_tokens(shape, or_layer, 3, first=10), "mx full T=3")


# ------------------------------------------------------------------ the instruction's rounding
#
# The MX batch bounds above rest on one property of v_mfma_scale_f32_16x16x128_f8f6f4:
# a 32-element block's sum (both operands' E8M0 scales applied) is within
# EPS_BLOCK of the block's largest |product| of the exact sum, and sums across
# blocks and chunks add fp32 roundings.  The test hook runs the instruction with
# the MX kernels' operand mapping on plain matrices and checks that bound against
# the exact (float64) products, on random full-range operands and on blocks built
# to expose the truncation (one large product beside 31 small ones).

def _mx_dot_case(a_codes, a_scales, b_codes, b_scales):
    n, m = a_codes.shape[0], b_codes.shape[0]
    A = w4.QMatrix.upload(MX, a_codes, a_scales, DEV)
    out = w4.w4_mx_dot_device(A, torch.from_numpy(b_codes).to(DEV), torch.from_numpy(b_scales).to(DEV))
    dev = out.cpu().numpy().astype(np.float64)
    wa = oracle.dequant(F.FMT_MXFP4, a_codes, a_scales).astype(np.float64)
    wb = _e4m3(b_codes) * np.repeat(np.exp2(b_scales.astype(np.float64) - 127.0), 32, axis=1)
    exact = wa @ wb.T
    p = np.abs(wa)[:, None, :] * np.abs(wb)[None, :, :]  # [n][m][k]
    blocks = p.reshape(n, m, -1, 32)
    bmax = blocks.max(axis=3).sum(axis=2)
    bound = EPS_BLOCK * bmax + EPS_ADD * blocks.shape[2] * p.sum(axis=2)
    err = np.abs(dev - exact)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bmax > 0, err / bmax, 0.0)
    return err, bound, float(ratio.max()), int((err > 0).sum())


def _valid_e4m3(rng, shape):
    b = rng.integers(0, 256, size=shape, dtype=np.uint8)
    b[(b & 0x7F) == 0x7F] = 0x70  # no NaN codes
    return b


def test_scaled_mfma_error_model_random():
    rng = np.random.default_rng(2027)
    n, m, k = 64, 64, 1024
    a = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    sa = rng.integers(118, 137, size=(n, k // 32), dtype=np.uint8)
    b = _valid_e4m3(rng, (m, k))
    sb = rng.integers(118, 137, size=(m, k // 32), dtype=np.uint8)
    err, bound, worst, inexact = _mx_dot_case(a, sa, b, sb)
    print(f"scaled MFMA, random operands: {inexact} of {n * m} sums inexact, worst |error| / "
          f"sum of block maxima = 2^{np.log2(worst) if worst > 0 else -np.inf:.2f}", flush=True)
    assert np.all(err <= bound), (float((err / bound).max()),)
    assert worst <= EPS_BLOCK


def test_scaled_mfma_error_model_directed():
    # A = 1.0 everywhere (code 0x2, scale byte 127); column j of B holds, in each
    # 32-block, 256 at one position and v_j at the 31 others (E4M3 bytes with
    # scale byte 127), so the block sums are 256 + 31 v_j.
    n, k = 16, 256
    a = np.full((n, k // 2), 0x22, dtype=np.uint8)
    sa = np.full((n, k // 32), 127, dtype=np.uint8)
    smalls = [2.0 ** -9, 2.0 ** -8, 2.0 ** -7, 2.0 ** -6, 0.0234375, 2.0 ** -3, 0.75, 3.0, 2.0 ** -9 * 3,
              2.0 ** -5 * 1.125, 2.0 ** -4 * 1.875, 1.0, 0.5, 2.0 ** -2 * 1.25, 0.0, 7.0]
    m = len(smalls)
    vals = np.empty((m, k))
    for j, v in enumerate(smalls):
        vals[j] = v
        vals[j, (np.arange(k // 32) * 32 + (j % 32))] = 256.0
    b = _e4m3_codes(vals)
    assert np.array_equal(_e4m3(b), vals)
    sb = np.full((m, k // 32), 127, dtype=np.uint8)
    err, bound, worst, inexact = _mx_dot_case(a, sa, b, sb)
    print(f"scaled MFMA, one large product per block: {inexact} of {n * m} sums inexact, worst |error| / sum of "
          f"block maxima = 2^{np.log2(worst) if worst > 0 else -np.inf:.2f}", flush=True)
    assert np.all(err <= bound), (float((err / bound).max()),)
    assert worst <= EPS_BLOCK
