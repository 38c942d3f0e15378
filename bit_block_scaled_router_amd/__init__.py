"""W4A16 mixture-of-experts decode layer and dense W4A16 GEMV for MI355X (gfx950).

Python binding of the w4moe C ABI (include/w4moe.h).  The functions below keep
the C names and only marshal arguments: torch tensors (device memory, streams)
and numpy arrays (host helpers) become the plain pointers and sizes the library
takes.  All computation runs in the HIP library; if it is not built, importing
the binding's entry points raises.
"""

import ctypes as C

import numpy as np

from ._lib import (  # noqa: F401
    EXPORTS,
    W4_ERR_ALIGNMENT,
    W4_ERR_HIP,
    W4_ERR_INVALID_ARG,
    W4_ERR_LAYOUT,
    W4_ERR_NONFINITE,
    W4_ERR_RANGE,
    W4_ERR_UNSUPPORTED,
    W4_ERR_WORKSPACE,
    W4_FMT_E2M1_F16S16,
    W4_FMT_INT4_F16S128,
    W4_FMT_NVFP4_E4M3S16,
    W4_FMT_BF16,
    W4_FMT_MXFP4_E8M0S32,
    W4_LAYOUT_CANONICAL,
    W4_LAYOUT_GFX950_V1,
    W4_LAYOUT_GFX950_KT16,
    W4_OK,
    MoELayerDesc,
    W4Error,
    W4Matrix,
    check,
    lib,
)

GROUP = {W4_FMT_E2M1_F16S16: 16, W4_FMT_INT4_F16S128: 128, W4_FMT_NVFP4_E4M3S16: 16, W4_FMT_MXFP4_E8M0S32: 32}
FORMATS = {"e2m1": W4_FMT_E2M1_F16S16, "int4": W4_FMT_INT4_F16S128, "nvfp4": W4_FMT_NVFP4_E4M3S16,
           "bf16": W4_FMT_BF16, "mxfp4": W4_FMT_MXFP4_E8M0S32}
# numpy dtype of one block scale per format (FP16 bit patterns, UE4M3 or E8M0 bytes)
SCALE_DTYPE = {W4_FMT_E2M1_F16S16: np.uint16, W4_FMT_INT4_F16S128: np.uint16, W4_FMT_NVFP4_E4M3S16: np.uint8,
               W4_FMT_MXFP4_E8M0S32: np.uint8}


def _torch():
    import torch

    return torch


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _require(t, name, dtype, shape, device=None, check_device=True):
    """Raise ValueError unless t is a contiguous device tensor of this dtype and shape
    (on `device` when given).  The C ABI takes raw pointers and cannot see buffer
    sizes, so every shape and layout promise is checked here before the call."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not check_device:
        return
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor, got device {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _stream(stream):
    if stream is None:
        return _torch().cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


# ------------------------------------------------------------------ host helpers


def w4_version():
    return lib().w4_version().decode()


def w4_status_string(status):
    return lib().w4_status_string(status).decode()


def w4_last_error():
    return lib().w4_last_error().decode()


def w4_codes_bytes(fmt, groups, n, k, layout=W4_LAYOUT_CANONICAL):
    return lib().w4_codes_bytes(fmt, layout, groups, n, k)


def w4_scales_bytes(fmt, groups, n, k, layout=W4_LAYOUT_CANONICAL):
    return lib().w4_scales_bytes(fmt, layout, groups, n, k)


def w4_quantize(fmt, w, codes=None, scales=None):
    """Quantise host fp32 w[n][k] (one matrix).

    Returns (codes uint8 [n][k/2], scales [n][k/G]): FP16 bit patterns (uint16)
    for E2M1/int4; for NVFP4 (codes, UE4M3 bytes uint8, global scale float);
    for MXFP4 (codes, E8M0 bytes uint8 [n][k/32]);
    for bf16 (bf16 bits uint16 [n][k],)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    if w.ndim != 2:
        raise ValueError("w must be 2-D")
    n, k = w.shape
    if fmt == W4_FMT_BF16:
        out = np.empty((n, k), dtype=np.uint16) if codes is None else codes
        check(lib().w4_quantize(fmt, _ptr(w), n, k, _ptr(out), None, None))
        return (out,)
    g = GROUP.get(fmt, 1)
    if codes is None:
        codes = np.empty((n, k // 2), dtype=np.uint8)
    if scales is None:
        scales = np.empty((n, max(k // g, 1)), dtype=SCALE_DTYPE.get(fmt, np.uint16))
    gs = np.zeros(1, dtype=np.float32)
    check(lib().w4_quantize(fmt, _ptr(w), n, k, _ptr(codes), _ptr(scales), _ptr(gs)))
    if fmt == W4_FMT_NVFP4_E4M3S16:
        return codes, scales, np.float32(gs[0])
    return codes, scales


def w4_pack(fmt, codes, scales, layout=W4_LAYOUT_GFX950_V1):
    """Canonical host arrays codes [G][n][k/2] (or [n][k/2]; bf16: bits [G][n][k])
    and scales [G][n][k/Gs] -> (codes, scales) in `layout`.  GFX950_V1 returns
    (records uint8 [G][n][R], None): each row's codes then its scales, padded to a
    multiple of 16 bytes; GFX950_KT16 returns (records uint8 [G][k/16][R], None):
    per 16-wide K tile, every row's 8 code bytes, then every row's scale."""
    c = np.ascontiguousarray(codes)
    if c.ndim == 2:
        c = c[None]
    groups, n, kc = c.shape
    k = kc if fmt == W4_FMT_BF16 else 2 * kc
    s = None if scales is None else np.ascontiguousarray(scales)
    nb = lib().w4_codes_bytes(fmt, layout, groups, n, k)
    if nb == 0:  # let the library name what is wrong (tag or shape)
        check(lib().w4_pack(fmt, groups, n, k, _ptr(c), _ptr(s), layout, None, None))
        check(W4_ERR_INVALID_ARG)
    out = np.empty(nb, dtype=np.uint8)
    sb = lib().w4_scales_bytes(fmt, layout, groups, n, k)
    sout = np.empty(sb, dtype=np.uint8) if sb else None
    check(lib().w4_pack(fmt, groups, n, k, _ptr(c), _ptr(s), layout, _ptr(out), _ptr(sout)))
    if layout == W4_LAYOUT_GFX950_V1:
        return out.reshape(groups, n, -1), None
    if layout == W4_LAYOUT_GFX950_KT16:
        return out.reshape(groups, k // 16, -1), None
    return out.view(c.dtype).reshape(c.shape), (sout.view(s.dtype).reshape(s.shape) if sout is not None else None)


def w4_unpack(fmt, groups, n, k, codes, scales=None, layout=W4_LAYOUT_GFX950_V1):
    """Arrays in `layout` -> canonical (codes uint8 [G][n][k/2], scales [G][n][k/Gs]
    in the format's scale dtype; bf16: (bits uint16 [G][n][k], None))."""
    c = np.ascontiguousarray(codes)
    s = None if scales is None else np.ascontiguousarray(scales)
    if fmt == W4_FMT_BF16:
        oc, osc = np.empty((groups, n, k), dtype=np.uint16), None
    else:
        oc = np.empty((groups, n, k // 2), dtype=np.uint8)
        osc = np.empty((groups, n, k // GROUP[fmt]), dtype=SCALE_DTYPE[fmt])
    check(lib().w4_unpack(fmt, groups, n, k, layout, _ptr(c), _ptr(s), _ptr(oc), _ptr(osc)))
    return oc, osc


def w4_pack_nibbles(nibbles):
    nib = np.ascontiguousarray(nibbles, dtype=np.uint8)
    n, k = nib.shape
    out = np.empty((n, k // 2), dtype=np.uint8)
    check(lib().w4_pack_nibbles(_ptr(nib), n, k, _ptr(out)))
    return out


def w4_unpack_nibbles(packed):
    p = np.ascontiguousarray(packed, dtype=np.uint8)
    n, kh = p.shape
    out = np.empty((n, 2 * kh), dtype=np.uint8)
    check(lib().w4_unpack_nibbles(_ptr(p), n, 2 * kh, _ptr(out)))
    return out


# ------------------------------------------------------------------ device matrices


class QMatrix:
    """A stack of quantised matrices in device memory plus its w4_matrix descriptor."""

    def __init__(self, fmt, groups, n, k, codes, scales, global_scales=None, layout=W4_LAYOUT_CANONICAL):
        self.fmt, self.groups, self.n, self.k = fmt, groups, n, k
        # torch device tensors: uint8 codes, int16 (FP16 bits) or uint8 (UE4M3) scales,
        # uint8 (E8M0) for MXFP4, fp32 [groups] global scales (NVFP4)
        self.codes, self.scales, self.global_scales = codes, scales, global_scales
        self.layout = layout
        self.desc = W4Matrix(fmt, layout, groups, n, k, _ptr(codes), _ptr(scales), _ptr(global_scales))

    @classmethod
    def upload_bf16(cls, bits_np, device="cuda"):
        """bf16 bits [G][n][k] (or [n][k]) -> a W4_FMT_BF16 matrix (no scales)."""
        b = np.ascontiguousarray(bits_np, dtype=np.uint16)
        if b.ndim == 2:
            b = b[None]
        groups, n, k = b.shape
        return cls(W4_FMT_BF16, groups, n, k, _torch().from_numpy(b.view(np.int16)).to(device), None)

    @classmethod
    def upload(cls, fmt, codes_np, scales_np, device="cuda", global_np=None, layout=W4_LAYOUT_CANONICAL):
        """codes_np [G][n][k/2] (or [n][k/2]), scales_np [G][n][k/Gs] (uint16 FP16 bits,
        or uint8 UE4M3 / E8M0 for NVFP4 / MXFP4), global_np fp32 [G] (NVFP4) -> device,
        in `layout` (GFX950_V1: packed on the host by w4_pack; the matrix then has
        row records in `codes` and no separate scales)."""
        torch = _torch()
        c = np.ascontiguousarray(codes_np)
        s = np.ascontiguousarray(scales_np)
        if c.ndim == 2:
            c, s = c[None], s[None]
        groups, n, kh = c.shape
        tg = None
        if global_np is not None:
            tg = torch.from_numpy(np.ascontiguousarray(global_np, dtype=np.float32).reshape(-1)).to(device)
        if layout != W4_LAYOUT_CANONICAL:
            rec, _ = w4_pack(fmt, c, s, layout)
            return cls(fmt, groups, n, 2 * kh, torch.from_numpy(rec).to(device), None, tg, layout=layout)
        tc = torch.from_numpy(c).to(device)
        ts = torch.from_numpy(s.view(np.int16) if s.dtype == np.uint16 else s).to(device)
        return cls(fmt, groups, n, 2 * kh, tc, ts, tg)


def w4a16_gemv(W, x, y=None, stream=None):
    """y[m][n] = x[m][k] . W^T (bf16 in and out); x is a [k] or [m][k] bf16 device tensor."""
    torch = _torch()
    if not isinstance(x, torch.Tensor) or x.dim() not in (1, 2):
        raise ValueError("x must be a [k] or [m][k] bf16 device tensor")
    x2 = x if x.dim() == 2 else x.unsqueeze(0)
    m = x2.shape[0]
    _require(x2, "x", torch.bfloat16, (m, W.k))
    if y is None:
        y = torch.empty((m, W.n) if x.dim() == 2 else (W.n,), dtype=torch.bfloat16, device=x.device)
    if not isinstance(y, torch.Tensor) or y.dim() != x.dim():
        raise ValueError("y must have as many dimensions as x ([n] or [m][n])")
    _require(y if y.dim() == 2 else y.unsqueeze(0), "y", torch.bfloat16, (m, W.n), x.device)
    check(lib().w4a16_gemv(C.byref(W.desc), _ptr(x2), m, _ptr(y), _stream(stream)))
    return y if x.dim() == 2 else y.view(-1)


def w4_dequant_device(W, out=None, stream=None):
    torch = _torch()
    if out is None:
        out = torch.empty((W.groups, W.n, W.k), dtype=torch.float32, device=W.codes.device)
    _require(out, "out", torch.float32, (W.groups, W.n, W.k), W.codes.device)
    check(lib().w4_dequant_device(C.byref(W.desc), _ptr(out), _stream(stream)))
    return out


def w4_mx_dot_device(A, b_codes, b_scales, out=None, stream=None):
    """out[n][m] = A (MXFP4 QMatrix, one group) x B^T on the scaled FP4 MFMA, B given
    as E4M3 codes uint8 [m][k] and E8M0 bytes uint8 [m][k/32] device tensors (test hook)."""
    torch = _torch()
    if not isinstance(b_codes, torch.Tensor) or b_codes.dim() != 2:
        raise ValueError("b_codes must be a [m][k] uint8 device tensor")
    m = b_codes.shape[0]
    _require(b_codes, "b_codes", torch.uint8, (m, A.k), A.codes.device)
    _require(b_scales, "b_scales", torch.uint8, (m, A.k // 32), A.codes.device)
    if out is None:
        out = torch.empty((A.n, m), dtype=torch.float32, device=A.codes.device)
    _require(out, "out", torch.float32, (A.n, m), A.codes.device)
    check(lib().w4_mx_dot_device(C.byref(A.desc), _ptr(b_codes), _ptr(b_scales), m, _ptr(out), _stream(stream)))
    return out


def w4_bench_stream_read(src, sink, stream=None):
    """Read all of the device tensor `src` (contiguous, size a multiple of 16 bytes)
    with the library's streaming-read probe; sink: a one-element int32/uint32 device
    tensor (measurement aid)."""
    torch = _torch()
    if not isinstance(src, torch.Tensor) or not src.is_contiguous() or src.device.type != "cuda":
        raise ValueError("src must be a contiguous device tensor")
    if not isinstance(sink, torch.Tensor) or sink.numel() < 1 or sink.element_size() != 4 or sink.device != src.device:
        raise ValueError("sink must be a 4-byte device tensor on src's device")
    check(lib().w4_bench_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink), _stream(stream)))


# ------------------------------------------------------------------ MoE layer


class MoELayer:
    """Device tensors of one MoE layer plus its moe_w4a16_layer descriptor."""

    def __init__(self, hidden, inter, num_experts, top_k, router_w, w13, w2, router_bias=None,
                 shared_w13=None, shared_w2=None, shared_gate_w=None):
        self.hidden, self.inter, self.num_experts, self.top_k = hidden, inter, num_experts, top_k
        self.router_w, self.router_bias = router_w, router_bias
        self.w13, self.w2 = w13, w2
        self.shared_w13, self.shared_w2, self.shared_gate_w = shared_w13, shared_w2, shared_gate_w
        has_shared = shared_w13 is not None
        empty = W4Matrix(0, 0, 0, 0, 0, None, None, None)
        self.desc = MoELayerDesc(
            hidden, inter, num_experts, top_k, inter if has_shared else 0,
            _ptr(router_w), _ptr(router_bias), w13.desc, w2.desc, 1 if has_shared else 0,
            shared_w13.desc if has_shared else empty, shared_w2.desc if has_shared else empty,
            _ptr(shared_gate_w),
        )

    @property
    def has_shared(self):
        return self.shared_w13 is not None


def _check_moe_args(layer, x, y, ws, ids=None, w=None, ids_name="topk_ids", w_name="topk_w"):
    """Validate the tensors of one MoE call (dtypes and shapes first, then devices);
    returns T."""
    torch = _torch()
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError("x must be a [T][hidden] bf16 device tensor")
    T = x.shape[0]
    need = [(x, "x", torch.bfloat16, (T, layer.hidden)), (y, "y", torch.bfloat16, (T, layer.hidden))]
    if ids is not None:
        need.append((ids, ids_name, torch.int32, (T, layer.top_k)))
    if w is not None:
        need.append((w, w_name, torch.float32, (T, layer.top_k)))
    for t, name, dt, shape in need:
        _require(t, name, dt, shape, check_device=False)
    if ws is not None:
        if not isinstance(ws, torch.Tensor) or ws.dtype != torch.uint8 or ws.dim() != 1 or not ws.is_contiguous():
            raise ValueError("ws must be a contiguous 1-D uint8 device tensor")
    dev = x.device
    for t, name, dt, shape in need:
        _require(t, name, dt, shape, dev)
    if ws is not None and ws.device != dev:
        raise ValueError(f"ws is on {ws.device}, expected {dev}")
    if layer.router_w.device != dev:
        raise ValueError(f"the layer's weights are on {layer.router_w.device}, x on {dev}")
    return T


def moe_w4a16_workspace_bytes(layer, T):
    n = lib().moe_w4a16_workspace_bytes(C.byref(layer.desc), T)
    if n == 0:
        check(W4_ERR_INVALID_ARG)
    return n


def alloc_workspace(layer, T, device="cuda"):
    torch = _torch()
    n = moe_w4a16_workspace_bytes(layer, T)
    return torch.empty(n, dtype=torch.uint8, device=device)


def moe_w4a16_forward(layer, x, y=None, topk_ids=None, topk_w=None, ws=None, stream=None):
    """Full MoE layer for x bf16 [T][H]; returns y bf16 [T][H]."""
    torch = _torch()
    if y is None and isinstance(x, torch.Tensor):
        y = torch.empty_like(x)
    T = _check_moe_args(layer, x, y, ws, topk_ids, topk_w)
    if ws is None:
        ws = alloc_workspace(layer, T, x.device)
    check(lib().moe_w4a16_forward(C.byref(layer.desc), _ptr(x), T, _ptr(y), _ptr(topk_ids), _ptr(topk_w),
                                  _ptr(ws), ws.numel(), _stream(stream)))
    return y


def moe_w4a16_forward_noalloc(layer, x, y, topk_ids=None, topk_w=None, stream=None):
    """moe_w4a16_forward on the library's per-GPU scratch: nothing is allocated,
    so y (bf16 [T][H]) must be given."""
    T = _check_moe_args(layer, x, y, None, topk_ids, topk_w)
    check(lib().moe_w4a16_forward_noalloc(C.byref(layer.desc), _ptr(x), T, _ptr(y), _ptr(topk_ids), _ptr(topk_w),
                                          _stream(stream)))
    return y


def moe_w4a16_stage_count(layer, T):
    n = lib().moe_w4a16_stage_count(C.byref(layer.desc), T)
    if n == 0:
        check(W4_ERR_INVALID_ARG)
    return n


def moe_w4a16_forward_timed(layer, x, y, ws, events, topk_ids=None, topk_w=None, stream=None):
    """moe_w4a16_forward with start/stop events per kernel (2 hipEvent_t per kernel)."""
    _check_moe_args(layer, x, y, ws, topk_ids, topk_w)
    arr = (C.c_void_p * len(events))(*events)
    check(lib().moe_w4a16_forward_timed(C.byref(layer.desc), _ptr(x), x.shape[0], _ptr(y), _ptr(topk_ids),
                                        _ptr(topk_w), _ptr(ws), ws.numel(), _stream(stream), arr, len(events)))
    return y


def moe_w4a16_experts(layer, x, ids, w, y=None, ws=None, stream=None):
    """Experts + combine with given routing: ids int32 [T][k], w fp32 [T][k]."""
    torch = _torch()
    if y is None and isinstance(x, torch.Tensor):
        y = torch.empty_like(x)
    T = _check_moe_args(layer, x, y, ws, ids, w, "ids", "w")
    if ws is None:
        ws = alloc_workspace(layer, T, x.device)
    check(lib().moe_w4a16_experts(C.byref(layer.desc), _ptr(x), T, _ptr(ids), _ptr(w), _ptr(y),
                                  _ptr(ws), ws.numel(), _stream(stream)))
    return y
