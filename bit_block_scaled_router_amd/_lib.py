"""ctypes binding of the w4moe C ABI (include/w4moe.h): argument marshalling only.

Every computation happens in the HIP library; this module only converts torch
tensors and numpy arrays into the plain pointers and sizes the C functions take.
Loading fails loudly when the library has not been built: there is no fallback.
"""

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libw4moe.so")

# status codes and tags (include/w4moe.h)
W4_OK = 0
W4_ERR_INVALID_ARG = -1
W4_ERR_LAYOUT = -2
W4_ERR_ALIGNMENT = -3
W4_ERR_UNSUPPORTED = -4
W4_ERR_WORKSPACE = -5
W4_ERR_NONFINITE = -6
W4_ERR_RANGE = -7
W4_ERR_HIP = -8
W4_FMT_E2M1_F16S16 = 1
W4_FMT_INT4_F16S128 = 2
W4_FMT_NVFP4_E4M3S16 = 3
W4_FMT_BF16 = 4
W4_FMT_MXFP4_E8M0S32 = 5
W4_LAYOUT_CANONICAL = 0
W4_LAYOUT_GFX950_V1 = 1
W4_LAYOUT_GFX950_KT16 = 2

# every symbol the header declares
EXPORTS = (
    "w4_status_string", "w4_last_error", "w4_version",
    "w4_codes_bytes", "w4_scales_bytes", "w4_quantize",
    "w4_pack_nibbles", "w4_unpack_nibbles", "w4_pack", "w4_unpack",
    "w4a16_gemv", "w4_dequant_device", "w4_mx_dot_device", "w4_bench_stream_read",
    "moe_w4a16_workspace_bytes", "moe_w4a16_forward", "moe_w4a16_forward_timed", "moe_w4a16_stage_count",
    "moe_w4a16_experts", "moe_w4a16_forward_noalloc",
)


class W4Matrix(C.Structure):
    _fields_ = [
        ("format", C.c_int32),
        ("layout", C.c_int32),
        ("groups", C.c_int64),
        ("n", C.c_int64),
        ("k", C.c_int64),
        ("codes", C.c_void_p),
        ("scales", C.c_void_p),
        ("global_scales", C.c_void_p),
    ]


class MoELayerDesc(C.Structure):
    _fields_ = [
        ("hidden", C.c_int64),
        ("inter", C.c_int64),
        ("num_experts", C.c_int64),
        ("top_k", C.c_int64),
        ("shared_inter", C.c_int64),
        ("router_w", C.c_void_p),
        ("router_bias", C.c_void_p),
        ("w13", W4Matrix),
        ("w2", W4Matrix),
        ("has_shared", C.c_int32),
        ("shared_w13", W4Matrix),
        ("shared_w2", W4Matrix),
        ("shared_gate_w", C.c_void_p),
    ]


class W4Error(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{message} (status {status})")
        self.status = status


_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        try:  # share the HIP runtime torch loads (one runtime per process)
            import torch  # noqa: F401
        except ImportError:
            pass
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m bit_block_scaled_router_amd.build`"
            )
        L = C.CDLL(LIB_PATH)
        P, I64, I32, SZ = C.c_void_p, C.c_int64, C.c_int32, C.c_size_t
        sig = {
            "w4_status_string": (C.c_char_p, [C.c_int]),
            "w4_last_error": (C.c_char_p, []),
            "w4_version": (C.c_char_p, []),
            "w4_codes_bytes": (SZ, [I32, I32, I64, I64, I64]),
            "w4_scales_bytes": (SZ, [I32, I32, I64, I64, I64]),
            "w4_quantize": (C.c_int, [I32, P, I64, I64, P, P, P]),
            "w4_pack_nibbles": (C.c_int, [P, I64, I64, P]),
            "w4_unpack_nibbles": (C.c_int, [P, I64, I64, P]),
            "w4_pack": (C.c_int, [I32, I64, I64, I64, P, P, I32, P, P]),
            "w4_unpack": (C.c_int, [I32, I64, I64, I64, I32, P, P, P, P]),
            "w4a16_gemv": (C.c_int, [C.POINTER(W4Matrix), P, I64, P, P]),
            "w4_dequant_device": (C.c_int, [C.POINTER(W4Matrix), P, P]),
            "w4_mx_dot_device": (C.c_int, [C.POINTER(W4Matrix), P, P, I64, P, P]),
            "w4_bench_stream_read": (C.c_int, [P, SZ, P, P]),
            "moe_w4a16_workspace_bytes": (SZ, [C.POINTER(MoELayerDesc), I64]),
            "moe_w4a16_forward": (C.c_int, [C.POINTER(MoELayerDesc), P, I64, P, P, P, P, SZ, P]),
            "moe_w4a16_forward_timed": (C.c_int, [C.POINTER(MoELayerDesc), P, I64, P, P, P, P, SZ, P, P, I32]),
            "moe_w4a16_stage_count": (C.c_int, [C.POINTER(MoELayerDesc), I64]),
            "moe_w4a16_experts": (C.c_int, [C.POINTER(MoELayerDesc), P, I64, P, P, P, P, SZ, P]),
            "moe_w4a16_forward_noalloc": (C.c_int, [C.POINTER(MoELayerDesc), P, I64, P, P, P, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def check(status):
    if status != W4_OK:
        L = lib()
        raise W4Error(status, f"{L.w4_status_string(status).decode()}: {L.w4_last_error().decode()}")
    return status
