"""ctypes binding of libmoe.so: the C ABI of include/moe.h, marshalled.

Every function here only checks and converts arguments and calls the
library; all of the layer's arithmetic runs in the HIP kernels.  torch
tensors provide device memory, and the stream is torch's current stream on
the tensors' device.  If the library has not been built this module raises
ImportError: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

from . import build as _build

c_i32 = ctypes.c_int32
c_vp = ctypes.c_void_p

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_WORKSPACE = -3
MOE_ERR_HIP = -4
MOE_ERR_SCRATCH = -5
NOALLOC_SCRATCH_BYTES = 16 << 20
MOE_F32 = 0
MOE_BF16 = 1
MOE_ROUTE_TOPK = 0
MOE_ROUTE_EXPERT_CHOICE = 1
MOE_ACT_GELU = 0
MOE_ACT_SILU = 1
MOE_ACT_SWIGLU = 2


class MoeDesc(ctypes.Structure):
    _fields_ = [("T", c_i32), ("d", c_i32), ("E", c_i32), ("k", c_i32),
                ("d_ff", c_i32), ("n_shared", c_i32), ("dtype", c_i32),
                ("capacity", c_i32), ("aux_alpha", ctypes.c_float),
                ("routing", c_i32), ("expert_fp8", c_i32),
                ("activation", c_i32)]


class MoeWeights(ctypes.Structure):
    _fields_ = [("w_router", c_vp), ("b_router", c_vp),
                ("expert_bias", c_vp), ("w1", c_vp), ("b1", c_vp),
                ("w2", c_vp), ("b2", c_vp), ("ws1", c_vp), ("bs1", c_vp),
                ("ws2", c_vp), ("bs2", c_vp), ("w1_scale", c_vp),
                ("w2_scale", c_vp), ("ws1_scale", c_vp), ("ws2_scale", c_vp),
                ("w3", c_vp), ("b3", c_vp), ("ws3", c_vp), ("bs3", c_vp),
                ("w3_scale", c_vp), ("ws3_scale", c_vp)]


class MoeRouting(ctypes.Structure):
    _fields_ = [("topk_idx", c_vp), ("topk_w", c_vp), ("counts", c_vp),
                ("kept", c_vp), ("offsets", c_vp), ("slot_token", c_vp),
                ("slot_of", c_vp), ("f", c_vp), ("p", c_vp),
                ("l_aux", c_vp), ("monitor", c_vp)]


# (name, restype, argtypes) of every entry point of include/moe.h
SIGNATURES = {
    "moe_capacity": (c_i32, [c_i32, c_i32, ctypes.c_double]),
    "moe_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(MoeDesc)]),
    "moe_gemm_variant": (ctypes.c_int, [ctypes.POINTER(MoeDesc), ctypes.c_int]),
    "moe_gemm_tail_split": (ctypes.c_int, [ctypes.POINTER(MoeDesc),
                                           ctypes.c_int]),
    "moe_router_topk": (ctypes.c_int, [ctypes.POINTER(MoeDesc), c_vp,
                                       ctypes.POINTER(MoeWeights),
                                       ctypes.POINTER(MoeRouting), c_vp,
                                       ctypes.c_size_t, c_vp]),
    "moe_route_dispatch": (ctypes.c_int, [ctypes.POINTER(MoeDesc), c_vp,
                                          ctypes.POINTER(MoeWeights),
                                          ctypes.POINTER(MoeRouting), c_vp,
                                          ctypes.c_size_t, c_vp]),
    "moe_permute": (ctypes.c_int, [ctypes.POINTER(MoeDesc),
                                   ctypes.POINTER(MoeRouting), c_vp,
                                   ctypes.c_size_t, c_vp]),
    "moe_grouped_ffn": (ctypes.c_int, [ctypes.POINTER(MoeDesc), c_vp,
                                       ctypes.POINTER(MoeWeights),
                                       ctypes.POINTER(MoeRouting), c_vp,
                                       ctypes.c_size_t, c_vp]),
    "moe_ffn_up": (ctypes.c_int, [ctypes.POINTER(MoeDesc), c_vp,
                                  ctypes.POINTER(MoeWeights),
                                  ctypes.POINTER(MoeRouting), c_vp,
                                  ctypes.c_size_t, c_vp]),
    "moe_ffn_down": (ctypes.c_int, [ctypes.POINTER(MoeDesc),
                                    ctypes.POINTER(MoeWeights),
                                    ctypes.POINTER(MoeRouting), c_vp,
                                    ctypes.c_size_t, c_vp]),
    "moe_combine": (ctypes.c_int, [ctypes.POINTER(MoeDesc),
                                   ctypes.POINTER(MoeRouting), c_vp, c_vp,
                                   ctypes.c_size_t, c_vp]),
    "moe_forward": (ctypes.c_int, [ctypes.POINTER(MoeDesc), c_vp,
                                   ctypes.POINTER(MoeWeights),
                                   ctypes.POINTER(MoeRouting), c_vp, c_vp,
                                   ctypes.c_size_t, c_vp]),
    "moe_forward_noalloc": (ctypes.c_int, [ctypes.POINTER(MoeDesc), c_vp,
                                           ctypes.POINTER(MoeWeights),
                                           ctypes.POINTER(MoeRouting), c_vp,
                                           c_vp]),
    "moe_bias_update": (ctypes.c_int, [c_i32, c_vp, ctypes.c_float,
                                       ctypes.c_float, c_vp, c_vp]),
    "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_version": (ctypes.c_char_p, []),
}

_LIB = None


def library_path() -> str:
    return _build.library_path()


def lib() -> ctypes.CDLL:
    """The loaded HIP library; ImportError if it was never built."""
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise ImportError(
                f"{path} is missing: build it first with "
                "`python -m sparse_mixture_experts_50_amd.build` "
                "(there is no non-HIP fallback)")
        L = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = lib().moe_status_string(status).decode()
        super().__init__(f"{fn} returned {status} ({msg})")
        self.status = status


def check(fn: str, status: int) -> None:
    if status != MOE_OK:
        raise MoeError(fn, status)
