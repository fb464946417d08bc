"""ctypes binding of libmoe_mi355x.so: the C-ABI functions under the same names.

Argument marshalling only.  The library must have been built (see build.py);
nothing here falls back to another implementation.
"""
from __future__ import annotations

import ctypes
import os
import re
from ctypes import POINTER, c_char_p, c_int32, c_int64, c_size_t, c_void_p

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB_PATH = os.path.join(PKG, "libmoe_mi355x.so")
HEADER = os.path.join(ROOT, "include", "moe.h")

MOE_OK = 0
MOE_ERR_INVALID_ARGUMENT = 1
MOE_ERR_NONFINITE_LOGIT = 2
MOE_ERR_WORKSPACE_TOO_SMALL = 3
MOE_ERR_UNSUPPORTED = 4
MOE_ERR_HIP = 5

MOE_F32 = 0
MOE_BF16 = 1
MOE_GATE_RENORM = 0
MOE_GATE_SWITCH = 1

MOE_STAT_OVERFLOW = 0
MOE_STAT_ACCEPTED = 1
MOE_STAT_MAX_LOAD = 2
MOE_STAT_TOKENS_DROPPED = 3
MOE_STAT_TOKENS_AFFECTED = 4
MOE_STAT_REROUTED = 5
MOE_STAT_COUNT = 8

MOE_SYNC_BYTES = 256   # zeroed once at the start of route / route-stats / forward workspaces
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20

MOE_WS_DISPATCH = 0
MOE_WS_FFN = 1
MOE_WS_SHARED = 2
MOE_WS_FORWARD = 3
MOE_WS_ROUTE = 4
MOE_WS_ROUTE_STATS = 5

MOE_BAL_VALUE = 0
MOE_BAL_PATH_REJECTION = 1
MOE_BAL_TOKENS_AFFECTED = 2
MOE_BAL_TOKENS_DROPPED = 3
MOE_BAL_RHO_MAX = 4
MOE_BAL_COUNT = 5


class MoeShape(ctypes.Structure):
    _fields_ = [("T", c_int64), ("d", c_int32), ("m", c_int32), ("E", c_int32), ("k", c_int32),
                ("capacity", c_int32), ("gate_mode", c_int32), ("dtype", c_int32), ("m_shared", c_int32),
                ("accept_by_gate", c_int32), ("renorm_survivors", c_int32), ("reroute", c_int32)]


class MoeError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {moe_status_str(code)}")


_SIGS = {
    "moe_capacity": (c_int32, [c_int64, c_int32, c_int32, c_int32, c_int32]),
    "moe_max_rows": (c_int64, [POINTER(MoeShape)]),
    "moe_workspace_bytes": (c_size_t, [POINTER(MoeShape), c_int32]),
    "moe_check_shape": (c_int32, [POINTER(MoeShape)]),
    "moe_status_str": (c_char_p, [c_int32]),
    "moe_route": (c_int32, [POINTER(MoeShape), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                            c_void_p, c_size_t, c_void_p]),
    "moe_route_stats": (c_int32, [POINTER(MoeShape), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                  c_void_p, c_void_p, c_size_t, c_void_p]),
    "moe_balance": (c_int32, [POINTER(MoeShape), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "moe_dispatch": (c_int32, [POINTER(MoeShape), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                               c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "moe_expert_ffn": (c_int32, [POINTER(MoeShape), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                 c_void_p, c_size_t, c_void_p]),
    "moe_expert_gemm1": (c_int32, [POINTER(MoeShape), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                   c_void_p, c_size_t, c_void_p]),
    "moe_expert_gemm2": (c_int32, [POINTER(MoeShape), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                   c_size_t, c_void_p]),
    "moe_shared_ffn": (c_int32, [POINTER(MoeShape), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                 c_size_t, c_void_p]),
    "moe_combine": (c_int32, [POINTER(MoeShape), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "moe_forward": (c_int32, [POINTER(MoeShape)] + [c_void_p] * 16 + [c_void_p, c_size_t, c_void_p]),
    "moe_forward_noalloc": (c_int32, [POINTER(MoeShape)] + [c_void_p] * 16 + [c_void_p]),
    "moe_pack_weights": (c_int32, [c_void_p, c_void_p, c_int64, c_int64, c_int64, c_int32, c_void_p]),
}

_lib = None


def declared_functions() -> list:
    """Names of the functions include/moe.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:[A-Za-z_][A-Za-z0-9_]*\s*\*?\s+)+\**(moe_[a-z0-9_]+)\s*\(", text, re.M)))


def lib():
    """Load the built library (raises if it is missing: there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sparse_mixture_experts_23_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def moe_status_str(code: int) -> str:
    return lib().moe_status_str(int(code)).decode()


def check(code: int, where: str) -> None:
    if code != MOE_OK:
        raise MoeError(code, where)


# Thin same-name wrappers (raw integers / device addresses).

def moe_capacity(T, k, E, cf_num, cf_den) -> int:
    return lib().moe_capacity(T, k, E, cf_num, cf_den)


def moe_max_rows(shape: MoeShape) -> int:
    return lib().moe_max_rows(ctypes.byref(shape))


def moe_workspace_bytes(shape: MoeShape, kind: int) -> int:
    return lib().moe_workspace_bytes(ctypes.byref(shape), kind)


def moe_check_shape(shape: MoeShape) -> int:
    return lib().moe_check_shape(ctypes.byref(shape))


def moe_route(shape, x, w_r, b_r, topk_ids, topk_w, status, ws, ws_bytes, stream) -> int:
    return lib().moe_route(ctypes.byref(shape), x, w_r, b_r, topk_ids, topk_w, status, ws, ws_bytes, stream)


def moe_route_stats(shape, x, w_r, b_r, topk_ids, topk_w, status, prob_sum, ws, ws_bytes, stream) -> int:
    return lib().moe_route_stats(ctypes.byref(shape), x, w_r, b_r, topk_ids, topk_w, status, prob_sum, ws, ws_bytes,
                                 stream)


def moe_balance(shape, load, stats, prob_sum, out, stream) -> int:
    return lib().moe_balance(ctypes.byref(shape), load, stats, prob_sum, out, stream)


def moe_dispatch(shape, x, topk_ids, topk_w, load, offsets, slot, row_of, src_token, x_perm, stats, ws, ws_bytes,
                 stream) -> int:
    return lib().moe_dispatch(ctypes.byref(shape), x, topk_ids, topk_w, load, offsets, slot, row_of, src_token, x_perm,
                              stats, ws, ws_bytes, stream)


def moe_expert_ffn(shape, x_perm, offsets, w_gate, w_up, w_down, H, ws, ws_bytes, stream) -> int:
    return lib().moe_expert_ffn(ctypes.byref(shape), x_perm, offsets, w_gate, w_up, w_down, H, ws, ws_bytes, stream)


def moe_expert_gemm1(shape, x_perm, offsets, w_gate, w_up, h, ws, ws_bytes, stream) -> int:
    return lib().moe_expert_gemm1(ctypes.byref(shape), x_perm, offsets, w_gate, w_up, h, ws, ws_bytes, stream)


def moe_expert_gemm2(shape, h, offsets, w_down, H, ws, ws_bytes, stream) -> int:
    return lib().moe_expert_gemm2(ctypes.byref(shape), h, offsets, w_down, H, ws, ws_bytes, stream)


def moe_shared_ffn(shape, x, s_gate, s_up, s_down, s, ws, ws_bytes, stream) -> int:
    return lib().moe_shared_ffn(ctypes.byref(shape), x, s_gate, s_up, s_down, s, ws, ws_bytes, stream)


def moe_combine(shape, H, row_of, topk_w, shared_out, y, stream) -> int:
    return lib().moe_combine(ctypes.byref(shape), H, row_of, topk_w, shared_out, y, stream)


def moe_forward(shape, x, w_r, b_r, w_gate, w_up, w_down, s_gate, s_up, s_down, y, topk_ids, topk_w, load, slot,
                stats, status, ws, ws_bytes, stream) -> int:
    return lib().moe_forward(ctypes.byref(shape), x, w_r, b_r, w_gate, w_up, w_down, s_gate, s_up, s_down, y,
                             topk_ids, topk_w, load, slot, stats, status, ws, ws_bytes, stream)


def moe_forward_noalloc(shape, x, w_r, b_r, w_gate, w_up, w_down, s_gate, s_up, s_down, y, topk_ids, topk_w, load,
                        slot, stats, status, stream) -> int:
    return lib().moe_forward_noalloc(ctypes.byref(shape), x, w_r, b_r, w_gate, w_up, w_down, s_gate, s_up, s_down,
                                     y, topk_ids, topk_w, load, slot, stats, status, stream)


def moe_pack_weights(src, dst, batch, rows, cols, elem_bytes, stream) -> int:
    return lib().moe_pack_weights(src, dst, batch, rows, cols, elem_bytes, stream)
