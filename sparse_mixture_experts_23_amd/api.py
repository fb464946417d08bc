"""Torch-tensor front end of the HIP library.

Every step of the layer runs in the library's HIP kernels; this module only
allocates device tensors (through PyTorch), passes their addresses and the
current HIP stream, and raises on error codes.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib as L


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return L.MOE_F32
    if dt == torch.bfloat16:
        return L.MOE_BF16
    raise TypeError(f"unsupported activation dtype {dt}")


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, shape: tuple):
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name}: expected contiguous {dtype} {shape} on the GPU, got "
                         f"{t.dtype} {tuple(t.shape)} on {t.device}")


def make_shape(T: int, d: int, m: int, E: int, k: int, capacity: int = 0, gate_mode: int = L.MOE_GATE_RENORM,
               dtype=torch.bfloat16, m_shared: int = 0, accept_by_gate: bool = False,
               renorm_survivors: bool = False, reroute: bool = False) -> L.MoeShape:
    s = L.MoeShape(T, d, m, E, k, capacity, gate_mode,
                   _dtype_code(dtype) if isinstance(dtype, torch.dtype) else int(dtype), m_shared,
                   int(accept_by_gate), int(renorm_survivors), int(reroute))
    L.check(L.moe_check_shape(s), "moe_check_shape")
    return s


def capacity(T: int, k: int, E: int, cf_num: int, cf_den: int) -> int:
    c = L.moe_capacity(T, k, E, cf_num, cf_den)
    if c < 0:
        raise ValueError("invalid capacity arguments")
    return c


def _torch_dtype(shape: L.MoeShape):
    return torch.bfloat16 if shape.dtype == L.MOE_BF16 else torch.float32


def paths(shape: L.MoeShape) -> int:
    """Routing records per token: k, or 2k with rerouting (the k selected
    experts, then the next k in rank order)."""
    return 2 * shape.k if shape.reroute else shape.k


def workspace(shape: L.MoeShape, kind: int, device="cuda") -> torch.Tensor:
    """Workspace for the named call; the router's sync words at the start of a
    route, route-stats or forward workspace are zeroed once here (the library
    leaves them at zero after every call)."""
    n = L.moe_workspace_bytes(shape, kind)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device=device)
    if kind in (L.MOE_WS_ROUTE, L.MOE_WS_ROUTE_STATS, L.MOE_WS_FORWARD):
        ws[:L.MOE_SYNC_BYTES].zero_()
    return ws


def pack_weights(w: torch.Tensor) -> torch.Tensor:
    """A weight in the pages' in x out layout, [rows, cols] or [batch, rows, cols]
    (bf16 or fp32), as the library's out x in layout [.., cols, rows]:
    W_r [d,E] -> w_r [E,d]; W_gate, W_up [E,d,m] -> [E,m,d]; W_down [E,m,d] -> [E,d,m]."""
    if w.dtype not in (torch.bfloat16, torch.float32) or w.dim() not in (2, 3) or not w.is_cuda \
            or not w.is_contiguous():
        raise ValueError(f"pack_weights: expected a contiguous 2-D or 3-D bf16/fp32 GPU tensor, got "
                         f"{w.dtype} {tuple(w.shape)} on {w.device}")
    batch, rows, cols = (1,) + tuple(w.shape) if w.dim() == 2 else tuple(w.shape)
    out = torch.empty(w.shape[:-2] + (cols, rows), dtype=w.dtype, device=w.device)
    L.check(L.moe_pack_weights(_ptr(w), _ptr(out), batch, rows, cols, w.element_size(), _stream()),
            "moe_pack_weights")
    return out


def route(shape: L.MoeShape, x, w_r, b_r=None):
    """Returns (topk_ids [T,P] int32, topk_w [T,P] fp32, status [1] int32), P = paths(shape)."""
    dev = x.device
    T, k = shape.T, paths(shape)
    _need(x, "x", _torch_dtype(shape), (T, shape.d))
    _need(w_r, "w_r", torch.float32, (shape.E, shape.d))
    if b_r is not None:
        _need(b_r, "b_r", torch.float32, (shape.E,))
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    status = torch.empty(1, dtype=torch.int32, device=dev)
    ws = workspace(shape, L.MOE_WS_ROUTE, dev)
    L.check(L.moe_route(shape, _ptr(x), _ptr(w_r), _ptr(b_r), _ptr(ids), _ptr(w), _ptr(status), _ptr(ws),
                        ws.numel(), _stream()), "moe_route")
    return ids, w, status


def route_stats(shape: L.MoeShape, x, w_r, b_r=None):
    """moe_route_stats: (topk_ids, topk_w, status, prob_sum [E] fp32)."""
    dev = x.device
    T, k = shape.T, paths(shape)
    _need(x, "x", _torch_dtype(shape), (T, shape.d))
    _need(w_r, "w_r", torch.float32, (shape.E, shape.d))
    if b_r is not None:
        _need(b_r, "b_r", torch.float32, (shape.E,))
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    status = torch.empty(1, dtype=torch.int32, device=dev)
    prob_sum = torch.empty(shape.E, dtype=torch.float32, device=dev)
    ws = workspace(shape, L.MOE_WS_ROUTE_STATS, dev)
    L.check(L.moe_route_stats(shape, _ptr(x), _ptr(w_r), _ptr(b_r), _ptr(ids), _ptr(w), _ptr(status),
                              _ptr(prob_sum), _ptr(ws), ws.numel(), _stream()), "moe_route_stats")
    return ids, w, status, prob_sum


def balance(shape: L.MoeShape, load, stats, prob_sum):
    """moe_balance: fp32 [2E + MOE_BAL_COUNT] = f_e, p_bar_e, then the MOE_BAL_* values."""
    E = shape.E
    _need(load, "load", torch.int32, (E,))
    _need(stats, "stats", torch.int32, (L.MOE_STAT_COUNT,))
    _need(prob_sum, "prob_sum", torch.float32, (E,))
    out = torch.empty(2 * E + L.MOE_BAL_COUNT, dtype=torch.float32, device=load.device)
    L.check(L.moe_balance(shape, _ptr(load), _ptr(stats), _ptr(prob_sum), _ptr(out), _stream()), "moe_balance")
    return out


@dataclass
class DispatchOut:
    load: torch.Tensor
    offsets: torch.Tensor
    slot: torch.Tensor
    row_of: torch.Tensor
    src_token: torch.Tensor
    x_perm: torch.Tensor
    stats: torch.Tensor


def dispatch(shape: L.MoeShape, x, topk_ids, topk_w=None) -> DispatchOut:
    """topk_w (the routing weights) is needed only with shape.accept_by_gate.
    topk_ids and the slot / row_of outputs have P = paths(shape) columns."""
    dev = x.device
    T, k, E = shape.T, paths(shape), shape.E
    R = L.moe_max_rows(shape)
    _need(x, "x", _torch_dtype(shape), (T, shape.d))
    _need(topk_ids, "topk_ids", torch.int32, (T, k))
    if topk_w is not None:
        _need(topk_w, "topk_w", torch.float32, (T, k))
    out = DispatchOut(
        load=torch.empty(E, dtype=torch.int32, device=dev),
        offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
        slot=torch.empty((T, k), dtype=torch.int32, device=dev),
        row_of=torch.empty((T, k), dtype=torch.int32, device=dev),
        src_token=torch.empty(max(R, 1), dtype=torch.int32, device=dev),
        x_perm=torch.empty((max(R, 1), shape.d), dtype=x.dtype, device=dev),
        stats=torch.empty(L.MOE_STAT_COUNT, dtype=torch.int32, device=dev),
    )
    ws = workspace(shape, L.MOE_WS_DISPATCH, dev)
    L.check(L.moe_dispatch(shape, _ptr(x), _ptr(topk_ids), _ptr(topk_w), _ptr(out.load), _ptr(out.offsets),
                           _ptr(out.slot),
                           _ptr(out.row_of), _ptr(out.src_token), _ptr(out.x_perm), _ptr(out.stats), _ptr(ws),
                           ws.numel(), _stream()), "moe_dispatch")
    return out


def expert_ffn(shape: L.MoeShape, x_perm, offsets, w_gate, w_up, w_down):
    dev = x_perm.device
    R = L.moe_max_rows(shape)
    dt = _torch_dtype(shape)
    _need(w_gate, "w_gate", dt, (shape.E, shape.m, shape.d))
    _need(w_up, "w_up", dt, (shape.E, shape.m, shape.d))
    _need(w_down, "w_down", dt, (shape.E, shape.d, shape.m))
    H = torch.empty((max(R, 1), shape.d), dtype=torch.float32, device=dev)
    ws = workspace(shape, L.MOE_WS_FFN, dev)
    L.check(L.moe_expert_ffn(shape, _ptr(x_perm), _ptr(offsets), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(H),
                             _ptr(ws), ws.numel(), _stream()), "moe_expert_ffn")
    return H


def expert_gemm1(shape: L.MoeShape, x_perm, offsets, w_gate, w_up, ws=None):
    dev = x_perm.device
    R = L.moe_max_rows(shape)
    h = torch.empty((max(R, 1), shape.m), dtype=_torch_dtype(shape), device=dev)
    ws = workspace(shape, L.MOE_WS_FFN, dev) if ws is None else ws
    L.check(L.moe_expert_gemm1(shape, _ptr(x_perm), _ptr(offsets), _ptr(w_gate), _ptr(w_up), _ptr(h), _ptr(ws),
                               ws.numel(), _stream()), "moe_expert_gemm1")
    return h


def expert_gemm2(shape: L.MoeShape, h, offsets, w_down, ws=None):
    dev = h.device
    R = L.moe_max_rows(shape)
    H = torch.empty((max(R, 1), shape.d), dtype=torch.float32, device=dev)
    ws = workspace(shape, L.MOE_WS_FFN, dev) if ws is None else ws
    L.check(L.moe_expert_gemm2(shape, _ptr(h), _ptr(offsets), _ptr(w_down), _ptr(H), _ptr(ws), ws.numel(),
                               _stream()), "moe_expert_gemm2")
    return H


def shared_ffn(shape: L.MoeShape, x, s_gate, s_up, s_down):
    dev = x.device
    s = torch.empty((shape.T, shape.d), dtype=torch.float32, device=dev)
    ws = workspace(shape, L.MOE_WS_SHARED, dev)
    L.check(L.moe_shared_ffn(shape, _ptr(x), _ptr(s_gate), _ptr(s_up), _ptr(s_down), _ptr(s), _ptr(ws), ws.numel(),
                             _stream()), "moe_shared_ffn")
    return s


def combine(shape: L.MoeShape, H, row_of, topk_w, shared_out=None):
    dev = row_of.device
    y = torch.empty((shape.T, shape.d), dtype=torch.float32, device=dev)
    L.check(L.moe_combine(shape, _ptr(H), _ptr(row_of), _ptr(topk_w), _ptr(shared_out), _ptr(y), _stream()),
            "moe_combine")
    return y


class MoELayer:
    """Pre-allocated outputs and workspace for repeated whole-layer forwards."""

    def __init__(self, shape: L.MoeShape, device="cuda"):
        self.shape = shape
        T, k, E, d = shape.T, paths(shape), shape.E, shape.d
        self.y = torch.empty((T, d), dtype=torch.float32, device=device)
        self.topk_ids = torch.empty((T, k), dtype=torch.int32, device=device)
        self.topk_w = torch.empty((T, k), dtype=torch.float32, device=device)
        self.load = torch.empty(E, dtype=torch.int32, device=device)
        self.slot = torch.empty((T, k), dtype=torch.int32, device=device)
        self.stats = torch.empty(L.MOE_STAT_COUNT, dtype=torch.int32, device=device)
        self.status = torch.empty(1, dtype=torch.int32, device=device)
        self.ws = workspace(shape, L.MOE_WS_FORWARD, device)

    def forward(self, x, w_r, b_r, w_gate, w_up, w_down, s_gate=None, s_up=None, s_down=None):
        L.check(L.moe_forward(self.shape, _ptr(x), _ptr(w_r), _ptr(b_r), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
                              _ptr(s_gate), _ptr(s_up), _ptr(s_down), _ptr(self.y), _ptr(self.topk_ids),
                              _ptr(self.topk_w), _ptr(self.load), _ptr(self.slot), _ptr(self.stats),
                              _ptr(self.status), _ptr(self.ws), self.ws.numel(), _stream()), "moe_forward")
        return self.y

    def check_status(self):
        code = int(self.status.item())
        if code != L.MOE_OK:
            raise L.MoeError(code, "device status")


def forward(shape: L.MoeShape, x, w_r, b_r, w_gate, w_up, w_down, s_gate=None, s_up=None, s_down=None,
            check_status: bool = True):
    """One whole-layer forward; returns the MoELayer holding y and the routing outputs."""
    layer = MoELayer(shape, x.device)
    layer.forward(x, w_r, b_r, w_gate, w_up, w_down, s_gate, s_up, s_down)
    if check_status:
        torch.cuda.current_stream().synchronize()
        layer.check_status()
    return layer
