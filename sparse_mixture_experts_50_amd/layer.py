"""torch-facing wrappers of the C ABI, with the C entry points' names.

Only argument checking and marshalling happens here; each call enqueues the
HIP kernels on torch's current stream for the tensors' device.  Shapes and
layouts are those of include/moe.h:
  x [T][d]; w_router [E][d]; w1 [E][d_ff][d]; w2 [E][d][d_ff];
  b1 [E][d_ff]; b2 [E][d]; shared expert ws1 [d_ff][d], ws2 [d][d_ff];
  b_router / expert_bias float32 [E].
FP8 expert matrices: uint8 (or float8_e4m3fn) tensors of the same shapes
holding OCP E4M3 codes, with float32 per-output-channel scales
w1_scale [E][d_ff], w2_scale [E][d], ws1_scale [d_ff], ws2_scale [d].
SwiGLU experts add the up projection w3 [E][d_ff][d], b3 [E][d_ff] (ws3,
bs3 for the shared expert; w3_scale, ws3_scale for FP8); W1 is the gate.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib
from ._lib import MoeDesc, MoeRouting, MoeWeights, check

_DT = {torch.float32: _lib.MOE_F32, torch.bfloat16: _lib.MOE_BF16}
_ROUTING = {"topk": _lib.MOE_ROUTE_TOPK,
            "expert_choice": _lib.MOE_ROUTE_EXPERT_CHOICE}
_ACT = {"gelu": _lib.MOE_ACT_GELU, "silu": _lib.MOE_ACT_SILU,
        "swiglu": _lib.MOE_ACT_SWIGLU}


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _need(t: Optional[torch.Tensor], name: str, shape, dtype, device):
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype} != {dtype}")
    if t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _opt(t, name, shape, dtype, device):
    if t is not None:
        _need(t, name, shape, dtype, device)


def make_desc(T: int, d: int, E: int, k: int, d_ff: int, dtype: torch.dtype,
              n_shared: int = 0, capacity: int = -1,
              aux_alpha: float = 0.01, routing: str = "topk",
              expert_fp8: bool = False, activation: str = "gelu") -> MoeDesc:
    """``routing`` is "topk" or "expert_choice" (then k must be E and
    capacity the tokens each expert picks); ``expert_fp8`` marks E4M3
    expert matrices; ``activation`` is "gelu", "silu" or "swiglu"."""
    if dtype not in _DT:
        raise ValueError(f"unsupported dtype {dtype}")
    if routing not in _ROUTING:
        raise ValueError(f"unknown routing {routing!r}")
    if activation not in _ACT:
        raise ValueError(f"unknown activation {activation!r}")
    return MoeDesc(T, d, E, k, d_ff, n_shared, _DT[dtype], capacity,
                   aux_alpha, _ROUTING[routing], int(bool(expert_fp8)),
                   _ACT[activation])


def moe_capacity(T: int, E: int, capacity_factor: Optional[float]) -> int:
    """floor(T / E * cf); -1 (no limit) when cf is None."""
    if capacity_factor is None:
        return -1
    c = _lib.lib().moe_capacity(T, E, float(capacity_factor))
    if c < -1:
        check("moe_capacity", c)
    return c


def moe_workspace_size(desc: MoeDesc) -> int:
    n = _lib.lib().moe_workspace_size(ctypes.byref(desc))
    if n == 0:
        raise _lib.MoeError("moe_workspace_size", _lib.MOE_ERR_INVALID_ARG)
    return n


def moe_gemm_variant(desc: MoeDesc, up: bool) -> int:
    """Internal id of the grouped-GEMM kernel the up (or down) projection
    runs for this descriptor (diagnostics, benchmark reports)."""
    v = _lib.lib().moe_gemm_variant(ctypes.byref(desc), 1 if up else 0)
    check("moe_gemm_variant", min(v, 0))
    return v


def moe_gemm_tail_split(desc: MoeDesc, up: bool) -> int:
    """K ranges per half-height tile of the four-wave 256-row GEMM for the
    up (or down) projection (1: no split, or another kernel runs)."""
    v = _lib.lib().moe_gemm_tail_split(ctypes.byref(desc), 1 if up else 0)
    check("moe_gemm_tail_split", min(v, 0))
    return v


def _codes(t):
    """float8_e4m3fn tensors are passed as their uint8 codes."""
    if t is not None and t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8)
    return t


class Weights:
    """Device weight tensors of one layer (see module docstring).  The
    expert matrices are FP8 when given as uint8 / float8_e4m3fn codes, and
    then need their scales."""

    def __init__(self, w_router, w1, w2, b_router=None, expert_bias=None,
                 b1=None, b2=None, ws1=None, bs1=None, ws2=None, bs2=None,
                 w1_scale=None, w2_scale=None, ws1_scale=None,
                 ws2_scale=None, w3=None, b3=None, ws3=None, bs3=None,
                 w3_scale=None, ws3_scale=None):
        w1, w2, ws1, ws2 = _codes(w1), _codes(w2), _codes(ws1), _codes(ws2)
        w3, ws3 = _codes(w3), _codes(ws3)
        self.w3, self.b3, self.ws3, self.bs3 = w3, b3, ws3, bs3
        self.w3_scale, self.ws3_scale = w3_scale, ws3_scale
        self.gated = w3 is not None
        self.w_router, self.w1, self.w2 = w_router, w1, w2
        self.b_router, self.expert_bias = b_router, expert_bias
        self.b1, self.b2 = b1, b2
        self.ws1, self.bs1, self.ws2, self.bs2 = ws1, bs1, ws2, bs2
        self.w1_scale, self.w2_scale = w1_scale, w2_scale
        self.ws1_scale, self.ws2_scale = ws1_scale, ws2_scale
        E, d_ff, d = w1.shape
        self.E, self.d, self.d_ff = E, d, d_ff
        self.dtype = w_router.dtype
        self.device = w1.device
        self.n_shared = 0 if ws1 is None else 1
        self.expert_fp8 = w1.dtype == torch.uint8
        dt, dev = self.dtype, self.device
        wdt = torch.uint8 if self.expert_fp8 else dt
        f32 = torch.float32
        _need(w_router, "w_router", (E, d), dt, dev)
        _need(w1, "w1", (E, d_ff, d), wdt, dev)
        _need(w2, "w2", (E, d, d_ff), wdt, dev)
        _opt(b_router, "b_router", (E,), f32, dev)
        _opt(expert_bias, "expert_bias", (E,), f32, dev)
        _opt(b1, "b1", (E, d_ff), dt, dev)
        _opt(b2, "b2", (E, d), dt, dev)
        if self.expert_fp8:
            _need(w1_scale, "w1_scale", (E, d_ff), f32, dev)
            _need(w2_scale, "w2_scale", (E, d), f32, dev)
        if self.gated:
            _need(w3, "w3", (E, d_ff, d), wdt, dev)
            _opt(b3, "b3", (E, d_ff), dt, dev)
            if self.expert_fp8:
                _need(w3_scale, "w3_scale", (E, d_ff), f32, dev)
        if self.n_shared:
            _need(ws1, "ws1", (d_ff, d), wdt, dev)
            _need(ws2, "ws2", (d, d_ff), wdt, dev)
            _opt(bs1, "bs1", (d_ff,), dt, dev)
            _opt(bs2, "bs2", (d,), dt, dev)
            if self.expert_fp8:
                _need(ws1_scale, "ws1_scale", (d_ff,), f32, dev)
                _need(ws2_scale, "ws2_scale", (d,), f32, dev)
            if self.gated:
                _need(ws3, "ws3", (d_ff, d), wdt, dev)
                _opt(bs3, "bs3", (d_ff,), dt, dev)
                if self.expert_fp8:
                    _need(ws3_scale, "ws3_scale", (d_ff,), f32, dev)

    @staticmethod
    def from_dict(inp: dict, device=None) -> "Weights":
        def g(key):
            t = inp.get(key)
            if t is None:
                return None
            return t.to(device).contiguous() if device is not None else t
        return Weights(g("wr"), g("w1"), g("w2"), b_router=g("br"),
                       expert_bias=g("ebias"), b1=g("b1"), b2=g("b2"),
                       ws1=g("ws1"), bs1=g("bs1"), ws2=g("ws2"),
                       bs2=g("bs2"), w1_scale=g("w1_scale"),
                       w2_scale=g("w2_scale"), ws1_scale=g("ws1_scale"),
                       ws2_scale=g("ws2_scale"), w3=g("w3"), b3=g("b3"),
                       ws3=g("ws3"), bs3=g("bs3"), w3_scale=g("w3_scale"),
                       ws3_scale=g("ws3_scale"))

    def struct(self) -> MoeWeights:
        return MoeWeights(*[_ptr(t) for t in (
            self.w_router, self.b_router, self.expert_bias, self.w1, self.b1,
            self.w2, self.b2, self.ws1, self.bs1, self.ws2, self.bs2,
            self.w1_scale, self.w2_scale, self.ws1_scale, self.ws2_scale,
            self.w3, self.b3, self.ws3, self.bs3, self.w3_scale,
            self.ws3_scale)])


class Routing:
    """Device buffers of the routing results and statistics (k = E for
    expert choice)."""

    def __init__(self, T: int, E: int, k: int, device,
                 slots: Optional[int] = None):
        """``slots``: length of slot_token, T*k by default (expert choice
        uses E*C)."""
        i32, f32 = torch.int32, torch.float32
        z = lambda *s, dt: torch.empty(s, dtype=dt, device=device)
        self.topk_idx = z(T, k, dt=i32)
        self.topk_w = z(T, k, dt=f32)
        self.counts = z(E, dt=i32)
        self.kept = z(E, dt=i32)
        self.offsets = z(E + 1, dt=i32)
        self.slot_token = z(T * k if slots is None else slots, dt=i32)
        self.slot_of = z(T, k, dt=i32)
        self.f = z(E, dt=f32)
        self.p = z(E, dt=f32)
        self.l_aux = z(1, dt=f32)
        # z-loss, entropy (bits), load imbalance, utilization, drop rate,
        # max share
        self.monitor = z(6, dt=f32)

    def struct(self) -> MoeRouting:
        return MoeRouting(*[_ptr(getattr(self, n)) for n, _ in
                            MoeRouting._fields_])


def _ws(desc, ws: torch.Tensor):
    need = moe_workspace_size(desc)
    if ws.numel() * ws.element_size() < need or not ws.is_contiguous():
        raise ValueError(f"workspace needs {need} contiguous bytes")
    return ws.data_ptr(), ws.numel() * ws.element_size()


def moe_router_topk(desc, x, w: Weights, r: Routing, ws) -> None:
    _need(x, "x", (desc.T, desc.d), w.dtype, w.device)
    p, n = _ws(desc, ws)
    rs, wsct = r.struct(), w.struct()
    check("moe_router_topk", _lib.lib().moe_router_topk(
        ctypes.byref(desc), x.data_ptr(), ctypes.byref(wsct),
        ctypes.byref(rs), p, n, _stream(x)))


def moe_permute(desc, r: Routing, ws) -> None:
    p, n = _ws(desc, ws)
    rs = r.struct()
    check("moe_permute", _lib.lib().moe_permute(
        ctypes.byref(desc), ctypes.byref(rs), p, n, _stream(ws)))


def moe_route_dispatch(desc, x, w: Weights, r: Routing, ws) -> None:
    """moe_router_topk + moe_permute (one launch for decode-sized steps)."""
    _need(x, "x", (desc.T, desc.d), w.dtype, w.device)
    p, n = _ws(desc, ws)
    rs, wsct = r.struct(), w.struct()
    check("moe_route_dispatch", _lib.lib().moe_route_dispatch(
        ctypes.byref(desc), x.data_ptr(), ctypes.byref(wsct),
        ctypes.byref(rs), p, n, _stream(x)))


def moe_grouped_ffn(desc, x, w: Weights, r: Routing, ws) -> None:
    _need(x, "x", (desc.T, desc.d), w.dtype, w.device)
    p, n = _ws(desc, ws)
    rs, wsct = r.struct(), w.struct()
    check("moe_grouped_ffn", _lib.lib().moe_grouped_ffn(
        ctypes.byref(desc), x.data_ptr(), ctypes.byref(wsct),
        ctypes.byref(rs), p, n, _stream(x)))


def moe_ffn_up(desc, x, w: Weights, r: Routing, ws) -> None:
    _need(x, "x", (desc.T, desc.d), w.dtype, w.device)
    p, n = _ws(desc, ws)
    rs, wsct = r.struct(), w.struct()
    check("moe_ffn_up", _lib.lib().moe_ffn_up(
        ctypes.byref(desc), x.data_ptr(), ctypes.byref(wsct),
        ctypes.byref(rs), p, n, _stream(x)))


def moe_ffn_down(desc, w: Weights, r: Routing, ws) -> None:
    p, n = _ws(desc, ws)
    rs, wsct = r.struct(), w.struct()
    check("moe_ffn_down", _lib.lib().moe_ffn_down(
        ctypes.byref(desc), ctypes.byref(wsct), ctypes.byref(rs), p, n,
        _stream(ws)))


def moe_combine(desc, r: Routing, y, ws) -> None:
    _need(y, "y", (desc.T, desc.d), y.dtype, ws.device)
    p, n = _ws(desc, ws)
    rs = r.struct()
    check("moe_combine", _lib.lib().moe_combine(
        ctypes.byref(desc), ctypes.byref(rs), y.data_ptr(), p, n,
        _stream(y)))


def moe_forward(desc, x, w: Weights, r: Routing, y, ws) -> None:
    _need(x, "x", (desc.T, desc.d), w.dtype, w.device)
    _need(y, "y", (desc.T, desc.d), w.dtype, w.device)
    p, n = _ws(desc, ws)
    rs, wsct = r.struct(), w.struct()
    check("moe_forward", _lib.lib().moe_forward(
        ctypes.byref(desc), x.data_ptr(), ctypes.byref(wsct),
        ctypes.byref(rs), y.data_ptr(), p, n, _stream(x)))


def moe_forward_noalloc(desc, x, w: Weights, r: Routing, y) -> None:
    """moe_forward with the library's static device scratch instead of a
    workspace (no allocation; raises MoeError with MOE_ERR_SCRATCH when the
    shape needs more than the static buffer)."""
    _need(x, "x", (desc.T, desc.d), w.dtype, w.device)
    _need(y, "y", (desc.T, desc.d), w.dtype, w.device)
    rs, wsct = r.struct(), w.struct()
    check("moe_forward_noalloc", _lib.lib().moe_forward_noalloc(
        ctypes.byref(desc), x.data_ptr(), ctypes.byref(wsct),
        ctypes.byref(rs), y.data_ptr(), _stream(x)))


def moe_bias_update(counts, target: float, gamma: float,
                    expert_bias) -> None:
    E = expert_bias.numel()
    if counts.dtype != torch.int32 or counts.numel() != E:
        raise ValueError("counts must be int32 [E]")
    if expert_bias.dtype != torch.float32 or not expert_bias.is_contiguous():
        raise ValueError("expert_bias must be contiguous float32 [E]")
    check("moe_bias_update", _lib.lib().moe_bias_update(
        E, counts.data_ptr(), float(target), float(gamma),
        expert_bias.data_ptr(), _stream(expert_bias)))


class MoeLayer:
    """One sparse MoE FFN layer on a GPU: weights plus reusable buffers.

    ``routing="topk"``: each token picks ``k`` experts, with an optional
    capacity floor(T/E * capacity_factor).  ``routing="expert_choice"``:
    each expert picks floor(T/E * capacity_factor) tokens (``k`` is then E
    and a capacity factor is required).  ``activation``: "gelu", "silu",
    or "swiglu" (the default when the weights carry w3).

    ``forward(x)`` returns ``(y, routing)``; the routing buffers are reused
    by the next call with the same T (copy them to keep them)."""

    def __init__(self, weights: Weights, k: int,
                 capacity_factor: Optional[float] = None,
                 aux_alpha: float = 0.01, routing: str = "topk",
                 activation: Optional[str] = None):
        if routing not in _ROUTING:
            raise ValueError(f"unknown routing {routing!r}")
        if activation is None:
            activation = "swiglu" if weights.gated else "gelu"
        if (activation == "swiglu") != weights.gated:
            raise ValueError("swiglu needs w3, and w3 needs swiglu")
        self.activation = activation
        if routing == "expert_choice":
            if capacity_factor is None:
                raise ValueError("expert choice needs a capacity factor")
            k = weights.E
        self.w = weights
        self.k = k
        self.capacity_factor = capacity_factor
        self.aux_alpha = aux_alpha
        self.routing = routing
        self._bufs = {}

    def desc(self, T: int) -> MoeDesc:
        w = self.w
        cap = moe_capacity(T, w.E, self.capacity_factor)
        if self.routing == "expert_choice":
            cap = min(cap, T)
        return make_desc(T, w.d, w.E, self.k, w.d_ff, w.dtype,
                         n_shared=w.n_shared, capacity=cap,
                         aux_alpha=self.aux_alpha, routing=self.routing,
                         expert_fp8=w.expert_fp8, activation=self.activation)

    def buffers(self, T: int):
        if T not in self._bufs:
            desc = self.desc(T)
            nbytes = moe_workspace_size(desc)
            ws = torch.empty(nbytes, dtype=torch.uint8, device=self.w.device)
            slots = None
            if self.routing == "expert_choice":
                slots = self.w.E * desc.capacity
            r = Routing(T, self.w.E, self.k, self.w.device, slots=slots)
            y = torch.empty((T, self.w.d), dtype=self.w.dtype,
                            device=self.w.device)
            self._bufs[T] = (desc, r, ws, y)
        return self._bufs[T]

    def forward(self, x: torch.Tensor):
        if x.dim() == 3:                    # (B, S, H) -> (B*S, H)
            shape = x.shape
            y, r = self.forward(x.reshape(-1, shape[-1]))
            return y.reshape(shape), r
        desc, r, ws, y = self.buffers(x.shape[0])
        moe_forward(desc, x.contiguous(), self.w, r, y, ws)
        return y, r

    def bias_update(self, routing: Routing, gamma: float) -> None:
        """One aux-loss-free step on weights.expert_bias from the counts of
        the last forward: target is T*k/E."""
        if self.w.expert_bias is None:
            raise ValueError("layer has no expert_bias")
        T = routing.topk_idx.shape[0]
        moe_bias_update(routing.counts, T * self.k / self.w.E, gamma,
                        self.w.expert_bias)
