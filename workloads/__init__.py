"""Seeded synthetic workloads for the sparse MoE FFN layer forward.

This module only describes shapes and draws random inputs.  It holds none of
the layer's arithmetic (no routing, no capacity formula, no FFN): the HIP
library and the CPU oracle each compute those on their own.  Both sides are
handed the very same tensors produced here.

Distributions.  ``N(0, v)`` in a workload description is read with ``v`` as
the variance, so ``N(0, 1/fan_in)`` draws with standard deviation
``fan_in ** -0.5``.  Every tensor is drawn in float32 from its own
``torch.Generator`` stream, seeded from ``(seed, tag, index)`` so that any
tensor (for example one expert's weights) can be regenerated alone, then
rounded to the workload dtype (round-to-nearest-even for bfloat16).

The five named workloads follow the layer shapes of the models the pages
discuss: a tiny top-2 layer, a Switch-style top-1 layer with an expert
capacity, Mixtral-8x7B-shaped prefill and decode, and a DeepSeek-V3-shaped
fine-grained layer with one shared expert and a per-expert balancing bias.
"""
from __future__ import annotations

import dataclasses
import zlib
from typing import Dict, Optional

import torch

__all__ = ["Workload", "WORKLOADS", "get", "scaled", "make_inputs", "make_x",
           "make_expert", "tensor_seed"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int                      # tokens in one call
    d: int                      # model width
    E: int                      # routed experts
    k: int                      # experts per token
    d_ff: int                   # expert hidden width
    dtype: str                  # "f32" or "bf16" (x, weights, y)
    n_shared: int = 0           # 0 or 1 always-on shared expert
    capacity_factor: Optional[float] = None   # None = no capacity limit
    alpha: float = 0.01         # auxiliary-loss coefficient
    router_var: Optional[float] = None        # None = 1/d
    router_bias: str = "none"   # "none" | "linear" (nn.Linear bias) | "skew"
    skew_var: float = 1.0       # variance of the fixed per-expert logit skew
    expert_bias: str = "none"   # "none" | "zipf" (subtracted balancing bias)
    zipf_s: float = 1.1
    zipf_scale: float = 0.5
    linear_biases: bool = False  # expert Linear biases b1, b2
    bias_var: float = 0.01       # variance of every Linear bias
    bias_update_gamma: Optional[float] = None  # one balancing-bias step
    calls: int = 1              # distinct x per timed run (decode)
    routing: str = "topk"       # "topk" | "expert_choice" (then k == E)
    expert_fp8: bool = False    # expert matrices stored as E4M3 + scales
    activation: str = "gelu"    # "gelu" | "silu" | "swiglu" (adds W3, b3)
    seed: int = 0

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


WORKLOADS: Dict[str, Workload] = {
    # T = 2 x 128 tokens, fp32, top-2 of 8, biases on the router and experts.
    "tiny_top2_f32": Workload(
        name="tiny_top2_f32", T=256, d=64, E=8, k=2, d_ff=256, dtype="f32",
        router_bias="linear", linear_biases=True),
    # Switch-style top-1 with capacity floor(T/E * 1.25); skewed logits.
    "switch_top1_cap": Workload(
        name="switch_top1_cap", T=8192, d=768, E=64, k=1, d_ff=3072,
        dtype="bf16", capacity_factor=1.25, router_bias="skew", skew_var=1.0),
    # Mixtral-8x7B-shaped prefill: 4 x 1024 tokens.
    "mixtral_prefill": Workload(
        name="mixtral_prefill", T=4096, d=4096, E=8, k=2, d_ff=14336,
        dtype="bf16", router_var=0.02),
    # Mixtral-8x7B-shaped decode: 32 tokens per call, 200 distinct calls.
    "mixtral_decode": Workload(
        name="mixtral_decode", T=32, d=4096, E=8, k=2, d_ff=14336,
        dtype="bf16", router_var=0.02, calls=200),
    # DeepSeek-V3-shaped: 256 routed + 1 shared expert, top-8, Zipf bias.
    "deepseek_v3": Workload(
        name="deepseek_v3", T=8192, d=7168, E=256, k=8, d_ff=2048,
        dtype="bf16", n_shared=1, expert_bias="zipf", bias_update_gamma=0.001),
    # Mixtral-8x7B-shaped decode with E4M3 expert weights (per-channel
    # scales): half the weight bytes of the bf16 layer.
    "mixtral_decode_fp8": Workload(
        name="mixtral_decode_fp8", T=32, d=4096, E=8, k=2, d_ff=14336,
        dtype="bf16", router_var=0.02, calls=200, expert_fp8=True),
    # Mixtral-8x7B's gated expert (SwiGLU: W2 (SiLU(W1 x) * W3 x)), prefill
    # and decode shapes.
    "mixtral_prefill_swiglu": Workload(
        name="mixtral_prefill_swiglu", T=4096, d=4096, E=8, k=2, d_ff=14336,
        dtype="bf16", router_var=0.02, activation="swiglu"),
    "mixtral_decode_swiglu": Workload(
        name="mixtral_decode_swiglu", T=32, d=4096, E=8, k=2, d_ff=14336,
        dtype="bf16", router_var=0.02, calls=200, activation="swiglu"),
    # Expert choice: each of 64 experts picks C = floor(T/E * 2) = 256
    # tokens, the compute of top-2 routing on the Switch-sized layer.
    "expert_choice_c2": Workload(
        name="expert_choice_c2", T=8192, d=768, E=64, k=64, d_ff=3072,
        dtype="bf16", capacity_factor=2.0, router_bias="skew", skew_var=1.0,
        routing="expert_choice"),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def scaled(w: Workload, **changes) -> Workload:
    """A copy of ``w`` with some fields changed (smaller parity cases)."""
    return dataclasses.replace(w, **changes)


def tensor_seed(seed: int, tag: str, index: int = 0) -> int:
    """Seed of one tensor's private random stream."""
    return zlib.crc32(f"{seed}:{tag}:{index}".encode()) & 0x7FFFFFFF


def _gen(device) -> torch.Generator:
    return torch.Generator(device=torch.device(device))


def _normal(shape, var, seed, tag, index, device, dtype, chunk_rows=None):
    """float32 N(0, var) draws rounded to ``dtype``."""
    g = _gen(device)
    g.manual_seed(tensor_seed(seed, tag, index))
    std = float(var) ** 0.5
    if chunk_rows is None:
        t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        return (t * std).to(dtype)
    out = torch.empty(shape, device=device, dtype=dtype)
    rows = shape[0]
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        t = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=g,
                        device=device, dtype=torch.float32)
        out[r0:r1] = (t * std).to(dtype)
    return out


def make_x(w: Workload, device="cpu", call: int = 0) -> torch.Tensor:
    """Activations x[T, d] ~ N(0, 1); call i of a multi-call run uses its own
    stream (seed offset 1 + i)."""
    return _normal((w.T, w.d), 1.0, w.seed + call, "x", call, device,
                   w.torch_dtype)


def make_expert(w: Workload, e: int, device="cpu", shared: bool = False):
    """One expert's (W1[d_ff,d], b1[d_ff] | None, W2[d,d_ff], b2[d] | None).
    ``shared`` selects the shared expert's own streams."""
    tag = "s" if shared else "r"
    dt = w.torch_dtype
    w1 = _normal((w.d_ff, w.d), 1.0 / w.d, w.seed, tag + "w1", e, device, dt)
    w2 = _normal((w.d, w.d_ff), 1.0 / w.d_ff, w.seed, tag + "w2", e, device,
                 dt)
    b1 = b2 = None
    if w.linear_biases:
        b1 = _normal((w.d_ff,), w.bias_var, w.seed, tag + "b1", e, device, dt)
        b2 = _normal((w.d,), w.bias_var, w.seed, tag + "b2", e, device, dt)
    return w1, b1, w2, b2


def make_expert_up3(w: Workload, e: int, device="cpu", shared: bool = False):
    """The SwiGLU up projection of one expert: (W3[d_ff,d], b3[d_ff] | None),
    from streams of its own."""
    tag = "s" if shared else "r"
    w3 = _normal((w.d_ff, w.d), 1.0 / w.d, w.seed, tag + "w3", e, device,
                 w.torch_dtype)
    b3 = None
    if w.linear_biases:
        b3 = _normal((w.d_ff,), w.bias_var, w.seed, tag + "b3", e, device,
                     w.torch_dtype)
    return w3, b3


def quantize_e4m3(wt: torch.Tensor):
    """Checkpoint conversion of one [N, K] matrix to FP8: per-row scale
    amax / 448 (1 for an all-zero row) and E4M3 codes of w / scale by
    torch's float8_e4m3fn cast (round to nearest even).  Returns (uint8
    codes, float32 scales)."""
    wf = wt.to(torch.float32)
    amax = wf.abs().amax(dim=1)
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (wf / scale[:, None]).to(torch.float8_e4m3fn).view(torch.uint8)
    return q, scale


def make_router(w: Workload, device="cpu"):
    """Router weight Wr[E, d] plus the float32 additive logit term (the
    router Linear bias, or a fixed per-expert skew) and the float32
    subtracted balancing bias, each None when the workload has none."""
    var = w.router_var if w.router_var is not None else 1.0 / w.d
    wr = _normal((w.E, w.d), var, w.seed, "wr", 0, device, w.torch_dtype)
    br = None
    if w.router_bias == "linear":
        br = _normal((w.E,), w.bias_var, w.seed, "br", 0, device,
                     torch.float32)
    elif w.router_bias == "skew":
        br = _normal((w.E,), w.skew_var, w.seed, "skew", 0, device,
                     torch.float32)
    ebias = None
    if w.expert_bias == "zipf":
        g = _gen("cpu")
        g.manual_seed(tensor_seed(w.seed, "zipf_perm", 0))
        perm = torch.randperm(w.E, generator=g)
        ranks = torch.arange(1, w.E + 1, dtype=torch.float64)
        vals = (w.zipf_scale * ranks.pow(-w.zipf_s)).to(torch.float32)
        ebias = torch.empty(w.E, dtype=torch.float32)
        ebias[perm] = vals
        ebias = ebias.to(device)
    return wr, br, ebias


def make_inputs(w: Workload, device="cpu", call: int = 0) -> dict:
    """All tensors of one layer call, stacked per expert:
    x[T,d]; wr[E,d]; br[E] f32|None; ebias[E] f32|None;
    w1[E,d_ff,d]; b1[E,d_ff]|None; w2[E,d,d_ff]; b2[E,d]|None;
    ws1, bs1, ws2, bs2 for the shared expert (None when absent)."""
    dt = w.torch_dtype
    out = {"x": make_x(w, device, call)}
    out["wr"], out["br"], out["ebias"] = make_router(w, device)
    if w.expert_fp8:
        return _fp8_experts(w, device, out)
    w1 = torch.empty((w.E, w.d_ff, w.d), device=device, dtype=dt)
    w2 = torch.empty((w.E, w.d, w.d_ff), device=device, dtype=dt)
    b1 = torch.empty((w.E, w.d_ff), device=device, dtype=dt) \
        if w.linear_biases else None
    b2 = torch.empty((w.E, w.d), device=device, dtype=dt) \
        if w.linear_biases else None
    for e in range(w.E):
        e1, eb1, e2, eb2 = make_expert(w, e, device)
        w1[e].copy_(e1)
        w2[e].copy_(e2)
        if b1 is not None:
            b1[e].copy_(eb1)
            b2[e].copy_(eb2)
        del e1, e2
    out.update(w1=w1, b1=b1, w2=w2, b2=b2)
    if w.activation == "swiglu":
        w3 = torch.empty((w.E, w.d_ff, w.d), device=device, dtype=dt)
        b3 = torch.empty((w.E, w.d_ff), device=device, dtype=dt) \
            if w.linear_biases else None
        for e in range(w.E):
            e3, eb3 = make_expert_up3(w, e, device)
            w3[e].copy_(e3)
            if b3 is not None:
                b3[e].copy_(eb3)
        out.update(w3=w3, b3=b3)
    if w.n_shared:
        s1, sb1, s2, sb2 = make_expert(w, 0, device, shared=True)
        out.update(ws1=s1, bs1=sb1, ws2=s2, bs2=sb2)
        if w.activation == "swiglu":
            s3, sb3 = make_expert_up3(w, 0, device, shared=True)
            out.update(ws3=s3, bs3=sb3)
    else:
        out.update(ws1=None, bs1=None, ws2=None, bs2=None)
    return out


def _fp8_experts(w: Workload, device, out: dict) -> dict:
    """The expert part of make_inputs for FP8 workloads: the layer-dtype
    weights of make_expert, converted by quantize_e4m3 (adds w1_scale,
    w2_scale and, with a shared expert, ws1_scale, ws2_scale)."""
    dt = w.torch_dtype
    u8, f32 = torch.uint8, torch.float32
    w1 = torch.empty((w.E, w.d_ff, w.d), device=device, dtype=u8)
    w2 = torch.empty((w.E, w.d, w.d_ff), device=device, dtype=u8)
    s1 = torch.empty((w.E, w.d_ff), device=device, dtype=f32)
    s2 = torch.empty((w.E, w.d), device=device, dtype=f32)
    b1 = torch.empty((w.E, w.d_ff), device=device, dtype=dt) \
        if w.linear_biases else None
    b2 = torch.empty((w.E, w.d), device=device, dtype=dt) \
        if w.linear_biases else None
    for e in range(w.E):
        e1, eb1, e2, eb2 = make_expert(w, e, device)
        q, s = quantize_e4m3(e1)
        w1[e].copy_(q)
        s1[e].copy_(s)
        q, s = quantize_e4m3(e2)
        w2[e].copy_(q)
        s2[e].copy_(s)
        if b1 is not None:
            b1[e].copy_(eb1)
            b2[e].copy_(eb2)
        del e1, e2, q
    out.update(w1=w1, b1=b1, w2=w2, b2=b2, w1_scale=s1, w2_scale=s2)
    if w.activation == "swiglu":
        w3 = torch.empty((w.E, w.d_ff, w.d), device=device, dtype=u8)
        s3 = torch.empty((w.E, w.d_ff), device=device, dtype=f32)
        b3 = torch.empty((w.E, w.d_ff), device=device, dtype=dt) \
            if w.linear_biases else None
        for e in range(w.E):
            e3, eb3 = make_expert_up3(w, e, device)
            q, sc = quantize_e4m3(e3)
            w3[e].copy_(q)
            s3[e].copy_(sc)
            if b3 is not None:
                b3[e].copy_(eb3)
        out.update(w3=w3, b3=b3, w3_scale=s3)
    if w.n_shared:
        e1, sb1, e2, sb2 = make_expert(w, 0, device, shared=True)
        q1, t1 = quantize_e4m3(e1)
        q2, t2 = quantize_e4m3(e2)
        out.update(ws1=q1, bs1=sb1, ws2=q2, bs2=sb2, ws1_scale=t1,
                   ws2_scale=t2)
        if w.activation == "swiglu":
            e3, sb3 = make_expert_up3(w, 0, device, shared=True)
            q3, t3 = quantize_e4m3(e3)
            out.update(ws3=q3, bs3=sb3, ws3_scale=t3)
    else:
        out.update(ws1=None, bs1=None, ws2=None, bs2=None)
    return out
