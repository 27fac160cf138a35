"""The C-ABI library on a host without a GPU: it loads, exports every
entry point that include/moe.h declares, and rejects bad arguments before
any HIP call (so these run on the CPU)."""
import ctypes
import os
import re

import pytest

import sparse_mixture_experts_50_amd as moe
from sparse_mixture_experts_50_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

FAKE = 0x1000      # never dereferenced: every call below fails validation


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(moe_[a-z_]+)\s*\(", text)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("moe_router_topk", "moe_permute", "moe_grouped_ffn",
                     "moe_combine", "moe_forward"):
        assert required in names


def test_library_exports_every_declared_symbol():
    L = _lib.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert set(declared_functions()) == set(_lib.SIGNATURES)


def test_version_and_status_strings():
    L = _lib.lib()
    assert L.moe_version().startswith(b"moe-gfx950")
    assert L.moe_status_string(0) == b"ok"
    assert L.moe_status_string(-3).startswith(b"workspace")
    assert L.moe_status_string(123) == b"unknown status"


def test_capacity_formula():
    L = _lib.lib()
    assert L.moe_capacity(8192, 64, 1.25) == 160
    assert L.moe_capacity(100, 8, 1.25) == 15
    assert L.moe_capacity(7, 8, 1.0) == 0
    assert L.moe_capacity(10, 2, -1.0) == -1
    assert L.moe_capacity(-1, 2, 1.0) == _lib.MOE_ERR_INVALID_ARG
    assert L.moe_capacity(10, 0, 1.0) == _lib.MOE_ERR_INVALID_ARG


def desc(**kw):
    base = dict(T=64, d=128, E=8, k=2, d_ff=256, n_shared=0, dtype=1,
                capacity=-1, aux_alpha=0.01)
    base.update(kw)
    return _lib.MoeDesc(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), _lib.MOE_ERR_INVALID_ARG),
    (dict(k=0), _lib.MOE_ERR_INVALID_ARG),
    (dict(k=9), _lib.MOE_ERR_INVALID_ARG),
    (dict(E=0), _lib.MOE_ERR_INVALID_ARG),
    (dict(n_shared=2), _lib.MOE_ERR_INVALID_ARG),
    (dict(capacity=-2), _lib.MOE_ERR_INVALID_ARG),
    (dict(dtype=7), _lib.MOE_ERR_UNSUPPORTED),
    (dict(d=100), _lib.MOE_ERR_UNSUPPORTED),
    (dict(d_ff=96), _lib.MOE_ERR_UNSUPPORTED),
    (dict(E=300, k=2), _lib.MOE_ERR_UNSUPPORTED),
    (dict(E=128, k=65), _lib.MOE_ERR_UNSUPPORTED),
    (dict(routing=2), _lib.MOE_ERR_INVALID_ARG),
    # expert choice: k must be E, 0 <= capacity <= T
    (dict(routing=1, k=2, capacity=16), _lib.MOE_ERR_INVALID_ARG),
    (dict(routing=1, k=8, capacity=-1), _lib.MOE_ERR_INVALID_ARG),
    (dict(routing=1, k=8, capacity=65), _lib.MOE_ERR_INVALID_ARG),
    # FP8 expert weights: bf16 layers with d, d_ff multiples of 1024
    (dict(expert_fp8=2), _lib.MOE_ERR_INVALID_ARG),
    (dict(expert_fp8=1, d=1024, d_ff=1024, dtype=0), _lib.MOE_ERR_UNSUPPORTED),
    (dict(expert_fp8=1, d=512, d_ff=1024), _lib.MOE_ERR_UNSUPPORTED),
    (dict(expert_fp8=1, d=1024, d_ff=1536), _lib.MOE_ERR_UNSUPPORTED),
    # activations: gelu, silu, swiglu; gated bf16 needs d_ff % 128 == 0
    (dict(activation=3), _lib.MOE_ERR_INVALID_ARG),
    (dict(activation=2, d_ff=192), _lib.MOE_ERR_UNSUPPORTED),
])
def test_descriptor_rejected_before_any_launch(kw, status):
    L = _lib.lib()
    d = desc(**kw)
    assert L.moe_workspace_size(ctypes.byref(d)) == 0
    w = _lib.MoeWeights(FAKE, None, None, FAKE, None, FAKE, None,
                        None, None, None, None)
    r = _lib.MoeRouting(*([FAKE] * 10))
    rc = L.moe_forward(ctypes.byref(d), FAKE, ctypes.byref(w),
                       ctypes.byref(r), FAKE, FAKE, 1 << 40, None)
    assert rc == status


def test_null_pointers_and_workspace():
    L = _lib.lib()
    d = desc()
    ws = L.moe_workspace_size(ctypes.byref(d))
    assert ws > 0
    w = _lib.MoeWeights(FAKE, None, None, FAKE, None, FAKE, None,
                        None, None, None, None)
    r = _lib.MoeRouting(*([FAKE] * 10))
    # missing x / y
    assert L.moe_forward(ctypes.byref(d), None, ctypes.byref(w),
                         ctypes.byref(r), FAKE, FAKE, ws, None) == -1
    assert L.moe_forward(ctypes.byref(d), FAKE, ctypes.byref(w),
                         ctypes.byref(r), None, FAKE, ws, None) == -1
    # missing weights
    w2 = _lib.MoeWeights(FAKE, None, None, None, None, FAKE, None,
                         None, None, None, None)
    assert L.moe_forward(ctypes.byref(d), FAKE, ctypes.byref(w2),
                         ctypes.byref(r), FAKE, FAKE, ws, None) == -1
    # shared expert declared but absent
    ds = desc(n_shared=1)
    wss = L.moe_workspace_size(ctypes.byref(ds))
    assert L.moe_forward(ctypes.byref(ds), FAKE, ctypes.byref(w),
                         ctypes.byref(r), FAKE, FAKE, wss, None) == -1
    # missing routing buffer
    r2 = _lib.MoeRouting(*([FAKE] * 9 + [None]))
    assert L.moe_permute(ctypes.byref(d), ctypes.byref(r2), FAKE, ws,
                         None) == -1
    # workspace too small / absent
    assert L.moe_forward(ctypes.byref(d), FAKE, ctypes.byref(w),
                         ctypes.byref(r), FAKE, FAKE, ws - 1, None) == -3
    assert L.moe_forward(ctypes.byref(d), FAKE, ctypes.byref(w),
                         ctypes.byref(r), FAKE, None, ws, None) == -3
    assert L.moe_bias_update(0, FAKE, 1.0, 0.001, FAKE, None) == -1
    assert L.moe_bias_update(8, None, 1.0, 0.001, FAKE, None) == -1


def test_zero_tokens_is_a_no_op():
    L = _lib.lib()
    d = desc(T=0)
    ws = L.moe_workspace_size(ctypes.byref(d))
    assert ws > 0
    w = _lib.MoeWeights(FAKE, None, None, FAKE, None, FAKE, None,
                        None, None, None, None)
    r = _lib.MoeRouting(*([FAKE] * 10))
    for fn, args in [
        ("moe_forward", (FAKE, ctypes.byref(w), ctypes.byref(r), FAKE, FAKE,
                         ws, None)),
        ("moe_router_topk", (FAKE, ctypes.byref(w), ctypes.byref(r), FAKE,
                             ws, None)),
        ("moe_permute", (ctypes.byref(r), FAKE, ws, None)),
        ("moe_grouped_ffn", (FAKE, ctypes.byref(w), ctypes.byref(r), FAKE,
                             ws, None)),
        ("moe_combine", (ctypes.byref(r), FAKE, FAKE, ws, None)),
    ]:
        assert getattr(L, fn)(ctypes.byref(d), *args) == 0, fn


def test_workspace_grows_with_tokens():
    L = _lib.lib()
    a = L.moe_workspace_size(ctypes.byref(desc(T=64)))
    b = L.moe_workspace_size(ctypes.byref(desc(T=4096)))
    c = L.moe_workspace_size(ctypes.byref(desc(T=4096, n_shared=1)))
    assert 0 < a < b < c


def test_expert_choice_descriptor_and_workspace():
    L = _lib.lib()
    # k = E = 128 > 64 is fine for expert choice
    big = desc(routing=1, E=128, k=128, capacity=16)
    assert L.moe_workspace_size(ctypes.byref(big)) > 0
    # the routed rows are E*C, not T*k: fewer than top-k with k = E
    a = L.moe_workspace_size(ctypes.byref(desc(routing=1, k=8, capacity=16)))
    b = L.moe_workspace_size(ctypes.byref(desc(routing=1, k=8, capacity=32)))
    assert 0 < a < b
    assert L.moe_workspace_size(ctypes.byref(desc(k=8))) > b
    # topk_idx is not needed by the expert-choice permute, but T = 0 is
    # still a no-op and a missing slot map is still rejected
    d = desc(routing=1, k=8, capacity=16)
    ws = L.moe_workspace_size(ctypes.byref(d))
    r = _lib.MoeRouting(*([FAKE] * 6 + [None] + [FAKE] * 3))
    assert L.moe_permute(ctypes.byref(d), ctypes.byref(r), FAKE, ws,
                         None) == -1


def test_fp8_needs_scales():
    L = _lib.lib()
    d = desc(expert_fp8=1, d=1024, d_ff=1024)
    ws = L.moe_workspace_size(ctypes.byref(d))
    assert ws > 0
    r = _lib.MoeRouting(*([FAKE] * 10))
    no_scale = _lib.MoeWeights(FAKE, None, None, FAKE, None, FAKE, None,
                               None, None, None, None)
    assert L.moe_forward(ctypes.byref(d), FAKE, ctypes.byref(no_scale),
                         ctypes.byref(r), FAKE, FAKE, ws, None) == -1
    one_scale = _lib.MoeWeights(FAKE, None, None, FAKE, None, FAKE, None,
                                None, None, None, None, FAKE, None)
    assert L.moe_grouped_ffn(ctypes.byref(d), FAKE, ctypes.byref(one_scale),
                             ctypes.byref(r), FAKE, ws, None) == -1


def test_swiglu_needs_w3():
    L = _lib.lib()
    d = desc(activation=2)
    ws = L.moe_workspace_size(ctypes.byref(d))
    assert ws > 0
    r = _lib.MoeRouting(*([FAKE] * 10))
    w = _lib.MoeWeights(FAKE, None, None, FAKE, None, FAKE, None,
                        None, None, None, None)
    assert L.moe_grouped_ffn(ctypes.byref(d), FAKE, ctypes.byref(w),
                             ctypes.byref(r), FAKE, ws, None) == -1
    # fp32 SwiGLU runs any d_ff the fp32 kernel runs
    assert L.moe_workspace_size(ctypes.byref(
        desc(activation=2, dtype=0, d_ff=192))) > 0


def test_python_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_LIB", None)
    monkeypatch.setattr(_lib, "library_path",
                        lambda: str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        _lib.lib()


def test_binding_checks_tensor_shapes():
    import torch
    w1 = torch.zeros(2, 64, 64, dtype=torch.bfloat16)
    w2 = torch.zeros(2, 64, 64, dtype=torch.bfloat16)
    wr = torch.zeros(2, 64, dtype=torch.bfloat16)
    moe.Weights(wr, w1, w2)
    with pytest.raises(ValueError):
        moe.Weights(wr, w1, torch.zeros(2, 64, 32, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        moe.Weights(wr.float(), w1, w2)
    with pytest.raises(ValueError):
        moe.Weights(wr, w1, w2, b_router=torch.zeros(2,
                                                     dtype=torch.bfloat16))


def _desc_of(w):
    import torch
    cap = (moe.moe_capacity(w.T, w.E, w.capacity_factor)
           if w.capacity_factor is not None else -1)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    return moe.make_desc(w.T, w.d, w.E, w.k, w.d_ff, dt, n_shared=w.n_shared,
                         capacity=cap, routing=w.routing,
                         expert_fp8=w.expert_fp8,
                         activation=w.activation or "gelu")


# (up, down) grouped-GEMM kernel ids the host picks on a 256-CU device
# (host side only: no GPU needed).  4: fp32 SIMT; 8 / 13: eight-wave
# 256- / 320-row tiles; 11 / 12: bf16 / FP8 weight streaming; 14: four-wave
# 256-row tiles with half-height tails; 15: four-wave 128-row tiles; 23:
# four-wave 256-row tiles of 192 columns; 24: four-wave 320 x 192 tiles.
PICKS = {
    "tiny_top2_f32": (4, 4),
    "switch_top1_cap": (2, 24),
    "mixtral_prefill": (14, 14),
    "mixtral_decode": (18, 18),
    "deepseek_v3": (24, 24),
    "mixtral_decode_fp8": (19, 19),
    "mixtral_prefill_swiglu": (14, 14),
    "mixtral_decode_swiglu": (11, 18),
    "expert_choice_c2": (8, 23),
}


@pytest.mark.parametrize("name", list(PICKS))
def test_gemm_variant_choice(name, monkeypatch):
    import workloads
    monkeypatch.delenv("MOE_GEMM_VARIANT_UP", raising=False)
    monkeypatch.delenv("MOE_GEMM_VARIANT_DOWN", raising=False)
    d = _desc_of(workloads.WORKLOADS[name])
    assert (moe.moe_gemm_variant(d, True),
            moe.moe_gemm_variant(d, False)) == PICKS[name]


def test_tall_tile_variants_are_validated(monkeypatch):
    """The tall-tile kernel (24, 25) takes a ragged last column tile (N not
    a multiple of 192 or 224), unlike the fixed-width kernels; it is
    refused for a gated (SwiGLU) up projection, whose waves must hold whole
    64-column gate/up chunks, and where the four-wave K rule fails."""
    import dataclasses
    import workloads
    ds = workloads.WORKLOADS["deepseek_v3"]
    d = _desc_of(ds)                         # up N = 2048, down N = 7168
    for v in ("24", "25"):
        monkeypatch.setenv("MOE_GEMM_VARIANT_UP", v)
        monkeypatch.setenv("MOE_GEMM_VARIANT_DOWN", v)
        assert moe.moe_gemm_variant(d, True) == int(v)
        assert moe.moe_gemm_variant(d, False) == int(v)
    # the 192-column four-wave form needs N % 192 == 0: refused for up
    # (2048), back to the pick
    monkeypatch.setenv("MOE_GEMM_VARIANT_UP", "23")
    assert moe.moe_gemm_variant(d, True) == 24
    # gated up projection: refused (the pick is a gate-capable kernel)
    sw = _desc_of(workloads.WORKLOADS["mixtral_prefill_swiglu"])
    monkeypatch.setenv("MOE_GEMM_VARIANT_UP", "24")
    assert moe.moe_gemm_variant(sw, True) == 14
    # K % 128 != 0: refused
    odd = _desc_of(dataclasses.replace(ds, d=7168 + 64))
    assert moe.moe_gemm_variant(odd, True) not in (24, 25)


def test_gemm_variant_override_is_validated(monkeypatch):
    import workloads
    d = _desc_of(workloads.WORKLOADS["mixtral_prefill"])
    monkeypatch.setenv("MOE_GEMM_VARIANT_UP", "15")
    assert moe.moe_gemm_variant(d, True) == 15
    # the four-wave kernels need K % 128 == 0: refused, back to the pick
    import dataclasses
    w = dataclasses.replace(workloads.WORKLOADS["mixtral_prefill"], d=4096 + 64)
    assert moe.moe_gemm_variant(_desc_of(w), True) != 15
    # an id out of range is ignored
    monkeypatch.setenv("MOE_GEMM_VARIANT_UP", "99")
    assert moe.moe_gemm_variant(d, True) == 14
    # the weight ring stages at most 1024 routed slots' tokens: refused for
    # this up projection (8192 slots), accepted for the down projection
    monkeypatch.setenv("MOE_GEMM_VARIANT_UP", "16")
    monkeypatch.setenv("MOE_GEMM_VARIANT_DOWN", "16")
    assert moe.moe_gemm_variant(d, True) == 14
    assert moe.moe_gemm_variant(d, False) == 16
    # ... and takes K in whole 2 KB row runs
    assert moe.moe_gemm_variant(_desc_of(w), False) == 16
    w2 = dataclasses.replace(workloads.WORKLOADS["mixtral_prefill"],
                             d_ff=14336 + 512)
    assert moe.moe_gemm_variant(_desc_of(w2), False) != 16
    # the FP8 ring needs FP8 weights
    monkeypatch.setenv("MOE_GEMM_VARIANT_DOWN", "17")
    assert moe.moe_gemm_variant(d, False) == 14
    # the two-block kernel takes K in 32-deep stages
    monkeypatch.setenv("MOE_GEMM_VARIANT_UP", "20")
    assert moe.moe_gemm_variant(d, True) == 20
    assert moe.moe_gemm_variant(_desc_of(w), True) == 20
    # (K % 32 != 0: refused; no tile kernel takes such a K at all)
    w3 = dataclasses.replace(workloads.WORKLOADS["mixtral_prefill"], d=4096 + 16)
    try:
        assert moe.moe_gemm_variant(_desc_of(w3), True) != 20
    except moe.MoeError:
        pass


@pytest.mark.parametrize("shape", [
    dict(name="mixtral_prefill"),                          # K 4096 / 14336
    dict(name="mixtral_prefill", T=2400, d=1024, d_ff=2048),   # K 1024 / 2048
    dict(name="mixtral_prefill", T=1200, d=2048, d_ff=1536),   # K 2048 / 1536
    dict(name="deepseek_v3", T=600, d=512, E=16, k=4, d_ff=512,
         expert_bias="none", linear_biases=True),
])
def test_tail_split_covers_whole_stage_pairs(shape, monkeypatch):
    # A split unit walks KT / S 64-deep stages two at a time: every cap of
    # MOE_TAIL_SPLIT must leave (K / 64) divisible by 2 S, or the units
    # would drop (or repeat) the last stages of K.
    import workloads
    shape = dict(shape)
    w = workloads.WORKLOADS[shape.pop("name")]
    if shape:
        w = workloads.scaled(w, **shape)
    monkeypatch.setenv("MOE_GEMM_VARIANT_UP", "14")
    monkeypatch.setenv("MOE_GEMM_VARIANT_DOWN", "14")
    d = _desc_of(w)
    seen = set()
    for cap in [None] + [str(c) for c in range(1, 9)]:
        if cap is None:
            monkeypatch.delenv("MOE_TAIL_SPLIT", raising=False)
        else:
            monkeypatch.setenv("MOE_TAIL_SPLIT", cap)
        for up in (True, False):
            K = w.d if up else w.d_ff
            S = moe.moe_gemm_tail_split(d, up)
            assert 1 <= S <= 8
            assert (K // 64) % (2 * S) == 0 or S == 1, (cap, up, K, S)
            if cap is not None:
                assert S <= int(cap)
            seen.add((up, S))
    # the Mixtral down projection (K = 14336, 224 stages) splits its 64
    # half tiles four ways by default; a cap of 3 must fall back to 2
    if w.name == "mixtral_prefill" and w.d_ff == 14336:
        monkeypatch.delenv("MOE_TAIL_SPLIT", raising=False)
        assert moe.moe_gemm_tail_split(d, False) == 4
        monkeypatch.setenv("MOE_TAIL_SPLIT", "3")
        assert moe.moe_gemm_tail_split(d, False) == 2
