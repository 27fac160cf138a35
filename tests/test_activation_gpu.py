"""SiLU and gated SwiGLU experts on the HIP layer vs the CPU oracle,
through the C ABI, on MI355X.  The gated up GEMM runs over a virtual
2*d_ff-column panel (64-column chunks: 32 rows of W1, then the same 32 rows
of W3), so every kernel that may run it is forced once on a shape with
ragged groups; the full Mixtral shapes are checked on sampled rows."""
import sys

import numpy as np
import pytest
import torch

import workloads
from workloads import scaled

from parity import (check_expert_choice, check_layer, device, gpu_forward,
                    inputs_on, sample_tokens)

pytestmark = pytest.mark.gpu

W = workloads.WORKLOADS
PRE = W["mixtral_prefill_swiglu"]
DEC = W["mixtral_decode_swiglu"]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


SMALL = {
    # fp32, router and expert biases (b3 too), SiLU and SwiGLU
    "silu_f32": scaled(W["tiny_top2_f32"], activation="silu"),
    "swiglu_f32": scaled(W["tiny_top2_f32"], activation="swiglu"),
    "swiglu_f32_shared_cap": scaled(W["tiny_top2_f32"], T=333, d=128, E=6,
                                    d_ff=192, capacity_factor=1.0,
                                    n_shared=1, activation="swiglu"),
    # bf16 prefill-like (256-row tiles), ragged tails
    "swiglu_prefill_small": scaled(PRE, T=1000, d=512, d_ff=1024),
    "silu_prefill_small": scaled(PRE, T=1000, d=512, d_ff=1024,
                                 activation="silu"),
    # decode: 64-column streaming units with the gate/up pair
    "swiglu_decode_small": scaled(DEC, T=32, d=512, d_ff=1024, calls=1),
    # shared gated expert, top-4 of 16, biases
    "swiglu_shared_biases": scaled(W["deepseek_v3"], T=200, d=512, E=16,
                                   k=4, d_ff=256, activation="swiglu",
                                   linear_biases=True),
    # FP8 gated experts (W1, W3, W2 all E4M3)
    "swiglu_fp8_decode": scaled(DEC, T=32, d=1024, d_ff=1024, calls=1,
                                expert_fp8=True, n_shared=1),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_activation_small_full_parity(name):
    w = SMALL[name]
    say(f"[act small] {name}: {w}")
    inp = inputs_on(w, device())
    gpu = gpu_forward(w, inp)
    rep = check_layer(w, inp, gpu)
    say(f"[act small] {name}: {rep}")


@pytest.mark.parametrize("variant", ["0", "1", "2", "5", "6", "8", "9", "11",
                                     "13", "14", "15", "16", "20", "21", "22"])
def test_swiglu_every_gate_capable_variant(variant, monkeypatch):
    monkeypatch.setenv("MOE_GEMM_VARIANT_UP", variant)
    monkeypatch.setenv("MOE_GEMM_VARIANT_DOWN", variant)
    w = scaled(PRE, T=150, d=512, E=6, k=2, d_ff=1024, n_shared=1,
               linear_biases=True)
    inp = inputs_on(w, device())
    gpu = gpu_forward(w, inp)
    say(f"[swiglu variant {variant}] {check_layer(w, inp, gpu)}")


def test_swiglu_expert_choice():
    w = scaled(W["expert_choice_c2"], T=512, d=256, E=8, k=8, d_ff=256,
               activation="swiglu")
    inp = inputs_on(w, device())
    gpu = gpu_forward(w, inp)
    say(f"[swiglu ec] {check_expert_choice(w, inp, gpu)}")


@pytest.mark.parametrize("name", ["mixtral_prefill_swiglu",
                                  "mixtral_decode_swiglu"])
def test_swiglu_full_size_sampled(name):
    w = W[name]
    say(f"[swiglu full] {name}: generating inputs")
    inp = inputs_on(w, device())
    gpu = gpu_forward(w, inp)
    tokens = sample_tokens(w.T, 12, seed=4)
    say(f"[swiglu full] {name}: oracle on {len(tokens)} rows")
    rep = check_layer(w, inp, gpu, tokens=tokens)
    say(f"[swiglu full] {name}: {rep}")
    del inp, gpu
    torch.cuda.empty_cache()


@pytest.mark.parametrize("act", ["gelu", "silu", "swiglu"])
def test_activation_accuracy_through_identity_experts(act):
    # E = 1, W1 = W3 = W2 = I: y = bf16(act(x)) (swiglu: SiLU(x) * x), so
    # every element checks the device activation against its definition
    # (the hidden rounding to bf16 is the only loss)
    d = 1024
    w = workloads.Workload(name="identity", T=512, d=d, E=1, k=1, d_ff=d,
                           dtype="bf16", activation=act)
    dev = device()
    inp = inputs_on(w, dev)
    grid = torch.linspace(-9.0, 9.0, w.T * d, device=dev)
    inp["x"] = grid.view(w.T, d).to(torch.bfloat16)
    eye = torch.eye(d, device=dev, dtype=torch.bfloat16)[None]
    inp["w1"] = eye.clone()
    inp["w2"] = eye.clone()
    if act == "swiglu":
        inp["w3"] = eye.clone()
    gpu = gpu_forward(w, inp)
    x = inp["x"].double().cpu()
    if act == "gelu":
        # Phi(x) = erfc(-x / sqrt 2) / 2: 1 + erf(x / sqrt 2) cancels to 0
        # in float64 for x below about -6
        ref = x * 0.5 * torch.special.erfc(-x / 2.0 ** 0.5)
    elif act == "silu":
        ref = x * torch.sigmoid(x)
    else:
        ref = x * torch.sigmoid(x) * x
    ref = ref.numpy()
    y = gpu["y"]
    # one rounding of the hidden unit to bf16 (relative 2^-9), then W2 = I
    # passes it on exactly; allow one bf16 ulp plus the approximation
    err = np.abs(y - ref)
    bound = np.abs(ref) * 2.0 ** -8 + 1e-6 * (1 + np.abs(x.numpy()))
    assert np.all(err <= bound), float(np.max(err / np.maximum(bound, 1e-30)))
    exact = (torch.from_numpy(ref).to(torch.bfloat16).double().numpy() == y)
    say(f"[act accuracy] {act}: max err {err.max():.3g}, "
        f"bf16-exact {exact.mean():.4f}")
    assert exact.mean() > 0.99
