"""FP8 (OCP E4M3, per-output-channel scales) expert weights on the HIP
layer vs the CPU oracle, through the C ABI, on MI355X.  The GPU decodes
the codes exactly to bf16 and applies the scale after the dot product;
the oracle dequantises to double first, so the comparison bound is the
bf16 layer's."""
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
F8 = W["mixtral_decode_fp8"]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


SMALL = {
    # decode: 8 rows per expert on average (single 16-row half)
    "fp8_decode_small": scaled(F8, T=32, d=1024, d_ff=2048),
    # groups of ~75 rows: several 32-row chunks per unit, both halves
    "fp8_chunks_shared": scaled(W["deepseek_v3"], T=300, d=1024, E=8, k=2,
                                d_ff=1024, expert_fp8=True, n_shared=1,
                                expert_bias="none"),
    # expert Linear biases and a ragged T
    "fp8_biases_ragged": scaled(F8, T=45, d=1024, E=4, k=2, d_ff=1024,
                                linear_biases=True, calls=1),
    # capacity drops
    "fp8_capacity": scaled(F8, T=64, d=2048, E=8, k=2, d_ff=1024,
                           capacity_factor=1.0, calls=1),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_fp8_small_full_parity(name):
    w = SMALL[name]
    say(f"[fp8 small] {name}: {w}")
    inp = inputs_on(w, device())
    assert inp["w1"].dtype == torch.uint8
    gpu = gpu_forward(w, inp)
    rep = check_layer(w, inp, gpu)
    say(f"[fp8 small] {name}: {rep}")


@pytest.mark.parametrize("variant", ["10", "12", "17"])
def test_fp8_every_kernel_variant(variant, monkeypatch):
    """Both FP8 streaming forms (split-K block, wave per unit) forced on a
    shape with 32-row chunks, a 16-row tail and a shared expert."""
    monkeypatch.setenv("MOE_GEMM_VARIANT_UP", variant)
    monkeypatch.setenv("MOE_GEMM_VARIANT_DOWN", variant)
    w = SMALL["fp8_chunks_shared"]
    inp = inputs_on(w, device())
    gpu = gpu_forward(w, inp)
    say(f"[fp8 variant {variant}] {check_layer(w, inp, gpu)}")


def test_fp8_expert_choice():
    w = scaled(F8, T=64, d=1024, E=4, k=4, d_ff=1024, capacity_factor=2.0,
               routing="expert_choice", calls=1)
    inp = inputs_on(w, device())
    gpu = gpu_forward(w, inp)
    say(f"[fp8 ec] {check_expert_choice(w, inp, gpu)}")


def test_fp8_full_size_decode_sampled():
    w = F8
    say(f"[fp8 full] {w.name}: generating inputs")
    inp = inputs_on(w, device())
    gpu = gpu_forward(w, inp)
    tokens = sample_tokens(w.T, 12, seed=3)
    say(f"[fp8 full] oracle on {len(tokens)} rows")
    rep = check_layer(w, inp, gpu, tokens=tokens)
    say(f"[fp8 full] {rep}")
    del inp, gpu
    torch.cuda.empty_cache()


def test_fp8_every_finite_code():
    # W1 cycles through all 254 finite codes (subnormals, both signs, the
    # largest magnitudes), so every code goes through the GPU decode
    w = scaled(F8, T=16, d=1024, E=1, k=1, d_ff=1024, calls=1)
    inp = inputs_on(w, device())
    codes = torch.arange(256, dtype=torch.uint8)
    vals = codes.view(torch.float8_e4m3fn).to(torch.float64)
    ok = codes[torch.isfinite(vals)]
    q = ok.repeat(1024 * 1024 // len(ok) + 1)[:1024 * 1024].view(1024, 1024)
    inp["w1"] = q.view(1, 1024, 1024).to(inp["w1"].device)
    gpu = gpu_forward(w, inp)
    rep = check_layer(w, inp, gpu)
    say(f"[fp8 codes] {rep}")
