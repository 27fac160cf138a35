"""The two-block grouped GEMM (128 x 256 tiles, 32-deep stages in a ring of
three LDS slots) forced on shapes that exercise its step loop and tile walk:
K of 8, 16 and 24 stages (trips of three steps with 2, 1 and 0 steps left
over), groups of one to several 128-row tiles with ragged tails, empty
experts, a shared expert, linear biases, GELU, SiLU and the gated SwiGLU
pairing, and the full Mixtral-shaped prefill layer on sampled rows.  Each
case checks that the forced kernel is the one that runs, then compares the
layer with the CPU oracle."""
import sys

import pytest
import torch

import sparse_mixture_experts_50_amd as moe
import workloads
from workloads import scaled

from parity import check_layer, device, gpu_forward, inputs_on, sample_tokens

pytestmark = pytest.mark.gpu

W = workloads.WORKLOADS
PRE = W["mixtral_prefill"]
PRE_SW = W["mixtral_prefill_swiglu"]
X2 = "20"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


CASES = {
    # up K = 256 (8 stages: two trips and 2 left), down K = 768 (24: none
    # left); ~300 rows per expert: three tiles, the last ragged
    "k8_k24": scaled(PRE, T=600, d=256, d_ff=768, E=4, k=2, calls=1),
    # up K = 512 (16 stages: 1 left), down K = 256 (8: 2 left)
    "k16_k8": scaled(PRE, T=300, d=512, d_ff=256, E=4, k=2, calls=1),
    # up K = 768 (24), down K = 512 (16); SiLU
    "k24_k16_silu": scaled(PRE, T=300, d=768, d_ff=512, E=4, k=2, calls=1,
                           activation="silu"),
    # 16 experts, 40 tokens, top-1: most groups empty, the rest a few rows
    "empty_experts": scaled(PRE, T=40, d=512, d_ff=512, E=16, k=1, calls=1),
    # shared expert (one more group, every token) and biases
    "shared_biases": scaled(PRE, T=200, d=512, d_ff=1024, E=4, k=2,
                            n_shared=1, linear_biases=True, calls=1),
    # gated: gate and up rows of each 32 features in one wave's 64 columns
    "swiglu_shared_biases": scaled(PRE_SW, T=200, d=512, d_ff=512, E=4, k=2,
                                   n_shared=1, linear_biases=True, calls=1),
    # gated with d_ff = 128: the down projection's K is 4 stages
    "swiglu_k4": scaled(PRE_SW, T=160, d=256, d_ff=128, E=4, k=2, calls=1),
}


@pytest.mark.parametrize("name", list(CASES))
def test_x2_forced(name, monkeypatch):
    w = CASES[name]
    monkeypatch.setenv("MOE_GEMM_VARIANT_UP", X2)
    monkeypatch.setenv("MOE_GEMM_VARIANT_DOWN", X2)
    say(f"[x2] {name}: {w}")
    inp = inputs_on(w, device())
    gpu = gpu_forward(w, inp)
    desc = gpu["layer"].desc(w.T)
    assert moe.moe_gemm_variant(desc, True) == int(X2)
    assert moe.moe_gemm_variant(desc, False) == int(X2)
    rep = check_layer(w, inp, gpu)
    say(f"[x2] {name}: {rep}")


@pytest.mark.parametrize("name", ["mixtral_prefill", "mixtral_prefill_swiglu"])
def test_x2_full_size_sampled(name, monkeypatch):
    monkeypatch.setenv("MOE_GEMM_VARIANT_UP", X2)
    monkeypatch.setenv("MOE_GEMM_VARIANT_DOWN", X2)
    w = W[name]
    say(f"[x2 full] {name}: generating inputs")
    inp = inputs_on(w, device())
    gpu = gpu_forward(w, inp)
    desc = gpu["layer"].desc(w.T)
    assert moe.moe_gemm_variant(desc, True) == int(X2)
    tokens = sample_tokens(w.T, 12, seed=8)
    rep = check_layer(w, inp, gpu, tokens=tokens)
    say(f"[x2 full] {name}: {rep}")
    del inp, gpu
    torch.cuda.empty_cache()


def test_x2_matches_four_wave_kernel(monkeypatch):
    """Same layer through the two-block and the four-wave kernel: identical
    routing, outputs equal to accumulation order."""
    w = scaled(PRE, T=400, d=1024, d_ff=1024, E=4, k=2, calls=1, n_shared=1,
               linear_biases=True)
    inp = inputs_on(w, device())
    outs = {}
    for v in ("14", X2):
        monkeypatch.setenv("MOE_GEMM_VARIANT_UP", v)
        monkeypatch.setenv("MOE_GEMM_VARIANT_DOWN", v)
        outs[v] = gpu_forward(w, inp)
    a, b = outs["14"], outs[X2]
    assert (a["slot_token"] == b["slot_token"]).all()
    scale = float(abs(a["y"]).max())
    err = float(abs(a["y"] - b["y"]).max())
    say(f"[x2 vs w4] max |diff| {err:.3g} of max |y| {scale:.3g}")
    assert err <= 1e-2 * scale
