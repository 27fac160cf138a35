"""The weight-ring grouped GEMM (bf16 and FP8 weights) forced on shapes
that exercise its unit walk: 16-row chunks with ragged tails, groups of
several chunks, empty experts, a shared expert, linear biases, the gated
SwiGLU pairing, blocks with many units, and the largest routed slot count
whose tokens it stages.  Each case checks that the forced kernel is the one
that runs, then compares the layer with the CPU oracle."""
import sys

import pytest
import torch

import sparse_mixture_experts_50_amd as moe
import workloads
from workloads import scaled

from parity import check_layer, device, gpu_forward, inputs_on, sample_tokens

pytestmark = pytest.mark.gpu

W = workloads.WORKLOADS
DEC = W["mixtral_decode"]
DEC_SW = W["mixtral_decode_swiglu"]
DEC_F8 = W["mixtral_decode_fp8"]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


CASES = {
    # ~20 rows per expert: a full chunk and a 4-row one; shared expert of
    # 40 rows (three chunks); biases on both projections
    "chunks_shared_biases": (scaled(DEC, T=40, d=1024, E=4, k=2, d_ff=2048,
                                    n_shared=1, linear_biases=True,
                                    calls=1), 16),
    # decode shape at a reduced width: 8 rows per expert
    "decode_small": (scaled(DEC, T=32, d=2048, d_ff=3072, calls=1), 16),
    # 16 experts, 8 tokens, top-1: most experts empty
    "empty_experts": (scaled(DEC, T=8, E=16, k=1, d=1024, d_ff=1024,
                             calls=1), 16),
    # gated up projection (gate rows then up rows of each 16 features)
    "swiglu_biases": (scaled(DEC_SW, T=32, d=1024, d_ff=1024, calls=1,
                             linear_biases=True, n_shared=1), 16),
    # 1024 routed slots, the most whose tokens are staged: 256 rows (16
    # chunks) per expert
    "max_slots": (scaled(DEC, T=512, d=1024, E=4, k=2, d_ff=1024,
                         calls=1), 16),
    # FP8 weights: ungated with a shared expert, and gated
    "fp8_shared": (scaled(DEC_F8, T=40, d=1024, E=4, k=2, d_ff=2048,
                          n_shared=1, calls=1), 17),
    "fp8_swiglu": (scaled(DEC_SW, T=32, d=1024, d_ff=1024, calls=1,
                          expert_fp8=True, n_shared=1), 17),
}


# each ring case on both forms: 2 KB bf16 row runs with one block per CU
# (16; FP8 17) and 1 KB runs with two blocks per CU (18; FP8 19)
FORMS = {16: 18, 17: 19}


@pytest.mark.parametrize("name,form", [(n, f) for n in CASES for f in (0, 1)])
def test_ring_forced(name, form, monkeypatch):
    w, variant = CASES[name]
    if form:
        variant = FORMS[variant]
    monkeypatch.setenv("MOE_GEMM_VARIANT_UP", str(variant))
    monkeypatch.setenv("MOE_GEMM_VARIANT_DOWN", str(variant))
    say(f"[ring {variant}] {name}: {w}")
    inp = inputs_on(w, device())
    gpu = gpu_forward(w, inp)
    desc = gpu["layer"].desc(w.T)
    assert moe.moe_gemm_variant(desc, True) == variant
    assert moe.moe_gemm_variant(desc, False) == variant
    rep = check_layer(w, inp, gpu)
    say(f"[ring {variant}] {name}: {rep}")


@pytest.mark.parametrize("name,variant", [("mixtral_decode", 16),
                                          ("mixtral_decode", 18),
                                          ("mixtral_decode_swiglu", 16),
                                          ("mixtral_decode_swiglu", 18),
                                          ("mixtral_decode_fp8", 17),
                                          ("mixtral_decode_fp8", 19)])
def test_ring_full_size_sampled(name, variant, monkeypatch):
    monkeypatch.setenv("MOE_GEMM_VARIANT_UP", str(variant))
    monkeypatch.setenv("MOE_GEMM_VARIANT_DOWN", str(variant))
    w = W[name]
    say(f"[ring full {variant}] {name}: generating inputs")
    inp = inputs_on(w, device())
    gpu = gpu_forward(w, inp)
    desc = gpu["layer"].desc(w.T)
    assert moe.moe_gemm_variant(desc, True) == variant
    tokens = sample_tokens(w.T, 12, seed=6)
    rep = check_layer(w, inp, gpu, tokens=tokens)
    say(f"[ring full {variant}] {name}: {rep}")
    del inp, gpu
    torch.cuda.empty_cache()


def test_ring_matches_streaming_kernel(monkeypatch):
    """Same layer through the ring and the register-streaming kernel: the
    routing is identical and the outputs agree to accumulation order."""
    w = scaled(DEC, T=32, d=1024, d_ff=2048, calls=1, n_shared=1,
               linear_biases=True)
    inp = inputs_on(w, device())
    outs = {}
    for v in ("11", "16"):
        monkeypatch.setenv("MOE_GEMM_VARIANT_UP", v)
        monkeypatch.setenv("MOE_GEMM_VARIANT_DOWN", v)
        outs[v] = gpu_forward(w, inp)
    a, b = outs["11"], outs["16"]
    assert (a["slot_token"] == b["slot_token"]).all()
    scale = float(abs(a["y"]).max())
    err = float(abs(a["y"] - b["y"]).max())
    say(f"[ring vs stream] max |diff| {err:.3g} of max |y| {scale:.3g}")
    assert err <= 1e-2 * scale
