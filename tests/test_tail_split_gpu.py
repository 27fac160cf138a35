"""Split tails of the four-wave 256-row GEMM vs the CPU oracle, through
the C ABI, on MI355X.  A group's last 1..128 rows (a half-height tile) run
as S units over consecutive ranges of K with fp32 partial sums, finished
by the tail reduction (bias, GELU / SwiGLU, bf16) when the half tiles
would otherwise form a sparse last round.  MOE_TAIL_SPLIT=1 turns the
split off, so both forms run on the same shapes and are compared."""
import sys

import numpy as np
import pytest
import torch

import sparse_mixture_experts_50_amd as moe
import workloads
from workloads import scaled

from parity import check_layer, device, gpu_forward, inputs_on, \
    sample_tokens

pytestmark = pytest.mark.gpu

W = workloads.WORKLOADS


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


CASES = {
    # ~600 rows per expert: two full tiles and a ~90-row half tile each
    "gelu_600": scaled(W["mixtral_prefill"], T=2400, d=1024, d_ff=2048),
    # gated experts, same group sizes
    "swiglu_600": scaled(W["mixtral_prefill_swiglu"], T=2400, d=1024,
                         d_ff=2048),
    # K = 1536 (24 stages): splits of 2, 3 and 4 all cover whole stage
    # pairs, so a cap of 3 really runs three units per half tile
    "gelu_k1536": scaled(W["mixtral_prefill"], T=2400, d=1536, d_ff=1536),
    # shared expert (T = 600 rows: 2 full + an 88-row tail) and Linear
    # biases, top-4 of 16
    "shared_biases": scaled(W["deepseek_v3"], T=600, d=512, E=16, k=4,
                            d_ff=512, expert_bias="none",
                            linear_biases=True),
}


# the four-wave kernel in its two MFMA forms: 16x16x32 (14), 32x32x16 (21)
FOUR_WAVE = ["14", "21"]


@pytest.mark.parametrize("kernel", FOUR_WAVE)
@pytest.mark.parametrize("split", ["8", "3", "1"])
@pytest.mark.parametrize("name", list(CASES))
def test_tail_split_parity(name, split, kernel, monkeypatch):
    monkeypatch.setenv("MOE_GEMM_VARIANT_UP", kernel)
    monkeypatch.setenv("MOE_GEMM_VARIANT_DOWN", kernel)
    monkeypatch.setenv("MOE_TAIL_SPLIT", split)
    w = CASES[name]
    d = moe.make_desc(w.T, w.d, w.E, w.k, w.d_ff, torch.bfloat16,
                      n_shared=w.n_shared, activation=w.activation)
    S = (moe.moe_gemm_tail_split(d, True), moe.moe_gemm_tail_split(d, False))
    if name == "gelu_k1536" and split == "3":
        assert S == (3, 3), S
    inp = inputs_on(w, device())
    gpu = gpu_forward(w, inp)
    tokens = sample_tokens(w.T, 64, seed=5)
    rep = check_layer(w, inp, gpu, tokens=tokens)
    say(f"[tail split <= {split}, S up/down {S}, kernel {kernel}] {name}: {rep}")


@pytest.mark.parametrize("kernel", FOUR_WAVE)
@pytest.mark.parametrize("name", ["gelu_600", "swiglu_600"])
def test_tail_split_matches_unsplit(name, kernel, monkeypatch):
    w = CASES[name]
    inp = inputs_on(w, device())
    monkeypatch.setenv("MOE_GEMM_VARIANT_UP", kernel)
    monkeypatch.setenv("MOE_GEMM_VARIANT_DOWN", kernel)
    out = {}
    for split in ("8", "1"):
        monkeypatch.setenv("MOE_TAIL_SPLIT", split)
        out[split] = gpu_forward(w, inp)
    assert np.array_equal(out["8"]["slot_token"], out["1"]["slot_token"])
    # the same products summed in another order: bf16-level agreement
    y0, y1 = out["8"]["y"], out["1"]["y"]
    scale = float(np.max(np.abs(y1)))
    err = float(np.max(np.abs(y0 - y1)))
    say(f"[tail split vs tiles] {name}: max diff {err:.3g} of {scale:.3g}")
    assert err <= 0.02 * scale
