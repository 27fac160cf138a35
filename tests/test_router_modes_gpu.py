"""The two bf16 router forms against the CPU oracle, through the C ABI, on
MI355X, each forced on every shape (MOE_ROUTER_SPLIT): fused (logits and
routing in one 32-token block) and split (partial logits over depth ranges,
then routing: one lane per token for E <= 32, 64-lane waves above).  Shapes
cover E = 8, 64, 100 and 256, ragged T, several token blocks and depth
ranges of the staged logits kernel, router and balancing biases, a shared
expert and expert choice.  Both forms must also agree on every routing
decision that is not a near-tie."""
import sys

import numpy as np
import pytest

import workloads
from workloads import scaled

from parity import check_expert_choice, check_layer, device, gpu_forward, \
    inputs_on

pytestmark = pytest.mark.gpu

W = workloads.WORKLOADS


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


CASES = {
    # E = 8, one lane per token in the split form; ragged T, k = 2
    "e8_ragged": scaled(W["mixtral_prefill"], T=77, d=512, d_ff=512),
    # E = 8, 32 decode tokens over a deep d (split into 8 depth ranges)
    "e8_decode": scaled(W["mixtral_decode"], T=32, d=2048, d_ff=512),
    # E = 64 with the skewed additive router bias, top-1 with capacity
    "e64_switch": scaled(W["switch_top1_cap"], T=300, d=256, d_ff=512),
    # E = 256 with the balancing bias and a shared expert, top-8
    "e256_deepseek": scaled(W["deepseek_v3"], T=200, d=512, d_ff=256),
    # E = 256 over three 256-token blocks (the last ragged) and eight
    # depth ranges of the staged logits kernel
    "e256_blocks": scaled(W["deepseek_v3"], T=600, d=2048, d_ff=256),
    # E = 100: the 128-expert staged kernel with experts past E clamped
    "e100_ragged": scaled(W["deepseek_v3"], T=300, d=1024, E=100, k=6,
                          d_ff=256),
    # E = 16 with router Linear biases and expert Linear biases
    "e16_biases": scaled(W["deepseek_v3"], T=150, d=256, E=16, k=4,
                         d_ff=256, n_shared=0, router_bias="linear",
                         linear_biases=True),
}


@pytest.mark.parametrize("mode", ["0", "1"])
@pytest.mark.parametrize("name", list(CASES))
def test_router_mode_parity(name, mode, monkeypatch):
    monkeypatch.setenv("MOE_ROUTER_SPLIT", mode)
    w = CASES[name]
    inp = inputs_on(w, device())
    gpu = gpu_forward(w, inp)
    rep = check_layer(w, inp, gpu)
    say(f"[router split={mode}] {name}: {rep}")


@pytest.mark.parametrize("mode", ["0", "1"])
def test_router_mode_expert_choice(mode, monkeypatch):
    monkeypatch.setenv("MOE_ROUTER_SPLIT", mode)
    for E in (8, 64):
        w = scaled(W["expert_choice_c2"], T=256, d=256, E=E, k=E, d_ff=256)
        inp = inputs_on(w, device())
        gpu = gpu_forward(w, inp)
        say(f"[router split={mode}] ec E={E}: {check_expert_choice(w, inp, gpu)}")


@pytest.mark.parametrize("name", ["e8_decode", "e64_switch", "e256_deepseek",
                                  "e256_blocks", "e100_ragged"])
def test_router_modes_agree(name, monkeypatch):
    w = CASES[name]
    inp = inputs_on(w, device())
    out = {}
    for mode in ("0", "1"):
        monkeypatch.setenv("MOE_ROUTER_SPLIT", mode)
        out[mode] = gpu_forward(w, inp)
    a, b = out["0"], out["1"]
    # identical picks wherever the fp32 logits are not within rounding of a
    # tie (the two forms sum the logits in different orders)
    same = np.all(a["topk_idx"] == b["topk_idx"], axis=1)
    assert same.mean() > 0.98, same.mean()
    rows = np.nonzero(same)[0]
    np.testing.assert_allclose(a["topk_w"][rows], b["topk_w"][rows],
                               rtol=1e-4, atol=1e-6)
    say(f"[router modes agree] {name}: {same.mean():.4f} of tokens identical")
