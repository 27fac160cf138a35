"""HIP layer vs CPU oracle, through the C ABI, on MI355X.

Small cases run the oracle on every token; the full workload sizes (the
launch configurations the benchmark times) check routing, counts, dispatch
and statistics on every token and the layer output on a sample of rows.
Edge cases: ragged T, E = 1, k = E, zero capacity, everything on one
expert, empty experts, identical experts, determinism, exact scaling, the
balancing-bias step and T = 0.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import sparse_mixture_experts_50_amd as moe
import workloads
from workloads import scaled

from parity import (check_expert_choice, check_layer, device, gpu_forward,
                    inputs_on, sample_tokens)

pytestmark = pytest.mark.gpu

W = workloads.WORKLOADS


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


SMALL = {
    # full-size tiny layer (fp32)
    "tiny_top2_f32": W["tiny_top2_f32"],
    # Switch top-1 with capacity; 128x256 tiles, 16 experts
    "switch_small": scaled(W["switch_top1_cap"], T=2000, d=256, E=16,
                           d_ff=512),
    # Mixtral top-2, 250 rows per expert: 256x256 tiles, ragged tails
    "mixtral_small": scaled(W["mixtral_prefill"], T=1000, d=512, d_ff=1024),
    # decode: 8 rows per expert, 32x256 tiles
    "decode_small": scaled(W["mixtral_decode"], T=32, d=512, d_ff=1024),
    # DeepSeek-shaped: top-8 of 64 + shared expert, Zipf bias
    "deepseek_small": scaled(W["deepseek_v3"], T=600, d=512, E=64,
                             d_ff=256),
    # widths that are not multiples of 256: 64x64 tiles
    "narrow_64": scaled(W["mixtral_prefill"], T=300, d=320, E=4, d_ff=448),
    # fp32 with capacity and a shared expert
    "f32_cap_shared": scaled(W["tiny_top2_f32"], T=333, d=128, E=6,
                             d_ff=192, capacity_factor=1.0, n_shared=1),
    # ragged T, k = 3
    "ragged": scaled(W["mixtral_prefill"], T=77, d=256, E=8, k=3,
                     d_ff=512),
    # decode shape with a shared expert (48-row shared group)
    "stream_shared": scaled(W["deepseek_v3"], T=48, d=512, E=16, k=4,
                            d_ff=512),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_full_parity(name):
    w = SMALL[name]
    say(f"[parity small] {name}: {w}")
    inp = inputs_on(w, device())
    gpu = gpu_forward(w, inp)
    rep = check_layer(w, inp, gpu)
    say(f"[parity small] {name}: {rep}")


@pytest.mark.parametrize("variant", ["0", "1", "2", "3", "5", "6", "7", "8",
                                     "9", "11", "13", "14", "15", "16", "20"])
def test_every_gemm_variant(variant, monkeypatch):
    """Each bf16 tile variant forced on a shape with groups of 0 to ~100
    rows (several row chunks for the small-tile kernels)."""
    monkeypatch.setenv("MOE_GEMM_VARIANT_UP", variant)
    monkeypatch.setenv("MOE_GEMM_VARIANT_DOWN", variant)
    w = scaled(W["deepseek_v3"], T=150, d=512, E=6, k=2, d_ff=1024)
    inp = inputs_on(w, device())
    gpu = gpu_forward(w, inp)
    rep = check_layer(w, inp, gpu)
    say(f"[variant {variant}] {rep}")


@pytest.mark.parametrize("variant", ["13", "14", "15", "20"])
def test_large_tile_variants_multi_tile_groups(variant, monkeypatch):
    """The 320- and four-wave 256-row kernels on groups of ~600 rows (three
    row tiles, the last ragged), eight column tiles and 16 stages of K,
    sampled rows against the oracle."""
    monkeypatch.setenv("MOE_GEMM_VARIANT_UP", variant)
    monkeypatch.setenv("MOE_GEMM_VARIANT_DOWN", variant)
    w = scaled(W["mixtral_prefill"], T=2400, d=1024, d_ff=2048)
    inp = inputs_on(w, device())
    gpu = gpu_forward(w, inp)
    tokens = sample_tokens(w.T, 48, seed=3)
    rep = check_layer(w, inp, gpu, tokens=tokens)
    say(f"[large tiles {variant}] {rep}")


def test_step_entry_points_match_forward():
    w = SMALL["deepseek_small"]
    inp = inputs_on(w, device())
    a = gpu_forward(w, inp, steps=False)
    b = gpu_forward(w, inp, steps=True)
    for key in ("topk_idx", "topk_w", "counts", "slot_token", "slot_of",
                "f", "p", "l_aux", "y"):
        assert np.array_equal(a[key], b[key]), key
    check_layer(w, inp, b)


FULL = {
    "switch_top1_cap": 96,
    "mixtral_prefill": 24,
    "mixtral_decode": 32,
    "deepseek_v3": 12,
}


@pytest.mark.parametrize("name", list(FULL))
def test_full_size_sampled_parity(name):
    w = W[name]
    say(f"[parity full] {name}: generating inputs")
    inp = inputs_on(w, device())
    gpu = gpu_forward(w, inp)
    must = []
    if w.capacity_factor is not None:
        dropped = np.nonzero(np.any(gpu["slot_of"] < 0, axis=1))[0]
        must = dropped[:8].tolist()
    tokens = sample_tokens(w.T, FULL[name], seed=1, must=must)
    say(f"[parity full] {name}: oracle on {len(tokens)} rows")
    rep = check_layer(w, inp, gpu, tokens=tokens)
    say(f"[parity full] {name}: {rep}")
    del inp, gpu
    torch.cuda.empty_cache()


def test_decode_distinct_calls():
    w = W["mixtral_decode"]
    dev = device()
    base = inputs_on(w, dev)
    for call in (1, 57, 199):
        inp = dict(base)
        inp["x"] = workloads.make_x(w, dev, call)
        gpu = gpu_forward(w, inp)
        rep = check_layer(w, inp, gpu, tokens=sample_tokens(w.T, 8, call))
        say(f"[decode call {call}] {rep}")


def test_deepseek_bias_update_step():
    w = scaled(W["deepseek_v3"], T=600, d=512, E=64, d_ff=256)
    dev = device()
    inp = inputs_on(w, dev)
    gpu = gpu_forward(w, inp)
    layer = gpu["layer"]
    before = inp["ebias"].cpu().numpy().copy()
    _, r = layer.forward(inp["x"])
    layer.bias_update(r, w.bias_update_gamma)
    torch.cuda.synchronize()
    after = layer.w.expert_bias.cpu().numpy()
    expect = oracle.bias_update(r.counts.cpu().numpy(),
                                w.T * w.k / w.E, w.bias_update_gamma, before)
    assert np.array_equal(after, expect)
    assert not np.array_equal(after, before)
    # the next call routes with the updated bias, still matching the oracle
    inp2 = dict(inp)
    inp2["ebias"] = layer.w.expert_bias
    gpu2 = gpu_forward(w, inp2)
    check_layer(w, inp2, gpu2)


# ------------------------------------------------------------ edge cases
def edge(w, mutate, tokens=None):
    inp = inputs_on(w, device())
    mutate(inp)
    gpu = gpu_forward(w, inp)
    return inp, gpu, check_layer(w, inp, gpu, tokens=tokens)


def test_single_expert_is_dense():
    w = scaled(W["mixtral_prefill"], T=100, d=256, E=1, k=1, d_ff=512)
    inp, gpu, rep = edge(w, lambda i: None)
    assert np.all(gpu["topk_idx"] == 0) and np.all(gpu["topk_w"] == 1.0)


def test_soft_mixture_k_equals_E():
    w = scaled(W["mixtral_prefill"], T=64, d=256, E=8, k=8, d_ff=256)
    edge(w, lambda i: None)


def test_zero_capacity_gives_zero_output():
    w = scaled(W["switch_top1_cap"], T=200, d=256, E=16, d_ff=256,
               capacity_factor=0.01)
    inp, gpu, rep = edge(w, lambda i: None)
    assert np.all(gpu["kept"] == 0) and np.all(gpu["slot_of"] == -1)
    assert np.all(gpu["y"] == 0.0)


def test_all_tokens_on_one_expert():
    w = scaled(W["mixtral_prefill"], T=300, d=256, E=8, k=2, d_ff=256)

    def mutate(inp):
        inp["wr"].zero_()
        br = torch.zeros(8, dtype=torch.float32, device=inp["wr"].device)
        br[5] = 4.0
        br[2] = 2.0
        inp["br"] = br
    inp, gpu, rep = edge(w, mutate)
    assert gpu["counts"][5] == 300 and gpu["counts"][2] == 300


def test_empty_experts():
    w = scaled(W["mixtral_prefill"], T=256, d=256, E=16, k=2, d_ff=512)

    def mutate(inp):
        br = torch.zeros(16, dtype=torch.float32, device=inp["wr"].device)
        br[::2] = -30.0        # even experts never chosen
        inp["br"] = br
    inp, gpu, rep = edge(w, mutate)
    assert np.all(gpu["counts"][::2] == 0)


def test_identical_experts_full_width():
    w = scaled(W["mixtral_prefill"], T=512, d=1024, E=8, k=2, d_ff=2048)

    def mutate(inp):
        inp["w1"][1:] = inp["w1"][0]
        inp["w2"][1:] = inp["w2"][0]
    edge(w, mutate)


def test_deterministic_and_exact_scaling():
    w = SMALL["deepseek_small"]
    inp = inputs_on(w, device())
    a = gpu_forward(w, inp)
    b = gpu_forward(w, inp)
    for key in ("topk_idx", "topk_w", "slot_token", "f", "p", "l_aux", "y"):
        assert np.array_equal(a[key], b[key]), key
    inp2 = dict(inp)
    inp2["w2"] = inp["w2"] * 2
    inp2["ws2"] = inp["ws2"] * 2
    c = gpu_forward(w, inp2)
    assert np.array_equal(c["y"], 2 * a["y"])


def test_zero_tokens():
    w = scaled(W["mixtral_prefill"], T=0, d=256, E=8, d_ff=256)
    dev = device()
    inp = inputs_on(scaled(w, T=4), dev)
    weights = moe.Weights.from_dict(inp)
    layer = moe.MoeLayer(weights, w.k)
    y, r = layer.forward(inp["x"][:0])
    torch.cuda.synchronize()
    assert y.shape == (0, 256)


@pytest.mark.parametrize("C", [513, 640, 700, 257])
def test_four_wave_even_split_group_sizes(C, monkeypatch):
    """Expert-Choice routing gives every expert exactly C rows.  Without
    split tails, 513 and 640 rows run as three 224-row tiles (the last of
    65 / 192 rows); 700 rows (a 188-row last block) and 257 rows (two
    tiles) keep 256-row and half-height tiles."""
    monkeypatch.setenv("MOE_GEMM_VARIANT_UP", "14")
    monkeypatch.setenv("MOE_GEMM_VARIANT_DOWN", "14")
    monkeypatch.setenv("MOE_TAIL_SPLIT", "1")
    w = scaled(W["expert_choice_c2"], T=2 * C, d=256, E=2, k=2, d_ff=512,
               capacity_factor=1.0)
    inp = inputs_on(w, device())
    gpu = gpu_forward(w, inp)
    # (expert choice: every expert keeps exactly C rows)
    assert int(gpu["kept"].max()) == C and int(gpu["kept"].min()) == C
    say(f"[even split C={C}] {check_expert_choice(w, inp, gpu)}")
