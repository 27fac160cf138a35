"""HIP layer vs CPU oracle, through the C ABI, on MI355X.

Small cases run the oracle on every token; the full workload sizes (the
launch configurations the benchmark times) check routing, counts, dispatch
and statistics on every token and the layer output on every row (or, for
the DeepSeek-shaped layer, on rows covering every row tile of both GEMMs).
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
                    inputs_on, sample_tokens, tile_cover_tokens)

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
                                     "9", "11", "13", "14", "15", "16", "20",
                                     "21", "22", "24", "25"])
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


@pytest.mark.parametrize("variant", ["13", "14", "15", "20", "21", "22",
                                     "24", "25"])
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


# Decode-sized steps (bf16, E <= 32, T <= 32, T*k <= 256): moe_forward runs
# the router and the permute as one launch; the separate entry points run
# the split router (logits over S depth ranges, then routing) and the
# single-launch permute.  Both must agree bit for bit, and with the oracle.
FUSED_ROUTE = {
    "mixtral_decode": W["mixtral_decode"],                      # S = 8
    "ragged_e16_k4": scaled(W["mixtral_decode"], T=20, d=1024, E=16, k=4,
                            d_ff=512),                          # S = 2
    "e32_k8_whole_chunk": scaled(W["mixtral_decode"], T=32, d=512, E=32,
                                 k=8, d_ff=256),                # S = 1
    "capacity_skew": scaled(W["switch_top1_cap"], T=32, d=768, E=8,
                            d_ff=512, capacity_factor=1.0),     # C = 4
    "zipf_shared_d7168": scaled(W["deepseek_v3"], T=16, d=7168, E=32, k=4,
                                d_ff=256),                      # kc = 896
    "uneven_ranges": scaled(W["mixtral_decode"], T=24, d=4160, E=8,
                            d_ff=256),       # last range shorter than kc
    "single_token": scaled(W["mixtral_decode"], T=1, d=1024, E=8,
                           d_ff=256),
}


@pytest.mark.parametrize("name", list(FUSED_ROUTE))
def test_fused_decode_routing_matches_entry_points(name):
    w = FUSED_ROUTE[name]
    say(f"[fused route] {name}: {w}")
    inp = inputs_on(w, device())
    a = gpu_forward(w, inp, steps=False)
    b = gpu_forward(w, inp, steps=True)
    for key in ("topk_idx", "topk_w", "counts", "kept", "offsets",
                "slot_token", "slot_of", "f", "p", "l_aux", "monitor", "y"):
        assert np.array_equal(a[key], b[key]), key
    rep = check_layer(w, inp, a)
    if w.capacity_factor is not None:
        assert np.any(a["slot_of"] < 0)
    say(f"[fused route] {name}: {rep}")


# Full workload sizes, in the launch configuration the benchmark times.
# Where the oracle finishes the whole layer in well under a minute on the
# host cores every output row is checked; the DeepSeek-shaped layer (257
# groups, ~50 oracle tokens/s) checks every row tile of both GEMMs instead:
# each group's first and last row, each tile's first, middle and last rows
# (tile_cover_tokens), plus random rows.
FULL_ALL_ROWS = {"switch_top1_cap", "mixtral_prefill", "mixtral_decode"}
FULL = ["switch_top1_cap", "mixtral_prefill", "mixtral_decode",
        "deepseek_v3"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_parity(name):
    w = W[name]
    say(f"[parity full] {name}: generating inputs")
    inp = inputs_on(w, device())
    gpu = gpu_forward(w, inp)
    desc = gpu["layer"].desc(w.T)
    variants = (moe.moe_gemm_variant(desc, True),
                moe.moe_gemm_variant(desc, False))
    if name in FULL_ALL_ROWS:
        tokens = np.arange(w.T, dtype=np.int32)
    else:
        cover = tile_cover_tokens(w, gpu, variants)
        tokens = np.union1d(cover, sample_tokens(w.T, 32, seed=1))
    if w.capacity_factor is not None:
        assert np.any(gpu["slot_of"] < 0)       # drops are exercised
    say(f"[parity full] {name}: variants {variants}, oracle on "
        f"{len(tokens)} rows")
    rep = check_layer(w, inp, gpu, tokens=tokens.astype(np.int32))
    # near-tie flips are allowed by the rules; report them, and require
    # the decided tokens to be identical (checked inside check_layer)
    say(f"[parity full] {name}: {rep}")
    del inp, gpu
    torch.cuda.empty_cache()


def test_deepseek_bias_update_full_shape():
    """One balancing-bias step at the DeepSeek-shaped layer's own size
    (E = 256, T = 8192, top-8: target exactly 256, so an expert on target
    takes the sign(0) case), from the counts of a full forward, bit-exact
    against the oracle's float32 step; then the same step on constructed
    counts around the target (256, 255, 257, 0, 8192)."""
    w = W["deepseek_v3"]
    dev = device()
    inp = inputs_on(w, dev)
    gpu = gpu_forward(w, inp)
    # routing, counts and dispatch against the oracle (no output rows)
    check_layer(w, inp, gpu, tokens=np.arange(0, dtype=np.int32))
    layer = gpu["layer"]
    before = inp["ebias"].cpu().numpy().copy()
    _, r = layer.forward(inp["x"])
    counts = r.counts.cpu().numpy().copy()
    assert np.array_equal(counts, gpu["counts"])
    target = w.T * w.k / w.E
    assert target == 256.0
    layer.bias_update(r, w.bias_update_gamma)
    torch.cuda.synchronize()
    after = layer.w.expert_bias.cpu().numpy()
    expect = oracle.bias_update(counts, target, w.bias_update_gamma, before)
    assert np.array_equal(after, expect)
    say(f"[bias step full] experts above / on / below target: "
        f"{int((counts > 256).sum())} / {int((counts == 256).sum())} / "
        f"{int((counts < 256).sum())}")
    # constructed counts: every sign, including exactly on target
    c = np.full(256, 256, np.int32)
    c[1::4] = 255
    c[2::4] = 257
    c[3] = 0
    c[7] = 8192
    b0 = torch.from_numpy(before.copy()).to(dev)
    moe.moe_bias_update(torch.from_numpy(c).to(dev), target,
                        w.bias_update_gamma, b0)
    torch.cuda.synchronize()
    want = oracle.bias_update(c, target, w.bias_update_gamma, before)
    assert np.array_equal(b0.cpu().numpy(), want)
    assert np.array_equal(want[0::4], before[0::4])     # sign(0): unchanged


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


# The multi-chunk dispatch (T*k above the one-block limit): every chunk's
# block derives its rank bases and the expert offsets from the router's
# per-tile histogram, split over 1024 / E segments of its threads.
DISPATCH = {
    # 258 assignments: 5 chunks, the last holding one token; E = 48 gives
    # 21 segments, most of them empty; capacity overflow
    "just_above_one_block": scaled(W["switch_top1_cap"], T=129, d=256, E=48,
                                   k=2, d_ff=256, capacity_factor=1.0),
    # E = 256, k = 8: 4 segments of 4 chunks each, capacity overflow
    "e256_k8_capacity": scaled(W["deepseek_v3"], T=100, d=256, E=256, k=8,
                               d_ff=256, capacity_factor=1.0),
    # E = 3: 341 segments for 32 chunks (one chunk or none each)
    "e3_many_segments": scaled(W["mixtral_prefill"], T=1000, d=256, E=3,
                               k=2, d_ff=256),
}


@pytest.mark.parametrize("name", list(DISPATCH))
def test_multi_chunk_dispatch(name):
    w = DISPATCH[name]
    say(f"[dispatch] {name}: {w}")
    inp, gpu, rep = edge(w, lambda i: None)
    assert w.T * w.k > 256
    say(f"[dispatch] {name}: {rep}")


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


@pytest.mark.parametrize("C", [129, 192, 193, 257, 321, 513])
def test_four_wave_trimmed_tiles_swiglu(C, monkeypatch):
    """The gated (SwiGLU) epilogue on the four-wave kernel's shorter tiles:
    one-tile groups of 129..224 rows (160-, 192- and 224-row tiles), the
    two-tile even split (257 rows: 2 x 160, 321 rows: 2 x 192) and three
    224-row tiles (513 rows), Expert-Choice groups of exactly C rows."""
    monkeypatch.setenv("MOE_GEMM_VARIANT_UP", "14")
    monkeypatch.setenv("MOE_GEMM_VARIANT_DOWN", "14")
    monkeypatch.setenv("MOE_TAIL_SPLIT", "1")
    w = scaled(W["expert_choice_c2"], T=2 * C, d=256, E=2, k=2, d_ff=512,
               capacity_factor=1.0, activation="swiglu")
    inp = inputs_on(w, device())
    gpu = gpu_forward(w, inp)
    assert int(gpu["kept"].max()) == C and int(gpu["kept"].min()) == C
    say(f"[trimmed swiglu C={C}] {check_expert_choice(w, inp, gpu)}")


@pytest.mark.parametrize("C", [100, 128, 129, 160, 161, 200, 224, 225, 256,
                               300, 513])
def test_four_wave_192_column_tiles(C, monkeypatch):
    """The four-wave kernel with 192-column tiles (23) on Expert-Choice
    groups of exactly C rows, d = 768 and d_ff = 1536 (both GEMMs' N a
    multiple of 192): up to 128 rows a half tile, 129..224 rows one tile
    of 160, 192 or 224 rows, 225..256 a full tile, 300 rows two 192-row
    tiles, 513 rows three 224-row tiles."""
    monkeypatch.setenv("MOE_GEMM_VARIANT_UP", "23")
    monkeypatch.setenv("MOE_GEMM_VARIANT_DOWN", "23")
    monkeypatch.setenv("MOE_TAIL_SPLIT", "1")
    w = scaled(W["expert_choice_c2"], T=2 * C, d=768, E=2, k=2, d_ff=1536,
               capacity_factor=1.0)
    d = moe.make_desc(w.T, w.d, w.E, w.k, w.d_ff, torch.bfloat16,
                      capacity=C, routing="expert_choice")
    assert (moe.moe_gemm_variant(d, True), moe.moe_gemm_variant(d, False)) \
        == (23, 23)
    inp = inputs_on(w, device())
    gpu = gpu_forward(w, inp)
    assert int(gpu["kept"].max()) == C and int(gpu["kept"].min()) == C
    say(f"[192 columns C={C}] {check_expert_choice(w, inp, gpu)}")


def test_switch_down_192_column_tiles(monkeypatch):
    """A Switch-shaped layer (capacity 160 rows: groups of 0..160 rows, half
    tiles and trimmed 160-row tiles; N = 768 for the down GEMM) with the
    192-column four-wave kernel forced on its down GEMM; every output row
    against the oracle."""
    monkeypatch.setenv("MOE_GEMM_VARIANT_DOWN", "23")
    w = scaled(W["switch_top1_cap"], T=2048, E=16)
    d = moe.make_desc(w.T, w.d, w.E, w.k, w.d_ff, torch.bfloat16,
                      capacity=moe.moe_capacity(w.T, w.E, w.capacity_factor))
    assert moe.moe_gemm_variant(d, False) == 23
    inp = inputs_on(w, device())
    gpu = gpu_forward(w, inp)
    rep = check_layer(w, inp, gpu)
    say(f"[switch 192 columns] {rep}")


@pytest.mark.parametrize("kernel", ["14", "21"])
@pytest.mark.parametrize("C", [513, 640, 700, 257, 300, 320, 321, 384, 385,
                               129, 192, 193, 1049])
def test_four_wave_even_split_group_sizes(C, kernel, monkeypatch):
    """Expert-Choice routing gives every expert exactly C rows.  Without
    split tails, the 16x16x32 four-wave kernel (14) runs 513 and 640 rows
    as three 224-row tiles (the last of 65 / 192 rows); 700 rows (a 188-row
    last block) keep 256-row tiles; 257..320 rows run as two 160-row tiles
    and 321..384 as two 192-row tiles; 385 rows (a 129-row last block) as
    two full-height tiles.  The 32x32x16 form (21) mixes 256-, 192- and
    128-row tiles: 129..192 rows one 192-row tile, 257 rows 192 + 128, 385
    rows 256 + 192, 1049 rows 2 x 256 + 3 x 192.  (A one-tile group of
    129..224 rows runs as one tile of 160, 192 or 224 rows in form 14.)"""
    monkeypatch.setenv("MOE_GEMM_VARIANT_UP", kernel)
    monkeypatch.setenv("MOE_GEMM_VARIANT_DOWN", kernel)
    monkeypatch.setenv("MOE_TAIL_SPLIT", "1")
    w = scaled(W["expert_choice_c2"], T=2 * C, d=256, E=2, k=2, d_ff=512,
               capacity_factor=1.0)
    inp = inputs_on(w, device())
    gpu = gpu_forward(w, inp)
    # (expert choice: every expert keeps exactly C rows)
    assert int(gpu["kept"].max()) == C and int(gpu["kept"].min()) == C
    say(f"[even split C={C}, kernel {kernel}] {check_expert_choice(w, inp, gpu)}")


@pytest.mark.parametrize("kernel", ["24", "25"])
@pytest.mark.parametrize("C", [1, 64, 65, 128, 129, 193, 256, 257, 288, 289,
                               320, 321, 577, 641])
def test_tall_tile_group_sizes(C, kernel, monkeypatch):
    """The tall-tile kernel (24: 320 x 192 tiles, 25: 288 x 224) on
    Expert-Choice groups of exactly C rows: a group runs as
    ceil(C / 320) (or / 288) row tiles of the smallest height in 64, 128,
    192, 256, 288, 320 that holds its share, so C covers each height, one
    row either side of a boundary, one-tile groups (non-temporal weights)
    and two or three tiles (577, 641).  d = 256 and d_ff = 512 make every
    GEMM's last column tile ragged (512 = 2 x 192 + 128 = 2 x 224 + 64;
    256 = 192 + 64 = 224 + 32)."""
    monkeypatch.setenv("MOE_GEMM_VARIANT_UP", kernel)
    monkeypatch.setenv("MOE_GEMM_VARIANT_DOWN", kernel)
    w = scaled(W["expert_choice_c2"], T=2 * C, d=256, E=2, k=2, d_ff=512,
               capacity_factor=1.0)
    d = moe.make_desc(w.T, w.d, w.E, w.k, w.d_ff, torch.bfloat16,
                      capacity=C, routing="expert_choice")
    assert (moe.moe_gemm_variant(d, True), moe.moe_gemm_variant(d, False)) \
        == (int(kernel), int(kernel))
    inp = inputs_on(w, device())
    gpu = gpu_forward(w, inp)
    assert int(gpu["kept"].max()) == C and int(gpu["kept"].min()) == C
    say(f"[tall {kernel} C={C}] {check_expert_choice(w, inp, gpu)}")


@pytest.mark.parametrize("up,down,act", [("24", "25", "gelu"),
                                         ("25", "24", "gelu"),
                                         ("24", "14", "silu")])
def test_tall_tiles_deepseek_shaped(up, down, act, monkeypatch):
    """A DeepSeek-shaped layer at reduced size (top-8 of 64 experts, about
    256 rows each, the Zipf balancing bias, a shared expert of all 2048
    tokens: seven or eight row tiles sharing each panel, plain loads) with
    the tall-tile kernels on both GEMMs (and the SiLU epilogue), N = 512
    and 1024 (ragged last column tiles); every output row against the
    oracle."""
    monkeypatch.setenv("MOE_GEMM_VARIANT_UP", up)
    monkeypatch.setenv("MOE_GEMM_VARIANT_DOWN", down)
    w = scaled(W["deepseek_v3"], T=2048, d=1024, E=64, d_ff=512,
               activation=act)
    inp = inputs_on(w, device())
    gpu = gpu_forward(w, inp)
    rep = check_layer(w, inp, gpu)
    say(f"[tall deepseek {up}/{down} {act}] {rep}")


@pytest.mark.parametrize("C", [100, 256, 300])
def test_tall_tile_wide_ragged_columns(C, monkeypatch):
    """The 320 x 192 kernel's up GEMM runs a one-tile group of at most 256
    rows on 256-column tiles: with d_ff = 640 those are two full column
    tiles and a ragged one of 128 columns (a 300-row group keeps 192-column
    tiles: three full and one of 64), every output row against the
    oracle."""
    monkeypatch.setenv("MOE_GEMM_VARIANT_UP", "24")
    monkeypatch.setenv("MOE_GEMM_VARIANT_DOWN", "24")
    w = scaled(W["expert_choice_c2"], T=2 * C, d=256, E=2, k=2, d_ff=640,
               capacity_factor=1.0)
    inp = inputs_on(w, device())
    gpu = gpu_forward(w, inp)
    assert int(gpu["kept"].max()) == C and int(gpu["kept"].min()) == C
    say(f"[tall wide C={C}] {check_expert_choice(w, inp, gpu)}")
