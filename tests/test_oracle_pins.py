"""Pins of the CPU oracle against things other than itself.

Each test ties one oracle step to a value the pages print, a closed form, an
invariant, brute force on a tiny input, or a special case that reduces to a
library routine (torch's float64 Linear / GELU / softmax, numpy's stable
sort and bincount).  Every test is chosen so that a plausible slip in the
oracle (a dropped bias term, a flipped sign, a transposed weight, a wrong
tie rule, an off-by-one in the capacity rank) fails at least one of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden",
                      "page_examples.json")


def golden(name):
    with open(GOLDEN) as fh:
        return json.load(fh)[name]


def dense_ffn_torch(x, w1, b1, w2, b2):
    """Textbook two-layer MLP with exact GELU via torch float64 library
    calls (the dense FFN the layer reduces to)."""
    f = lambda a: None if a is None else torch.as_tensor(a).double()
    h = torch.nn.functional.linear(f(x), f(w1), f(b1))
    h = torch.nn.functional.gelu(h, approximate="none")
    return torch.nn.functional.linear(h, f(w2), f(b2)).numpy()


def tiny_inputs(T=16, d=8, E=4, d_ff=12, seed=3, biases=True):
    w = workloads.Workload(name="t", T=T, d=d, E=E, k=1, d_ff=d_ff,
                           dtype="f32", router_bias="linear" if biases
                           else "none", linear_biases=biases, seed=seed)
    return w, workloads.make_inputs(w)


# ----------------------------------------------------------------- router
def test_router_closed_form_permutation_weights():
    # Wr is a permutation matrix: logit_e = x[pi(e)] exactly, so softmax is
    # q / sum(q) for x = log q.  A transposed Wr gives x[pi^-1(e)] instead.
    E = 5
    pi = [2, 0, 4, 1, 3]                    # not an involution
    wr = np.zeros((E, E), np.float32)
    for e, c in enumerate(pi):
        wr[e, c] = 1.0
    q = np.array([1, 2, 3, 4, 6], np.float64)
    x = np.log(q).astype(np.float32)[None, :]
    logits, probs = oracle.router(x, wr)
    xq = np.exp(x.astype(np.float64)[0])
    expect = xq[pi] / xq.sum()
    assert np.allclose(probs[0], expect, rtol=1e-15, atol=0)
    assert np.allclose(logits[0], x.astype(np.float64)[0][pi], rtol=0,
                       atol=0)


def test_router_bias_signs():
    # Additive router bias shifts logits up, the balancing bias shifts them
    # down: with add == sub the probabilities are unchanged, and a
    # subtracted log r divides each probability by r (then renormalises).
    rng = np.random.default_rng(0)
    x = rng.standard_normal((6, 8)).astype(np.float32)
    wr = rng.standard_normal((4, 8)).astype(np.float32)
    r = np.array([1.0, 2.0, 4.0, 0.5], np.float32)
    add = rng.standard_normal(4).astype(np.float32)
    _, p0 = oracle.router(x, wr)
    la, pa = oracle.router(x, wr, add_bias=add)
    logr = np.log(r).astype(np.float32)
    ls, ps = oracle.router(x, wr, sub_bias=logr)
    _, pboth = oracle.router(x, wr, add_bias=add, sub_bias=add)
    l0, _ = oracle.router(x, wr)
    assert np.allclose(la - l0, add.astype(np.float64)[None, :], atol=1e-12)
    assert np.allclose(pboth, p0, rtol=1e-13, atol=1e-16)
    expect = p0 / np.exp(logr.astype(np.float64))[None, :]
    expect /= expect.sum(1, keepdims=True)
    assert np.allclose(ps, expect, rtol=1e-12, atol=1e-16)
    assert not np.allclose(pa, p0)


def test_router_softmax_shift_invariance_and_uniform():
    x = np.ones((3, 4), np.float32)
    wr = np.zeros((8, 4), np.float32)
    _, p = oracle.router(x, wr, add_bias=np.full(8, 7.5, np.float32))
    assert np.all(p == 1.0 / 8)             # exp(0)/8 is exact
    # huge logits must not overflow: max subtraction
    wr2 = np.zeros((3, 4), np.float32)
    wr2[1, 0] = 1.0
    _, p2 = oracle.router(np.full((1, 4), 1000.0, np.float32), wr2)
    assert p2[0, 1] == 1.0 and p2[0, 0] == 0.0


# ------------------------------------------------------------------ top-k
def brute_topk(p, k):
    """Every k-subset; the best has the largest sum, ties to the
    lexicographically smallest sorted index set; order by (-p, index)."""
    best = None
    for sub in itertools.combinations(range(len(p)), k):
        s = sum(p[i] for i in sub)
        if best is None or s > best[0]:
            best = (s, sub)
    sel = sorted(best[1], key=lambda i: (-p[i], i))
    return sel


@settings(max_examples=200, deadline=None)
@given(st.integers(1, 9).flatmap(lambda E: st.tuples(
    st.just(E), st.integers(1, E),
    st.lists(st.integers(1, 6), min_size=E, max_size=E))))
def test_topk_brute_force_with_ties(args):
    E, k, ints = args
    # small-integer probabilities make exact ties common
    p = np.array(ints, np.float64) / 64.0
    idx, w, margin = oracle.topk(p[None, :], k)
    assert list(idx[0]) == brute_topk(list(p), k)
    sel = p[idx[0]]
    assert np.allclose(w[0], sel / sel.sum(), rtol=1e-15)
    assert abs(w[0].sum() - 1.0) < 1e-12
    if k < E:
        rest = np.delete(p, idx[0])
        assert margin[0] == sel[-1] - rest.max()
    else:
        assert math.isinf(margin[0])


def test_topk_golden_renorm_figure():
    g = golden("renorm_figure")
    p = np.array(g["probs"], np.float64)
    assert abs(p.sum() - 1.0) < 1e-15
    idx, w, _ = oracle.topk(p[None, :], g["k"])
    assert list(idx[0]) == g["topk_idx"]
    assert np.allclose(w[0], g["topk_w"], rtol=1e-15, atol=1e-15)


def test_topk_golden_router_vector():
    g = golden("router_vector")
    E = g["E"]
    p = np.full(E, g["tail"])
    p[:3] = g["head"]
    p /= p.sum()
    idx, w, _ = oracle.topk(p[None, :], g["k"])
    assert idx[0, 0] == g["top1_idx"] and w[0, 0] == g["top1_w"]


def test_activation_ratio_golden():
    g = golden("activation_ratio")
    rng = np.random.default_rng(1)
    p = rng.random((100, g["E"]))
    idx, _, _ = oracle.topk(p, g["k"])
    d = oracle.dispatch(idx, g["E"], -1)
    assert d["counts"].sum() == 100 * g["k"]
    # every token activates exactly k distinct experts
    assert all(len(set(r)) == g["k"] for r in idx.tolist())
    assert g["k"] / g["E"] == g["ratio"]


def test_renorm_single_expert_is_one():
    rng = np.random.default_rng(2)
    p = rng.random((50, 16))
    p /= p.sum(1, keepdims=True)
    idx, w, _ = oracle.topk(p, 1)
    assert np.all(w == 1.0)
    assert np.array_equal(idx[:, 0], np.argmax(p, axis=1))   # argmax routing


# --------------------------------------------------------------- dispatch
def test_capacity_golden():
    g = golden("capacity")
    for c in g["cases"]:
        assert oracle.capacity(c["T"], c["E"], c["cf"]) == c["C"], c
    assert oracle.capacity(10, 2, None) == -1


@settings(max_examples=150, deadline=None)
@given(st.integers(1, 40), st.integers(1, 6), st.integers(1, 3),
       st.integers(-1, 12), st.integers(0, 10_000))
def test_dispatch_against_stable_sort(T, E, k, cap, seed):
    k = min(k, E)
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(
        np.int32)
    d = oracle.dispatch(idx, E, cap)
    flat = idx.reshape(-1)
    counts = np.bincount(flat, minlength=E)
    assert np.array_equal(d["counts"], counts)
    kept = counts if cap < 0 else np.minimum(counts, cap)
    assert np.array_equal(d["kept"], kept)
    assert np.array_equal(d["offsets"], np.concatenate([[0],
                                                        np.cumsum(kept)]))
    # token-major order of assignments, grouped stably by expert
    order = np.argsort(flat, kind="stable")
    rank = np.empty_like(flat)
    for e in range(E):
        members = order[flat[order] == e]
        rank[members] = np.arange(len(members))
    keep = (rank < cap) if cap >= 0 else np.ones_like(flat, bool)
    slot_of = np.where(keep, d["offsets"][flat] + rank, -1)
    assert np.array_equal(d["slot_of"].reshape(-1), slot_of)
    st_ = np.full(T * k, -1, np.int32)
    st_[slot_of[keep]] = (np.arange(T * k) // k)[keep]
    assert np.array_equal(d["slot_token"], st_)
    # structure: increasing tokens within each segment
    for e in range(E):
        seg = d["slot_token"][d["offsets"][e]:d["offsets"][e + 1]]
        assert np.all(np.diff(seg) > 0)


def test_dispatch_zero_capacity_and_empty():
    idx = np.array([[0], [1], [0]], np.int32)
    d = oracle.dispatch(idx, 2, 0)
    assert np.all(d["slot_of"] == -1) and d["offsets"][-1] == 0
    d0 = oracle.dispatch(np.zeros((0, 2), np.int32), 3, -1)
    assert np.all(d0["counts"] == 0) and d0["offsets"][-1] == 0


# ------------------------------------------------------------------ stats
def test_aux_loss_uniform_golden():
    g = golden("aux_loss_uniform")
    # zero router weights: every probability is exactly 1/E
    T, d, E, k = 64, 8, 8, 2
    x = np.random.default_rng(0).standard_normal((T, d)).astype(np.float32)
    _, probs = oracle.router(x, np.zeros((E, d), np.float32))
    idx, _, _ = oracle.topk(probs, k)
    disp = oracle.dispatch(idx, E, -1)
    f, p, l_aux = oracle.stats(probs, disp["counts"], k, g["alpha"])
    assert abs(l_aux - g["l_aux"]) < 1e-15
    assert abs(f.sum() - 1) < 1e-15 and abs(p.sum() - 1) < 1e-15


def test_aux_loss_collapse_and_sums():
    # all tokens on expert 2 with probability 1: L = alpha * E
    T, E = 10, 4
    probs = np.zeros((T, E))
    probs[:, 2] = 1.0
    counts = np.array([0, 0, T, 0], np.int32)
    f, p, l = oracle.stats(probs, counts, 1, 0.01)
    assert abs(l - 0.01 * E) < 1e-15
    # f is before capacity and normalised by T*k
    rng = np.random.default_rng(5)
    pr = rng.random((30, 6))
    pr /= pr.sum(1, keepdims=True)
    idx, _, _ = oracle.topk(pr, 3)
    c = oracle.dispatch(idx, 6, 2)["counts"]
    f, p, l = oracle.stats(pr, c, 3, 0.5)
    assert np.allclose(f, np.bincount(idx.reshape(-1), minlength=6) / 90)
    assert np.allclose(p, pr.mean(0))
    assert abs(l - 0.5 * 6 * float(np.dot(f, p))) < 1e-14


# -------------------------------------------------------------- expert FFN
def test_single_expert_is_dense_ffn():
    # E = 1, k = 1: p = w = 1 and the layer is the dense FFN
    w, inp = tiny_inputs(E=1)
    out = oracle.forward(inp, k=1)
    ref = dense_ffn_torch(inp["x"], inp["w1"][0], inp["b1"][0],
                          inp["w2"][0], inp["b2"][0])
    assert np.allclose(out["y"], ref, rtol=1e-12, atol=1e-13)


def test_gelu_textbook_values():
    # one hidden unit, identity read-out: y = GELU(z) for chosen z
    zs = np.array([-3.0, -1.0, 0.0, 0.5, 1.0, 2.0], np.float32)
    x = zs[:, None]
    w1 = np.ones((1, 1), np.float32)
    w2 = np.ones((1, 1), np.float32)
    ex = oracle.Experts(1, lambda e: (w1, None, w2, None))
    y = oracle.layer_rows(range(len(zs)), x, np.zeros((6, 1), np.int32),
                          np.ones((6, 1)), None, ex)
    phi = np.array([0.0013498980316301, 0.15865525393145707, 0.5,
                    0.6914624612740131, 0.8413447460685429,
                    0.9772498680518208])            # standard normal CDF
    assert np.allclose(y[:, 0], zs * phi, rtol=1e-13, atol=1e-15)


def test_identical_experts_independent_of_routing():
    w, inp = tiny_inputs(E=6, T=40)
    for key in ("w1", "b1", "w2", "b2"):
        inp[key] = inp[key][:1].repeat(6, *([1] * (inp[key].dim() - 1)))
    out = oracle.forward(inp, k=3)
    ref = dense_ffn_torch(inp["x"], inp["w1"][0], inp["b1"][0],
                          inp["w2"][0], inp["b2"][0])
    assert np.allclose(out["y"], ref, rtol=1e-12, atol=1e-13)


def test_soft_mixture_k_equals_E():
    w, inp = tiny_inputs(E=4, T=20)
    out = oracle.forward(inp, k=4)
    logits = torch.nn.functional.linear(inp["x"].double(),
                                        inp["wr"].double(),
                                        inp["br"].double())
    p = torch.softmax(logits, -1).numpy()
    ref = sum(p[:, e:e + 1] * dense_ffn_torch(
        inp["x"], inp["w1"][e], inp["b1"][e], inp["w2"][e], inp["b2"][e])
        for e in range(4))
    assert np.allclose(out["y"], ref, rtol=1e-11, atol=1e-12)
    assert np.allclose(out["probs"], p, rtol=1e-12)


def test_shared_expert_alone():
    w, inp = tiny_inputs(E=4, T=20)
    sh = workloads.make_expert(w, 0, shared=True)
    inp.update(ws1=sh[0], bs1=sh[1], ws2=sh[2], bs2=sh[3])
    inp["w2"].zero_()
    inp["b2"].zero_()
    out = oracle.forward(inp, k=2)
    ref = dense_ffn_torch(inp["x"], *sh)
    assert np.allclose(out["y"], ref, rtol=1e-12, atol=1e-13)
    # and shared + routed is the sum of both parts
    w_, inp2 = tiny_inputs(E=4, T=20)
    routed = oracle.forward(inp2, k=2)["y"]
    inp2.update(ws1=sh[0], bs1=sh[1], ws2=sh[2], bs2=sh[3])
    both = oracle.forward(inp2, k=2)["y"]
    assert np.allclose(both, routed + ref, rtol=1e-12, atol=1e-13)


def test_top2_combine_by_definition_of_pages():
    # y_t = w0 * FFN_{i0}(x) + w1 * FFN_{i1}(x) with the renormalised
    # top-2 weights: each term from the torch dense reduction.
    w, inp = tiny_inputs(E=5, T=12)
    out = oracle.forward(inp, k=2)
    for t in range(12):
        ref = 0
        for j in range(2):
            e = out["topk_idx"][t, j]
            ref = ref + out["topk_w"][t, j] * dense_ffn_torch(
                inp["x"][t:t + 1], inp["w1"][e], inp["b1"][e], inp["w2"][e],
                inp["b2"][e])[0]
        assert np.allclose(out["y"][t], ref, rtol=1e-12, atol=1e-13)


def test_capacity_drops_give_exact_zero():
    w, inp = tiny_inputs(E=4, T=64, biases=False)
    out = oracle.forward(inp, k=1, capacity_factor=0.5)   # C = 8
    assert out["capacity"] == 8
    dropped = out["slot_of"][:, 0] < 0
    assert dropped.any() and (~dropped).any()
    assert np.all(out["y"][dropped] == 0.0)
    kept_rows = ~dropped
    e0 = out["topk_idx"][kept_rows, 0]
    xs = inp["x"][kept_rows]
    for i, e in enumerate(e0):
        ref = dense_ffn_torch(xs[i:i + 1], inp["w1"][e], None, inp["w2"][e],
                              None)
        assert np.allclose(out["y"][kept_rows][i], ref[0], rtol=1e-12,
                           atol=1e-13)
    # the first C tokens in token order are the kept ones, per expert
    for e in range(4):
        toks = np.nonzero(out["topk_idx"][:, 0] == e)[0]
        assert np.array_equal(out["slot_of"][toks[:8], 0] >= 0,
                              np.ones(min(8, len(toks)), bool))
        assert np.all(out["slot_of"][toks[8:], 0] == -1)
    zero = oracle.forward(inp, k=1, capacity_factor=0.01)  # C = 0
    assert zero["capacity"] == 0 and np.all(zero["y"] == 0.0)


def test_scaling_second_layer_by_two_is_exact():
    w, inp = tiny_inputs(E=4, T=16)
    y1 = oracle.forward(inp, k=2)["y"]
    inp["w2"] = inp["w2"] * 2
    inp["b2"] = inp["b2"] * 2
    y2 = oracle.forward(inp, k=2)["y"]
    assert np.array_equal(y2, 2 * y1)


def test_bf16_inputs_widen_exactly():
    # bf16 bit patterns are widened exactly: same result as the float32
    # copy of the same values
    w, inp = tiny_inputs(E=4, T=16)
    bf = {k: (v.to(torch.bfloat16) if isinstance(v, torch.Tensor) and
              k not in ("br", "ebias") else v) for k, v in inp.items()}
    f32 = {k: (v.float() if isinstance(v, torch.Tensor) else v)
           for k, v in bf.items()}
    a = oracle.forward(bf, k=2)
    b = oracle.forward(f32, k=2)
    assert np.array_equal(a["y"], b["y"])
    assert np.array_equal(a["probs"], b["probs"])


# -------------------------------------------------------------- bias step
def test_bias_update_golden():
    g = golden("bias_update")
    b = np.array(g["bias_in"], np.float32)
    nb = oracle.bias_update(np.array(g["counts"], np.int32), g["target"],
                            g["gamma"], b)
    expect = b + np.float32(g["gamma"]) * np.array(g["sign"], np.float32)
    assert np.array_equal(nb, expect.astype(np.float32))
    assert nb[1] == b[1]                     # exactly on target: unchanged
    # the higher bias lowers the adjusted logit of an overloaded expert
    x = np.ones((1, 2), np.float32)
    wr = np.ones((4, 2), np.float32)
    _, p_before = oracle.router(x, wr, sub_bias=np.zeros(4, np.float32))
    _, p_after = oracle.router(x, wr, sub_bias=nb - b)
    assert p_after[0, 0] < p_before[0, 0] and p_after[0, 2] > p_before[0, 2]


def test_capacity_top2_keeps_pre_drop_weight():
    # A dropped assignment adds nothing and the surviving weight is not
    # renormalised: y_t = w_kept * FFN_kept(x_t).
    w, inp = tiny_inputs(E=3, T=48, biases=False)
    out = oracle.forward(inp, k=2, capacity_factor=1.0)     # C = 16
    so = out["slot_of"]
    part = (so[:, 0] >= 0) ^ (so[:, 1] >= 0)
    assert part.any()
    for t in np.nonzero(part)[0]:
        j = 0 if so[t, 0] >= 0 else 1
        e = out["topk_idx"][t, j]
        ref = out["topk_w"][t, j] * dense_ffn_torch(
            inp["x"][t:t + 1], inp["w1"][e], None, inp["w2"][e], None)[0]
        assert out["topk_w"][t, j] < 1.0
        assert np.allclose(out["y"][t], ref, rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------- monitors
def test_monitor_uniform_closed_forms():
    # zero router weights: logits all 0, so logsumexp = ln E and the
    # entropy is log2 E bits ([GROUP] 4.4 compares against log2(16) = 4)
    for E in (4, 8, 16):
        T, d, k = 10, 8, 2
        x = np.random.default_rng(E).standard_normal((T, d)).astype(np.float32)
        lg, pr = oracle.router(x, np.zeros((E, d), np.float32))
        idx, _, _ = oracle.topk(pr, k)
        disp = oracle.dispatch(idx, E, -1)
        m = oracle.monitor(lg, pr, disp["counts"], disp["kept"], k)
        assert abs(m[0] - math.log(E) ** 2) < 1e-12
        assert abs(m[1] - math.log2(E)) < 1e-12
    assert abs(math.log2(16) - 4.0) == 0.0


def test_monitor_confident_router_has_zero_entropy():
    wr = np.zeros((4, 2), np.float32)
    wr[2, 0] = 1.0
    x = np.array([[800.0, 0.0]], np.float32)
    lg, pr = oracle.router(x, wr)
    m = oracle.monitor(lg, pr, np.array([0, 0, 1, 0], np.int32),
                       np.array([0, 0, 1, 0], np.int32), 1)
    assert m[1] == 0.0
    assert abs(m[0] - 800.0 ** 2) < 1e-6 * 800.0 ** 2


def test_monitor_count_statistics_golden():
    # [SKILL] 10.1: imbalance max/min (healthy near 1, act above 2),
    # utilization used/E, drop rate dropped/total; [DIVE] 4: collapse when
    # one expert takes over 40 percent of the tokens
    T, E, k = 10, 4, 2
    probs = np.full((T, E), 0.25)
    logits = np.zeros((T, E))
    counts = np.array([8, 6, 4, 2], np.int32)
    kept = np.array([5, 5, 4, 2], np.int32)
    m = oracle.monitor(logits, probs, counts, kept, k)
    assert m[2] == 4.0 and m[3] == 1.0
    assert abs(m[4] - 4 / 20) < 1e-15
    assert m[5] == 0.8
    m2 = oracle.monitor(logits, probs, np.array([10, 10, 0, 0], np.int32),
                        np.array([10, 10, 0, 0], np.int32), k)
    assert math.isinf(m2[2]) and m2[3] == 0.5 and m2[4] == 0.0


def test_monitor_matches_direct_definitions():
    # library re-statement on random routing: scipy logsumexp and entropy
    from scipy.special import logsumexp
    from scipy.stats import entropy
    w, inp = tiny_inputs(E=6, T=30)
    out = oracle.forward(inp, k=2, capacity_factor=0.5)
    lg = out["logits"]
    assert abs(out["monitor"][0] - np.mean(logsumexp(lg, axis=1) ** 2)) \
        < 1e-12
    assert abs(out["monitor"][1] -
               np.mean(entropy(out["probs"], base=2, axis=1))) < 1e-12
    c, kp = out["counts"], out["kept"]
    assert out["monitor"][4] == (60 - kp.sum()) / 60


# ---------------------------------------------------------- expert choice
def _ec_brute(logits, C):
    """Per expert, the C-subset of tokens with the largest score sum; among
    equal sums the lexicographically smallest token set (the lower-index
    tie rule).  Exhaustive over all subsets: independent of any sort."""
    T, E = logits.shape
    out = []
    for e in range(E):
        best, best_set = None, None
        for sub in itertools.combinations(range(T), C):
            s = sum(logits[t, e] for t in sub)
            if best is None or s > best:
                best, best_set = s, sub
        out.append(best_set)
    return out


@settings(max_examples=40, deadline=None)
@given(st.integers(1, 7), st.integers(1, 4), st.data())
def test_expert_choice_brute_force(T, E, data):
    # integer scores make ties frequent; the tie rule is the lower token
    C = data.draw(st.integers(0, T))
    vals = data.draw(st.lists(st.integers(-2, 2), min_size=T * E,
                              max_size=T * E))
    logits = np.array(vals, np.float64).reshape(T, E)
    probs = np.exp(logits) / np.exp(logits).sum(1, keepdims=True)
    ec = oracle.expert_choice(logits, probs, C)
    want = _ec_brute(logits, C)
    for e in range(E):
        got = ec["slot_token"][e * C:(e + 1) * C]
        assert tuple(got.tolist()) == tuple(want[e])
        for r, t in enumerate(got.tolist()):
            assert ec["slot_of"][t, e] == e * C + r
            assert ec["gate"][t, e] == probs[t, e]
    assert ec["picks"].sum() == E * C
    assert np.count_nonzero(ec["slot_of"] >= 0) == E * C
    assert np.all((ec["gate"] == 0) == (ec["slot_of"] < 0)) or \
        np.any(probs == 0)


def test_expert_choice_perfect_balance():
    # the pages' claim: every expert gets exactly its capacity
    w, inp = tiny_inputs(E=6, T=48)
    out = oracle.forward_expert_choice(inp, capacity=10)
    assert np.all(out["kept"] == 10)
    for e in range(6):
        assert np.count_nonzero(out["slot_of"][:, e] >= 0) == 10
    assert np.array_equal(out["offsets"], np.arange(7) * 10)
    # Every token is a candidate of every expert: f = 1/E, L_aux = alpha.
    assert np.allclose(out["f"], 1 / 6, rtol=1e-15)
    assert abs(out["l_aux"] - 0.01) < 1e-15
    # drop rate = assignments not kept = 1 - C/T
    i = oracle.MONITOR_NAMES.index("drop_rate")
    assert abs(out["monitor"][i] - (1 - 10 / 48)) < 1e-12


def test_expert_choice_ranks_by_logit_not_probability():
    # expert 1 scores token 0 with logit 0 (prob 0.119) and token 1 with
    # logit 1 (prob 0.018): the transposed router output ranks by logit
    logits = np.array([[2.0, 0.0], [5.0, 1.0]])
    probs = np.exp(logits) / np.exp(logits).sum(1, keepdims=True)
    ec = oracle.expert_choice(logits, probs, 1)
    assert ec["slot_token"].tolist() == [1, 1]
    assert ec["picks"].tolist() == [0, 2]
    assert ec["gate"][1].tolist() == probs[1].tolist()


def test_expert_choice_full_capacity_is_soft_mixture():
    # C = T: every expert takes every token, y = sum_e p_e FFN_e(x) (+ the
    # shared expert), the dense softmax mixture
    w, inp = tiny_inputs(E=4, T=20)
    out = oracle.forward_expert_choice(inp, capacity=20)
    logits = torch.nn.functional.linear(inp["x"].double(),
                                        inp["wr"].double(),
                                        inp["br"].double())
    p = torch.softmax(logits, -1).numpy()
    ref = sum(p[:, e:e + 1] * dense_ffn_torch(
        inp["x"], inp["w1"][e], inp["b1"][e], inp["w2"][e], inp["b2"][e])
        for e in range(4))
    assert np.allclose(out["y"], ref, rtol=1e-11, atol=1e-12)
    assert np.all(out["picks"] == 4)


def test_expert_choice_rows_partial_picks():
    # C < T: each row sums only the experts that picked it, unrenormalised;
    # a row nobody picked is zero
    w, inp = tiny_inputs(E=4, T=24)
    out = oracle.forward_expert_choice(inp, capacity=3)
    ffn = [dense_ffn_torch(inp["x"], inp["w1"][e], inp["b1"][e],
                           inp["w2"][e], inp["b2"][e]) for e in range(4)]
    logits = torch.nn.functional.linear(inp["x"].double(),
                                        inp["wr"].double(),
                                        inp["br"].double()).numpy()
    p = np.exp(logits) / np.exp(logits).sum(1, keepdims=True)
    ref = np.zeros_like(out["y"])
    for e in range(4):
        top = np.argsort(-logits[:, e], kind="stable")[:3]
        ref[top] += p[top, e:e + 1] * ffn[e][top]
    assert np.allclose(out["y"], ref, rtol=1e-11, atol=1e-12)
    assert np.any(out["picks"] == 0)
    assert np.all(out["y"][out["picks"] == 0] == 0.0)


def test_expert_choice_zero_capacity_and_bounds():
    w, inp = tiny_inputs(E=3, T=10)
    out = oracle.forward_expert_choice(inp, capacity=0)
    assert out["slot_token"].size == 0 and np.all(out["slot_of"] == -1)
    assert np.all(out["y"] == 0.0)
    lg = np.zeros((4, 2))
    with pytest.raises(ValueError):
        oracle.expert_choice(lg, lg, 5)


# ------------------------------------------------------------ FP8 weights
def test_fp8_e4m3_every_code_matches_torch():
    # torch's float8_e4m3fn decoding is the library special case
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(
        torch.float64).numpy()
    got = oracle.fp8_e4m3(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_fp8_e4m3_format_values():
    # values fixed by the format: largest finite, smallest normal and
    # subnormal, one, a mantissa pattern, signed zero, the NaN codes
    v = oracle.fp8_e4m3
    assert v(0x7E) == 448.0 and v(0xFE) == -448.0
    assert v(0x08) == 2.0 ** -6 and v(0x01) == 2.0 ** -9
    # 0x4D: exponent 9, mantissa 5 -> 1.625 * 2^2
    assert v(0x38) == 1.0 and v(0x37) == 0.9375 and v(0x4D) == 6.5
    assert v(0x00) == 0.0 and np.signbit(v(0x80))
    assert np.isnan(v(0x7F)) and np.isnan(v(0xFF))
    assert v(0x77) == 240.0      # exponent 14 is finite (no infinities)


def test_fp8_layer_equals_bf16_layer_on_representable_weights():
    # per-output-channel scales 2^(n%5 - 2): decode(q) * s is exactly a
    # bf16 value, so the FP8 layer must equal the bf16 layer bit for bit;
    # a scale on the wrong axis or divided instead of multiplied fails
    w, inp = tiny_inputs(E=3, T=24, d=16, d_ff=32, biases=False)
    g = np.random.default_rng(5)
    table = torch.arange(256, dtype=torch.uint8).view(
        torch.float8_e4m3fn).to(torch.float64).numpy()
    finite = np.nonzero(np.isfinite(table) & (np.abs(table) <= 64))[0]

    def quant(E, N, K):
        q = g.choice(finite, size=(E, N, K)).astype(np.uint8)
        s = (2.0 ** (np.arange(N) % 5 - 2)).astype(np.float32)
        s = np.tile(s, (E, 1))
        deq = table[q] * s[:, :, None].astype(np.float64)
        return q, s, torch.from_numpy(deq.astype(np.float32))
    x16 = dict(inp)
    x16["x"] = inp["x"].to(torch.bfloat16)
    x16["wr"] = inp["wr"].to(torch.bfloat16)
    q1, s1, d1 = quant(3, 32, 16)
    q2, s2, d2 = quant(3, 16, 32)
    bf = dict(x16, w1=d1.to(torch.bfloat16), w2=d2.to(torch.bfloat16))
    assert torch.equal(bf["w1"].float(), d1) and torch.equal(bf["w2"].float(), d2)
    f8 = dict(x16, w1=torch.from_numpy(q1), w1_scale=torch.from_numpy(s1),
              w2=torch.from_numpy(q2), w2_scale=torch.from_numpy(s2))
    a = oracle.forward(bf, k=2)
    b = oracle.forward(f8, k=2)
    assert np.array_equal(a["y"], b["y"])
    assert np.any(a["y"] != 0)


# ------------------------------------------------- SiLU / SwiGLU experts
def test_silu_textbook_values():
    # one hidden unit, identity read-out: y = SiLU(z) = z * sigma(z)
    zs = np.array([-3.0, -1.0, 0.0, 0.5, 1.0, 2.0], np.float32)
    x = zs[:, None]
    one = np.ones((1, 1), np.float32)
    ex = oracle.Experts(1, lambda e: (one, None, one, None))
    y = oracle.layer_rows(range(len(zs)), x, np.zeros((6, 1), np.int32),
                          np.ones((6, 1)), None, ex, activation="silu")
    sigma = np.array([0.04742587317756678, 0.2689414213699951, 0.5,
                      0.6224593312018546, 0.7310585786300049,
                      0.8807970779778823])          # logistic function
    assert np.allclose(y[:, 0], zs * sigma, rtol=1e-13, atol=1e-15)


def _dense(x, w1, b1, w2, b2, w3=None, b3=None, act="gelu"):
    f = lambda a: None if a is None else torch.as_tensor(a).double()
    z = torch.nn.functional.linear(f(x), f(w1), f(b1))
    if act == "silu":
        h = torch.nn.functional.silu(z)
    else:
        h = torch.nn.functional.silu(z) * torch.nn.functional.linear(
            f(x), f(w3), f(b3))
    return torch.nn.functional.linear(h, f(w2), f(b2)).numpy()


def test_single_expert_silu_and_swiglu_are_torch_ffns():
    for act in ("silu", "swiglu"):
        w = workloads.Workload(name="t", T=16, d=8, E=1, k=1, d_ff=12,
                               dtype="f32", linear_biases=True,
                               activation=act, seed=4)
        inp = workloads.make_inputs(w)
        out = oracle.forward(inp, k=1, activation=act)
        ref = _dense(inp["x"], inp["w1"][0], inp["b1"][0], inp["w2"][0],
                     inp["b2"][0], None if act == "silu" else inp["w3"][0],
                     None if act == "silu" else inp["b3"][0], act)
        assert np.allclose(out["y"], ref, rtol=1e-12, atol=1e-13), act


def test_swiglu_with_unit_up_projection_is_silu():
    # W3 = 0, b3 = 1: the up branch is 1, so SwiGLU reduces to SiLU
    # exactly; a swapped gate/up (SiLU on the up branch) gives SiLU(1)*z
    w = workloads.Workload(name="t", T=20, d=8, E=3, k=2, d_ff=12,
                           dtype="f32", linear_biases=True,
                           activation="swiglu", seed=6)
    inp = workloads.make_inputs(w)
    inp["w3"] = torch.zeros_like(inp["w3"])
    inp["b3"] = torch.ones_like(inp["b3"])
    a = oracle.forward(inp, k=2, activation="swiglu")
    b = oracle.forward(inp, k=2, activation="silu")
    assert np.array_equal(a["y"], b["y"])
    c = oracle.forward(inp, k=2, activation="gelu")
    assert not np.allclose(a["y"], c["y"])


def test_swiglu_shared_expert_and_fp8_up_projection():
    # the shared expert is gated too; FP8 W3 dequantises like W1
    w = workloads.Workload(name="t", T=12, d=1024, E=2, k=1, d_ff=1024,
                           dtype="bf16", n_shared=1, activation="swiglu",
                           expert_fp8=True, seed=7)
    inp = workloads.make_inputs(w)
    out = oracle.forward(inp, k=1, activation="swiglu",
                         tokens=np.array([0, 5], np.int32))
    x = inp["x"][[0, 5]].float()
    deq = lambda q, s: oracle.fp8_dequant(q, s)
    e = out["topk_idx"][[0, 5], 0]
    ref = np.stack([
        _dense(x[i:i + 1], deq(inp["w1"][e[i]], inp["w1_scale"][e[i]]), None,
               deq(inp["w2"][e[i]], inp["w2_scale"][e[i]]), None,
               deq(inp["w3"][e[i]], inp["w3_scale"][e[i]]), None,
               "swiglu")[0] for i in range(2)])
    ref += _dense(x, deq(inp["ws1"], inp["ws1_scale"]), None,
                  deq(inp["ws2"], inp["ws2_scale"]), None,
                  deq(inp["ws3"], inp["ws3_scale"]), None, "swiglu")
    assert np.allclose(out["y"], ref, rtol=1e-10, atol=1e-10)


# ---------------------------------------------- selection-conditioned path
# A checker that adopts the GPU's choice at a near-tie re-runs the layer on
# a given selection: the weights are then the renormalised probabilities of
# the chosen experts ("MoE architecture deep dive", sec. 1.3 steps 2-3) and
# everything after is the ordinary dispatch, FFN and combine.
@settings(max_examples=200, deadline=None)
@given(st.integers(1, 9).flatmap(lambda E: st.tuples(
    st.just(E), st.integers(1, E),
    st.lists(st.integers(1, 6), min_size=E, max_size=E))))
def test_renorm_selection_of_own_topk_is_topk_weights(args):
    E, k, ints = args
    p = np.array(ints, np.float64) / 64.0
    idx, w, _ = oracle.topk(p[None, :], k)
    assert np.array_equal(oracle.renorm_selection(p[None, :], idx), w)


def test_renorm_selection_golden_figure_and_non_top_pairs():
    g = golden("renorm_figure")
    p = np.array(g["probs"], np.float64)[None, :]
    # the figure's pair, in either order: the weights follow the selection
    w = oracle.renorm_selection(p, np.array([g["topk_idx"]], np.int32))
    assert np.allclose(w[0], g["topk_w"], rtol=1e-15, atol=1e-15)
    w = oracle.renorm_selection(p, np.array([[5, 1]], np.int32))
    assert np.allclose(w[0], [0.4, 0.6], rtol=1e-15, atol=1e-15)
    # a pair that is not the top-2: renormalised over the chosen two only
    # (dividing by the sum over all E would give 0.1 each)
    w = oracle.renorm_selection(p, np.array([[0, 2]], np.int32))
    assert np.array_equal(w[0], [0.5, 0.5])
    w = oracle.renorm_selection(p, np.array([[2, 6]], np.int32))
    assert np.allclose(w[0], [2 / 3, 1 / 3], rtol=1e-15)
    # one expert: weight 1 whatever its probability
    w = oracle.renorm_selection(p, np.array([[7]], np.int32))
    assert w[0, 0] == 1.0


def test_forward_with_own_selection_is_bit_equal():
    for cf in (None, 0.75):
        w, inp = tiny_inputs(E=5, T=40)
        a = oracle.forward(inp, k=2, capacity_factor=cf)
        b = oracle.forward(inp, k=2, capacity_factor=cf,
                           selection=a["topk_idx"])
        for key in ("topk_idx", "topk_w", "counts", "kept", "offsets",
                    "slot_token", "slot_of", "f", "p", "y"):
            assert np.array_equal(a[key], b[key]), (cf, key)
        assert a["l_aux"] == b["l_aux"]


def test_forward_with_foreign_selection_follows_definition():
    # Every token takes experts (t mod E, (t + 2) mod E), mostly not its own
    # top-2: y_t = sum_j p_sel_j / (sum p_sel) * FFN_sel_j(x_t) by torch's
    # float64 Linear -> GELU -> Linear, and the counts follow the selection.
    E, T = 5, 30
    w, inp = tiny_inputs(E=E, T=T)
    sel = np.stack([np.arange(T) % E, (np.arange(T) + 2) % E], 1).astype(
        np.int32)
    out = oracle.forward(inp, k=2, selection=sel)
    logits = torch.nn.functional.linear(inp["x"].double(),
                                        inp["wr"].double(),
                                        inp["br"].double())
    p = torch.softmax(logits, -1).numpy()
    assert np.array_equal(out["counts"], np.bincount(sel.ravel(),
                                                     minlength=E))
    for t in range(T):
        ps = p[t, sel[t]]
        ref = 0
        for j in range(2):
            e = sel[t, j]
            ref = ref + ps[j] / ps.sum() * dense_ffn_torch(
                inp["x"][t:t + 1], inp["w1"][e], inp["b1"][e], inp["w2"][e],
                inp["b2"][e])[0]
        assert np.allclose(out["topk_w"][t], ps / ps.sum(), rtol=1e-13)
        assert np.allclose(out["y"][t], ref, rtol=1e-12, atol=1e-13)


def test_expert_choice_with_own_selection_is_bit_equal():
    w, inp = tiny_inputs(E=4, T=24)
    a = oracle.forward_expert_choice(inp, capacity=5)
    b = oracle.forward_expert_choice(inp, capacity=5,
                                     selection=a["slot_token"])
    for key in ("slot_token", "slot_of", "gate", "picks", "y"):
        assert np.array_equal(a[key], b[key]), key


def test_expert_choice_with_foreign_selection_follows_definition():
    # Expert e picks tokens e, e+4, e+8 (ascending): y_t sums p[t,e] *
    # FFN_e(x_t) over the experts that picked t, unrenormalised.
    E, T, C = 4, 20, 3
    w, inp = tiny_inputs(E=E, T=T)
    sel = np.concatenate([np.arange(C) * E + e for e in range(E)]).astype(
        np.int32)
    out = oracle.forward_expert_choice(inp, capacity=C, selection=sel)
    logits = torch.nn.functional.linear(inp["x"].double(),
                                        inp["wr"].double(),
                                        inp["br"].double())
    p = torch.softmax(logits, -1).numpy()
    ref = np.zeros((T, inp["x"].shape[1]))
    for e in range(E):
        toks = sel[e * C:(e + 1) * C]
        ref[toks] += p[toks, e:e + 1] * dense_ffn_torch(
            inp["x"][toks], inp["w1"][e], inp["b1"][e], inp["w2"][e],
            inp["b2"][e])
        for r, t in enumerate(toks):
            assert out["slot_of"][t, e] == e * C + r
    assert np.allclose(out["y"], ref, rtol=1e-12, atol=1e-13)
    assert np.array_equal(out["picks"], (np.arange(T) < E * C).astype(
        np.int32))
