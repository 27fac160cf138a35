"""The checker's own rules, on the CPU: the logit-gap criterion that marks a
near-tie token as decided must rest on a real bound of fp32 logit error."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import logit_decided


def _bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16)


def _fp32_logits_orders(x: torch.Tensor, wr: torch.Tensor, chunks: int):
    """fp32 logits summed in three different orders: forward over d,
    backward over d, and `chunks` depth-range partials added in order."""
    xf, wf = x.float(), wr.float()
    prod = xf[:, None, :] * wf[None, :, :]           # exact for bf16 inputs
    fwd = torch.zeros(prod.shape[:2])
    for i in range(prod.shape[2]):
        fwd = fwd + prod[:, :, i]
    bwd = torch.zeros(prod.shape[:2])
    for i in reversed(range(prod.shape[2])):
        bwd = bwd + prod[:, :, i]
    parts = [p.sum(dim=2) for p in torch.chunk(prod, chunks, dim=2)]
    split = parts[0]
    for p in parts[1:]:
        split = split + p
    return [fwd.double().numpy(), bwd.double().numpy(),
            split.double().numpy()]


def test_logit_bound_holds_for_fp32_sums():
    """Every fp32 summation order lands within the bound that
    logit_decided uses, on every (token, expert) pair."""
    rng = np.random.default_rng(5)
    T, E, d = 48, 8, 512
    x = _bf16(rng.standard_normal((T, d)))
    wr = _bf16(rng.standard_normal((E, d)) * 0.3)
    logits, _ = oracle.router(x, wr)
    xd = x.double().numpy()
    wd = wr.double().numpy()
    bound = (2 * d + 64) * 2.0 ** -23 * (np.abs(xd) @ np.abs(wd).T) \
        + 4 * 2.0 ** -23 * np.abs(logits)
    for got in _fp32_logits_orders(x, wr, chunks=8):
        assert np.all(np.abs(got - logits) <= bound)


def test_sharp_router_ties_in_probability_are_decided_by_logits():
    """A token whose 2nd and 3rd probabilities are both tiny (margin far
    under 1e-4) but whose logits are several units apart is decided; a
    true logit tie is not."""
    d, E = 64, 4
    wr = np.zeros((E, d), np.float32)
    # logits of token 0: 40, 10, 4, 0 (p2, p3 ~ 1e-13, 1e-16)
    # logits of token 1: 40, 10, 10, 0 (an exact tie for the 2nd pick)
    for e in range(E):
        wr[e, e] = 1.0
    x = np.zeros((2, d), np.float32)
    x[0, :4] = [40.0, 10.0, 4.0, 0.0]
    x[1, :4] = [40.0, 10.0, 10.0, 0.0]
    inp = {"x": _bf16(x), "wr": _bf16(wr)}
    logits, probs = oracle.router(inp["x"], inp["wr"])
    _, _, margin = oracle.topk(probs, 2)
    assert margin[0] < 1e-4 and margin[1] == 0.0
    decided = logit_decided(inp, logits, 2)
    assert decided.tolist() == [True, False]


def test_logit_decided_with_biases_and_k_equal_e():
    """The router and balancing biases widen the bound (they are terms of
    the fp32 sum); with k = E every token is decided."""
    w = workloads.scaled(workloads.get("deepseek_v3"), T=64, d=256, E=16,
                         k=4, d_ff=64)
    inp = workloads.make_inputs(w, "cpu")
    logits, probs = oracle.router(inp["x"], inp["wr"], inp.get("br"),
                                  inp.get("ebias"))
    with_b = logit_decided(inp, logits, w.k)
    bare = dict(inp)
    bare["ebias"] = None
    bare["br"] = None
    without_b = logit_decided(bare, logits, w.k)
    # a bigger bound can only mark fewer tokens decided
    assert np.all(without_b[with_b])
    assert logit_decided(inp, logits, w.E).all()
