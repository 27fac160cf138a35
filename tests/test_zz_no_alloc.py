"""moe_forward_noalloc (the static-scratch entry point, for callers that
cannot allocate) against moe_forward with a caller workspace, through the C
ABI on MI355X: two calls in a row on the same GPU, the second with fewer
tokens, each bit-identical to moe_forward's results; the same forward
captured in a HIP graph and replayed with new inputs; a shape whose scratch
exceeds the static buffer is refused before any GPU work."""
import numpy as np
import pytest
import torch

import sparse_mixture_experts_50_amd as moe
import workloads
from sparse_mixture_experts_50_amd import _lib
from workloads import scaled

from parity import check_layer, device, inputs_on

pytestmark = pytest.mark.gpu

KEYS = ("topk_idx", "topk_w", "counts", "kept", "offsets", "slot_token",
        "slot_of", "f", "p", "l_aux", "monitor")


def _host(r, y):
    out = {k: getattr(r, k).cpu().numpy().copy() for k in KEYS}
    out["y"] = y.float().cpu().numpy().astype(np.float64)
    return out


def test_noalloc_matches_workspace_forward_twice():
    dev = device()
    w = workloads.WORKLOADS["mixtral_decode"]
    inp = inputs_on(w, dev)
    weights = moe.Weights.from_dict(inp)
    layer = moe.MoeLayer(weights, w.k, w.capacity_factor, w.alpha)
    # second call: fewer tokens, other x, same weights
    x2 = workloads.make_x(scaled(w, T=20), dev, 7)
    cases = [(inp["x"], w), (x2, scaled(w, T=20))]
    # every buffer the calls write, allocated before the first call
    bufs = []
    for x, wl in cases:
        T = x.shape[0]
        desc = layer.desc(T)
        assert moe.moe_workspace_size(desc) <= _lib.NOALLOC_SCRATCH_BYTES
        bufs.append((desc, moe.Routing(T, w.E, w.k, dev),
                     torch.empty((T, w.d), dtype=torch.bfloat16, device=dev)))
    torch.cuda.synchronize()
    got = []
    for (x, wl), (desc, r, y) in zip(cases, bufs):
        moe.moe_forward_noalloc(desc, x, weights, r, y)
        torch.cuda.synchronize()
        got.append(_host(r, y))
    for (x, wl), g in zip(cases, got):
        y_ref, r_ref = layer.forward(x)
        torch.cuda.synchronize()
        ref = _host(r_ref, y_ref)
        for k in KEYS + ("y",):
            assert np.array_equal(g[k], ref[k]), (wl.T, k)
        # and the oracle's rules on the no-allocation results
        g_in = dict(inp)
        g_in["x"] = x
        check_layer(wl, g_in, dict(g, layer=layer))


def test_noalloc_forward_replays_in_a_hip_graph():
    """The callers moe_forward_noalloc is for include HIP graph capture: the
    decode-shaped forward captured once (torch.cuda.graph, on its capture
    stream: the layer's kernels only, no allocation and no memset node),
    then replayed five times with a new x copied into the captured input
    before each replay and eager work between the replays; every replay's
    routing, statistics and output bit-identical to the eager moe_forward
    (with a workspace) on the same x."""
    dev = device()
    w = workloads.WORKLOADS["mixtral_decode"]
    inp = inputs_on(w, dev)
    weights = moe.Weights.from_dict(inp)
    layer = moe.MoeLayer(weights, w.k, w.capacity_factor, w.alpha)
    desc = layer.desc(w.T)
    x_static = inp["x"].clone()
    r = moe.Routing(w.T, w.E, w.k, dev)
    y = torch.empty((w.T, w.d), dtype=torch.bfloat16, device=dev)
    # an eager call first: the scratch's address is looked up outside capture
    moe.moe_forward_noalloc(desc, x_static, weights, r, y)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        moe.moe_forward_noalloc(desc, x_static, weights, r, y)
    torch.cuda.synchronize()
    for i in range(5):
        xi = workloads.make_x(w, dev, 100 + i)
        x_static.copy_(xi)
        graph.replay()
        torch.cuda.synchronize()
        got = _host(r, y)
        y_ref, r_ref = layer.forward(xi)
        torch.cuda.synchronize()
        ref = _host(r_ref, y_ref)
        for k in KEYS + ("y",):
            assert np.array_equal(got[k], ref[k]), (i, k)


def test_noalloc_refuses_a_shape_beyond_the_static_scratch():
    dev = device()
    w = scaled(workloads.WORKLOADS["mixtral_prefill"], T=1024, d=1024,
               d_ff=4096)
    inp = inputs_on(w, dev)
    weights = moe.Weights.from_dict(inp)
    layer = moe.MoeLayer(weights, w.k)
    desc = layer.desc(w.T)
    assert moe.moe_workspace_size(desc) > _lib.NOALLOC_SCRATCH_BYTES
    r = moe.Routing(w.T, w.E, w.k, dev)
    y = torch.full((w.T, w.d), 7.0, dtype=torch.bfloat16, device=dev)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_forward_noalloc(desc, inp["x"], weights, r, y)
    assert ei.value.status == _lib.MOE_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool(torch.all(y == 7.0))          # nothing was enqueued
