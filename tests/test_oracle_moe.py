"""Pins for the oracle router and forward pass (section "Dynamic Paging" of
the PagedWeight page): closed forms, a lossless special case computed with
torch's own dense layers, and invariances of the layer."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

import synth
from oracle import moe, quant


def test_router_ties_go_to_lower_index():
    logits = torch.tensor([[0.5, 2.0, -1.0, 2.0]])
    ids, g = moe.route(logits, 2)
    assert ids.tolist() == [[1, 3]]
    # textbook softmax over all four
    ex = [math.exp(v - 2.0) for v in (0.5, 2.0, -1.0, 2.0)]
    assert g[0].tolist() == pytest.approx([ex[1] / sum(ex), ex[3] / sum(ex)], rel=1e-15)


def test_router_closed_forms():
    ids, g = moe.route(torch.zeros(3, 8), 2)
    assert ids.tolist() == [[0, 1]] * 3
    assert torch.all(g == 0.125)
    _, g = moe.route(torch.zeros(3, 8), 2, renorm=True)
    assert torch.all(g == 0.5)
    # logits (0, ln 3) -> (1/4, 3/4) up to the fp32 rounding of ln 3
    l = torch.tensor([[0.0, math.log(3.0)]])
    ids, g = moe.route(l, 1)
    assert ids.tolist() == [[1]] and g.item() == pytest.approx(0.75, rel=1e-7)


def test_router_matches_topk_on_distinct_logits():
    g = torch.Generator().manual_seed(1)
    logits = torch.randn(50, 16, generator=g)
    ids, w = moe.route(logits, 4)
    ref = torch.topk(logits, 4, dim=1)
    assert torch.equal(ids, ref.indices)
    sm = torch.softmax(logits.double(), dim=1)
    assert torch.allclose(w, torch.gather(sm, 1, ids), rtol=1e-14, atol=0)


def on_grid_layer(E, d, F, seed):
    """Masters that are exactly s * q at 8 bits (q integer, |q| <= 127)."""
    g = torch.Generator().manual_seed(seed)
    mats = []
    for shape in ((E, F, d), (E, F, d), (E, d, F)):
        mats.append(torch.randint(-60, 61, shape, generator=g).float())
    for e in range(E):
        mats[0][e, 0, 0] = 127.0     # make max|w| = 127 * s for each expert
    s = torch.tensor([2.0 ** -9 * (1 + e) for e in range(E)])
    w1 = mats[0] * s.view(E, 1, 1)
    w3 = mats[1] * s.view(E, 1, 1)
    w2 = mats[2] * s.view(E, 1, 1)
    return w1, w3, w2


def dense_reference(x, logits, k, w1, w3, w2):
    """Independent dense evaluation with torch's own layers, float64."""
    x64 = x.double()
    top = torch.topk(logits, k, dim=1)
    gates = torch.softmax(logits.double(), dim=1)
    y = torch.zeros(x.shape, dtype=torch.float64)
    for t in range(x.shape[0]):
        for j in range(k):
            e = int(top.indices[t, j])
            a = Fn.linear(x64[t], w1[e].double())
            c = Fn.linear(x64[t], w3[e].double())
            o = Fn.linear(Fn.silu(a) * c, w2[e].double())
            y[t] += gates[t, e] * o
    return y


def test_lossless_special_case_matches_dense_layers():
    E, d, F, k, T = 4, 32, 48, 2, 6
    w1, w3, w2 = on_grid_layer(E, d, F, 3)
    g = torch.Generator().manual_seed(4)
    x = torch.randn(T, d, generator=g).to(torch.bfloat16).float()
    logits = torch.randn(T, E, generator=g)
    bits = [8] * E
    for e in range(E):   # quantization at 8 bits reproduces the masters
        m = quant.expert_absmax((w1[e], w3[e], w2[e]))
        s = quant.scale(m, 8)
        assert torch.equal(quant.dequant(w1[e], s, 8), w1[e].double())
    y = moe.moe_forward_quantized(x, logits, k, w1, w3, w2, bits)
    ref = dense_reference(x, logits, k, w1, w3, w2)
    assert torch.allclose(y, ref, rtol=1e-12, atol=1e-12 * float(ref.abs().max()))


def test_single_expert_is_dense_swiglu():
    d, F, T = 16, 24, 5
    w1, w3, w2 = on_grid_layer(1, d, F, 5)
    x = torch.randn(T, d).to(torch.bfloat16).float()
    y = moe.moe_forward_quantized(x, torch.zeros(T, 1), 1, w1, w3, w2, [8])
    ref = Fn.linear(Fn.silu(Fn.linear(x.double(), w1[0].double())) *
                    Fn.linear(x.double(), w3[0].double()), w2[0].double())
    assert torch.allclose(y, ref, rtol=1e-12, atol=1e-13)


def small_layer():
    wl = synth.WORKLOADS["tiny"].scaled(E=6, d=128, F=128, k=2, T=7, bits=(8, 4, 3, 3, 4, 8))
    w1, w3, w2 = synth.expert_weights(wl)
    x, logits = synth.tokens(wl)
    return wl, w1, w3, w2, x, logits


def test_zero_input_gives_zero_output():
    wl, w1, w3, w2, x, logits = small_layer()
    y = moe.moe_forward_quantized(torch.zeros_like(x), logits, wl.k, w1, w3, w2, wl.bits)
    assert torch.count_nonzero(y) == 0


def test_token_permutation_invariance():
    wl, w1, w3, w2, x, logits = small_layer()
    y = moe.moe_forward_quantized(x, logits, wl.k, w1, w3, w2, wl.bits)
    perm = torch.randperm(x.shape[0], generator=torch.Generator().manual_seed(9))
    yp = moe.moe_forward_quantized(x[perm], logits[perm], wl.k, w1, w3, w2, wl.bits)
    assert torch.allclose(yp, y[perm], rtol=1e-13, atol=1e-15)


def test_expert_permutation_invariance():
    wl, w1, w3, w2, x, logits = small_layer()
    y = moe.moe_forward_quantized(x, logits, wl.k, w1, w3, w2, wl.bits)
    perm = torch.tensor([3, 0, 5, 1, 4, 2])
    bits = [wl.bits[i] for i in perm.tolist()]
    yp = moe.moe_forward_quantized(x, logits[:, perm], wl.k, w1[perm], w3[perm], w2[perm], bits)
    assert torch.allclose(yp, y, rtol=1e-13, atol=1e-15)


def test_unrouted_expert_does_not_matter():
    wl, w1, w3, w2, x, logits = small_layer()
    logits = logits.clone()
    logits[:, 2] = -100.0      # expert 2 is never chosen
    y = moe.moe_forward_quantized(x, logits, wl.k, w1, w3, w2, wl.bits)
    w1b = w1.clone()
    w1b[2] = torch.randn_like(w1b[2])
    y2 = moe.moe_forward_quantized(x, logits, wl.k, w1b, w3, w2, wl.bits)
    assert torch.equal(y, y2)


def test_output_is_linear_in_up_projection_sign():
    # silu(a) * c: flipping W3 flips c and hence y (quantization is symmetric)
    wl, w1, w3, w2, x, logits = small_layer()
    y = moe.moe_forward_quantized(x, logits, wl.k, w1, w3, w2, wl.bits)
    y2 = moe.moe_forward_quantized(x, logits, wl.k, w1, -w3, w2, wl.bits)
    assert torch.allclose(y2, -y, rtol=1e-14, atol=1e-16)


def test_renorm_weights_sum_to_one():
    _, w = moe.route(torch.randn(20, 9), 3, renorm=True)
    assert torch.allclose(w.sum(1), torch.ones(20, dtype=torch.float64), rtol=1e-15)
    _, w = moe.route(torch.randn(20, 9), 9, renorm=False)
    assert torch.allclose(w.sum(1), torch.ones(20, dtype=torch.float64), rtol=1e-15)


def test_brute_force_scalar_loops_tiny():
    """Scalar re-evaluation with math.exp on a 2-token, 3-expert layer."""
    E, d, F, k = 3, 4, 3, 2
    g = torch.Generator().manual_seed(21)
    w1 = torch.randn(E, F, d, generator=g) * 0.3
    w3 = torch.randn(E, F, d, generator=g) * 0.3
    w2 = torch.randn(E, d, F, generator=g) * 0.3
    x = torch.randn(2, d, generator=g).to(torch.bfloat16).float()
    logits = torch.tensor([[0.1, 0.7, -0.2], [1.5, -1.0, 0.4]])
    bits = [3, 8, 4]
    y = moe.moe_forward_quantized(x, logits, k, w1, w3, w2, bits)
    for t in range(2):
        ls = logits[t].tolist()
        order = sorted(range(E), key=lambda e: (-np.float32(ls[e]), e))[:k]
        den = sum(math.exp(v - max(ls)) for v in ls)
        want = [0.0] * d
        for e in order:
            mats = (w1[e], w3[e], w2[e])
            m = max(abs(v) for M in mats for v in M.reshape(-1).tolist())
            s = float(np.float32(m / (2 ** (bits[e] - 1) - 1)))
            def qd(v):
                q = round(v / s)            # Python round(): half to even
                return s * max(-(2 ** (bits[e] - 1) - 1), min(2 ** (bits[e] - 1) - 1, q))
            h = []
            for f in range(F):
                a = sum(qd(w1[e, f, i].item()) * x[t, i].item() for i in range(d))
                c = sum(qd(w3[e, f, i].item()) * x[t, i].item() for i in range(d))
                h.append(a / (1 + math.exp(-a)) * c)
            gw = math.exp(ls[e] - max(ls)) / den
            for i in range(d):
                want[i] += gw * sum(qd(w2[e, i, f].item()) * h[f] for f in range(F))
        assert y[t].tolist() == pytest.approx(want, rel=1e-12, abs=1e-14)
