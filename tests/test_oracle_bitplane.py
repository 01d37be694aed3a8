"""Pins for the bitplane (nested) quantizer of oracle/bitplane.py: the PagedMoE
page's prefix-compatible tree codebook and bitplane layout (Abstract) read on
top of Eq. 2 at 8 bits.

The pins do not re-run the oracle's own formulas: hand-worked vectors, exact
rational arithmetic for the codes and the error bound, an independent
big-integer unpacker reassembling u8 from the planes, the nesting of the
pages, and the reduction to Eq. 2 at depth 8."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import bitplane, moe, quant
from test_oracle_quant import bigint_unpack, exact_round_half_even, f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def vectors():
    with open(os.path.join(GOLDEN, "bitplane_vectors.json")) as f:
        return json.load(f)["vectors"]


@pytest.mark.parametrize("vec", vectors(), ids=lambda v: v["id"])
def test_hand_vectors(vec):
    w = torch.tensor([f32(x) for x in vec["w"]], dtype=torch.float32)
    m = quant.expert_absmax([w])
    s8 = bitplane.scale8(m)
    assert s8 == float(vec["s8"])
    u = bitplane.u8(w, s8)
    assert u.tolist() == vec["u8"]
    for b, c in vec["c"].items():
        b = int(b)
        assert bitplane.centre2(bitplane.prefix(u, b), b).tolist() == c, b
    for b, wh in vec["w_hat"].items():
        assert bitplane.dequant(w, s8, int(b)).tolist() == [float(x) for x in wh]
    # the planes of one row, packed
    for j, byte in enumerate(vec["plane_bytes"]):
        row = quant.pack_rows(bitplane.plane(u, j)[None, :], 1)[0]
        assert row.numel() == 16
        assert row[0].item() == int(byte, 16), j
        assert int(row[1:].sum()) == 0


def _expert(seed, F=128, d=256, std=0.02):
    g = torch.Generator().manual_seed(seed)
    w1 = torch.randn(F, d, generator=g) * std
    w3 = torch.randn(F, d, generator=g) * std
    w2 = torch.randn(d, F, generator=g) * std
    return w1, w3, w2


def test_codes_are_eq2_at_8_bits_exactly():
    # u8 from exact rational rounding of w / s8 (half to even), clamped
    w1, _, _ = _expert(1)
    w = w1.reshape(-1)[:4000]
    m = quant.expert_absmax([w])
    s8 = bitplane.scale8(m)
    u = bitplane.u8(w, s8).tolist()
    for wi, ui in zip(w.tolist(), u):
        q = max(-127, min(127, exact_round_half_even(Fraction(wi) / Fraction(s8))))
        assert ui == q + 128


@pytest.mark.parametrize("b", bitplane.DEPTHS)
def test_error_bound_and_node_containment(b):
    # |w - w^| <= s8 2^(7-b) exactly, and q8 lies inside the node whose
    # centre is used
    w1, w3, w2 = _expert(2)
    w = torch.cat([w1.reshape(-1), w2.reshape(-1)])[:6000]
    m = quant.expert_absmax([w])
    s8 = bitplane.scale8(m)
    wh = bitplane.dequant(w, s8, b).tolist()
    u = bitplane.u8(w, s8)
    p = bitplane.prefix(u, b).tolist()
    bound = Fraction(s8) * Fraction(2) ** (7 - b)
    for wi, whi, ui, pi in zip(w.tolist(), wh, u.tolist(), p):
        assert abs(Fraction(wi) - Fraction(whi)) <= bound
        lo, hi = pi << (8 - b), ((pi + 1) << (8 - b)) - 1
        assert lo <= ui <= hi
        assert Fraction(whi) == Fraction(s8) * (Fraction(lo + hi, 2) - 128)


def test_depth_8_is_eq2_at_8_bits():
    w1, w3, w2 = _expert(3)
    m = quant.expert_absmax((w1, w3, w2))
    s8 = bitplane.scale8(m)
    for w in (w1, w3, w2):
        assert torch.equal(bitplane.dequant(w, s8, 8), quant.dequant(w, quant.scale(m, 8), 8))
    assert bitplane.loss((w1, w3, w2), m, 8) == quant.loss((w1, w3, w2), m, 8)


def test_pages_are_nested_and_planes_reassemble_u8():
    w1, w3, w2 = _expert(4, F=128, d=256)
    F, d = w1.shape
    m = quant.expert_absmax((w1, w3, w2))
    s8 = bitplane.scale8(m)
    full = bitplane.expert_page(w1, w3, w2, 8, s8)
    plane_bytes = 3 * F * d // 8
    assert full.numel() == bitplane.page_nbytes(d, F, 8) == 8 * plane_bytes
    for b in bitplane.DEPTHS:
        page = bitplane.expert_page(w1, w3, w2, b, s8)
        assert page.numel() == bitplane.page_nbytes(d, F, b)
        assert torch.equal(page[:b * plane_bytes], full[:b * plane_bytes]), b
    # independent reassembly of u8 from the planes of the full page, row by
    # row with a big-integer unpacker
    fb = bytes(full.tolist())
    for mi, (w, rows, K) in enumerate(((w1, F, d), (w3, F, d), (w2, d, F))):
        want = bitplane.u8(w, s8)
        mat_off = sum((F * d, F * d, d * F)[:mi]) // 8
        for r in (0, 7, rows - 1):
            got = [0] * K
            for j in range(8):
                at = j * plane_bytes + mat_off + r * K // 8
                bits = bigint_unpack(fb[at:at + K // 8], 1, K)
                got = [g | (bit << (7 - j)) for g, bit in zip(got, bits)]
            assert got == want[r].tolist(), (mi, r)


def test_loss_decreases_with_depth_on_gaussian_weights():
    w1, w3, w2 = _expert(5)
    m = quant.expert_absmax((w1, w3, w2))
    L = [bitplane.loss((w1, w3, w2), m, b) for b in bitplane.DEPTHS]
    assert all(a > b for a, b in zip(L, L[1:])), L
    # depth b's error is uniform over nodes of 2^(8-b) codes once they are
    # small against the spread of the weights: about s8^2 4^(8-b) / 12
    s8 = bitplane.scale8(m)
    for b in (5, 6, 7):
        assert L[b - 1] == pytest.approx(s8 * s8 * 4.0 ** (8 - b) / 12, rel=0.05)


def test_depth_8_forward_is_the_8_bit_eq2_forward():
    g = torch.Generator().manual_seed(6)
    E, d, F, k, T = 3, 128, 128, 2, 5
    w1 = torch.randn(E, F, d, generator=g) * 0.05
    w3 = torch.randn(E, F, d, generator=g) * 0.05
    w2 = torch.randn(E, d, F, generator=g) * 0.05
    x = torch.randn(T, d, generator=g).to(torch.bfloat16)
    logits = torch.randn(T, E, generator=g)
    y8 = moe.forward(x, logits, k, bitplane.experts(w1, w3, w2, [8] * E))
    yq = moe.moe_forward_quantized(x, logits, k, w1, w3, w2, [8] * E)
    assert torch.equal(y8, yq)
    y3 = moe.forward(x, logits, k, bitplane.experts(w1, w3, w2, [3] * E))
    assert float((y3 - yq).norm() / yq.norm()) > 1e-3      # a coarser layer, not the same one
