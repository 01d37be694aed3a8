"""Pins for the plain C++ CPU oracle (oracle/cpu_oracle.cpp through
oracle/c_oracle.py): Eq. 2 of the PagedWeight page (section "Implementation
Details"), Eq. 1 (section "Quality-Aware Quantization") and the forward pass
of section "Dynamic Paging".

As for the Python oracle, the pins do not re-run the oracle's formulas:
hand-worked vectors, exact rational rounding, a big-integer unpacker,
enumeration of every allocation, torch's own dense layers on a lossless
layer, scalar loops on a tiny one, and invariants. The two oracles are
written independently; they are also compared with each other (bit-exact
codes, scales, pages and allocations; outputs to 1e-12).
"""
import json
import math
import os
import random
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

import synth
from oracle import alloc, c_oracle as C, moe, quant
from test_oracle_moe import dense_reference, on_grid_layer
from test_oracle_quant import bigint_unpack, exact_round_half_even, f32, load_vectors, nearest_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("vec", load_vectors(), ids=lambda v: v["id"])
def test_hand_vectors(vec):
    b = vec["b"]
    w = np.array([f32(x) for x in vec["w"]], dtype=np.float32)
    s = C.scale(C.absmax(w), b)
    if "s" in vec:
        assert s == float(vec["s"])
    else:
        assert np.float32(s).tobytes()[::-1].hex() == vec["s_hex"]
    q = C.codes(w, s, b)
    assert q.tolist() == vec["q"]
    packed = C.pack_rows(q.reshape(1, -1), b)
    assert packed.shape == (1, 128 * b // 8)
    prefix = bytes.fromhex(vec["packed_prefix"])
    assert bytes(packed[0, :len(prefix)].tolist()) == prefix
    assert not packed[0, len(prefix):].any()


def test_e4_exact_quotient_not_fp32_division():
    assert C.codes(np.array([f32("0.35")], dtype=np.float32), f32("0.1"), 4).tolist() == [3]


def test_codes_match_exact_rational_rounding():
    rng = random.Random(101)
    for b in (3, 4, 8):
        qm = C.qmax(b)
        ws, want = [], []
        m = f32(rng.uniform(1e-3, 10.0))
        s = C.scale(m, b)
        for _ in range(600):
            if rng.random() < 0.5:
                w = f32(rng.uniform(-m, m))
            else:   # on and next to half-grid points
                k = rng.randint(-qm, qm - 1) + 0.5
                w = float(np.nextafter(np.float32(k * s), np.float32(rng.choice([-np.inf, np.inf]))))
                if rng.random() < 0.3:
                    w = f32(k * s)
                w = max(-m, min(m, w))
            ws.append(w)
            want.append(max(-qm, min(qm, exact_round_half_even(Fraction(w) / Fraction(s)))))
        assert C.codes(np.array(ws, dtype=np.float32), s, b).tolist() == want


def test_codes_clamp_to_qmax():
    # values beyond +-qmax s (not reachable from an expert's own maximum)
    # clamp: Eq. 2's codes stay within +-(2^(b-1) - 1)
    w = np.array([10.0, -10.0, 3.49, -3.51, 7.6], dtype=np.float32)
    assert C.codes(w, 1.0, 3).tolist() == [3, -3, 3, -3, 3]
    assert C.codes(w, 1.0, 4).tolist() == [7, -7, 3, -4, 7]
    assert C.codes(w * 20, 1.0, 8).tolist() == [127, -127, 70, -70, 127]


def test_scale_is_nearest_fp32_of_exact_quotient():
    rng = random.Random(102)
    for b in (3, 4, 8):
        for _ in range(200):
            m = f32(rng.uniform(1e-6, 1e3))
            assert C.scale(m, b) == nearest_f32(Fraction(m) / C.qmax(b))
    assert C.scale(0.0, 3) == 0.0


def test_zero_expert():
    z = np.zeros((8, 128), dtype=np.float32)
    s, q, page = C.quantize_expert(z, z, z.T.copy(), 4)
    assert s == 0.0 and not q.any()
    # every stored code is the offset 2^(b-1) (nibbles of 8); W2's 128 rows
    # of 8 codes are padded with zero codes to 128 (4 + 60 bytes)
    assert set(page[:2 * 8 * 128 // 2].tolist()) == {0x88}
    w2_rows = page[1024:1024 + 128 * 64].reshape(128, 64)
    assert set(w2_rows[:, :4].reshape(-1).tolist()) == {0x88} and not w2_rows[:, 4:].any()
    assert C.loss(z, z, z.T.copy(), 3) == 0.0


@pytest.mark.parametrize("b", (3, 4, 8))
@pytest.mark.parametrize("K", (7, 128, 200, 256))
def test_pack_against_bigint_unpacker(b, K):
    rng = np.random.default_rng(b * 100 + K)
    qm = C.qmax(b)
    q = rng.integers(-qm - 1, qm + 1, size=(4, K)).clip(-(2 ** (b - 1)), 2 ** (b - 1) - 1).astype(np.int8)
    packed = C.pack_rows(q, b)
    Kp = -(-K // 128) * 128
    assert packed.shape == (4, Kp * b // 8)
    for r in range(4):
        got = bigint_unpack(bytes(packed[r].tolist()), b, Kp)
        assert got[:K] == [int(v) + 2 ** (b - 1) for v in q[r]]
        assert all(v == 0 for v in got[K:])


def test_page_layout_rows_from_exact_rounding():
    d, F = 128, 256
    g = torch.Generator().manual_seed(55)
    w1 = torch.randn(F, d, generator=g) * 0.02
    w3 = torch.randn(F, d, generator=g) * 0.02
    w2 = torch.randn(d, F, generator=g) * 0.02
    w2[3, 4] = 0.3   # the expert's largest weight sits in W2
    for b in (3, 4, 8):
        s, _, page = C.quantize_expert(w1, w3, w2, b)
        assert s == nearest_f32(Fraction(f32(0.3)) / C.qmax(b))
        assert page.size == C.page_bytes(d, F, b) == 3 * d * F * b // 8
        pb = bytes(page.tolist())
        m1 = F * d * b // 8
        for mat, base, rows, K in ((w1, 0, (0, 99, F - 1), d), (w3, m1, (0, 17, F - 1), d),
                                   (w2, 2 * m1, (0, 3, d - 1), F)):
            rb = K * b // 8
            for r in rows:
                got = bigint_unpack(pb[base + r * rb:base + (r + 1) * rb], b, K)
                want = [exact_round_half_even(Fraction(float(v)) / Fraction(s)) + 2 ** (b - 1)
                        for v in mat[r].tolist()]
                assert got == want, (b, r)


def test_page_padding_to_256_bytes():
    # d = 64, F = 96 at 3 bits: rows pad to 128 codes (48 bytes); raw
    # 2 * 96 * 48 + 64 * 48 = 12288 bytes, already a multiple of 256;
    # d = 8, F = 8 at 3 bits: 24 rows of 48 bytes = 1152 -> 1280
    assert C.page_bytes(64, 96, 3) == 12288
    assert C.page_bytes(8, 8, 3) == 1280


def test_loss_closed_forms():
    w = np.array([f32(x) for x in ["0.75", "-0.375", "0.125", "0.1", "-0.625", "0"]], dtype=np.float32)
    z = np.zeros((1, 6), dtype=np.float32)
    # E1 at 3 bits: errors 0, 0.125, 0.125, fp32(0.1), -0.125, 0 over 18
    # weights (W3 and W2 are zero rows here)
    got = C.loss(w.reshape(1, 6), z, z.reshape(6, 1).copy(), 3)
    assert got == pytest.approx((3 * 0.125 ** 2 + f32("0.1") ** 2) / 18, rel=1e-15)
    grid = (np.array([[-7, -3, 0, 1, 5, 7]], dtype=np.float32) * 0.125)
    assert C.loss(grid, grid, grid.reshape(6, 1).copy(), 4) == 0.0


def test_loss_uniform_data_is_s2_over_12():
    w = torch.linspace(-1.0, 1.0, 3 * 1024 * 512, dtype=torch.float64).float().reshape(3, 512, 1024)
    for b in (3, 4, 8):
        s = C.scale(1.0, b)
        got = C.loss(w[0], w[1], w[2].T.contiguous(), b)
        assert got == pytest.approx(s * s / 12, rel=5e-3)


def golden_alloc():
    with open(os.path.join(GOLDEN, "eq1_allocation.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("solver", [C.allocate, C.allocate_brute])
def test_allocation_hand_worked_example(solver):
    g = golden_alloc()
    for case in g["cases"]:
        if case.get("infeasible"):
            with pytest.raises(C.Infeasible):
                solver(g["p"], g["L"], g["W"], case["B"])
            continue
        bits, obj = solver(g["p"], g["L"], g["W"], case["B"])
        assert bits == case["bits"], case
        assert obj == pytest.approx(case["objective"], rel=1e-12)


def test_allocation_dp_equals_enumeration_and_python_oracle():
    rng = random.Random(103)
    for trial in range(250):
        E = rng.randint(1, 7)
        W = [rng.choice([4, 6, 10])] * E if trial % 2 else [rng.choice([2, 3, 4, 6]) for _ in range(E)]
        p = [rng.random() for _ in range(E)]
        L = []
        for _ in range(E):
            l8 = rng.uniform(1e-4, 1e-2)
            l4 = l8 + rng.uniform(1e-3, 0.5)
            L.append([l4 + rng.uniform(1e-3, 1.0), l4, l8])
        B = rng.randint(3 * sum(W) - 2, 8 * sum(W) + 2)
        if 3 * sum(W) > B:
            for fn in (C.allocate, C.allocate_brute):
                with pytest.raises(C.Infeasible):
                    fn(p, L, W, B)
            continue
        b1, o1 = C.allocate_brute(p, L, W, B)
        b2, o2 = C.allocate(p, L, W, B)
        assert sum(b * w for b, w in zip(b2, W)) <= B
        assert o2 == o1 and b2 == b1, (trial, b1, b2)
        b3, o3 = alloc.solve_dp(p, L, W, B)
        assert b3 == b2 and o3 == o2


def test_allocation_exact_ties_follow_the_stated_conventions():
    """Several optimal allocations (worked by hand, W = 1, p = 1 each):
    with L = (1, 0.5, 0) per expert and B = 11, (8, 3), (3, 8) and (4, 4)
    all cost 1.0; the fewest bits, (4, 4), is taken. With L = (1, 0.6, 0),
    (4, 4) costs 1.2 and (8, 3) and (3, 8) tie at 1.0 with 11 bits each: the
    DP keeps the larger width at the later expert, (3, 8); enumeration takes
    the larger width at the lower index, (8, 3)."""
    p, W = [1.0, 1.0], [1, 1]
    for fn in (C.allocate, C.allocate_brute):
        assert fn(p, [[1.0, 0.5, 0.0]] * 2, W, 11) == ([4, 4], 1.0)
    assert C.allocate(p, [[1.0, 0.6, 0.0]] * 2, W, 11) == ([3, 8], 1.0)
    assert C.allocate_brute(p, [[1.0, 0.6, 0.0]] * 2, W, 11) == ([8, 3], 1.0)


def test_allocation_identical_experts_follow_importance():
    # equal W and L: the more important expert never gets fewer bits
    E = 10
    p = [1.0 / (e + 1) for e in range(E)]
    L = [[0.5, 0.2, 0.01]] * E
    for avg in (3, 3.5, 4, 5, 6, 8):
        bits, _ = C.allocate(p, L, [8] * E, int(avg * 8 * E))
        assert all(bits[e] >= bits[e + 1] for e in range(E - 1)), (avg, bits)


def test_allocation_over_several_layers():
    """One budget over two or three layers: enumeration over the union of
    their experts (importances times the layer weights) and the Python
    oracle's solver give the same bits and objective."""
    rng = random.Random(107)
    for trial in range(60):
        n = rng.randint(2, 3)
        ps, Ls, Ws = [], [], []
        for _ in range(n):
            E = rng.randint(1, 3)
            ps.append([rng.random() for _ in range(E)])
            Ls.append([[l4 + rng.uniform(1e-3, 1.0), l4, l4 - rng.uniform(1e-4, 1e-3)]
                       for l4 in (rng.uniform(0.01, 0.5) for _ in range(E))])
            Ws.append([rng.choice([2, 3, 4])] * E)
        lw = [rng.uniform(0.5, 2.0) for _ in range(n)]
        tot = sum(sum(W) for W in Ws)
        B = rng.randint(3 * tot, 8 * tot)
        got, obj = C.allocate_layers(ps, Ls, Ws, B, lw)
        flat_p = [lw[l] * v for l in range(n) for v in ps[l]]
        flat_L = [row for l in range(n) for row in Ls[l]]
        flat_W = [v for W in Ws for v in W]
        want_bits, want_obj = C.allocate_brute(flat_p, flat_L, flat_W, B)
        # random problems have a unique optimum; both sum the objective in
        # expert order
        assert [b for bl in got for b in bl] == want_bits, trial
        assert obj == want_obj
        py_bits, py_obj = alloc.solve_layers(ps, Ls, Ws, B, lw)
        assert obj == pytest.approx(py_obj, rel=1e-12, abs=0)


def test_router_ties_and_closed_forms():
    ids, g = C.route(np.array([[0.5, 2.0, -1.0, 2.0]], dtype=np.float32), 2)
    assert ids.tolist() == [[1, 3]]
    ex = [math.exp(v - 2.0) for v in (0.5, 2.0, -1.0, 2.0)]
    assert g[0].tolist() == pytest.approx([ex[1] / sum(ex), ex[3] / sum(ex)], rel=1e-15)
    ids, g = C.route(np.zeros((3, 8), dtype=np.float32), 2)
    assert ids.tolist() == [[0, 1]] * 3 and np.all(g == 0.125)
    _, g = C.route(np.zeros((3, 8), dtype=np.float32), 2, renorm=True)
    assert np.all(g == 0.5)


def test_router_matches_topk_and_softmax():
    gen = torch.Generator().manual_seed(104)
    logits = torch.randn(40, 24, generator=gen)
    ids, w = C.route(logits, 5)
    ref = torch.topk(logits, 5, dim=1)
    assert np.array_equal(ids, ref.indices.numpy())
    sm = torch.softmax(logits.double(), dim=1)
    assert np.allclose(w, torch.gather(sm, 1, ref.indices).numpy(), rtol=1e-14, atol=0)


def test_forward_lossless_layer_matches_dense_layers():
    E, d, F, k, T = 4, 32, 48, 2, 6
    w1, w3, w2 = on_grid_layer(E, d, F, 3)
    g = torch.Generator().manual_seed(105)
    x = torch.randn(T, d, generator=g).to(torch.bfloat16).float()
    logits = torch.randn(T, E, generator=g)
    y = C.moe_forward_quantized(x, logits, k, w1, w3, w2, [8] * E)
    ref = dense_reference(x, logits, k, w1, w3, w2).numpy()
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_forward_single_expert_is_dense_swiglu():
    d, F, T = 16, 24, 5
    w1, w3, w2 = on_grid_layer(1, d, F, 5)
    x = torch.randn(T, d).to(torch.bfloat16).float()
    y = C.moe_forward_quantized(x, torch.zeros(T, 1), 1, w1, w3, w2, [8])
    ref = Fn.linear(Fn.silu(Fn.linear(x.double(), w1[0].double())) * Fn.linear(x.double(), w3[0].double()),
                    w2[0].double()).numpy()
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-13)


def test_forward_scalar_loops_tiny():
    """Scalar re-evaluation with math.exp and Python's round() (half to
    even) on a 2-token, 3-expert layer at 3, 8 and 4 bits."""
    E, d, F, k = 3, 4, 3, 2
    g = torch.Generator().manual_seed(106)
    w1 = torch.randn(E, F, d, generator=g) * 0.3
    w3 = torch.randn(E, F, d, generator=g) * 0.3
    w2 = torch.randn(E, d, F, generator=g) * 0.3
    x = torch.randn(2, d, generator=g).to(torch.bfloat16).float()
    logits = torch.tensor([[0.1, 0.7, -0.2], [1.5, -1.0, 0.4]])
    bits = [3, 8, 4]
    y = C.moe_forward_quantized(x, logits, k, w1, w3, w2, bits)
    for t in range(2):
        ls = logits[t].tolist()
        order = sorted(range(E), key=lambda e: (-np.float32(ls[e]), e))[:k]
        den = sum(math.exp(v - max(ls)) for v in ls)
        want = [0.0] * d
        for e in order:
            qm = 2 ** (bits[e] - 1) - 1
            m = max(abs(v) for M in (w1[e], w3[e], w2[e]) for v in M.reshape(-1).tolist())
            s = float(np.float32(m / qm))

            def qd(v):
                return s * max(-qm, min(qm, round(v / s)))
            h = []
            for f in range(F):
                a = sum(qd(w1[e, f, i].item()) * x[t, i].item() for i in range(d))
                c = sum(qd(w3[e, f, i].item()) * x[t, i].item() for i in range(d))
                h.append(a / (1 + math.exp(-a)) * c)
            gw = math.exp(ls[e] - max(ls)) / den
            for i in range(d):
                want[i] += gw * sum(qd(w2[e, i, f].item()) * h[f] for f in range(F))
        assert y[t].tolist() == pytest.approx(want, rel=1e-12, abs=1e-14)


def test_forward_thread_count_does_not_change_the_result():
    wl = synth.WORKLOADS["tiny"].scaled(E=6, d=128, F=128, k=2, T=9, bits=(8, 4, 3, 3, 4, 8))
    w1, w3, w2 = synth.expert_weights(wl)
    x, logits = synth.tokens(wl)
    y1 = C.moe_forward_quantized(x, logits, 2, w1, w3, w2, wl.bits, nthreads=1)
    y4 = C.moe_forward_quantized(x, logits, 2, w1, w3, w2, wl.bits, nthreads=4)
    assert np.array_equal(y1, y4)


@pytest.mark.parametrize("renorm", [False, True])
def test_agrees_with_the_python_oracle(renorm):
    """Seeded layer with 0.1% outliers x20 (the fine-grained decode
    workload's weight recipe) at 3, 4 and 8 bits: scales, pages and loss
    rows against oracle.quant, y against oracle.moe."""
    wl = synth.WORKLOADS["decode_fine"].scaled(name="c_vs_py", E=6, d=256, F=128, k=3, T=11,
                                               bits=(3, 4, 8, 3, 8, 4))
    w1, w3, w2 = synth.expert_weights(wl)
    x, logits = synth.tokens(wl)
    for e in range(wl.E):
        b = wl.bits[e]
        s, _, page = C.quantize_expert(w1[e], w3[e], w2[e], b)
        m = quant.expert_absmax((w1[e], w3[e], w2[e]))
        assert s == quant.scale(m, b)
        assert np.array_equal(page, quant.expert_page(w1[e], w3[e], w2[e], b, s).numpy())
        for bb in (3, 4, 8):
            lp = quant.loss((w1[e], w3[e], w2[e]), m, bb)
            assert C.loss(w1[e], w3[e], w2[e], bb) == pytest.approx(lp, rel=1e-12)
    y = C.moe_forward_quantized(x, logits, wl.k, w1, w3, w2, wl.bits, renorm=renorm)
    yp = moe.moe_forward_quantized(x, logits, wl.k, w1, w3, w2, wl.bits, renorm=renorm).numpy()
    assert np.abs(y - yp).max() <= 1e-12 * np.abs(yp).max()
