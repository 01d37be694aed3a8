"""Pins for the oracle quantizer (Eq. 2 of the PagedWeight page, section
"Implementation Details") and its page layout.

The pins do not re-run the oracle's own formula: they use hand-worked
vectors, exact rational arithmetic, an independent big-integer unpacker and
invariants that Eq. 2 implies.
"""
import json
import os
import random
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import quant

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32(x) -> float:
    return float(np.float32(float(x)))


def load_vectors():
    with open(os.path.join(GOLDEN, "eq2_vectors.json")) as f:
        return json.load(f)["vectors"]


def exact_round_half_even(fr: Fraction) -> int:
    fl = fr.numerator // fr.denominator
    rem = fr - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def nearest_f32(fr: Fraction) -> float:
    """fp32 value nearest to the rational fr (ties to even), by comparison."""
    c = np.float32(float(fr))
    cands = [np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))]
    best = min(cands, key=lambda v: (abs(Fraction(float(v)) - fr),
                                     struct.unpack("<I", struct.pack("<f", v))[0] & 1))
    return float(best)


def bigint_unpack(row_bytes: bytes, b: int, K: int):
    """Independent unpacker: the row as one little-endian integer."""
    n = int.from_bytes(row_bytes, "little")
    return [(n >> (b * j)) & ((1 << b) - 1) for j in range(K)]


@pytest.mark.parametrize("vec", load_vectors(), ids=lambda v: v["id"])
def test_hand_vectors(vec):
    b = vec["b"]
    w = torch.tensor([f32(x) for x in vec["w"]], dtype=torch.float32)
    m = quant.expert_absmax([w])
    s = quant.scale(m, b)
    if "s" in vec:
        assert s == float(vec["s"])
    else:
        assert struct.pack(">f", s).hex() == vec["s_hex"]
    q = quant.codes(w, s, b)
    assert q.tolist() == vec["q"]
    u = quant.stored(q, b)
    assert u.tolist() == vec["u"]
    packed = quant.pack_rows(u.reshape(1, -1), b)
    assert packed.shape == (1, 128 * b // 8)
    prefix = bytes.fromhex(vec["packed_prefix"])
    assert bytes(packed[0].tolist()[:len(prefix)]) == prefix
    assert all(v == 0 for v in packed[0].tolist()[len(prefix):])


def test_e4_distinguishes_exact_from_fp32_division():
    # the fp32-division reading rounds fp32(0.35)/fp32(0.1) to 3.5 -> 4
    w = np.float32(0.35)
    s = np.float32(0.1)
    assert np.rint(np.float32(w / s)) == 4
    assert quant.codes(torch.tensor([float(w)]), float(s), 4).item() == 3


def test_codes_match_exact_rational_rounding():
    rng = random.Random(1)
    for b in quant.BITS:
        qm = quant.qmax(b)
        for _ in range(400):
            m = f32(rng.uniform(1e-3, 10.0))
            s = quant.scale(m, b)
            # mix random values with values on and next to exact half-grid points
            if rng.random() < 0.5:
                w = f32(rng.uniform(-m, m))
            else:
                k = rng.randint(-qm, qm - 1) + 0.5
                w = float(np.nextafter(np.float32(k * s),
                                       np.float32(rng.choice([-np.inf, np.inf]))))
                if abs(w) > m:
                    w = f32(m)
            q_exact = exact_round_half_even(Fraction(w) / Fraction(s))
            q_exact = max(-qm, min(qm, q_exact))
            assert quant.codes(torch.tensor([w]), s, b).item() == q_exact, (b, w, s)


def test_scale_is_nearest_fp32_of_exact_quotient():
    rng = random.Random(2)
    for b in quant.BITS:
        for _ in range(300):
            m = f32(rng.uniform(1e-6, 1e3))
            assert quant.scale(m, b) == nearest_f32(Fraction(m) / quant.qmax(b))
    assert quant.scale(0.0, 4) == 0.0


def test_code_invariants_on_random_expert():
    g = torch.Generator().manual_seed(3)
    w = torch.randn(50_000, generator=g) * 0.02
    w[123] = 0.5                       # the maximum
    w[456] = -0.5
    m = quant.expert_absmax([w])
    for b in quant.BITS:
        s = quant.scale(m, b)
        q = quant.codes(w, s, b)
        qm = quant.qmax(b)
        assert int(q.abs().max()) <= qm
        assert q[123].item() == qm and q[456].item() == -qm
        err = (w.double() - q.double() * s).abs()
        # |w - s q| <= s/2 holds exactly in fp64 where q is not clamped
        assert float(err.max()) <= s / 2 * (1 + 2 ** -20)
        u = quant.stored(q, b)
        assert int(u.min()) >= 1 and int(u.max()) <= 2 ** b - 1


def test_zero_expert():
    w = torch.zeros(300)
    m = quant.expert_absmax([w])
    assert m == 0.0 and quant.scale(m, 3) == 0.0
    assert quant.codes(w, 0.0, 3).abs().sum().item() == 0
    assert quant.loss([w], m, 4) == 0.0


@pytest.mark.parametrize("b", quant.BITS)
@pytest.mark.parametrize("K", [128, 256, 200, 7])
def test_pack_against_bigint_unpacker(b, K):
    g = torch.Generator().manual_seed(b * 1000 + K)
    u = torch.randint(0, 2 ** b, (5, K), generator=g, dtype=torch.int32).to(torch.uint8)
    packed = quant.pack_rows(u, b)
    Kp = -(-K // 128) * 128
    assert packed.shape == (5, Kp * b // 8)
    for r in range(5):
        row = bytes(packed[r].tolist())
        got = bigint_unpack(row, b, Kp)
        assert got[:K] == u[r].tolist()
        assert all(v == 0 for v in got[K:])          # zero padding codes
    assert torch.equal(quant.unpack_rows(packed, b, K), u)


@pytest.mark.parametrize("b", quant.BITS)
def test_tests_page_map_two_statements_agree(b):
    """The tests read device pages through pagemap.untile_matrix (a reshape
    of the tile layout the library's header describes); the loop-based
    address formula pagemap.tiled_row states the same map piece by piece."""
    import pagemap
    rows, K = 48, 384
    g = torch.Generator().manual_seed(40 + b)
    tiled = torch.randint(0, 256, (rows * K * b // 8,), generator=g, dtype=torch.int32).to(torch.uint8)
    rm = pagemap.untile_matrix(tiled, rows, K, b)
    assert rm.shape == (rows, K * b // 8)
    for r in range(rows):
        assert bytes(rm[r].tolist()) == pagemap.tiled_row(tiled, K, b, r), r
    # a permutation: every tiled byte lands exactly once
    assert sorted(rm.reshape(-1).tolist()) == sorted(tiled.tolist())


def test_page_layout_and_size():
    E, d, F = 1, 128, 256
    g = torch.Generator().manual_seed(5)
    w1 = torch.randn(F, d, generator=g) * 0.02
    w3 = torch.randn(F, d, generator=g) * 0.02
    w2 = torch.randn(d, F, generator=g) * 0.02
    for b in quant.BITS:
        m = quant.expert_absmax((w1, w3, w2))
        s = quant.scale(m, b)
        page = quant.expert_page(w1, w3, w2, b, s)
        assert page.numel() == quant.page_nbytes(d, F, b)
        assert page.numel() % 256 == 0
        assert page.numel() == 3 * d * F * b // 8       # 128-multiples: no padding
        pb = bytes(page.tolist())
        # row-major bitstreams: W3 starts after the F rows of W1, W2 after
        # both; a row of K codes takes K b / 8 bytes
        m1 = F * d * b // 8
        for r in (0, 17, F - 1):
            row = d * b // 8
            q3 = bigint_unpack(pb[m1 + r * row:m1 + (r + 1) * row], b, d)
            want3 = [exact_round_half_even(Fraction(float(v)) / Fraction(s)) + 2 ** (b - 1)
                     for v in w3[r].tolist()]
            assert q3 == want3
        for r in (0, 17, d - 1):
            row = F * b // 8
            q2 = bigint_unpack(pb[2 * m1 + r * row:2 * m1 + (r + 1) * row], b, F)
            want2 = [exact_round_half_even(Fraction(float(v)) / Fraction(s)) + 2 ** (b - 1)
                     for v in w2[r].tolist()]
            assert q2 == want2


def test_loss_closed_forms():
    # E1 at b=3: errors 0, 0.125, 0.125, fp32(0.1), -0.125, 0 (worked by hand)
    w = torch.tensor([f32(x) for x in ["0.75", "-0.375", "0.125", "0.1", "-0.625", "0"]])
    m = quant.expert_absmax([w])
    want = (3 * 0.125 ** 2 + f32("0.1") ** 2) / 6
    assert quant.loss([w], m, 3) == pytest.approx(want, rel=1e-15)
    # weights on the 4-bit grid of their own scale: Q is lossless at 4 bits
    grid = torch.tensor([-7, -3, 0, 1, 5, 7], dtype=torch.float32) * 0.125
    m = quant.expert_absmax([grid])
    assert quant.loss([grid], m, 4) == 0.0
    assert quant.loss([grid], m, 3) > 0.0


def test_loss_uniform_data_is_s2_over_12():
    # dense, evenly spread weights: the rounding error is uniform on
    # [-s/2, s/2], whose mean square is s^2 / 12
    w = torch.linspace(-1.0, 1.0, 2_000_001, dtype=torch.float64).to(torch.float32)
    m = quant.expert_absmax([w])
    for b in quant.BITS:
        s = quant.scale(m, b)
        assert quant.loss([w], m, b) == pytest.approx(s * s / 12, rel=2e-3)


def test_loss_ordering_on_gaussian_expert():
    g = torch.Generator().manual_seed(7)
    w = torch.randn(100_000, generator=g) * 0.02
    m = quant.expert_absmax([w])
    L3, L4, L8 = (quant.loss([w], m, b) for b in (3, 4, 8))
    assert L8 < L4 < L3
