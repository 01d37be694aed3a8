"""Oracle quantizer, page packer and loss table.

TEST INFRASTRUCTURE: imported only by tests, the smoke check and the
benchmark's CPU baseline; never by the GPU library.

Follows Eq. 2 of the PagedWeight page (section "Implementation Details"):
Q(w) = round(w / s) * s with s = max|w| / (2^(b-1) - 1), uniform and
symmetric, one scale per expert (the same section says "per-expert scaling
factors"), b in {3, 4, 8} (section "Dynamic Paging" names 8-, 4- and 3-bit
pages).

Readings where the page is silent (each is listed in the design notes):

* the max is over every weight of the expert (W1, W3 and W2 together);
* s is the fp32 value nearest to the exact quotient m / qmax; m = 0 gives
  s = 0 and all codes 0;
* round() is round-half-to-even of the exact real quotient w / s, then the
  code is clamped to [-qmax, qmax];
* a code q is stored as the unsigned value u = q + 2^(b-1);
* page layout: [W1 codes][W3 codes][W2 codes]; each matrix is [out, in]
  (W1, W3: F x d; W2: d x F), row after row; each row is a dense LSB-first
  bitstream (code j of the row occupies stream bits b*j .. b*j+b-1, stream
  bit i is bit i%8 of byte i//8), padded with zero bits to a multiple of
  128 codes. The page is padded with zero bytes to a multiple of 256. (How
  the library arranges these bytes in device memory is its own business;
  the tests map its pages back to this form.)
* the loss L(b) of the allocation problem is the mean squared error of
  Eq. 2 on the expert's own weights, in float64.
"""
from __future__ import annotations

import numpy as np
import torch

BITS = (3, 4, 8)
ROW_ALIGN_CODES = 128
PAGE_ALIGN_BYTES = 256


def qmax(b: int) -> int:
    """Largest code magnitude for b bits: 2^(b-1) - 1 (Eq. 2's denominator)."""
    return 2 ** (b - 1) - 1


def expert_absmax(mats) -> float:
    """m = max |w| over all weights of one expert. Exact in any order."""
    m = 0.0
    for t in mats:
        if t.numel():
            m = max(m, float(t.float().abs().max()))
    return m


def scale(m: float, b: int) -> float:
    """s = m / qmax rounded to the nearest fp32 value.

    Python's float division is the correctly rounded fp64 quotient; rounding
    that to fp32 equals rounding the exact quotient, because m / qmax with an
    odd qmax is either exact or not a dyadic rational, so it never sits on an
    fp32 rounding boundary.
    """
    if m == 0.0:
        return 0.0
    return float(np.float32(m / qmax(b)))


def codes(w: torch.Tensor, s: float, b: int) -> torch.Tensor:
    """Signed codes q = clamp(round_half_even(w / s), -qmax, qmax), int16.

    The fp64 quotient of two fp32 numbers rounds to a half-integer only when
    the exact quotient is one, so rounding it half-to-even gives the exact
    real quotient's rounding.
    """
    if s == 0.0:
        return torch.zeros(w.shape, dtype=torch.int16)
    q = torch.round(w.to(torch.float64) / s)  # torch.round: half to even
    return q.clamp_(-qmax(b), qmax(b)).to(torch.int16)


def stored(q: torch.Tensor, b: int) -> torch.Tensor:
    """Offset-binary stored code u = q + 2^(b-1), in [1, 2^b - 1]."""
    return (q.to(torch.int32) + (1 << (b - 1))).to(torch.uint8)


def pack_rows(u: torch.Tensor, b: int) -> torch.Tensor:
    """Pack a [rows, K] matrix of b-bit codes into [rows, Kp*b/8] bytes.

    Kp = K rounded up to 128; padding codes are 0. Bit i of code j becomes
    stream bit b*j + i; stream bit n is bit n%8 of byte n//8.
    """
    rows, K = u.shape
    Kp = -(-K // ROW_ALIGN_CODES) * ROW_ALIGN_CODES
    if Kp != K:
        u = torch.nn.functional.pad(u, (0, Kp - K))
    out = torch.empty((rows, Kp * b // 8), dtype=torch.uint8)
    shifts_b = torch.arange(b, dtype=torch.int32)
    shifts_8 = torch.arange(8, dtype=torch.int32)
    step = max(1, (1 << 22) // max(1, Kp))      # bound the temporary size
    for r0 in range(0, rows, step):
        chunk = u[r0:r0 + step].to(torch.int32)
        bits = (chunk.unsqueeze(-1) >> shifts_b) & 1           # [r, Kp, b]
        bits = bits.reshape(chunk.shape[0], Kp * b // 8, 8)    # stream order
        out[r0:r0 + step] = (bits << shifts_8).sum(-1).to(torch.uint8)
    return out


def unpack_rows(packed: torch.Tensor, b: int, K: int) -> torch.Tensor:
    """Inverse of pack_rows: [rows, nbytes] -> [rows, K] codes (uint8)."""
    rows, nbytes = packed.shape
    bits = (packed.to(torch.int32).unsqueeze(-1) >> torch.arange(8, dtype=torch.int32)) & 1
    bits = bits.reshape(rows, nbytes * 8 // b, b)
    u = (bits << torch.arange(b, dtype=torch.int32)).sum(-1)
    return u[:, :K].to(torch.uint8)


def matrix_bytes(rows: int, K: int, b: int) -> int:
    Kp = -(-K // ROW_ALIGN_CODES) * ROW_ALIGN_CODES
    return rows * Kp * b // 8


def page_nbytes(d: int, F: int, b: int) -> int:
    """Bytes of one expert's page: W1, W3 (F rows of d) and W2 (d rows of F)."""
    raw = 2 * matrix_bytes(F, d, b) + matrix_bytes(d, F, b)
    return -(-raw // PAGE_ALIGN_BYTES) * PAGE_ALIGN_BYTES


def expert_page(w1: torch.Tensor, w3: torch.Tensor, w2: torch.Tensor, b: int,
                s: float) -> torch.Tensor:
    """The page of one expert: the packed rows of W1, then of W3, then of W2,
    zero-padded to a multiple of 256 bytes."""
    parts = [pack_rows(stored(codes(w, s, b), b), b).reshape(-1) for w in (w1, w3, w2)]
    page = torch.cat(parts)
    n = page_nbytes(w1.shape[1], w1.shape[0], b)
    if page.numel() < n:
        page = torch.cat([page, torch.zeros(n - page.numel(), dtype=torch.uint8)])
    return page


def dequant(w: torch.Tensor, s: float, b: int) -> torch.Tensor:
    """Q(w) = s * q in float64 (exact: s has 24 and q at most 8 significant bits)."""
    return codes(w, s, b).to(torch.float64) * s


def loss(mats, m: float, b: int) -> float:
    """L(b) = mean over the expert's weights of (w - Q(w))^2, float64."""
    s = scale(m, b)
    total = 0.0
    count = 0
    for w in mats:
        err = w.to(torch.float64) - dequant(w, s, b)
        total += float((err * err).sum())
        count += w.numel()
    return total / count


def loss_table(w1: torch.Tensor, w3: torch.Tensor, w2: torch.Tensor):
    """Per-expert max|w| and loss table L[e][i] for b = BITS[i] (numpy)."""
    E = w1.shape[0]
    m = np.zeros(E)
    L = np.zeros((E, len(BITS)))
    for e in range(E):
        mats = (w1[e], w3[e], w2[e])
        m[e] = expert_absmax(mats)
        for i, b in enumerate(BITS):
            L[e, i] = loss(mats, m[e], b)
    return m, L


def quantize_layer(w1, w3, w2, bits):
    """Pages and scales for explicit per-expert bits.

    Returns (scales [E] fp32 values as floats, pages: list of uint8 tensors).
    """
    E = w1.shape[0]
    scales, pages = [], []
    for e in range(E):
        m = expert_absmax((w1[e], w3[e], w2[e]))
        s = scale(m, int(bits[e]))
        scales.append(s)
        pages.append(expert_page(w1[e], w3[e], w2[e], int(bits[e]), s))
    return scales, pages
