"""Oracle of the prefix-compatible bitplane layout (a nested quantizer).

TEST INFRASTRUCTURE: imported only by tests, the smoke check and the
benchmark's CPU baseline; never by the GPU library.

The PagedMoE page (Abstract) stores each expert once, with a
prefix-compatible tree codebook in a bitplane layout: a lower precision is a
prefix of a higher one, so precision can be lowered by dropping bitplanes
and raised by fetching only the missing ones. The page gives no formula.
Reading taken here, on top of Eq. 2 of the PagedWeight page (section
"Implementation Details"):

* every weight is coded once, by Eq. 2 at 8 bits: s8 = max|w| / 127 (the
  nearest fp32), q8 = round-half-even(w / s8) clamped to [-127, 127],
  u8 = q8 + 128 in [1, 255];
* the codebook is the binary tree over the 256 values of u8, most
  significant bit first: the first b bits of u8 (p = u8 >> (8 - b)) name a
  node at depth b, which covers the 2^(8-b) consecutive values
  p 2^(8-b) .. (p + 1) 2^(8-b) - 1;
* a depth-b weight is the centre of its node: q^ = (2p + 1) 2^(7-b) - 128.5
  (written below as twice that, the integer c = (2p + 1) 2^(8-b) - 257), so
  w^ = s8 q^ = s8 c / 2; at depth 8 this is Eq. 2's q8 exactly;
* bitplane j (j = 0 .. 7) holds bit 7 - j of every weight's u8; an expert's
  depth-b page is its first b planes, plane after plane, each plane the
  planes of W1, W3 and W2 ([out, in], row after row, each row an LSB-first
  bit stream padded to a multiple of 128 weights); the page is padded with
  zero bytes to a multiple of 256. A depth-b page is thus the first
  b W_e / 8 bytes of the depth-8 page;
* the loss of depth b is the mean squared error of w^ on the expert's own
  weights (float64), as for Eq. 2 pages.

Everything is float64 except the fp32 scale (Eq. 2's reading).
"""
from __future__ import annotations

import torch

from . import quant

DEPTHS = tuple(range(1, 9))
FULL = 8


def scale8(m: float) -> float:
    """s8: Eq. 2's scale at 8 bits (the nearest fp32 to m / 127)."""
    return quant.scale(m, FULL)


def u8(w: torch.Tensor, s8: float) -> torch.Tensor:
    """The stored 8-bit code u8 = q8 + 128 of Eq. 2 at 8 bits (int32)."""
    return quant.codes(w, s8, FULL).to(torch.int32) + 128


def prefix(u: torch.Tensor, b: int) -> torch.Tensor:
    """Node at depth b: the first (most significant) b bits of u8."""
    return u >> (FULL - b)


def centre2(p: torch.Tensor, b: int) -> torch.Tensor:
    """Twice the centre of node p at depth b, minus 2 * 128 (an integer)."""
    return (2 * p + 1) * (1 << (FULL - b)) - 257


def dequant(w: torch.Tensor, s8: float, b: int) -> torch.Tensor:
    """w^ at depth b, float64 (s8 c / 2 is exact in float64)."""
    return centre2(prefix(u8(w, s8), b), b).to(torch.float64) * (s8 / 2)


def plane(u: torch.Tensor, j: int) -> torch.Tensor:
    """Bitplane j: bit 7 - j of every code (j = 0 is the most significant)."""
    return ((u >> (FULL - 1 - j)) & 1).to(torch.uint8)


def expert_page(w1: torch.Tensor, w3: torch.Tensor, w2: torch.Tensor, b: int, s8: float) -> torch.Tensor:
    """The depth-b page of one expert: planes 0 .. b-1, each holding the
    packed bit rows of W1, then W3, then W2; zero-padded to 256 bytes."""
    codes = [u8(w, s8) for w in (w1, w3, w2)]
    parts = []
    for j in range(b):
        for u in codes:
            parts.append(quant.pack_rows(plane(u, j), 1).reshape(-1))
    page = torch.cat(parts)
    n = page_nbytes(w1.shape[1], w1.shape[0], b)
    if page.numel() < n:
        page = torch.cat([page, torch.zeros(n - page.numel(), dtype=torch.uint8)])
    return page


def page_nbytes(d: int, F: int, b: int) -> int:
    """Bytes of a depth-b page: b planes of the three matrices, 256-aligned."""
    raw = b * (2 * quant.matrix_bytes(F, d, 1) + quant.matrix_bytes(d, F, 1))
    return -(-raw // quant.PAGE_ALIGN_BYTES) * quant.PAGE_ALIGN_BYTES


def loss(mats, m: float, b: int) -> float:
    """Mean squared error of the depth-b weights over the expert, float64."""
    s8 = scale8(m)
    total, count = 0.0, 0
    for w in mats:
        err = w.to(torch.float64) - dequant(w, s8, b)
        total += float((err * err).sum())
        count += w.numel()
    return total / count


def loss_table(w1, w3, w2, depths=(3, 4, 8)):
    """Per-expert loss L[e][i] at depth depths[i] (numpy)."""
    import numpy as np
    E = w1.shape[0]
    L = np.zeros((E, len(depths)))
    for e in range(E):
        mats = (w1[e], w3[e], w2[e])
        m = quant.expert_absmax(mats)
        for i, b in enumerate(depths):
            L[e, i] = loss(mats, m, b)
    return L


def experts(w1, w3, w2, depth):
    """experts(e) callback for oracle.moe.forward: the depth[e] weights."""
    def get(e):
        m = quant.expert_absmax((w1[e], w3[e], w2[e]))
        s8 = scale8(m)
        b = int(depth[e])
        return dequant(w1[e], s8, b), dequant(w3[e], s8, b), dequant(w2[e], s8, b)
    return get
