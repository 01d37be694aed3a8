"""Address map of the library's device page layout, used by the tests (and the
smoke check) to turn a device page back into the oracle's plain form.

The oracle writes a page as row-major LSB-first bitstreams ([W1][W3][W2],
each matrix [out, in]). The library stores the same bytes tiled, as
include/pagedweight.h describes at pw_quantize_experts: tiles of 16 rows x
128 codes in (row block, K step) order; inside a tile the 32-code run g of
row r (4b bytes) belongs to lane l = 16 g + r, cut into pieces of
min(16, 4b) bytes, and piece p of all 64 lanes is stored together, lane
after lane. This module restates that description; it shares nothing with
the library's pack kernel or with the oracle.
"""
from __future__ import annotations

import torch

TILE_ROWS = 16
TILE_CODES = 128


def untile_matrix(tiled: torch.Tensor, rows: int, K: int, b: int) -> torch.Tensor:
    """Tiled bytes of one [rows, K] matrix of b-bit codes -> row-major
    bitstream bytes [rows, K b / 8] (rows a multiple of 16, K of 128)."""
    assert rows % TILE_ROWS == 0 and K % TILE_CODES == 0
    lane_bytes = 4 * b
    piece = min(16, lane_bytes)
    npiece = lane_bytes // piece
    steps = K // TILE_CODES
    t = tiled.reshape(rows // TILE_ROWS, steps, npiece, 4, TILE_ROWS, piece)
    #                  row block,        K step, piece, g,  r,         bytes
    t = t.permute(0, 4, 1, 3, 2, 5)      # row block, r, K step, g, piece, bytes
    return t.reshape(rows, K * b // 8)


def page_rows(page: torch.Tensor, d: int, F: int, b: int) -> torch.Tensor:
    """A device page (uint8, W1, W3, W2 tiled, then padding) in the oracle's
    layout: the row-major bitstreams of W1, W3 and W2, then the padding."""
    out = page.clone()
    off = 0
    for rows, K in ((F, d), (F, d), (d, F)):
        n = rows * K * b // 8
        out[off:off + n] = untile_matrix(page[off:off + n], rows, K, b).reshape(-1)
        off += n
    return out


def tiled_row(matrix: torch.Tensor, K: int, b: int, r: int) -> bytes:
    """Row r's bitstream gathered from a tiled matrix with the address
    formula, piece by piece (a second, loop-based statement of the map)."""
    steps = K // TILE_CODES
    piece = min(16, 4 * b)
    idx = []
    for s in range(steps):
        tile = ((r // TILE_ROWS) * steps + s) * (TILE_ROWS * TILE_CODES * b // 8)
        for g in range(4):
            for p in range(4 * b // piece):
                at = tile + p * 64 * piece + (16 * g + r % TILE_ROWS) * piece
                idx.extend(range(at, at + piece))
    return bytes(matrix[torch.tensor(idx)].tolist())


def bitplane_page_rows(page: torch.Tensor, d: int, F: int, depth: int) -> torch.Tensor:
    """A device bitplane page of `depth` planes in the oracle's layout: each
    plane is the W1, W3 and W2 bits, every matrix tiled as above at one bit
    per code (a 256-byte tile, lane l holding one 32-bit word)."""
    out = page.clone()
    off = 0
    for _ in range(depth):
        for rows, K in ((F, d), (F, d), (d, F)):
            n = rows * K // 8
            out[off:off + n] = untile_matrix(page[off:off + n], rows, K, 1).reshape(-1)
            off += n
    return out
