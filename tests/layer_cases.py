"""Shared helpers of the GPU tests: build a layer on cuda from synthetic
masters, compute the oracle's reference on the CPU, compare."""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

import synth
from oracle import alloc, moe, quant

YTOL_NORM = 2e-3        # normwise relative error of y
YTOL_MAX = 1e-2         # max |y - y_ref| relative to max |y_ref|


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def cpu_threads():
    n = min(16, os.cpu_count() or 1)
    torch.set_num_threads(n)
    return n


def make_layer(wl: synth.Workload, masters, max_tokens: int, pool_bytes: int = None):
    from mixed_precision_weight_page_amd import PagedMoELayer
    w1, w3, w2 = (m.to("cuda") for m in masters)
    layer = PagedMoELayer(wl.E, wl.d, wl.F, wl.k, max_tokens=max_tokens, renorm=wl.renorm,
                          master_dtype=wl.master)
    layer.bind_masters(w1, w3, w2)
    if pool_bytes is None:
        pool_bytes = layer.pool_bytes_for_bits([8] * wl.E)
    pool = layer.alloc_pool(pool_bytes)
    layer.alloc_workspace()
    return layer, pool


def compare_y(y: torch.Tensor, ref: torch.Tensor, what: str = ""):
    y = y.detach().cpu().double()
    diff = y - ref
    rn = float(ref.norm())
    norm_err = float(diff.norm()) / rn if rn > 0 else float(diff.norm())
    mref = float(ref.abs().max())
    max_err = float(diff.abs().max()) / mref if mref > 0 else float(diff.abs().max())
    log(f"  {what} normwise {norm_err:.3e} max-abs {max_err:.3e}")
    assert norm_err <= YTOL_NORM, (what, norm_err)
    assert max_err <= YTOL_MAX, (what, max_err)
    return norm_err, max_err


def check_pages(layer, pool: torch.Tensor, masters, bits, experts=None, rows_per_matrix=None,
                seed=0):
    """Page table entries and page bytes against the oracle.

    experts: which experts to compare (default all). rows_per_matrix: if set,
    compare that many random rows of each matrix instead of whole pages.
    """
    w1, w3, w2 = masters
    E = w1.shape[0]
    F, d = w1.shape[1], w1.shape[2]
    table = layer.get_page_table()
    pool_h = pool.cpu()
    rng = np.random.default_rng(seed)
    experts = range(E) if experts is None else experts
    for e in experts:
        b = int(bits[e])
        ent = table[e]
        m = quant.expert_absmax((w1[e], w3[e], w2[e]))
        s = quant.scale(m, b)
        assert ent["bits"] == b, (e, ent)
        assert ent["scale"] == s, (e, ent["scale"], s)
        assert ent["nbytes"] == quant.page_nbytes(d, F, b)
        assert ent["offset"] % 256 == 0
        page = pool_h[ent["offset"]:ent["offset"] + ent["nbytes"]]
        if rows_per_matrix is None:
            want = quant.expert_page(w1[e], w3[e], w2[e], b, s)
            if not torch.equal(page, want):
                bad = int((page != want).nonzero()[0])
                raise AssertionError(f"expert {e} ({b} bits): first differing byte {bad}")
        else:
            off = 0
            for mat in (w1[e], w3[e], w2[e]):
                rows, K = mat.shape
                nb = rows * K * b // 8
                for r in rng.choice(rows, size=min(rows, rows_per_matrix), replace=False):
                    want = quant.pack_rows(quant.stored(quant.codes(mat[r:r + 1], s, b), b), b)[0]
                    got = torch.tensor(list(tiled_row(page[off:off + nb], K, b, int(r))), dtype=torch.uint8)
                    assert torch.equal(got, want), (e, b, int(r))
                off += nb
    # placement invariants: aligned, inside the pool, no overlap
    spans = sorted((t["offset"], t["offset"] + t["nbytes"]) for t in table)
    for (a0, a1), (b0, b1) in zip(spans, spans[1:]):
        assert a1 <= b0
    assert spans[-1][1] <= pool.numel()


def tiled_row(matrix: torch.Tensor, K: int, b: int, r: int) -> bytes:
    """Bytes of row r's bitstream read back from a tiled matrix (tile =
    16 rows x 128 codes; lane 16 g + r holds codes 32g..32g+31 of row r in
    pieces of min(16, 4b) bytes, piece p of all 64 lanes together)."""
    steps = K // 128
    piece = min(16, 4 * b)
    idx = []
    for s in range(steps):
        tile = ((r // 16) * steps + s) * (16 * 128 * b // 8)
        for g in range(4):
            for p in range(4 * b // piece):
                at = tile + p * 64 * piece + (16 * g + r % 16) * piece
                idx.extend(range(at, at + piece))
    return bytes(matrix[torch.tensor(idx)].tolist())


def oracle_bits(wl, masters, B, L=None):
    w1, w3, w2 = masters
    if L is None:
        _, L = quant.loss_table(w1, w3, w2)
    p = synth.importance(wl)
    bits, _ = alloc.solve(p, L.tolist(), [wl.W_e] * wl.E, B)
    return bits, L


def oracle_y(x, logits, wl, masters, bits):
    w1, w3, w2 = masters
    return moe.moe_forward_quantized(x.float(), logits, wl.k, w1, w3, w2, bits, bool(wl.renorm))
