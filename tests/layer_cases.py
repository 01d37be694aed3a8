"""Shared helpers of the GPU tests: build a layer on cuda from synthetic
masters, compute the oracle's reference on the CPU, compare. The reference
pages, scales and outputs come from the plain C++ oracle (oracle/c_oracle.py);
the Python oracle, pinned and compared with it separately, serves the
bitplane layout, the scheduler and the host tier."""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

import synth
from oracle import alloc, c_oracle, moe, quant
from pagemap import page_rows, tiled_row

YTOL_NORM = 2e-3        # normwise relative error of y
YTOL_MAX = 1e-2         # max |y - y_ref| relative to max |y_ref|


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def cpu_threads():
    n = min(16, os.cpu_count() or 1)
    torch.set_num_threads(n)
    return n


def make_layer(wl: synth.Workload, masters, max_tokens: int, pool_bytes: int = None, layout: str = "eq2"):
    from mixed_precision_weight_page_amd import PagedMoELayer
    w1, w3, w2 = (m.to("cuda") for m in masters)
    layer = PagedMoELayer(wl.E, wl.d, wl.F, wl.k, max_tokens=max_tokens, renorm=wl.renorm,
                          master_dtype=wl.master, layout=layout)
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


def compare_y_rows(y: torch.Tensor, ref: torch.Tensor, what: str = ""):
    """The layer tolerance applied to every token row on its own (rows may
    differ in magnitude by many orders); an all-zero reference row must be
    matched exactly."""
    y = y.detach().cpu().double()
    worst_n, worst_m = 0.0, 0.0
    for t in range(ref.shape[0]):
        r, d = ref[t], y[t] - ref[t]
        rn = float(r.norm())
        if rn == 0.0:
            assert float(d.abs().max()) == 0.0, (what, t)
            continue
        n_err = float(d.norm()) / rn
        m_err = float(d.abs().max()) / float(r.abs().max())
        worst_n, worst_m = max(worst_n, n_err), max(worst_m, m_err)
        assert n_err <= YTOL_NORM and m_err <= YTOL_MAX, (what, t, n_err, m_err, rn)
    log(f"  {what} per row: worst normwise {worst_n:.3e} max-abs {worst_m:.3e}")
    return worst_n, worst_m


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
        s, q, want_page = c_oracle.quantize_expert(w1[e], w3[e], w2[e], b, want_page=rows_per_matrix is None)
        assert ent["bits"] == b, (e, ent)
        assert ent["scale"] == s, (e, ent["scale"], s)
        assert ent["nbytes"] == c_oracle.page_bytes(d, F, b)
        assert ent["offset"] % 256 == 0
        page = pool_h[ent["offset"]:ent["offset"] + ent["nbytes"]]
        if rows_per_matrix is None:
            # the device page read back through the tests' map of the tile
            # layout, against the oracle's row-major page
            want = torch.from_numpy(want_page)
            got = page_rows(page, d, F, b)
            if not torch.equal(got, want):
                bad = int((got != want).nonzero()[0])
                raise AssertionError(f"expert {e} ({b} bits): first differing byte {bad}")
        else:
            off = 0
            for mi, mat in enumerate((w1[e], w3[e], w2[e])):
                rows, K = mat.shape
                nb = rows * K * b // 8
                qm = q[mi * d * F:(mi + 1) * d * F].reshape(rows, K)
                for r in rng.choice(rows, size=min(rows, rows_per_matrix), replace=False):
                    want = torch.from_numpy(c_oracle.pack_rows(qm[r:r + 1], b)[0])
                    got = torch.tensor(list(tiled_row(page[off:off + nb], K, b, int(r))), dtype=torch.uint8)
                    assert torch.equal(got, want), (e, b, int(r))
                off += nb
    # placement invariants: aligned, inside the pool, no overlap
    spans = sorted((t["offset"], t["offset"] + t["nbytes"]) for t in table)
    for (a0, a1), (b0, b1) in zip(spans, spans[1:]):
        assert a1 <= b0
    assert spans[-1][1] <= pool.numel()


def oracle_bits(wl, masters, B, L=None):
    w1, w3, w2 = masters
    if L is None:
        L = c_oracle.loss_table(w1, w3, w2, nthreads=cpu_threads())
    p = synth.importance(wl)
    bits, _ = c_oracle.allocate(p, L, [wl.W_e] * wl.E, B)
    return bits, L


def oracle_y(x, logits, wl, masters, bits):
    """y of the plain C++ oracle (float64) for bf16 x, from the fp masters
    quantized at bits."""
    w1, w3, w2 = masters
    y = c_oracle.moe_forward_quantized(x, logits, wl.k, w1, w3, w2, bits, bool(wl.renorm), nthreads=cpu_threads())
    return torch.from_numpy(y)
