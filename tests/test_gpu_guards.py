"""Guard bands around every buffer the library writes.

The pool, the workspace and the output y each sit inside a larger device
buffer whose 64 KB on either side hold seeded random bytes; before the first
quantization the pool's own bytes hold them too. After quantization,
re-precision (lowering and raising bit-widths or bitplane depths, which
rewrite or move pages and write planes in place) and forwards on the
streaming and matrix-core paths (and the allocation-free forward), the bands
are unchanged, and so are the pool bytes between and after the pages of a
fresh quantization: nothing is written outside the pages, the workspace and
the output rows. Outputs are checked against the oracle as well.
"""
import numpy as np
import pytest
import torch

import synth
from layer_cases import compare_y, cpu_threads, log, oracle_y
from oracle import bitplane, moe

pytestmark = pytest.mark.gpu

G = 64 * 1024


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cpu_threads()


class Guarded:
    """A device uint8 buffer of n bytes inside guard bands of random bytes
    (`inner` also random when fill_inner)."""

    def __init__(self, n: int, seed: int, fill_inner: bool = True):
        gen = torch.Generator().manual_seed(seed)
        host = torch.randint(0, 256, (n + 2 * G,), dtype=torch.uint8, generator=gen)
        if not fill_inner:
            host[G:G + n] = 0
        self.ref = host.clone()
        self.buf = host.cuda()
        self.n = n
        self.view = self.buf[G:G + n]

    def check_bands(self, what: str):
        torch.cuda.synchronize()
        now = self.buf.cpu()
        assert torch.equal(now[:G], self.ref[:G]), f"{what}: bytes before the buffer changed"
        assert torch.equal(now[G + self.n:], self.ref[G + self.n:]), f"{what}: bytes after the buffer changed"

    def check_inner_outside(self, spans, what: str):
        """Bytes of the buffer outside the (offset, nbytes) spans unchanged."""
        torch.cuda.synchronize()
        now = self.buf[G:G + self.n].cpu()
        keep = torch.ones(self.n, dtype=torch.bool)
        for off, nb in spans:
            keep[off:off + nb] = False
        assert torch.equal(now[keep], self.ref[G:G + self.n][keep]), f"{what}: pool bytes outside the pages changed"


def guarded_layer(wl, masters, max_tokens, layout="eq2", seed=0):
    from mixed_precision_weight_page_amd import PagedMoELayer
    layer = PagedMoELayer(wl.E, wl.d, wl.F, wl.k, max_tokens=max_tokens, renorm=wl.renorm,
                          master_dtype=wl.master, layout=layout)
    layer.bind_masters(*(m.cuda() for m in masters))
    pool = Guarded(layer.pool_bytes_for_bits([8] * wl.E) + 4096, seed)
    layer.bind_pool(pool.view)
    ws = Guarded(max(256, layer.workspace_bytes()), seed + 1)
    layer.bind_workspace(ws.view)
    return layer, pool, ws


def guarded_forward(layer, x, logits, seed, what, noalloc=False):
    """The forward into rows 1 .. T of a guarded [T + 2, d] output; returns y."""
    T, d = x.shape
    yb = Guarded((T + 2) * d * 4, seed, fill_inner=False)
    y = yb.view.view(torch.float32).view(T + 2, d)
    if noalloc:
        layer.moe_forward_noalloc(x.cuda(), logits.cuda(), y[1:T + 1])
    else:
        layer.moe_forward(x.cuda(), logits.cuda(), y[1:T + 1])
    yb.check_bands(what + " (output)")
    torch.cuda.synchronize()
    assert torch.equal(y[0].cpu(), torch.zeros(d)) and torch.equal(y[T + 1].cpu(), torch.zeros(d)), \
        f"{what}: output rows outside the batch changed"
    return y[1:T + 1].clone()


def page_spans(layer):
    return [(e["offset"], e["nbytes"]) for e in layer.get_page_table()]


@pytest.mark.parametrize("layout", ["eq2", "bitplane"])
def test_streaming_path_writes_nothing_outside_its_buffers(layout):
    wl = synth.WORKLOADS["decode_fine"].scaled(name=f"guard_{layout}", E=32, d=256, F=384, T=40)
    masters = synth.expert_weights(wl)
    layer, pool, ws = guarded_layer(wl, masters, max_tokens=wl.T, layout=layout, seed=10)
    bits = [(8, 4, 3)[e % 3] for e in range(wl.E)]
    layer.quantize_experts(bits)
    pool.check_bands("quantize")
    pool.check_inner_outside(page_spans(layer), "quantize")
    experts = (bitplane.experts(*masters, bits) if layout == "bitplane" else None)
    for T, seed in ((40, 1), (8, 2), (1, 3)):
        x, logits = synth.tokens(wl, T=T, seed=seed)
        if T == 40:
            logits[:, 0] += 20.0          # one expert with every token: wide passes
        y = guarded_forward(layer, x, logits, 100 + seed, f"{layout} T={T}")
        ws.check_bands(f"{layout} T={T} (workspace)")
        pool.check_bands(f"{layout} T={T} (pool)")
        ref = (moe.forward(x.float(), logits, wl.k, experts) if experts
               else oracle_y(x, logits, wl, masters, bits))
        compare_y(y, ref, f"guarded {layout} T={T}")
    # re-precision: lower every width, then raise some (pages rewritten,
    # moved, or grown in place by planes)
    for step, new in enumerate(([3] * wl.E, [(8, 4)[e % 2] for e in range(wl.E)])):
        layer.quantize_experts(new)
        pool.check_bands(f"{layout} re-precision {step}")
        x, logits = synth.tokens(wl, T=16, seed=20 + step)
        guarded_forward(layer, x, logits, 200 + step, f"{layout} after re-precision {step}")
        ws.check_bands(f"{layout} after re-precision {step} (workspace)")
    log(f"guards intact ({layout})")


def test_matrix_core_path_writes_nothing_outside_its_buffers():
    wl = synth.WORKLOADS["tiny"].scaled(name="guard_gemm", E=8, d=512, F=384, k=2, T=600,
                                        bits=(8, 3, 4, 4, 3, 8, 4, 3))
    masters = synth.expert_weights(wl)
    layer, pool, ws = guarded_layer(wl, masters, max_tokens=wl.T, seed=30)
    layer.quantize_experts(wl.bits)
    pool.check_inner_outside(page_spans(layer), "quantize")
    x, logits = synth.tokens(wl)
    y = guarded_forward(layer, x, logits, 300, "matrix-core T=600")
    ws.check_bands("matrix-core (workspace)")
    pool.check_bands("matrix-core (pool)")
    compare_y(y, oracle_y(x, logits, wl, masters, wl.bits), "guarded matrix-core T=600")


def test_allocation_free_forward_writes_only_its_output():
    wl = synth.WORKLOADS["decode_fine"].scaled(name="guard_noalloc", E=32, d=256, F=384, T=24)
    masters = synth.expert_weights(wl)
    layer, pool, ws = guarded_layer(wl, masters, max_tokens=wl.T, seed=40)
    bits = [(3, 4, 8)[e % 3] for e in range(wl.E)]
    layer.quantize_experts(bits)
    torch.cuda.synchronize()
    before = ws.buf.cpu()
    x, logits = synth.tokens(wl)
    y = guarded_forward(layer, x, logits, 400, "allocation-free", noalloc=True)
    torch.cuda.synchronize()
    assert torch.equal(ws.buf.cpu(), before), "the bound workspace (or its bands) changed"
    pool.check_bands("allocation-free (pool)")
    compare_y(y, oracle_y(x, logits, wl, masters, bits), "guarded allocation-free forward")
