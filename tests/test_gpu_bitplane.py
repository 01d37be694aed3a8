"""GPU parity of the bitplane (prefix-compatible) pages against the oracle of
oracle/bitplane.py: page bytes bit-exact at every depth 1..8 (read back
through the tests' map of the device layout), the loss table, the
allocation and the layer's outputs; re-precision by plane count: lowering
depths drops planes without reading the masters (they are wiped first),
raising them writes the missing planes in place."""
import numpy as np
import pytest
import torch

import synth
from layer_cases import compare_y, compare_y_rows, cpu_threads, log, make_layer
from oracle import alloc, bitplane, moe, quant
from pagemap import bitplane_page_rows

pytestmark = pytest.mark.gpu

WL = synth.WORKLOADS["decode_fine"].scaled(name="bp_fine", E=16, d=256, F=384, T=40)


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cpu_threads()


def check_bp_pages(layer, pool, masters, depth, experts=None):
    w1, w3, w2 = masters
    F, d = w1.shape[1], w1.shape[2]
    table = layer.get_page_table()
    pool_h = pool.cpu()
    for e in (range(len(depth)) if experts is None else experts):
        b = int(depth[e])
        ent = table[e]
        m = quant.expert_absmax((w1[e], w3[e], w2[e]))
        s8 = bitplane.scale8(m)
        assert ent["bits"] == b and ent["scale"] == s8, (e, ent, b, s8)
        assert ent["nbytes"] == 3 * d * F * b // 8 and ent["offset"] % 256 == 0
        page = pool_h[ent["offset"]:ent["offset"] + bitplane.page_nbytes(d, F, b)]
        want = bitplane.expert_page(w1[e], w3[e], w2[e], b, s8)
        got = bitplane_page_rows(page, d, F, b)
        if not torch.equal(got, want):
            bad = int((got != want).nonzero()[0])
            raise AssertionError(f"expert {e} (depth {b}): first differing byte {bad}")
    spans = sorted((t["offset"], t["offset"] + t["nbytes"]) for t in table)
    for (a0, a1), (b0, b1) in zip(spans, spans[1:]):
        assert a1 <= b0


def oracle_y_bp(x, logits, wl, masters, depth):
    return moe.forward(x.float(), logits, wl.k, bitplane.experts(*masters, depth), bool(wl.renorm))


@pytest.mark.parametrize("T", [1, 12, 40, 300])
def test_every_depth_pages_and_forward(T):
    masters = synth.expert_weights(WL)
    depth = [1 + e % 8 for e in range(WL.E)]
    layer, pool = make_layer(WL, masters, max_tokens=T, layout="bitplane")
    log(f"bitplane: quantize depths {depth}")
    layer.quantize_experts(depth)
    torch.cuda.synchronize()
    check_bp_pages(layer, pool, masters, depth)
    x, logits = synth.tokens(WL, T=T)
    y = layer.moe_forward(x.cuda(), logits.cuda())
    compare_y(y, oracle_y_bp(x, logits, WL, masters, depth), f"bitplane T={T}")


def test_loss_table_and_budget():
    masters = synth.expert_weights(WL)
    layer, pool = make_layer(WL, masters, max_tokens=WL.T, layout="bitplane")
    got = layer.get_loss_table()
    want = bitplane.loss_table(*masters)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=0)
    B = WL.budget_bits(4.0)
    depth = layer.set_budget(B, synth.importance(WL))
    torch.cuda.synchronize()
    bits_want, _ = alloc.solve(synth.importance(WL), want.tolist(), [WL.W_e] * WL.E, B)
    assert depth.tolist() == list(bits_want)
    check_bp_pages(layer, pool, masters, depth)
    x, logits = synth.tokens(WL)
    y = layer.moe_forward(x.cuda(), logits.cuda())
    compare_y(y, oracle_y_bp(x, logits, WL, masters, depth), "bitplane after set_budget")


def test_lowering_depths_reads_no_masters_and_raising_writes_planes_in_place():
    masters = synth.expert_weights(WL)
    layer, pool = make_layer(WL, masters, max_tokens=WL.T, layout="bitplane")
    dev = layer._keep["masters"]
    layer.quantize_experts([8] * WL.E)
    torch.cuda.synchronize()
    offsets = [t["offset"] for t in layer.get_page_table()]
    # wipe the device masters: lowering must not read them
    saved = [m.clone() for m in dev]
    for m in dev:
        m.zero_()
    x, logits = synth.tokens(WL)
    for step, depth in enumerate(([6] * 8 + [5] * 8, [3, 4, 5, 5] * 4, [1, 2] * 8)):
        log(f"bitplane: lower to {depth}")
        layer.quantize_experts(depth)
        torch.cuda.synchronize()
        table = layer.get_page_table()
        assert [t["offset"] for t in table] == offsets          # nothing moved
        check_bp_pages(layer, pool, masters, depth)
        y = layer.moe_forward(x.cuda(), logits.cuda())
        compare_y(y, oracle_y_bp(x, logits, WL, masters, depth), f"lowered, step {step}")
    # raise again with the masters back: only the missing planes are written,
    # each page where it was (the planes it lost are free after it)
    for m, s_ in zip(dev, saved):
        m.copy_(s_)
    depth = [8, 3, 7, 4] * 4
    layer.quantize_experts(depth)
    torch.cuda.synchronize()
    table = layer.get_page_table()
    assert [t["offset"] for t in table] == offsets
    check_bp_pages(layer, pool, masters, depth)
    y = layer.moe_forward(x.cuda(), logits.cuda())
    compare_y(y, oracle_y_bp(x, logits, WL, masters, depth), "raised")


def test_growth_that_does_not_fit_moves_the_page():
    # dense depth-2 pages leave no room after each page: raising one expert
    # to depth 8 moves it (whole page rewritten), the others keep their bytes
    masters = synth.expert_weights(WL)
    depth = [2] * WL.E
    layer, pool = make_layer(WL, masters, max_tokens=WL.T, layout="bitplane",
                             pool_bytes=bitplane.page_nbytes(WL.d, WL.F, 2) * WL.E
                             + bitplane.page_nbytes(WL.d, WL.F, 8))
    layer.quantize_experts(depth)
    torch.cuda.synchronize()
    before = layer.get_page_table()
    keep = pool.clone()
    depth[3] = 8
    layer.quantize_experts(depth)
    torch.cuda.synchronize()
    after = layer.get_page_table()
    assert after[3]["offset"] != before[3]["offset"]
    for e in range(WL.E):
        if e != 3:
            assert after[e]["offset"] == before[e]["offset"]
            o, n = before[e]["offset"], before[e]["nbytes"]
            assert torch.equal(pool[o:o + n], keep[o:o + n])
    check_bp_pages(layer, pool, masters, depth)


def test_bitplane_rows_across_the_bf16_range():
    masters = synth.expert_weights(WL)
    depth = [8, 4, 3, 5] * 4
    layer, _ = make_layer(WL, masters, max_tokens=24, layout="bitplane")
    layer.quantize_experts(depth)
    x, logits = synth.tokens(WL, T=24)
    js = torch.tensor([-40, -12, 0, 12, 40])
    scale = torch.pow(2.0, js[torch.arange(24) % len(js)].double()).float()
    x = (x.float() * scale[:, None]).to(torch.bfloat16)
    y = layer.moe_forward(x.cuda(), logits.cuda())
    torch.cuda.synchronize()
    assert torch.isfinite(y).all()
    compare_y_rows(y, oracle_y_bp(x, logits, WL, masters, depth), "bitplane rows 2^-40..2^40")


def test_deep_experts_first_with_hot_experts_and_idle_slots():
    """The streaming kernels take bitplane experts deeper than 4 planes
    first: the router lists them from the front of its active list and the
    others from the back, with idle slots in between when fewer experts are
    routed than the grid has slots. 128 experts at every depth 1..8, d_model
    2048 (the down product walks row-block sequences), 200 tokens x top-2
    (128 slots; 108 experts routed), six hot experts (more than 16
    tokens), three deep and three shallow: the hot-expert scans (extra
    workgroups for the first ones) run over both ends of the list. Every
    output against the oracle."""
    wl = synth.WORKLOADS["decode_fine"].scaled(name="bp_hot_order", E=128, d=2048, F=384, k=2, T=200)
    masters = synth.expert_weights(wl)
    depth = [1 + (5 * e) % 8 for e in range(wl.E)]
    layer, _ = make_layer(wl, masters, max_tokens=wl.T, layout="bitplane")
    layer.quantize_experts(depth)
    x, logits = synth.tokens(wl)
    hot = [e for e in range(wl.E) if depth[e] > 4][:3] + [e for e in range(wl.E) if depth[e] <= 4][3:6]
    for h, e in enumerate(hot):
        logits[30 * h:30 * h + 30, e] += 10.0   # 30 tokens each
    counts = torch.bincount(moe.route(logits, wl.k)[0].reshape(-1), minlength=wl.E)
    assert sorted(torch.nonzero(counts > 16).reshape(-1).tolist()) == sorted(hot)
    routed = int((counts > 0).sum())
    log(f"routed experts {routed} of {wl.E} (slots {min(wl.E, wl.T * wl.k)}), hot {hot}, "
        f"deep routed {sum(1 for e in range(wl.E) if counts[e] > 0 and depth[e] > 4)}")
    assert routed < wl.E
    y = layer.moe_forward(x.cuda(), logits.cuda())
    compare_y(y, oracle_y_bp(x, logits, wl, masters, depth), "bitplane deep-first order, hot experts")
