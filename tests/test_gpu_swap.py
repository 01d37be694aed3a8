"""GPU tests of the host tier (pages in pinned CPU memory, the device pool a
cache of page slots): the forward equals the one without a host tier bit
for bit, the slot of every expert after each pass equals the residency
oracle's (oracle/swap.py), slot bytes equal the host pages, which equal the
oracle's pages, and every output is also checked against the float64
oracle's forward; requantizing empties exactly the rewritten experts'
slots."""
import numpy as np
import pytest
import torch

import synth
from layer_cases import check_pages, compare_y, cpu_threads, log, make_layer, oracle_y
from oracle import moe
from oracle import swap as oswap

pytestmark = pytest.mark.gpu

# decode_fine-shaped, scaled down: 32 experts, top-8
WL = synth.WORKLOADS["decode_fine"].scaled(name="swap_fine", E=32, d=256, F=384, T=64)


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cpu_threads()


def _pair(n_slots, bits, wl=WL):
    """Layer A (pages in the pool) and layer B (host tier + n_slots slots)."""
    masters = synth.expert_weights(wl)
    a, pool_a = make_layer(wl, masters, max_tokens=wl.T)
    a.quantize_experts(bits)
    b, _ = make_layer(wl, masters, max_tokens=wl.T, pool_bytes=256)
    host = b.alloc_host_tier(b.pool_bytes_for_bits([8] * wl.E))
    slots = b.alloc_pool(max(256, n_slots * b.slot_bytes()))
    b.quantize_experts(bits)
    torch.cuda.synchronize()
    return masters, a, b, host, slots


def _active(logits):
    ids, _ = moe.route(logits, WL.k)
    return sorted(set(ids.flatten().tolist()))


def _check_slots(b, host, slots, res):
    slot_of, stats = b.residency()
    assert slot_of.tolist() == res.slot_of
    assert stats == dict(hits=res.hits, copies=res.copies, host_reads=res.host_reads)
    table = b.get_page_table()
    sb = b.slot_bytes()
    sl = slots.cpu()
    for e, s in enumerate(res.slot_of):
        if s >= 0:
            t = table[e]
            assert torch.equal(sl[s * sb:s * sb + t["nbytes"]], host[t["offset"]:t["offset"] + t["nbytes"]]), e


def test_forward_equal_and_residency_follows_the_oracle():
    rng = np.random.default_rng(0)
    bits = rng.choice([3, 4, 8], size=WL.E).tolist()
    masters, a, b, host, slots = _pair(6, bits)
    check_pages(b, host, masters, bits)
    res = oswap.Residency(WL.E, 6)
    for step in range(14):
        T = [1, 2, 3, 5, 1, 8, 2][step % 7]
        x, logits = synth.tokens(WL, T=T, step=step)
        log(f"swap step {step}: T={T}")
        ya = a.moe_forward(x.cuda(), logits.cuda())
        yb = b.moe_forward(x.cuda(), logits.cuda())
        torch.cuda.synchronize()
        assert torch.equal(ya, yb), step
        compare_y(yb, oracle_y(x, logits, WL, masters, bits), f"host tier step {step}")
        res.forward(_active(logits))
        _check_slots(b, host, slots, res)
    assert res.copies > 6 and res.hits > 0 and res.host_reads > 0


def test_requantize_empties_rewritten_slots():
    bits = [4] * WL.E
    masters, a, b, host, slots = _pair(8, bits)
    res = oswap.Residency(WL.E, 8)
    for step in range(4):
        x, logits = synth.tokens(WL, T=2, step=100 + step)
        b.moe_forward(x.cuda(), logits.cuda())
        res.forward(_active(logits))
    torch.cuda.synchronize()
    _check_slots(b, host, slots, res)
    # new widths for a third of the experts; the host tier has room for
    # first-fit placement, so exactly those pages are rewritten
    new = list(bits)
    for e in range(0, WL.E, 3):
        new[e] = 3 if e % 2 else 8
    before = b.get_page_table()
    log("swap: requantize")
    b.quantize_experts(new)
    a.quantize_experts(new)
    torch.cuda.synchronize()
    after = b.get_page_table()
    rewritten = [e for e in range(WL.E) if before[e]["bits"] != after[e]["bits"]
                 or before[e]["offset"] != after[e]["offset"]]
    assert rewritten == [e for e in range(WL.E) if new[e] != bits[e]]
    res.invalidate(rewritten)
    _check_slots(b, host, slots, res)
    check_pages(b, host, masters, new)
    for step in range(4):
        x, logits = synth.tokens(WL, T=3, step=200 + step)
        ya = a.moe_forward(x.cuda(), logits.cuda())
        yb = b.moe_forward(x.cuda(), logits.cuda())
        torch.cuda.synchronize()
        assert torch.equal(ya, yb)
        compare_y(yb, oracle_y(x, logits, WL, masters, new), f"after requantization, step {step}")
        res.forward(_active(logits))
        _check_slots(b, host, slots, res)


def test_no_slots_reads_every_page_from_the_host_tier():
    bits = [8, 4, 3, 4] * (WL.E // 4)
    masters, a, b, host, slots = _pair(0, bits)
    x, logits = synth.tokens(WL, T=4, step=7)
    ya = a.moe_forward(x.cuda(), logits.cuda())
    yb = b.moe_forward(x.cuda(), logits.cuda())
    torch.cuda.synchronize()
    assert torch.equal(ya, yb)
    compare_y(yb, oracle_y(x, logits, WL, masters, bits), "no slots")
    slot_of, stats = b.residency()
    assert (slot_of == -1).all()
    assert stats == dict(hits=0, copies=0, host_reads=len(_active(logits)))


def test_matrix_core_path_through_the_host_tier():
    # 320 tokens x top-8 over 32 experts (80 per expert): the large-batch kernels
    wl = WL.scaled(name="swap_gemm", T=320)
    bits = [3, 4, 8, 4] * (wl.E // 4)
    masters, a, b, host, slots = _pair(20, bits, wl)
    res = oswap.Residency(wl.E, 20)
    for step in range(3):
        x, logits = synth.tokens(wl, T=320, step=300 + step)
        log(f"swap gemm step {step}")
        ya = a.moe_forward(x.cuda(), logits.cuda())
        yb = b.moe_forward(x.cuda(), logits.cuda())
        torch.cuda.synchronize()
        assert torch.equal(ya, yb)
        compare_y(yb, oracle_y(x, logits, wl, masters, bits), f"host tier, matrix cores, step {step}")
        res.forward(_active(logits))
        _check_slots(b, host, slots, res)


def test_unbinding_the_host_tier_needs_new_pages():
    from mixed_precision_weight_page_amd import PagedWeightError
    _, a, b, host, slots = _pair(4, [4] * WL.E)
    b.bind_host_tier(None)
    x, logits = synth.tokens(WL, T=2, step=1)
    with pytest.raises(PagedWeightError):
        b.moe_forward(x.cuda(), logits.cuda())
    with pytest.raises(PagedWeightError):
        b.residency()


def test_many_experts_and_slots():
    # 300 experts (one wave per token in the router), 100 slots: the plan
    # kernel's scans and ranks over more than 256 entries
    wl = synth.WORKLOADS["tiny"].scaled(name="swap_e300", E=300, k=6, T=48)
    rng = np.random.default_rng(3)
    bits = rng.choice([3, 4, 8], size=wl.E).tolist()
    masters, a, b, host, slots = _pair(100, bits, wl)
    res = oswap.Residency(wl.E, 100)
    for step in range(8):
        T = [48, 5, 30, 1][step % 4]
        x, logits = synth.tokens(wl, T=T, step=400 + step)
        log(f"swap e300 step {step}: T={T}")
        ya = a.moe_forward(x.cuda(), logits.cuda())
        yb = b.moe_forward(x.cuda(), logits.cuda())
        torch.cuda.synchronize()
        assert torch.equal(ya, yb)
        compare_y(yb, oracle_y(x, logits, wl, masters, bits), f"host tier e300 step {step}")
        ids, _ = moe.route(logits, wl.k)
        res.forward(sorted(set(ids.flatten().tolist())))
        _check_slots(b, host, slots, res)
    assert res.host_reads > 0 and res.copies > 100
