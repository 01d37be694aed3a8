"""GPU parity at the five workloads' full sizes, in the launch configuration
the benchmark times (same layer shapes, batches and budgets).

Masters are drawn on the GPU (seeded) and copied to the host for the
oracle. Where the oracle cannot redo everything in seconds, it checks a
sample: loss rows and whole pages of a few experts, random rows of every
other page. Allocation and forward outputs are compared in full: the oracle
computes the whole loss table (it needs it for Eq. 1) and the whole float64
forward pass.
"""
import time

import numpy as np
import pytest
import torch

import synth
from layer_cases import check_pages, compare_y, cpu_threads, log, make_layer, oracle_y
from oracle import c_oracle

pytestmark = pytest.mark.gpu

_cache = {}


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cpu_threads()


def layer_for(name, max_tokens):
    """(wl, device masters, host masters, oracle loss table), built once."""
    if name not in _cache:
        wl = synth.WORKLOADS[name]
        t0 = time.time()
        dev = synth.expert_weights(wl, device="cuda", seed=0)
        host = tuple(m.cpu() for m in dev)
        L = c_oracle.loss_table(*host, nthreads=cpu_threads())
        log(f"{name}: masters + oracle loss table {time.time() - t0:.1f}s")
        _cache[name] = (wl, dev, host, L)
    wl, dev, host, L = _cache[name]
    from mixed_precision_weight_page_amd import PagedMoELayer
    layer = PagedMoELayer(wl.E, wl.d, wl.F, wl.k, max_tokens=max_tokens, master_dtype=wl.master)
    layer.bind_masters(*dev)
    pool = layer.alloc_pool(layer.pool_bytes_for_bits([8] * wl.E))
    layer.alloc_workspace()
    return wl, layer, pool, host, L


def check_loss_rows(layer, host, L, experts):
    got = layer.get_loss_table()
    np.testing.assert_allclose(got[experts], L[experts], rtol=1e-12, atol=0)


def budget_and_pages(wl, layer, pool, host, L, B, sample_experts):
    p = synth.importance(wl)
    t0 = time.time()
    bits = layer.set_budget(B, p)
    torch.cuda.synchronize()
    want, _ = c_oracle.allocate(p, L, [wl.W_e] * wl.E, B)
    assert bits.tolist() == want
    assert int(bits.astype(np.int64).sum()) * wl.W_e <= B
    check_pages(layer, pool, host, bits, experts=sample_experts)
    others = [e for e in range(wl.E) if e not in sample_experts]
    if others:
        check_pages(layer, pool, host, bits, experts=others, rows_per_matrix=2)
    log(f"  bits {np.bincount(bits, minlength=9)[[3, 4, 8]].tolist()} (#3/#4/#8) checked in {time.time() - t0:.1f}s")
    return bits


def test_decode_coarse_full():
    wl, layer, pool, host, L = layer_for("decode_coarse", max_tokens=16)
    check_loss_rows(layer, host, L, [0, 5])
    bits = budget_and_pages(wl, layer, pool, host, L, wl.budget_bits(), sample_experts=[0, 5])
    for T in synth.DECODE_COARSE_BATCHES:
        x, logits = synth.tokens(wl, T=T, device="cuda", seed=1)
        y = layer.moe_forward(x, logits)
        compare_y(y, oracle_y(x.cpu(), logits.cpu(), wl, host, bits), f"decode_coarse T={T}")


def test_decode_fine_full():
    wl, layer, pool, host, L = layer_for("decode_fine", max_tokens=64)
    check_loss_rows(layer, host, L, list(range(0, wl.E, 9)))
    bits = budget_and_pages(wl, layer, pool, host, L, wl.budget_bits(),
                            sample_experts=list(range(0, wl.E, 16)))
    x, logits = synth.tokens(wl, device="cuda", seed=1)
    y = layer.moe_forward(x, logits)
    compare_y(y, oracle_y(x.cpu(), logits.cpu(), wl, host, bits), "decode_fine T=64")


def test_decode_fine_skewed_full():
    """decode_fine with routing skewed by importance (logits + log p_e, as
    the benchmark's skewed line): the most important experts take far more
    than 16 of the 64 tokens. Every output against the oracle."""
    wl, layer, pool, host, L = layer_for("decode_fine", max_tokens=64)
    bits = layer.set_budget(wl.budget_bits(), synth.importance(wl))
    want, _ = c_oracle.allocate(synth.importance(wl), L, [wl.W_e] * wl.E, wl.budget_bits())
    assert bits.tolist() == want
    x, logits = synth.tokens(wl, device="cuda", seed=2)
    logits = logits + torch.log(torch.tensor(synth.importance(wl), dtype=torch.float32, device="cuda"))
    counts = torch.bincount(torch.topk(logits, wl.k, dim=1).indices.reshape(-1), minlength=wl.E)
    log(f"  experts with more than 16 tokens: {int((counts > 16).sum())}, largest {int(counts.max())}")
    assert int((counts > 16).sum()) > 4
    y = layer.moe_forward(x, logits)
    compare_y(y, oracle_y(x.cpu(), logits.cpu(), wl, host, bits), "decode_fine skewed T=64")


def test_prefill_full():
    wl, layer, pool, host, L = layer_for("prefill", max_tokens=4096)
    check_loss_rows(layer, host, L, [0, 33, 63])
    bits = budget_and_pages(wl, layer, pool, host, L, wl.budget_bits(), sample_experts=[0, 63])
    x, logits = synth.tokens(wl, device="cuda", seed=1)
    t0 = time.time()
    y = layer.moe_forward(x, logits)
    torch.cuda.synchronize()
    ref = oracle_y(x.cpu(), logits.cpu(), wl, host, bits)
    log(f"  oracle prefill forward {time.time() - t0:.1f}s")
    compare_y(y, ref, "prefill T=4096")


def test_dynamic_schedule_full():
    """fp16 masters; budget stepped avg 8 -> 6 -> 4 -> 3.5 -> 5 bits, each for
    8 decode steps of 64 tokens; pages re-derived from the masters on the
    device between steps. After every budget change: allocation and pages
    against the oracle, untouched pages unchanged, one forward checked."""
    wl, layer, pool, host, L = layer_for("dynamic", max_tokens=64)
    p = synth.importance(wl)
    prev_bits = prev_table = prev_pool = None
    for phase, avg in enumerate(wl.schedule):
        B = wl.budget_bits(avg)
        bits = budget_and_pages(wl, layer, pool, host, L, B, sample_experts=[phase, 127 - phase])
        table = layer.get_page_table()
        if prev_bits is not None:
            kept = [e for e in range(wl.E) if bits[e] == prev_bits[e]
                    and table[e]["offset"] == prev_table[e]["offset"]]
            for e in kept[:8]:
                o, n = table[e]["offset"], table[e]["nbytes"]
                assert torch.equal(pool[o:o + n].cpu(), prev_pool[o:o + n])
        for step in range(wl.steps_per_phase):
            x, logits = synth.tokens(wl, device="cuda", seed=1, step=phase * wl.steps_per_phase + step)
            y = layer.moe_forward(x, logits)
            if step == 0:
                compare_y(y, oracle_y(x.cpu(), logits.cpu(), wl, host, bits), f"dynamic avg {avg}")
        torch.cuda.synchronize()
        prev_bits, prev_table, prev_pool = bits, table, pool.cpu()
