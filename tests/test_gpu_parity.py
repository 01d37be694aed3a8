"""GPU parity of the HIP path against the CPU oracle at sizes the oracle
finishes in seconds: codes, scales and pages bit-exact, router choices
exact, loss table within 1e-12 relative, outputs within the layer
tolerance (normwise 2e-3, max-abs 1e-2 of max |y_ref|)."""
import numpy as np
import pytest
import torch

import synth
from layer_cases import (check_pages, compare_y, cpu_threads, log, make_layer, oracle_bits,
                         oracle_y)
from oracle import sched as osched
from oracle import c_oracle, moe

pytestmark = pytest.mark.gpu

TINY = synth.WORKLOADS["tiny"]
# a decode_fine-shaped layer scaled down: outliers, many experts, top-8
SMALL_FINE = synth.WORKLOADS["decode_fine"].scaled(name="small_fine", E=32, d=256, F=384, T=40)
# fp16 masters, for the re-precision path
SMALL_DYN = synth.WORKLOADS["dynamic"].scaled(name="small_dyn", E=16, d=256, F=256, T=24)


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cpu_threads()


def test_tiny_pages_and_forward():
    wl = TINY
    masters = synth.expert_weights(wl)
    x, logits = synth.tokens(wl)
    layer, pool = make_layer(wl, masters, max_tokens=wl.T)
    log("tiny: quantize_experts")
    layer.quantize_experts(wl.bits)
    torch.cuda.synchronize()
    check_pages(layer, pool, masters, wl.bits)
    log("tiny: forward")
    y = layer.moe_forward(x.cuda(), logits.cuda())
    torch.cuda.synchronize()
    compare_y(y, oracle_y(x, logits, wl, masters, wl.bits), "tiny")


ROUTER_CASES = [
    # (workload, tokens): one-workgroup path with 16-lane rows (E <= 256,
    # T <= 64), router + one-workgroup grouping, and the multi-workgroup path
    # (more than 4096 pairs; 2500 tokens = three ranking chunks of 1024, the
    # last one ragged)
    (TINY, 16), (SMALL_FINE, 40), (synth.WORKLOADS["decode_fine"], 64),
    (synth.WORKLOADS["decode_fine"], 65), (synth.WORKLOADS["prefill"].scaled(E=64, d=128, F=128), 300),
    (SMALL_FINE, 700), (SMALL_FINE, 2500),
    # 256 experts: 16 logits per lane; k = 20 > 16 slots per row of lanes
    (TINY.scaled(name="e256", E=256, k=8), 64), (TINY.scaled(name="k20", E=64, k=20), 30),
    # more than 256 experts: a wave per token (fused up to 16 tokens)
    (TINY.scaled(name="e300", E=300, k=6), 12), (TINY.scaled(name="e300", E=300, k=6), 40),
    (TINY.scaled(name="e300", E=300, k=6), 800),
]


@pytest.mark.parametrize("wl,T", ROUTER_CASES, ids=lambda v: str(v) if isinstance(v, int) else v.name)
def test_router_matches_oracle(wl, T):
    from mixed_precision_weight_page_amd import PagedMoELayer
    layer = PagedMoELayer(wl.E, 128, 128, wl.k, max_tokens=T)
    layer.alloc_workspace()
    _, logits = synth.tokens(wl, T=T)
    # plant exact ties: equal logits must resolve to the lower index
    logits[0, :] = 0.25
    logits[1, 3] = logits[1, 5] = logits[1].max() + 1.0
    # -0 and +0 are equal logits too: the lower index (holding -0) first
    logits[2, :] = -1.0
    logits[2, 1], logits[2, 4] = -0.0, 0.0
    ids, g, counts = layer.route(logits.cuda())
    torch.cuda.synchronize()
    rid, rg = moe.route(logits, wl.k)
    assert torch.equal(ids.cpu().long(), rid), wl.name
    assert torch.allclose(g.cpu().double(), rg, rtol=2e-6, atol=1e-7), wl.name
    want = torch.bincount(rid.reshape(-1), minlength=wl.E)
    assert torch.equal(counts.cpu().long(), want)


def test_router_renorm():
    wl = SMALL_FINE.scaled(renorm=1)
    from mixed_precision_weight_page_amd import PagedMoELayer
    layer = PagedMoELayer(wl.E, wl.d, wl.F, wl.k, max_tokens=40, renorm=1)
    layer.alloc_workspace()
    _, logits = synth.tokens(wl, T=40)
    ids, g, _ = layer.route(logits.cuda())
    rid, rg = moe.route(logits, wl.k, renorm=True)
    assert torch.equal(ids.cpu().long(), rid)
    assert torch.allclose(g.cpu().double(), rg, rtol=2e-6, atol=1e-7)


@pytest.mark.parametrize("wl", [TINY, SMALL_FINE, SMALL_DYN], ids=lambda w: w.name)
def test_loss_table_matches_oracle(wl):
    masters = synth.expert_weights(wl)
    layer, _ = make_layer(wl, masters, max_tokens=8)
    got = layer.get_loss_table()
    want = c_oracle.loss_table(*masters, nthreads=cpu_threads())
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=0)
    assert np.all(got[:, 2] < got[:, 1])   # 8 bits beat 4 bits


@pytest.mark.parametrize("wl", [SMALL_FINE, SMALL_DYN], ids=lambda w: w.name)
def test_set_budget_pages_and_forward(wl):
    masters = synth.expert_weights(wl)
    x, logits = synth.tokens(wl)
    layer, pool = make_layer(wl, masters, max_tokens=wl.T)
    B = wl.budget_bits(4.0)
    log(f"{wl.name}: set_budget")
    bits = layer.set_budget(B, synth.importance(wl))
    torch.cuda.synchronize()
    want, _ = oracle_bits(wl, masters, B)
    assert bits.tolist() == want
    assert int(bits.astype(np.int64).sum()) * wl.W_e <= B
    check_pages(layer, pool, masters, bits)
    y = layer.moe_forward(x.cuda(), logits.cuda())
    compare_y(y, oracle_y(x, logits, wl, masters, bits), wl.name)


def test_budget_shared_by_two_layers():
    # two layers of different shapes under one budget of 4.5 bits per weight
    # on average: bits as the oracle's solve over the union of their
    # experts, pages bit-exact, outputs within tolerance
    from mixed_precision_weight_page_amd import set_budget_layers
    wls = [SMALL_FINE, TINY.scaled(name="tiny_b")]
    layers, pools, masters, ps, Ls = [], [], [], [], []
    for wl in wls:
        m = synth.expert_weights(wl)
        layer, pool = make_layer(wl, m, max_tokens=wl.T)
        layers.append(layer)
        pools.append(pool)
        masters.append(m)
        ps.append(list(synth.importance(wl)))
        Ls.append(c_oracle.loss_table(*m, nthreads=cpu_threads()))
    B = int(4.5 * sum(wl.E * wl.W_e for wl in wls))
    log("two layers: set_budget_layers")
    bits, obj = set_budget_layers(layers, B, ps, layer_weights=[1.0, 2.0])
    torch.cuda.synchronize()
    want, want_obj = c_oracle.allocate_layers(ps, Ls, [[wl.W_e] * wl.E for wl in wls], B, [1.0, 2.0])
    assert [b.tolist() for b in bits] == want
    assert obj == pytest.approx(want_obj, rel=1e-12)
    assert sum(int(b.astype(np.int64).sum()) * wl.W_e for b, wl in zip(bits, wls)) <= B
    for wl, layer, pool, m, b in zip(wls, layers, pools, masters, bits):
        check_pages(layer, pool, m, b)
        x, logits = synth.tokens(wl)
        y = layer.moe_forward(x.cuda(), logits.cuda())
        compare_y(y, oracle_y(x, logits, wl, m, b), wl.name)


def test_ragged_token_counts():
    # experts with more than 16 tokens (several token blocks), a ragged tail,
    # a single token, and T = 0
    wl = synth.WORKLOADS["tiny"].scaled(name="ragged", E=4, d=256, F=256, k=2, T=45,
                                        bits=(3, 4, 8, 4))
    masters = synth.expert_weights(wl)
    layer, pool = make_layer(wl, masters, max_tokens=64)
    layer.quantize_experts(wl.bits)
    for T in (45, 1, 17, 64):
        x, logits = synth.tokens(wl, T=T)
        y = layer.moe_forward(x.cuda(), logits.cuda())
        compare_y(y, oracle_y(x, logits, wl, masters, wl.bits), f"T={T}")
    empty = torch.empty(0, wl.d, dtype=torch.bfloat16, device="cuda")
    y0 = layer.moe_forward(empty, torch.empty(0, wl.E, device="cuda"))
    assert y0.shape == (0, wl.d)


def test_deterministic_outputs():
    wl = SMALL_FINE
    masters = synth.expert_weights(wl)
    x, logits = synth.tokens(wl)
    layer, pool = make_layer(wl, masters, max_tokens=wl.T)
    layer.set_budget(wl.budget_bits(4.0), synth.importance(wl))
    xc, lc = x.cuda(), logits.cuda()
    y1 = layer.moe_forward(xc, lc).clone()
    p1 = pool.clone()
    layer2, pool2 = make_layer(wl, masters, max_tokens=wl.T)
    layer2.set_budget(wl.budget_bits(4.0), synth.importance(wl))
    y2 = layer2.moe_forward(xc, lc)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    assert torch.equal(p1, pool2)
    assert layer.get_page_table() == layer2.get_page_table()


def test_reprecision_schedule():
    """Budget stepped through avg 8, 6, 4, 3.5, 5 bits on fp16 masters:
    after every step the pages equal a fresh oracle quantization from the
    masters, experts whose bits did not change keep their bytes, and the
    forward pass matches the oracle."""
    wl = SMALL_DYN
    masters = synth.expert_weights(wl)
    layer, pool = make_layer(wl, masters, max_tokens=wl.T)
    L = c_oracle.loss_table(*masters, nthreads=cpu_threads())
    p = synth.importance(wl)
    prev_bits, prev_pool, prev_table = None, None, None
    for step, avg in enumerate(wl.schedule):
        B = wl.budget_bits(avg)
        bits = layer.set_budget(B, p)
        torch.cuda.synchronize()
        want, _ = c_oracle.allocate(p, L, [wl.W_e] * wl.E, B)
        assert bits.tolist() == want, avg
        check_pages(layer, pool, masters, bits)
        table = layer.get_page_table()
        if prev_bits is not None:
            for e in range(wl.E):
                if bits[e] == prev_bits[e] and table[e]["offset"] == prev_table[e]["offset"]:
                    o, n = table[e]["offset"], table[e]["nbytes"]
                    assert torch.equal(pool[o:o + n].cpu(), prev_pool[o:o + n])
        x, logits = synth.tokens(wl, step=step)
        y = layer.moe_forward(x.cuda(), logits.cuda())
        compare_y(y, oracle_y(x, logits, wl, masters, bits), f"avg {avg}")
        prev_bits, prev_pool, prev_table = bits, pool.cpu(), table


def test_failed_budget_keeps_previous_table():
    wl = SMALL_DYN
    masters = synth.expert_weights(wl)
    from mixed_precision_weight_page_amd import PagedWeightError
    # a pool that holds everything at 4 bits but not at 8
    layer, pool = make_layer(wl, masters, max_tokens=wl.T,
                             pool_bytes=int(wl.E * wl.W_e * 4 // 8))
    p = synth.importance(wl)
    bits = layer.set_budget(wl.budget_bits(4.0), p)
    before = layer.get_page_table()
    snap = pool.cpu()
    with pytest.raises(PagedWeightError) as ei:
        layer.set_budget(wl.budget_bits(8.0), p)
    assert ei.value.status == -5
    assert layer.get_page_table() == before
    torch.cuda.synchronize()
    assert torch.equal(pool.cpu(), snap)
    x, logits = synth.tokens(wl)
    y = layer.moe_forward(x.cuda(), logits.cuda())
    compare_y(y, oracle_y(x, logits, wl, masters, bits), "after failed budget")


def test_nonfinite_masters_rejected():
    wl = TINY
    w1, w3, w2 = synth.expert_weights(wl)
    w2 = w2.clone()
    w2[3, 7, 9] = float("nan")
    from mixed_precision_weight_page_amd import PagedWeightError
    layer, _ = make_layer(wl, (w1, w3, w2), max_tokens=wl.T)
    with pytest.raises(PagedWeightError) as ei:
        layer.quantize_experts(wl.bits)
    assert ei.value.status == -4


def test_zero_expert_and_lossless_grid():
    # expert 1 all zero (s = 0); expert 0 on the 8-bit grid (lossless)
    wl = synth.WORKLOADS["tiny"].scaled(name="grid", E=3, d=128, F=128, k=2, T=8, bits=(8, 4, 3))
    w1, w3, w2 = (m.clone() for m in synth.expert_weights(wl))
    for m in (w1, w3, w2):
        m[1].zero_()
        m[0] = torch.round(m[0] / 2 ** -9).clamp(-127, 127) * 2 ** -9
    w1[0, 0, 0] = 127 * 2 ** -9
    masters = (w1, w3, w2)
    layer, pool = make_layer(wl, masters, max_tokens=wl.T)
    layer.quantize_experts(wl.bits)
    check_pages(layer, pool, masters, wl.bits)
    assert layer.get_page_table()[1]["scale"] == 0.0
    x, logits = synth.tokens(wl)
    y = layer.moe_forward(x.cuda(), logits.cuda())
    compare_y(y, oracle_y(x, logits, wl, masters, wl.bits), "grid")


def test_rounding_ties_and_neighbours():
    """Eq. 2 rounds half to even. With power-of-two scales (absmax = qmax *
    2^-j) the quotients w / s of weights (n + 1/2) s are exact ties, and their
    fp32 neighbours lie just above and below them; every code must match the
    oracle's exact rounding (bit-exact pages)."""
    wl = synth.WORKLOADS["tiny"].scaled(name="ties", E=3, d=128, F=128, k=2, T=8, bits=(8, 4, 3))
    w1, w3, w2 = (m.clone() for m in synth.expert_weights(wl))
    gen = torch.Generator().manual_seed(7)
    for e, (b, j) in enumerate(((8, 8), (4, 5), (3, 4))):
        qm = 2 ** (b - 1) - 1
        s = 2.0 ** -j
        for m in (w1, w3, w2):
            n = torch.randint(-qm, qm, m[e].shape, generator=gen).to(torch.float32)
            tie = (n + 0.5) * s                                  # exact in fp32
            kind = torch.randint(0, 4, m[e].shape, generator=gen)
            up = torch.nextafter(tie, torch.full_like(tie, float("inf")))
            down = torch.nextafter(tie, torch.full_like(tie, float("-inf")))
            m[e] = torch.where(kind == 0, up, torch.where(kind == 1, down, tie))
        w1[e, 0, 0] = qm * s                                     # absmax: s = 2^-j exactly
    masters = (w1, w3, w2)
    layer, pool = make_layer(wl, masters, max_tokens=wl.T)
    layer.quantize_experts(wl.bits)
    for e, j in enumerate((8, 5, 4)):
        assert layer.get_page_table()[e]["scale"] == 2.0 ** -j
    check_pages(layer, pool, masters, wl.bits)


def test_budget_scheduler_follows_a_kv_trace():
    """The KV-pressure scheduler (reading in include/pagedweight.h) on a
    layer with fp16 masters over 48 decode steps of a synthetic KV-cache
    trace: each step's action and budget equal the oracle's decision from
    the oracle's own state (the pool's size being the bytes its pages span);
    after every move the allocation (Eq. 1) and the pages are the oracle's,
    and without pressure the pages span at most the memory the KV cache
    leaves, so the pool's tail from pw_pool_used_bytes on is free for it."""
    wl = SMALL_DYN
    masters = synth.expert_weights(wl)
    layer, pool = make_layer(wl, masters, max_tokens=wl.T)
    p = synth.importance(wl)
    Ltab = c_oracle.loss_table(*masters, nthreads=cpu_threads())
    W = [wl.W_e] * wl.E
    pool8 = osched.pool_nbytes(W, [8] * wl.E)
    memory, reserve, h, n = pool8 + pool8 // 8, pool8 // 16, 0.05, 3
    trace = synth.kv_trace(48, pool8)
    o_pool = o_budget = None
    o_since = 0
    seen = set()
    shrinks_checked = 0
    for t, kv in enumerate(trace):
        got = layer.budget_step(memory, reserve, h, n, kv, p)
        want = osched.decide(memory, reserve, h, n, kv, W, o_pool, o_budget, o_since)
        assert got == want, (t, kv, got, want)
        action, B, pressure = got
        seen.add(action)
        if action != osched.KEEP:
            bits_want, _ = c_oracle.allocate(p, Ltab, W, B)
            table = layer.get_page_table()
            bits = [int(e["bits"]) for e in table]
            assert bits == list(bits_want), t
            assert sum(int(e["nbytes"]) for e in table) == osched.pool_nbytes(W, bits)
            used = layer.pool_used_bytes()
            assert used == max(e["offset"] + e["nbytes"] for e in table)
            if not pressure:
                assert used <= memory - kv - reserve, (t, used, memory - kv - reserve)
                if action == osched.SHRINK:
                    shrinks_checked += 1
            o_pool, o_budget, o_since = used, B, 0
            check_pages(layer, pool, masters, bits, rows_per_matrix=2)
        else:
            o_since += 1
    assert {osched.INIT, osched.SHRINK, osched.GROW, osched.KEEP} <= seen, seen
    assert shrinks_checked > 0
    x, logits = synth.tokens(wl)
    y = layer.moe_forward(x.cuda(), logits.cuda())
    compare_y(y, oracle_y(x, logits, wl, masters, bits), "after the KV trace")


def test_shrink_compacts_pages_below_the_kv_cache():
    """Importance rising with the expert index keeps the last expert's page,
    at the top of the pool, at 8 bits when the KV cache grows: first-fit
    placement of the shrunk pages would leave the pool spanning its whole
    all-8-bit size, above the memory left, so the scheduler rewrites the
    pages densely; they then span exactly their total size, within the
    memory left, bit-exact, and the layer's output is the oracle's."""
    wl = SMALL_DYN
    masters = synth.expert_weights(wl)
    layer, pool = make_layer(wl, masters, max_tokens=wl.T)
    p = synth.importance(wl)[::-1].copy()      # the last expert is the most important
    W = [wl.W_e] * wl.E
    pool8 = osched.pool_nbytes(W, [8] * wl.E)
    memory, reserve = pool8 + pool8 // 8, pool8 // 16
    act, B, pressure = layer.budget_step(memory, reserve, 0.05, 0, 0, p)
    assert act == osched.INIT and not pressure
    before = layer.get_page_table()
    assert [e["bits"] for e in before] == [8] * wl.E
    last_off = before[-1]["offset"]
    kv = pool8 // 2
    act, B, pressure = layer.budget_step(memory, reserve, 0.05, 0, kv, p)
    assert act == osched.SHRINK and not pressure
    table = layer.get_page_table()
    bits = [e["bits"] for e in table]
    assert bits[-1] == 8 and min(bits) < 8
    used = layer.pool_used_bytes()
    total = sum(e["nbytes"] for e in table)
    assert used == total <= memory - kv - reserve < last_off + table[-1]["nbytes"]
    assert table[-1]["offset"] < last_off    # the unchanged page moved down
    check_pages(layer, pool, masters, bits)
    x, logits = synth.tokens(wl)
    y = layer.moe_forward(x.cuda(), logits.cuda())
    compare_y(y, oracle_y(x, logits, wl, masters, bits), "after compaction")


def test_mostly_zero_codes_keep_precision():
    """Outliers x1000 make nearly every 3- and 4-bit code 0, so the true
    products sum only a few terms; the kernel must not let the code offset
    2^(b-1) sum(x) swamp them (long K = 4096 makes that visible)."""
    wl = synth.WORKLOADS["decode_fine"].scaled(name="sparse_codes", E=8, d=4096, F=256, k=2,
                                               T=16, outlier_rate=0.0005, outlier_mult=1000.0,
                                               bits=(3, 3, 3, 4, 4, 8, 3, 4))
    masters = synth.expert_weights(wl)
    x, logits = synth.tokens(wl)
    layer, pool = make_layer(wl, masters, max_tokens=wl.T)
    layer.quantize_experts(wl.bits)
    y = layer.moe_forward(x.cuda(), logits.cuda())
    ref = oracle_y(x, logits, wl, masters, wl.bits)
    norm_err, _ = compare_y(y, ref, "mostly-zero codes")
    assert norm_err < 1e-3


@pytest.mark.parametrize("T", [600, 257, 2100])
def test_large_batch_matrix_core_path(T):
    """Batches with many tokens per expert take the tiled matrix-core
    kernels (64 tokens x 128 or 256 rows per workgroup): ragged last token
    tile, 3/4/8-bit experts, an expert left without tokens, and (2100 tokens)
    a router that ranks pairs over several chunks of 1024 tokens."""
    wl = synth.WORKLOADS["tiny"].scaled(name="gemm_path", E=8, d=512, F=384, k=2, T=T,
                                        bits=(8, 3, 4, 4, 3, 8, 4, 3))
    masters = synth.expert_weights(wl)
    x, logits = synth.tokens(wl)
    logits[:, 6] = -50.0     # expert 6 gets no tokens
    layer, pool = make_layer(wl, masters, max_tokens=T)
    layer.quantize_experts(wl.bits)
    y = layer.moe_forward(x.cuda(), logits.cuda())
    compare_y(y, oracle_y(x, logits, wl, masters, wl.bits), f"matrix-core path T={T}")


def test_small_batch_sweep():
    """Seeded random small decode batches across the shapes whose routing
    and grouping the gate/up kernel does itself (1-16 tokens, 1-64 experts,
    top-1 to top-16, either normalisation, random widths), and just beyond
    them (17 tokens, 65 experts). Every output against the oracle."""
    rng = np.random.default_rng(7)
    cases = [(int(rng.integers(1, 17)), int(rng.integers(1, 65)), None, int(rng.integers(0, 2))) for _ in range(24)]
    cases += [(17, 12, 3, 0), (16, 65, 4, 1), (4, 64, 16, 0), (1, 1, 1, 0)]
    for T, E, k, renorm in cases:
        k = k or int(rng.integers(1, min(16, E) + 1))
        bits = tuple(int(b) for b in rng.choice([3, 4, 8], size=E))
        wl = synth.WORKLOADS["tiny"].scaled(name=f"sweep_{T}_{E}_{k}", E=E, d=256, F=128, k=k, T=T,
                                            renorm=renorm, bits=bits)
        masters = synth.expert_weights(wl)
        layer, _ = make_layer(wl, masters, max_tokens=T)
        layer.quantize_experts(wl.bits)
        x, logits = synth.tokens(wl, seed=T * 1000 + E)
        y = layer.moe_forward(x.cuda(), logits.cuda())
        compare_y(y, oracle_y(x, logits, wl, masters, wl.bits), f"T={T} E={E} k={k} renorm={renorm}")
        del layer


@pytest.mark.parametrize("E,k,renorm", [(8, 2, 0), (40, 1, 1), (64, 16, 0), (17, 8, 1)])
def test_small_batches_routed_by_the_gate_up_kernel(E, k, renorm):
    """Batches of at most 4 tokens over at most 64 experts are routed by the
    gate/up kernel itself (no router launch): 1-4 tokens with planted equal
    logits (ties go to the lower expert), 3/4/8-bit experts, then batches
    routed by the router kernel (16 and 40 tokens) and again by the gate/up
    kernel, so the counter sets each leaves behind serve the next. Every
    output against the oracle."""
    wl = synth.WORKLOADS["tiny"].scaled(name=f"own_route_{E}_{k}", E=E, d=256, F=384, k=k, T=40, renorm=renorm,
                                        bits=tuple((8, 4, 3)[e % 3] for e in range(E)))
    masters = synth.expert_weights(wl)
    layer, _ = make_layer(wl, masters, max_tokens=wl.T)
    layer.quantize_experts(wl.bits)
    for step, T in enumerate((1, 4, 16, 3, 40, 2, 4)):
        x, logits = synth.tokens(wl, T=T, seed=10 + step)
        logits[0, E - 1] = logits[0, 0] = logits[0].max() + 1.0   # a tie at the top
        if T > 1:
            logits[1, :] = 0.5                                   # every logit equal
        y = layer.moe_forward(x.cuda(), logits.cuda())
        compare_y(y, oracle_y(x, logits, wl, masters, wl.bits), f"E={E} k={k} T={T}")


@pytest.mark.parametrize("layout", ["eq2", "bitplane"])
def test_skewed_routing_on_the_streaming_path(layout):
    """Importance-skewed routing of a decode batch: expert 0 takes all 150
    tokens (three passes of 64 in the kernel for experts with more than 16
    tokens), experts 1-3 between 17 and 64, the rest few or none; every
    output against the oracle."""
    from oracle import bitplane
    wl = synth.WORKLOADS["decode_fine"].scaled(name=f"skew_{layout}", E=16, d=256, F=384, k=2, T=150)
    masters = synth.expert_weights(wl)
    layer, _ = make_layer(wl, masters, max_tokens=wl.T, layout=layout)
    bits = [8, 4, 3, 4, 8, 3, 4, 3, 3, 4, 8, 3, 4, 4, 3, 8]
    layer.quantize_experts(bits)
    x, logits = synth.tokens(wl)
    logits[:, 0] += 20.0                       # every token's first expert
    logits[:40, 1] += 10.0
    logits[40:90, 2] += 10.0
    logits[90:110, 3] += 10.0
    counts = torch.bincount(moe.route(logits, wl.k)[0].reshape(-1), minlength=wl.E)
    assert int(counts[0]) == 150 and 16 < int(counts[1]) <= 64 and int(counts[3]) > 16
    log(f"skewed ({layout}): counts {counts.tolist()}")
    y = layer.moe_forward(x.cuda(), logits.cuda())
    if layout == "eq2":
        ref = oracle_y(x, logits, wl, masters, bits)
    else:
        ref = moe.forward(x.float(), logits, wl.k, bitplane.experts(*masters, bits))
    compare_y(y, ref, f"skewed routing ({layout})")


def test_hot_experts_on_multi_tile_workgroups():
    """A layer wide enough (128 experts, d_model 2048) that each workgroup of
    the down product covers several 64-row tiles: six experts take more than
    16 tokens each (the first four get extra workgroups for their remaining
    tiles, the last two keep passes of 16 tokens over their tile
    sequences), the rest few; d_ff = 384 gives three K steps per tile, so
    several tiles end inside one prefetch group. Every output against the
    oracle."""
    wl = synth.WORKLOADS["decode_fine"].scaled(name="hot_multi_tile", E=128, d=2048, F=384, k=2, T=200)
    masters = synth.expert_weights(wl)
    layer, _ = make_layer(wl, masters, max_tokens=wl.T)
    bits = [(8, 4, 3)[e % 3] for e in range(wl.E)]
    layer.quantize_experts(bits)
    x, logits = synth.tokens(wl)
    for h in range(6):
        logits[30 * h:30 * h + 30, 7 * h + 1] += 10.0   # expert 7h+1: 30 tokens
    counts = torch.bincount(moe.route(logits, wl.k)[0].reshape(-1), minlength=wl.E)
    assert int((counts > 16).sum()) == 6
    log(f"hot experts {torch.nonzero(counts > 16).reshape(-1).tolist()}, counts {counts[counts > 16].tolist()}")
    y = layer.moe_forward(x.cuda(), logits.cuda())
    compare_y(y, oracle_y(x, logits, wl, masters, bits), "hot experts, multi-tile workgroups")


@pytest.mark.parametrize("layout", ["eq2", "bitplane"])
def test_more_hot_experts_than_shared_gate_up_tiles(layout):
    """Twenty experts take more than 16 tokens: the gate/up tiles of the
    first sixteen (in routed order) are shared by four workgroups, each
    taking every fourth pass of 16 tokens (one expert has 100 tokens: seven
    passes over its four shares if it is among them), the other four take
    wide passes of up to 64 tokens. Every output against the oracle."""
    from oracle import bitplane
    wl = synth.WORKLOADS["decode_fine"].scaled(name=f"hot_shares_{layout}", E=128, d=512, F=384, k=2, T=480)
    masters = synth.expert_weights(wl)
    layer, _ = make_layer(wl, masters, max_tokens=wl.T, layout=layout)
    bits = ([(8, 4, 3)[e % 3] for e in range(wl.E)] if layout == "eq2"
            else [1 + e % 8 for e in range(wl.E)])
    layer.quantize_experts(bits)
    x, logits = synth.tokens(wl)
    logits[:100, 2] += 10.0                             # expert 2: 100 tokens
    for h in range(1, 20):
        logits[100 + 20 * (h - 1):120 + 20 * (h - 1), 5 * h + 2] += 10.0   # expert 5h+2: 20 tokens
    counts = torch.bincount(moe.route(logits, wl.k)[0].reshape(-1), minlength=wl.E)
    assert int((counts > 16).sum()) == 20 and int(counts[2]) >= 100
    log(f"hot experts ({layout}) {torch.nonzero(counts > 16).reshape(-1).tolist()}, counts {counts[counts > 16].tolist()}")
    y = layer.moe_forward(x.cuda(), logits.cuda())
    if layout == "eq2":
        ref = oracle_y(x, logits, wl, masters, bits)
    else:
        ref = moe.forward(x.float(), logits, wl.k, bitplane.experts(*masters, bits))
    compare_y(y, ref, f"hot experts beyond the shared ones ({layout})")


def test_down_split_with_row_block_sequences():
    """A batch whose down product is both split along K and walked in
    sequences of row blocks per wave: 12 routed experts x 64 row tiles of
    d_model 4096 give 768 workgroups per split, so two K splits of d_ff 1536
    (6 steps each), and two row blocks per wave fill the 1024 resident
    workgroups as well as one does (the launch takes the larger); the code
    cursor then steps from one block's K range to the next block's.
    3/4/8-bit experts; every output against the oracle."""
    wl = TINY.scaled(name="split_seq", E=12, d=4096, F=1536, k=2, T=6,
                     bits=(8, 4, 3, 4, 3, 8, 3, 4, 8, 3, 4, 3))
    masters = synth.expert_weights(wl)
    layer, _ = make_layer(wl, masters, max_tokens=wl.T)
    layer.quantize_experts(wl.bits)
    x, logits = synth.tokens(wl)
    # every expert routed once: token t takes experts 2t and 2t + 1
    logits = torch.full((wl.T, wl.E), -5.0)
    for t in range(wl.T):
        logits[t, 2 * t] = 2.0
        logits[t, 2 * t + 1] = 1.0
    counts = torch.bincount(moe.route(logits, wl.k)[0].reshape(-1), minlength=wl.E)
    assert int((counts > 0).sum()) == 12
    y = layer.moe_forward(x.cuda(), logits.cuda())
    compare_y(y, oracle_y(x, logits, wl, masters, list(wl.bits)), "down split with row-block sequences")


def test_small_batches_on_a_context_sized_for_large_ones():
    """A context whose workspace is sized for 2048 tokens (its partial-output
    buffer holds one split per pair) still splits the down product of a
    1- or 3-token batch: the split stride is the batch's own pair count."""
    wl = synth.WORKLOADS["tiny"].scaled(name="big_ctx", E=4, d=256, F=1024, k=2, T=3, bits=(8, 4, 3, 4))
    masters = synth.expert_weights(wl)
    layer, pool = make_layer(wl, masters, max_tokens=2048)
    layer.quantize_experts(wl.bits)
    for T in (1, 3, 40):
        x, logits = synth.tokens(wl, T=T, step=T)
        log(f"large context: forward T={T}")
        y = layer.moe_forward(x.cuda(), logits.cuda())
        compare_y(y, oracle_y(x, logits, wl, masters, wl.bits), f"large context T={T}")


@pytest.mark.parametrize("F", [384, 640, 896, 1024])
def test_down_splits_summed_in_order(F):
    """Small batches split the down product along d_ff (here into 3, 5, 7
    and 8 parts for one and three tokens); the combine sums every split of
    every slot, two splits per round of loads, odd counts included."""
    wl = synth.WORKLOADS["tiny"].scaled(name=f"splits_F{F}", E=4, d=256, F=F, k=2, T=3,
                                        bits=(8, 4, 3, 4))
    masters = synth.expert_weights(wl)
    layer, pool = make_layer(wl, masters, max_tokens=wl.T)
    layer.quantize_experts(wl.bits)
    for T in (1, 3):
        x, logits = synth.tokens(wl, T=T)
        log(f"splits F={F}: forward T={T}")
        y = layer.moe_forward(x.cuda(), logits.cuda())
        compare_y(y, oracle_y(x, logits, wl, masters, wl.bits), f"splits F={F} T={T}")


EXTREME = [
    # one expert, top-1, the smallest rows (one 128-code step, two 64-row tiles)
    (synth.WORKLOADS["tiny"].scaled(name="one", E=1, d=128, F=128, k=1, T=5, bits=(3,)), (5, 1)),
    (synth.WORKLOADS["tiny"].scaled(name="one8", E=1, d=128, F=128, k=1, T=3, bits=(8,)), (3,)),
    # the most experts and the largest top-k the library takes
    (synth.WORKLOADS["tiny"].scaled(name="e1024", E=1024, d=128, F=128, k=32, T=40,
                                    bits=tuple([8, 4, 3, 4] * 256)), (40, 7)),
    # on both sides of the matrix-core threshold (mean 64 tokens per routed expert)
    (synth.WORKLOADS["tiny"].scaled(name="edge", E=2, d=256, F=128, k=1, T=128, bits=(4, 3)), (128, 127)),
]


@pytest.mark.parametrize("wl,Ts", EXTREME, ids=lambda v: v.name if hasattr(v, "name") else str(v))
def test_extreme_shapes(wl, Ts):
    masters = synth.expert_weights(wl)
    layer, pool = make_layer(wl, masters, max_tokens=max(Ts))
    log(f"{wl.name}: quantize")
    layer.quantize_experts(wl.bits)
    torch.cuda.synchronize()
    check_pages(layer, pool, masters, wl.bits)
    for T in Ts:
        x, logits = synth.tokens(wl, T=T)
        log(f"{wl.name}: forward T={T}")
        y = layer.moe_forward(x.cuda(), logits.cuda())
        compare_y(y, oracle_y(x, logits, wl, masters, wl.bits), f"{wl.name} T={T}")
