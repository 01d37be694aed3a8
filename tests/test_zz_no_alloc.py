"""GPU test of pw_moe_forward_noalloc (the forward whose scratch is the
library's static device array): through the C ABI, two calls in a row on
one context, the second with a smaller batch, each against pw_moe_forward on
the same inputs (to the layer tolerance; the two may split the down product
differently) and against the float64 oracle; then a batch on the
matrix-core path, and a batch too large for the array, which must fail
cleanly and leave the next call working."""
import pytest
import torch

import synth
from layer_cases import compare_y, cpu_threads, log, make_layer, oracle_y

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cpu_threads()


def test_noalloc_forward_matches_the_workspace_forward():
    from mixed_precision_weight_page_amd import PagedWeightError
    wl = synth.WORKLOADS["decode_fine"].scaled(name="noalloc", E=32, d=256, F=384, T=64)
    masters = synth.expert_weights(wl)
    layer, _ = make_layer(wl, masters, max_tokens=2048)
    bits = [(3, 4, 8)[e % 3] for e in range(wl.E)]
    layer.quantize_experts(bits)
    for step, T in enumerate((64, 9, 1, 600)):
        x, logits = synth.tokens(wl, T=T, step=step)
        xc, lc = x.cuda(), logits.cuda()
        log(f"noalloc: T={T}")
        y_ws = layer.moe_forward(xc, lc)
        y_st = torch.full((T, wl.d), float("nan"), device="cuda")
        layer.moe_forward_noalloc(xc, lc, y_st)
        torch.cuda.synchronize()
        ref = oracle_y(x, logits, wl, masters, bits)
        compare_y(y_st, y_ws.cpu().double(), f"noalloc vs workspace forward T={T}")
        compare_y(y_st, ref, f"noalloc vs oracle T={T}")


def test_noalloc_refuses_a_batch_larger_than_its_scratch():
    from mixed_precision_weight_page_amd import PagedWeightError
    # 4096 tokens x top-2 at d_model 4096: the partial outputs alone take
    # 128 MiB, more than the static array holds
    wl = synth.WORKLOADS["tiny"].scaled(name="noalloc_big", E=8, d=4096, F=256, k=2, T=4096,
                                        bits=(8, 4, 3, 4, 8, 4, 3, 4))
    masters = synth.expert_weights(wl)
    layer, _ = make_layer(wl, masters, max_tokens=4096)
    layer.quantize_experts(wl.bits)
    x, logits = synth.tokens(wl, T=4096, step=1)
    y = torch.empty((4096, wl.d), device="cuda")
    with pytest.raises(PagedWeightError) as err:
        layer.moe_forward_noalloc(x.cuda(), logits.cuda(), y)
    assert "scratch" in str(err.value)
    x, logits = synth.tokens(wl, T=3, step=2)
    y = torch.empty((3, wl.d), device="cuda")
    layer.moe_forward_noalloc(x.cuda(), logits.cuda(), y)
    torch.cuda.synchronize()
    compare_y(y, oracle_y(x, logits, wl, masters, wl.bits), "noalloc after a refused batch")
