"""GPU parity over the whole range of the inputs: the layer takes bf16
activations, whose range (up to about 3.4e38, subnormal down to about 9e-41)
is far wider than that of the fp16 operands of the matrix cores (largest
finite 65504, subnormal down to 6e-8), and the SwiGLU rows h between the two
products can be large. Every case is checked against the float64 oracle,
token row by token row (one row can be 10^30 times another, so a norm over
the batch would hide the small rows), on the streaming (decode) path and on
the matrix-core (large-batch) path."""
import pytest
import torch

import synth
from layer_cases import compare_y, compare_y_rows, cpu_threads, log, make_layer, oracle_y

pytestmark = pytest.mark.gpu

# a tiny-shaped layer with every bit-width; 24 tokens take the streaming
# kernels (48 pairs < 64 per routed expert), 300 tokens the matrix-core ones
WL = synth.WORKLOADS["tiny"].scaled(name="range", T=24)
PATHS = [("streaming", 24), ("matrix", 300)]


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cpu_threads()


def _run(wl, x, logits, masters, what):
    layer, _ = make_layer(wl, masters, max_tokens=x.shape[0])
    layer.quantize_experts(wl.bits)
    log(f"{what}: forward, T={x.shape[0]}")
    y = layer.moe_forward(x.cuda(), logits.cuda())
    torch.cuda.synchronize()
    ref = oracle_y(x, logits, wl, masters, wl.bits)
    assert torch.isfinite(y).all(), what
    return y, ref


@pytest.mark.parametrize("path,T", PATHS, ids=[p for p, _ in PATHS])
def test_token_rows_across_the_bf16_range(path, T):
    # row t is N(0, 1) times 2^j_t, j_t in [-56, 56]: the outputs (about
    # 0.05 |x|^2 here) stay inside fp32's normal range; fp16 operands without
    # scaling would flush the small rows to 0 and overflow the large ones
    masters = synth.expert_weights(WL)
    x, logits = synth.tokens(WL, T=T)
    js = torch.tensor([-56, -40, -24, -12, -4, 0, 4, 12, 24, 40, 56])
    scale = torch.pow(2.0, js[torch.arange(T) % len(js)].double()).float()
    x = (x.float() * scale[:, None]).to(torch.bfloat16)
    y, ref = _run(WL, x, logits, masters, f"{path}: rows 2^-56..2^56")
    compare_y_rows(y, ref, path)


@pytest.mark.parametrize("path,T", PATHS, ids=[p for p, _ in PATHS])
def test_activations_near_1e30_with_tiny_weights(path, T):
    # |x| around 1e30 (fp16 overflows at 65504) against weights N(0, 1e-20):
    # the SwiGLU rows reach about 1e22 and the outputs stay moderate
    wl = WL.scaled(name="range_e30", w_std=1e-20)
    masters = synth.expert_weights(wl)
    x, logits = synth.tokens(wl, T=T)
    x = (x.float() * 1e30).to(torch.bfloat16)
    y, ref = _run(wl, x, logits, masters, f"{path}: |x| ~ 1e30")
    compare_y_rows(y, ref, path)
    compare_y(y, ref, path)


@pytest.mark.parametrize("path,T", PATHS, ids=[p for p, _ in PATHS])
def test_swiglu_rows_beyond_fp16(path, T):
    # activations N(0, 1000): the gate and up sums reach a few hundred, so h
    # exceeds 1e5 (largest fp16: 65504)
    masters = synth.expert_weights(WL)
    x, logits = synth.tokens(WL, T=T)
    x = (x.float() * 1000.0).to(torch.bfloat16)
    y, ref = _run(WL, x, logits, masters, f"{path}: |h| > 1e5")
    # the largest |h| of the oracle's forward, recomputed for the record
    from oracle import moe, quant
    w1, w3, _ = masters
    ids, _ = moe.route(logits, WL.k)
    e = int(ids[0, 0])
    s = quant.scale(quant.expert_absmax((w1[e], w3[e], masters[2][e])), WL.bits[e])
    a = x[:1].double() @ quant.dequant(w1[e], s, WL.bits[e]).T
    c = x[:1].double() @ quant.dequant(w3[e], s, WL.bits[e]).T
    hmax = float((a / (1 + torch.exp(-a)) * c).abs().max())
    log(f"  token 0, expert {e}: max |h| = {hmax:.3e}")
    assert hmax > 1e5
    compare_y_rows(y, ref, path)
    compare_y(y, ref, path)


@pytest.mark.parametrize("path,T", PATHS, ids=[p for p, _ in PATHS])
def test_tiny_activations(path, T):
    # |x| around 1e-12 (below fp16's smallest subnormal, 6e-8)
    masters = synth.expert_weights(WL)
    x, logits = synth.tokens(WL, T=T)
    x = (x.float() * 1e-12).to(torch.bfloat16)
    y, ref = _run(WL, x, logits, masters, f"{path}: |x| ~ 1e-12")
    assert float(ref.abs().max()) > 0
    compare_y_rows(y, ref, path)


def test_zero_rows_and_zero_expert():
    # an all-zero token row gives an all-zero output row; an expert whose
    # weights are all zero contributes nothing
    masters = [m.clone() for m in synth.expert_weights(WL)]
    for m in masters:
        m[2].zero_()
    x, logits = synth.tokens(WL, T=24)
    x[3].zero_()
    logits[5, 2] = logits[5].max() + 1.0   # token 5's first expert is the zero expert
    y, ref = _run(WL, x, logits, masters, "zero row / zero expert")
    assert torch.equal(y[3].cpu(), torch.zeros(WL.d))
    compare_y_rows(y, ref, "zero row / zero expert")
