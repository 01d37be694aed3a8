"""GPU test: pw_moe_forward_noalloc captured in a HIP graph (through torch's
graph capture on its capture stream) and replayed. The forward records only
kernel launches on the caller's stream and clears its counters with a fill
kernel, so a captured forward is replayable; every replay gets new inputs
copied into the captured buffers, eager forwards and synchronisations run
between the replays, and each replay's y must equal the eager forward's y on
the same inputs bit for bit (the kernels are deterministic), and the first
must be within the layer tolerance of the oracle. Paths: the self-routing
decode kernel (4 and 12 tokens), the streaming kernels behind the router (40
tokens over 32 experts), the same with routing skewed so that experts take
passes of more than 16 tokens (150 tokens over 16 experts), bitplane pages
(24 tokens, depths 1 to 8) and the matrix-core kernels (600 tokens over 8
experts)."""
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


CASES = [
    ("own_route_T4", dict(E=8, d=256, F=512, k=2), 4, "eq2", False),
    ("own_group_T12", dict(E=8, d=256, F=512, k=2), 12, "eq2", False),
    ("router_T40", dict(E=32, d=256, F=384, k=2), 40, "eq2", False),
    ("skewed_T150", dict(E=16, d=256, F=384, k=2), 150, "eq2", True),
    ("bitplane_T24", dict(E=8, d=256, F=384, k=2), 24, "bitplane", False),
    ("matrix_core_T600", dict(E=8, d=512, F=384, k=2), 600, "eq2", False),
]


def skew(logits):
    """Every token's first expert is 0; experts 1-3 take runs of tokens."""
    logits[:, 0] += 20.0
    logits[:40, 1] += 10.0
    logits[40:90, 2] += 10.0
    logits[90:110, 3] += 10.0
    return logits


def reference(x, lg, wl, masters, bits, layout):
    if layout == "eq2":
        return oracle_y(x, lg, wl, masters, bits)
    from oracle import bitplane, moe
    return moe.forward(x.float(), lg, wl.k, bitplane.experts(*masters, bits), bool(wl.renorm))


@pytest.mark.parametrize("name,shape,T,layout,skewed", CASES, ids=[c[0] for c in CASES])
def test_captured_noalloc_forward_replays(name, shape, T, layout, skewed):
    wl = synth.WORKLOADS["decode_fine"].scaled(name=f"graph_{name}", T=T, **shape)
    masters = synth.expert_weights(wl)
    layer, _ = make_layer(wl, masters, max_tokens=T, layout=layout)
    bits = ([(3, 4, 8)[e % 3] for e in range(wl.E)] if layout == "eq2"
            else [1 + e % 8 for e in range(wl.E)])
    layer.quantize_experts(bits)
    batches = [synth.tokens(wl, T=T, step=i) for i in range(4)]
    if skewed:
        batches = [(x, skew(lg)) for x, lg in batches]
    xs = batches[0][0].cuda().clone()
    ls = batches[0][1].cuda().clone()
    ys = torch.zeros((T, wl.d), dtype=torch.float32, device="cuda")
    log(f"graph {name}: eager warm-up, then capture")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.moe_forward_noalloc(xs, ls, ys)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.moe_forward_noalloc(xs, ls, ys)
    torch.cuda.synchronize()
    for i in range(1, 4):
        x, lg = batches[i]
        xs.copy_(x.cuda())
        ls.copy_(lg.cuda())
        ys.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        y_graph = ys.clone()
        y_eager = torch.full((T, wl.d), float("nan"), device="cuda")
        layer.moe_forward_noalloc(x.cuda(), lg.cuda(), y_eager)
        torch.cuda.synchronize()
        log(f"  replay {i}")
        assert torch.equal(y_graph, y_eager), f"{name}: replay {i} differs from the eager forward"
        if i == 1:
            compare_y(y_graph, reference(x, lg, wl, masters, bits, layout), f"graph replay {name}")
    del g
    torch.cuda.synchronize()
