"""Oracle for the MoE expert layer forward pass.

TEST INFRASTRUCTURE: imported only by tests, the smoke check and the
benchmark's CPU baseline; never by the GPU library.

Follows section "Dynamic Paging" of the PagedWeight page: the router picks
the experts a token needs, their quantized weights are dequantized
(Q(w) = s * q, Eq. 2) and the experts run in full precision. Readings where
the page is silent:

* router: the k largest logits per token, equal logits resolved towards the
  lower expert index; routing weight g = softmax probability over all E
  experts (``renorm=False``) or renormalised over the k chosen
  (``renorm=True``);
* expert: SwiGLU, a = W1 x (gate), c = W3 x (up), h = silu(a) * c with
  silu(z) = z / (1 + exp(-z)), o = W2 h;
* combine: y_t = sum over the chosen experts of g * o.

Everything is float64; x enters as the exact value of its bf16 input.
"""
from __future__ import annotations

import torch

from . import quant


def route(logits: torch.Tensor, k: int, renorm: bool = False):
    """Top-k experts per token and their weights.

    Returns (ids int64 [T, k] in descending logit order, g float64 [T, k]).
    """
    l32 = logits.to(torch.float32)
    ids = torch.sort(l32, dim=1, descending=True, stable=True).indices[:, :k]
    l64 = l32.to(torch.float64)
    ex = torch.exp(l64 - l64.max(dim=1, keepdim=True).values)
    chosen = torch.gather(ex, 1, ids)
    den = chosen.sum(1, keepdim=True) if renorm else ex.sum(1, keepdim=True)
    return ids, chosen / den


def expert_ffn(x64: torch.Tensor, W1: torch.Tensor, W3: torch.Tensor,
               W2: torch.Tensor) -> torch.Tensor:
    """o = W2 (silu(W1 x) * (W3 x)) for the rows of x64 [n, d] (float64)."""
    a = x64 @ W1.T
    c = x64 @ W3.T
    h = a / (1.0 + torch.exp(-a)) * c
    return h @ W2.T


def forward(x: torch.Tensor, logits: torch.Tensor, k: int, experts,
            renorm: bool = False) -> torch.Tensor:
    """y [T, d] float64.

    ``experts(e)`` returns the float64 dequantized (W1 [F,d], W3 [F,d],
    W2 [d,F]) of expert e; it is called only for experts some token uses.
    """
    T = x.shape[0]
    x64 = x.to(torch.float64)
    ids, g = route(logits, k, renorm)
    y = torch.zeros((T, x.shape[1]), dtype=torch.float64)
    for e in torch.unique(ids).tolist():
        rows, slots = (ids == e).nonzero(as_tuple=True)
        W1, W3, W2 = experts(e)
        o = expert_ffn(x64[rows], W1, W3, W2)
        y.index_add_(0, rows, g[rows, slots].unsqueeze(1) * o)
    return y


def quantized_experts(w1, w3, w2, bits):
    """experts(e) callback returning s_e * q of each matrix at bits[e]."""
    def get(e):
        m = quant.expert_absmax((w1[e], w3[e], w2[e]))
        b = int(bits[e])
        s = quant.scale(m, b)
        return (quant.dequant(w1[e], s, b), quant.dequant(w3[e], s, b),
                quant.dequant(w2[e], s, b))
    return get


def moe_forward_quantized(x, logits, k, w1, w3, w2, bits, renorm=False):
    """The whole layer from fp masters: quantize at ``bits``, then forward."""
    return forward(x, logits, k, quantized_experts(w1, w3, w2, bits), renorm)
