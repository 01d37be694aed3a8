"""The plain C++ CPU oracle (``cpu_oracle.cpp``) through ctypes.

TEST INFRASTRUCTURE: imported only by tests, the smoke check and the
benchmark's CPU baseline; never by the GPU library.

``cpu_oracle.cpp`` computes Eq. 2 (scale, codes, page bytes, loss), Eq. 1
(the allocation) and the forward pass of section "Dynamic Paging" of the
PagedWeight page in plain double-precision loops. This module only moves
arrays in and out (numpy) and builds the shared library with g++ when it is
missing or older than its source.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "cpu_oracle.cpp")
LIB = os.path.join(HERE, "libcpu_oracle.so")
BITS = (3, 4, 8)

_lock = threading.Lock()
_lib = None


class Infeasible(Exception):
    """B < 3 sum_e W_e: even all-3-bit does not fit."""


def build(force: bool = False) -> str:
    """Compile cpu_oracle.cpp (g++, -O2, no fused multiply-add, OpenMP)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp%d" % os.getpid()
        cmd = ["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
               "-Wall", "-o", tmp, SRC]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("g++ failed for the CPU oracle:\n" + r.stdout + r.stderr)
        os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    with _lock:
        if _lib is None:
            L = ctypes.CDLL(build())
            P = ctypes.c_void_p
            i32, i64, u64, f32, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float, ctypes.c_double
            sig = {
                "orc_qmax": (i32, [i32]),
                "orc_absmax": (f64, [P, i64]),
                "orc_scale": (f32, [f64, i32]),
                "orc_codes": (None, [P, i64, f32, i32, P]),
                "orc_row_bytes": (i64, [i32, i32]),
                "orc_page_bytes": (i64, [i32, i32, i32]),
                "orc_pack_rows": (None, [P, i32, i32, i32, P]),
                "orc_quantize_expert": (i32, [P, P, P, i32, i32, i32, P, P, P]),
                "orc_loss": (f64, [P, P, P, i32, i32, i32]),
                "orc_allocate": (i32, [i32, P, P, P, u64, P, P]),
                "orc_allocate_brute": (i32, [i32, P, P, P, u64, P, P]),
                "orc_route": (i32, [P, i32, i32, i32, i32, P, P]),
                "orc_moe_forward": (i32, [P, P, i32, i32, i32, i32, i32, i32, P, P, P, i32]),
            }
            for name, (res, args) in sig.items():
                fn = getattr(L, name)
                fn.restype = res
                fn.argtypes = args
            _lib = L
    return _lib


def _f32(a) -> np.ndarray:
    """A contiguous float32 numpy array of a tensor or array (fp16 masters
    convert exactly)."""
    if hasattr(a, "detach"):
        a = a.detach().cpu().float().numpy()
    return np.ascontiguousarray(a, dtype=np.float32)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def qmax(b: int) -> int:
    return lib().orc_qmax(b)


def absmax(w) -> float:
    w = _f32(w)
    return lib().orc_absmax(_ptr(w), w.size)


def scale(m: float, b: int) -> float:
    return float(lib().orc_scale(float(m), int(b)))


def codes(w, s: float, b: int) -> np.ndarray:
    w = _f32(w)
    q = np.empty(w.shape, dtype=np.int8)
    lib().orc_codes(_ptr(w), w.size, float(s), int(b), _ptr(q))
    return q


def pack_rows(q: np.ndarray, b: int) -> np.ndarray:
    """[rows, K] signed codes -> [rows, row_bytes] packed stored codes."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    rows, K = q.shape
    out = np.empty((rows, lib().orc_row_bytes(K, b)), dtype=np.uint8)
    lib().orc_pack_rows(_ptr(q), rows, K, int(b), _ptr(out))
    return out


def page_bytes(d: int, F: int, b: int) -> int:
    return lib().orc_page_bytes(d, F, b)


def quantize_expert(w1, w3, w2, b: int, want_page: bool = True):
    """(s, codes [3 d F] int8 in W1, W3, W2 order, page uint8 or None) of
    one expert: w1, w3 [F, d], w2 [d, F]."""
    w1, w3, w2 = _f32(w1), _f32(w3), _f32(w2)
    F, d = w1.shape
    q = np.empty(3 * d * F, dtype=np.int8)
    page = np.empty(page_bytes(d, F, b), dtype=np.uint8) if want_page else None
    s = ctypes.c_float(0.0)
    rc = lib().orc_quantize_expert(_ptr(w1), _ptr(w3), _ptr(w2), d, F, int(b), ctypes.byref(s), _ptr(q),
                                   _ptr(page) if want_page else None)
    if rc != 0:
        raise ValueError(f"unsupported bit-width {b}")
    return float(s.value), q, page


def loss(w1, w3, w2, b: int) -> float:
    w1, w3, w2 = _f32(w1), _f32(w3), _f32(w2)
    F, d = w1.shape
    return lib().orc_loss(_ptr(w1), _ptr(w3), _ptr(w2), d, F, int(b))


def loss_table(w1, w3, w2, nthreads: int = 1) -> np.ndarray:
    """L [E, 3] for 3, 4 and 8 bits (w1, w3 [E, F, d], w2 [E, d, F]); the
    experts on up to nthreads threads (the C call releases the interpreter)."""
    E = w1.shape[0]
    L = np.zeros((E, len(BITS)))

    def one(e):
        L[e] = [loss(w1[e], w3[e], w2[e], b) for b in BITS]
    if nthreads > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(one, range(E)))
    else:
        for e in range(E):
            one(e)
    return L


def _solve(fn, p, L, W, B):
    E = len(p)
    p = np.ascontiguousarray(p, dtype=np.float64)
    L = np.ascontiguousarray(np.asarray(L, dtype=np.float64).reshape(E, 3))
    W = np.ascontiguousarray(W, dtype=np.uint64)
    bits = np.zeros(E, dtype=np.uint8)
    obj = ctypes.c_double(0.0)
    rc = fn(E, _ptr(p), _ptr(L), _ptr(W), int(B), _ptr(bits), ctypes.byref(obj))
    if rc == 1:
        raise Infeasible()
    if rc != 0:
        raise ValueError("allocation problem rejected (bad input or table too large)")
    return [int(b) for b in bits], float(obj.value)


def allocate(p, L, W, B):
    """Eq. 1 by the exact dynamic programme: (bits, objective)."""
    return _solve(lib().orc_allocate, p, L, W, B)


def allocate_brute(p, L, W, B):
    """Eq. 1 by enumeration (E <= 12): (bits, objective)."""
    return _solve(lib().orc_allocate_brute, p, L, W, B)


def allocate_layers(ps, Ls, Ws, B, layer_weights=None):
    """Eq. 1 with one budget B over the experts of several layers: the
    objective sum_l w_l sum_e p_{l,e} L_{l,e}(b) and the constraint are sums
    over the union of the layers' experts, so this is the DP above on that
    union with importances w_l p_{l,e}. Returns (per-layer bit lists,
    objective)."""
    n = len(ps)
    w = [1.0] * n if layer_weights is None else [float(v) for v in layer_weights]
    p_all = np.concatenate([w[l] * np.asarray(ps[l], dtype=np.float64) for l in range(n)])
    L_all = np.concatenate([np.asarray(Ls[l], dtype=np.float64).reshape(-1, 3) for l in range(n)])
    W_all = np.concatenate([np.asarray(Ws[l], dtype=np.uint64) for l in range(n)])
    bits, obj = allocate(p_all, L_all, W_all, B)
    out, i = [], 0
    for l in range(n):
        out.append(bits[i:i + len(ps[l])])
        i += len(ps[l])
    return out, obj


def route(logits, k: int, renorm: bool = False):
    """(ids int32 [T, k], g float64 [T, k])."""
    l = _f32(logits)
    T, E = l.shape
    ids = np.empty((T, k), dtype=np.int32)
    g = np.empty((T, k), dtype=np.float64)
    if lib().orc_route(_ptr(l), T, E, int(k), int(bool(renorm)), _ptr(ids), _ptr(g)) != 0:
        raise ValueError("bad k")
    return ids, g


def bf16_bits(x) -> np.ndarray:
    """bf16 bit patterns of x (a bf16 tensor, or values exactly representable
    in bf16)."""
    import torch
    t = x if hasattr(x, "detach") else torch.as_tensor(np.asarray(x, dtype=np.float32))
    t = t.detach().cpu().to(torch.bfloat16).contiguous()
    return np.ascontiguousarray(t.view(torch.int16).numpy().view(np.uint16))


def quantize_layer(w1, w3, w2, bits, experts=None, nthreads: int = 1):
    """Scales [E] and codes of the listed experts (all by default) at their
    bits; experts are quantized on up to nthreads threads (the C call
    releases the interpreter)."""
    E = w1.shape[0]
    experts = range(E) if experts is None else experts
    scales = np.zeros(E, dtype=np.float32)
    qs = [None] * E

    def one(e):
        s, q, _ = quantize_expert(w1[e], w3[e], w2[e], int(bits[e]), want_page=False)
        scales[e] = s
        qs[e] = q
    if nthreads > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(one, experts))
    else:
        for e in experts:
            one(e)
    return scales, qs


def moe_forward(x, logits, k: int, scales, qs, renorm: bool = False, nthreads: int = 1) -> np.ndarray:
    """y [T, d] float64 from bf16 x [T, d], logits [T, E] and the experts'
    codes (qs[e] None for experts no token routes to)."""
    xb = bf16_bits(x)
    l = _f32(logits)
    T, d = xb.shape
    E = l.shape[1]
    F = None
    for q in qs:
        if q is not None:
            F = q.size // (3 * d)
            break
    if F is None:
        raise ValueError("no expert codes given")
    ptrs = (ctypes.c_void_p * E)(*[q.ctypes.data if q is not None else None for q in qs])
    sc = np.ascontiguousarray(scales, dtype=np.float32)
    y = np.empty((T, d), dtype=np.float64)
    rc = lib().orc_moe_forward(_ptr(xb), _ptr(l), T, d, F, E, int(k), int(bool(renorm)),
                               ctypes.cast(ptrs, ctypes.c_void_p), _ptr(sc), _ptr(y), int(nthreads))
    if rc != 0:
        raise ValueError("forward rejected: bad k or a routed expert without codes")
    return y


def moe_forward_quantized(x, logits, k: int, w1, w3, w2, bits, renorm: bool = False, nthreads: int = 1):
    """The whole layer from fp masters: quantize the routed experts at their
    bits, then the forward pass."""
    ids, _ = route(logits, k, renorm)
    used = sorted(set(int(e) for e in ids.reshape(-1)))
    scales, qs = quantize_layer(w1, w3, w2, bits, used, nthreads)
    return moe_forward(x, logits, k, scales, qs, renorm, nthreads)
