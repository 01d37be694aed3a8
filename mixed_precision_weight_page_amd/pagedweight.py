"""ctypes binding of libpagedweight.so (include/pagedweight.h).

Argument marshalling only: every function checks dtypes, devices and
contiguity, passes raw pointers and the current HIP stream to the C ABI and
turns a negative status into ``PagedWeightError``. All computation happens in
the library's HIP kernels; if the library is not built, importing the
binding works but every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np
import torch

# PW_LIBRARY may name another build of the same library (the tests' host
# sanitizer build); by default the one built in-tree
_LIB_PATH = os.environ.get("PW_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                         "libpagedweight.so")
_lib = None

PW_MASTER_F32 = 0
PW_MASTER_F16 = 1
PW_LAYOUT_EQ2 = 0
PW_LAYOUT_BITPLANE = 1
BITS = (3, 4, 8)


class PagedWeightError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"pagedweight error {status}: {message}")
        self.status = status


class LayerDesc(ctypes.Structure):
    _fields_ = [("num_experts", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("d_ff", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("renorm", ctypes.c_int32), ("max_tokens", ctypes.c_int32),
                ("master_dtype", ctypes.c_int32), ("layout", ctypes.c_int32)]


class PageEntry(ctypes.Structure):
    _fields_ = [("offset", ctypes.c_uint64), ("nbytes", ctypes.c_uint64),
                ("scale", ctypes.c_float), ("bits", ctypes.c_uint8),
                ("pad_", ctypes.c_uint8 * 3)]


class ProfileData(ctypes.Structure):
    _fields_ = [("route_ms", ctypes.c_double), ("gate_up_ms", ctypes.c_double),
                ("down_ms", ctypes.c_double), ("combine_ms", ctypes.c_double),
                ("forwards", ctypes.c_int64)]


class BudgetPolicy(ctypes.Structure):
    """pw_budget_policy: memory shared by the pool and the KV cache, bytes
    kept free, headroom fraction, steps from a change to the next grow."""
    _fields_ = [("memory_bytes", ctypes.c_uint64), ("reserve_bytes", ctypes.c_uint64),
                ("headroom", ctypes.c_double), ("min_interval", ctypes.c_int32)]


BUDGET_KEEP, BUDGET_SHRINK, BUDGET_GROW, BUDGET_INIT = 0, 1, 2, 3

_P = ctypes.c_void_p
_SIGNATURES = {
    "pw_create": (ctypes.c_int, [ctypes.POINTER(LayerDesc), ctypes.POINTER(_P)]),
    "pw_destroy": (None, [_P]),
    "pw_bind_masters": (ctypes.c_int, [_P, _P, _P, _P]),
    "pw_pool_bytes_for_bits": (ctypes.c_uint64, [_P, _P]),
    "pw_bind_pool": (ctypes.c_int, [_P, _P, ctypes.c_uint64]),
    "pw_workspace_bytes": (ctypes.c_uint64, [_P]),
    "pw_bind_workspace": (ctypes.c_int, [_P, _P, ctypes.c_uint64]),
    "pw_quantize_experts": (ctypes.c_int, [_P, _P, _P]),
    "pw_set_budget": (ctypes.c_int, [_P, ctypes.c_uint64, _P, _P, _P, _P]),
    "pw_moe_forward": (ctypes.c_int, [_P, _P, _P, ctypes.c_int32, _P, _P]),
    "pw_moe_forward_noalloc": (ctypes.c_int, [_P, _P, _P, ctypes.c_int32, _P, _P]),
    "pw_route": (ctypes.c_int, [_P, _P, ctypes.c_int32, _P, _P, _P, _P]),
    "pw_get_page_table": (ctypes.c_int, [_P, ctypes.POINTER(PageEntry)]),
    "pw_get_loss_table": (ctypes.c_int, [_P, _P, _P]),
    "pw_solve_allocation": (ctypes.c_int, [ctypes.c_int32, _P, _P, _P, ctypes.c_uint64, _P]),
    "pw_solve_allocation_layers": (ctypes.c_int, [ctypes.c_int32, _P, _P, _P, _P, _P, ctypes.c_uint64, _P, _P]),
    "pw_proportional_bits": (ctypes.c_int, [ctypes.c_int32, _P, _P, ctypes.c_uint64, _P, _P]),
    "pw_budget_decide": (ctypes.c_int, [ctypes.POINTER(BudgetPolicy), ctypes.c_uint64, ctypes.c_int32, _P,
                                        ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int32, _P, _P, _P]),
    "pw_budget_step": (ctypes.c_int, [_P, ctypes.POINTER(BudgetPolicy), ctypes.c_uint64, _P, _P, _P, _P, _P, _P]),
    "pw_pool_used_bytes": (ctypes.c_uint64, [_P]),
    "pw_bind_host_tier": (ctypes.c_int, [_P, _P, ctypes.c_uint64]),
    "pw_get_residency": (ctypes.c_int, [_P, _P, _P, _P]),
    "pw_profile": (ctypes.c_int, [_P, ctypes.c_int32]),
    "pw_profile_read": (ctypes.c_int, [_P, ctypes.POINTER(ProfileData)]),
    "pw_last_error": (ctypes.c_char_p, [_P]),
    "pw_status_str": (ctypes.c_char_p, [ctypes.c_int32]),
}


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build()")
        handle = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def library_path() -> str:
    return _LIB_PATH


def _check(status: int, ctx=None):
    if status != 0:
        L = lib()
        msg = L.pw_last_error(ctx).decode() if ctx else ""
        if not msg:
            msg = L.pw_status_str(status).decode()
        raise PagedWeightError(status, msg)


def _stream(stream=None) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dev(t: torch.Tensor, dtype, name: str) -> int:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _host_array(a, dtype, n: int, name: str) -> np.ndarray:
    arr = np.ascontiguousarray(np.asarray(a, dtype=dtype))
    if arr.shape != (n,) and arr.size != n:
        raise ValueError(f"{name} must hold {n} values")
    return arr.reshape(-1)


def solve_allocation(W: Sequence[int], p: Sequence[float], L, budget_bits: int) -> np.ndarray:
    """pw_solve_allocation: exact host solver of Eq. 1 (no GPU needed)."""
    E = len(p)
    Wa = _host_array(W, np.uint64, E, "W")
    pa = _host_array(p, np.float64, E, "p")
    La = np.ascontiguousarray(np.asarray(L, dtype=np.float64).reshape(E * 3))
    out = np.zeros(E, dtype=np.uint8)
    _check(lib().pw_solve_allocation(E, Wa.ctypes.data, pa.ctypes.data, La.ctypes.data,
                                     int(budget_bits), out.ctypes.data))
    return out


def solve_allocation_layers(Ws, ps, Ls, budget_bits: int, layer_weights=None):
    """pw_solve_allocation_layers: one exact solve of Eq. 1 for several layers
    sharing budget_bits. Ws, ps, Ls hold one entry per layer (W[E_l], p[E_l],
    L[E_l][3]). Returns (list of per-layer bit arrays, objective)."""
    n = len(ps)
    if not (len(Ws) == len(Ls) == n) or n == 0:
        raise ValueError("Ws, ps and Ls need one entry per layer")
    E = np.array([len(v) for v in ps], dtype=np.int32)
    Wa = np.ascontiguousarray(np.concatenate([_host_array(W, np.uint64, int(e), "W") for W, e in zip(Ws, E)]))
    pa = np.ascontiguousarray(np.concatenate([_host_array(p, np.float64, int(e), "p") for p, e in zip(ps, E)]))
    La = np.ascontiguousarray(np.concatenate([np.asarray(L, dtype=np.float64).reshape(int(e) * 3)
                                              for L, e in zip(Ls, E)]))
    wa = None if layer_weights is None else _host_array(layer_weights, np.float64, n, "layer_weights")
    out = np.zeros(int(E.sum()), dtype=np.uint8)
    obj = ctypes.c_double(0.0)
    _check(lib().pw_solve_allocation_layers(n, E.ctypes.data, Wa.ctypes.data, pa.ctypes.data, La.ctypes.data,
                                            None if wa is None else wa.ctypes.data, int(budget_bits),
                                            out.ctypes.data, ctypes.byref(obj)))
    return np.split(out, np.cumsum(E)[:-1]), obj.value


def proportional_bits(W: Sequence[int], p: Sequence[float], budget_bits: int):
    """pw_proportional_bits: the pages' simplified proportional sketch (a
    comparison mode; may exceed the budget). Returns (bits, used_bits)."""
    E = len(p)
    Wa = _host_array(W, np.uint64, E, "W")
    pa = _host_array(p, np.float64, E, "p")
    out = np.zeros(E, dtype=np.uint8)
    used = ctypes.c_uint64(0)
    _check(lib().pw_proportional_bits(E, Wa.ctypes.data, pa.ctypes.data, int(budget_bits), out.ctypes.data,
                                      ctypes.byref(used)))
    return out, used.value


def set_budget_layers(layers, budget_bits: int, importances, layer_weights=None, stream=None):
    """One budget shared by several PagedMoELayer objects: each layer's loss
    table (pw_get_loss_table), one exact solve over all their experts
    (pw_solve_allocation_layers), then each layer quantized to its share
    (pw_quantize_experts; its pool must hold the new pages). Returns (list of
    per-layer bit arrays, objective)."""
    Ls = [layer.get_loss_table(stream) for layer in layers]
    Ws = [[3 * layer.d * layer.F] * layer.E for layer in layers]
    bits, obj = solve_allocation_layers(Ws, importances, Ls, budget_bits, layer_weights)
    for layer, b in zip(layers, bits):
        layer.quantize_experts(b, stream)
    return bits, obj


NO_POOL = (1 << 64) - 1   # pool_bytes_now before the first allocation


def _policy(memory_bytes, reserve_bytes, headroom, min_interval) -> BudgetPolicy:
    return BudgetPolicy(int(memory_bytes), int(reserve_bytes), float(headroom), int(min_interval))


def budget_decide(memory_bytes: int, reserve_bytes: int, headroom: float, min_interval: int,
                  kv_used_bytes: int, W: Sequence[int], pool_bytes_now: Optional[int],
                  budget_now: Optional[int], steps_since_change: int):
    """pw_budget_decide (host only): (action, budget_bits, pressure)."""
    E = len(W)
    Wa = _host_array(W, np.uint64, E, "W")
    pol = _policy(memory_bytes, reserve_bytes, headroom, min_interval)
    act, press = ctypes.c_int32(0), ctypes.c_int32(0)
    out = ctypes.c_uint64(0)
    _check(lib().pw_budget_decide(ctypes.byref(pol), int(kv_used_bytes), E, Wa.ctypes.data,
                                  NO_POOL if pool_bytes_now is None else int(pool_bytes_now),
                                  0 if budget_now is None else int(budget_now), int(steps_since_change),
                                  ctypes.byref(act), ctypes.byref(out), ctypes.byref(press)))
    return act.value, out.value, bool(press.value)


class PagedMoELayer:
    """One MoE expert layer bound to its masters, pool and workspace."""

    def __init__(self, num_experts: int, d_model: int, d_ff: int, top_k: int,
                 max_tokens: int, renorm: int = 0, master_dtype: str = "f32", layout: str = "eq2"):
        """layout: "eq2" (pages of Eq. 2 codes at 3/4/8 bits) or "bitplane"
        (prefix-compatible bitplane pages; bits are depths 1..8)."""
        self._ctx = None
        if layout not in ("eq2", "bitplane"):
            raise ValueError("layout must be 'eq2' or 'bitplane'")
        desc = LayerDesc(num_experts, d_model, d_ff, top_k, renorm, max_tokens,
                         PW_MASTER_F16 if master_dtype == "f16" else PW_MASTER_F32,
                         PW_LAYOUT_BITPLANE if layout == "bitplane" else PW_LAYOUT_EQ2)
        self.layout = layout
        ctx = _P()
        _check(lib().pw_create(ctypes.byref(desc), ctypes.byref(ctx)))
        self._ctx = ctx
        self.E, self.d, self.F, self.k = num_experts, d_model, d_ff, top_k
        self.max_tokens = max_tokens
        self.master_dtype = torch.float16 if master_dtype == "f16" else torch.float32
        self._keep = {}

    def __del__(self):
        if getattr(self, "_ctx", None) and _lib is not None:
            _lib.pw_destroy(self._ctx)
            self._ctx = None

    # ---- binding of caller-owned memory ----
    def bind_masters(self, w1: torch.Tensor, w3: torch.Tensor, w2: torch.Tensor):
        E, d, F = self.E, self.d, self.F
        if tuple(w1.shape) != (E, F, d) or tuple(w3.shape) != (E, F, d) or tuple(w2.shape) != (E, d, F):
            raise ValueError("masters must be w1, w3 [E, F, d] and w2 [E, d, F]")
        ptrs = [_dev(t, self.master_dtype, n) for t, n in ((w1, "w1"), (w3, "w3"), (w2, "w2"))]
        _check(lib().pw_bind_masters(self._ctx, *ptrs), self._ctx)
        self._keep["masters"] = (w1, w3, w2)

    def pool_bytes_for_bits(self, bits) -> int:
        b = _host_array(bits, np.uint8, self.E, "bits")
        return int(lib().pw_pool_bytes_for_bits(self._ctx, b.ctypes.data))

    def bind_pool(self, pool: torch.Tensor):
        _check(lib().pw_bind_pool(self._ctx, _dev(pool, torch.uint8, "pool"), pool.numel()), self._ctx)
        self._keep["pool"] = pool

    def bind_host_tier(self, host: Optional[torch.Tensor]):
        """Pages in pinned host memory, the pool a cache of page slots
        (pw_bind_host_tier); None goes back to pages in the pool."""
        if host is None:
            _check(lib().pw_bind_host_tier(self._ctx, None, 0), self._ctx)
            self._keep.pop("host", None)
            return
        if host.device.type != "cpu" or not host.is_pinned() or host.dtype != torch.uint8 or not host.is_contiguous():
            raise ValueError("host tier must be a contiguous pinned uint8 CPU tensor")
        _check(lib().pw_bind_host_tier(self._ctx, host.data_ptr(), host.numel()), self._ctx)
        self._keep["host"] = host

    def pool_used_bytes(self) -> int:
        """pw_pool_used_bytes: bytes of the pool the pages span (from its start)."""
        return int(lib().pw_pool_used_bytes(self._ctx))

    def slot_bytes(self) -> int:
        """Bytes of one page slot of the host tier's device cache (an 8-bit page)."""
        return (3 * self.d * self.F + 255) // 256 * 256

    def residency(self, stream=None):
        """pw_get_residency: (slot of each expert, -1 none; dict of hits,
        pages copied in, pages read from the host tier)."""
        slots = np.zeros(self.E, dtype=np.int32)
        stats = np.zeros(3, dtype=np.uint64)
        _check(lib().pw_get_residency(self._ctx, slots.ctypes.data, stats.ctypes.data, _stream(stream)),
               self._ctx)
        return slots, dict(hits=int(stats[0]), copies=int(stats[1]), host_reads=int(stats[2]))

    def workspace_bytes(self) -> int:
        return int(lib().pw_workspace_bytes(self._ctx))

    def bind_workspace(self, ws: torch.Tensor):
        _check(lib().pw_bind_workspace(self._ctx, _dev(ws, torch.uint8, "workspace"), ws.numel()),
               self._ctx)
        self._keep["workspace"] = ws

    # ---- the hot path ----
    def quantize_experts(self, bits, stream=None):
        b = _host_array(bits, np.uint8, self.E, "bits")
        _check(lib().pw_quantize_experts(self._ctx, b.ctypes.data, _stream(stream)), self._ctx)

    def set_budget(self, budget_bits: int, importance, loss=None, stream=None) -> np.ndarray:
        p = _host_array(importance, np.float64, self.E, "importance")
        L = None if loss is None else np.ascontiguousarray(np.asarray(loss, dtype=np.float64).reshape(self.E * 3))
        out = np.zeros(self.E, dtype=np.uint8)
        _check(lib().pw_set_budget(self._ctx, int(budget_bits), p.ctypes.data,
                                   None if L is None else L.ctypes.data, out.ctypes.data,
                                   _stream(stream)), self._ctx)
        return out

    def budget_step(self, memory_bytes: int, reserve_bytes: int, headroom: float, min_interval: int,
                    kv_used_bytes: int, importance, loss=None, stream=None):
        """pw_budget_step: one KV-pressure scheduler step (re-quantizes on
        INIT, SHRINK and GROW). Returns (action, budget_bits, pressure)."""
        p = _host_array(importance, np.float64, self.E, "importance")
        L = None if loss is None else np.ascontiguousarray(np.asarray(loss, dtype=np.float64).reshape(self.E * 3))
        pol = _policy(memory_bytes, reserve_bytes, headroom, min_interval)
        act, press = ctypes.c_int32(0), ctypes.c_int32(0)
        out = ctypes.c_uint64(0)
        _check(lib().pw_budget_step(self._ctx, ctypes.byref(pol), int(kv_used_bytes), p.ctypes.data,
                                    None if L is None else L.ctypes.data, ctypes.byref(act),
                                    ctypes.byref(out), ctypes.byref(press), _stream(stream)), self._ctx)
        return act.value, out.value, bool(press.value)

    def moe_forward(self, x: torch.Tensor, logits: torch.Tensor, y: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
        T = x.shape[0]
        if x.dim() != 2 or x.shape[1] != self.d or tuple(logits.shape) != (T, self.E):
            raise ValueError("x must be [T, d] and logits [T, E]")
        if y is None:
            y = torch.empty((T, self.d), dtype=torch.float32, device=x.device)
        elif tuple(y.shape) != (T, self.d):
            raise ValueError("y must be [T, d]")
        _check(lib().pw_moe_forward(self._ctx, _dev(x, torch.bfloat16, "x"),
                                    _dev(logits, torch.float32, "logits"), T,
                                    _dev(y, torch.float32, "y"), _stream(stream)), self._ctx)
        return y

    def moe_forward_noalloc(self, x: torch.Tensor, logits: torch.Tensor, y: torch.Tensor,
                            stream=None) -> torch.Tensor:
        """pw_moe_forward_noalloc: the forward with the library's static
        device scratch instead of the workspace (y is the caller's)."""
        T = x.shape[0]
        if x.dim() != 2 or x.shape[1] != self.d or tuple(logits.shape) != (T, self.E):
            raise ValueError("x must be [T, d] and logits [T, E]")
        if tuple(y.shape) != (T, self.d):
            raise ValueError("y must be [T, d]")
        _check(lib().pw_moe_forward_noalloc(self._ctx, _dev(x, torch.bfloat16, "x"),
                                            _dev(logits, torch.float32, "logits"), T,
                                            _dev(y, torch.float32, "y"), _stream(stream)), self._ctx)
        return y

    def route(self, logits: torch.Tensor, stream=None):
        T = logits.shape[0]
        ids = torch.empty((T, self.k), dtype=torch.int32, device=logits.device)
        g = torch.empty((T, self.k), dtype=torch.float32, device=logits.device)
        counts = torch.empty((self.E,), dtype=torch.int32, device=logits.device)
        _check(lib().pw_route(self._ctx, _dev(logits, torch.float32, "logits"), T,
                              ids.data_ptr(), g.data_ptr(), counts.data_ptr(), _stream(stream)),
               self._ctx)
        return ids, g, counts

    # ---- inspection ----
    def get_page_table(self):
        arr = (PageEntry * self.E)()
        _check(lib().pw_get_page_table(self._ctx, arr), self._ctx)
        return [dict(offset=int(e.offset), nbytes=int(e.nbytes), scale=float(e.scale),
                     bits=int(e.bits)) for e in arr]

    def get_loss_table(self, stream=None) -> np.ndarray:
        out = np.zeros(self.E * 3, dtype=np.float64)
        _check(lib().pw_get_loss_table(self._ctx, out.ctypes.data, _stream(stream)), self._ctx)
        return out.reshape(self.E, 3)

    def profile(self, mask):
        """Per-kernel timing: mask bits 0 router, 1 gate/up, 2 down, 3 combine
        (True = all, False/0 = off)."""
        m = 15 if mask is True else (0 if mask is False else int(mask))
        _check(lib().pw_profile(self._ctx, m), self._ctx)

    def profile_read(self) -> dict:
        d = ProfileData()
        _check(lib().pw_profile_read(self._ctx, ctypes.byref(d)), self._ctx)
        return dict(route_ms=d.route_ms, gate_up_ms=d.gate_up_ms, down_ms=d.down_ms,
                    combine_ms=d.combine_ms, forwards=d.forwards)

    # ---- convenience: caller-owned buffers allocated with torch ----
    def alloc_pool(self, nbytes: int, device="cuda") -> torch.Tensor:
        pool = torch.zeros(max(256, int(nbytes)), dtype=torch.uint8, device=device)
        self.bind_pool(pool)
        return pool

    def alloc_host_tier(self, nbytes: int) -> torch.Tensor:
        host = torch.zeros(max(256, int(nbytes)), dtype=torch.uint8, pin_memory=True)
        self.bind_host_tier(host)
        return host

    def alloc_workspace(self, device="cuda") -> torch.Tensor:
        ws = torch.empty(max(256, self.workspace_bytes()), dtype=torch.uint8, device=device)
        self.bind_workspace(ws)
        return ws
