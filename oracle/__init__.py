"""CPU oracle for the quantised MoE FFN layer (test infrastructure only).

Only the tests, the smoke check and the CPU-baseline leg of the benchmark
load this package.  The GPU library never imports, links or calls it.

The arithmetic lives in ``moe_oracle.cpp`` (plain C++, fp64, built with
``-O2 -ffp-contract=off``); this file only builds it and marshals arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.cpp")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with g++ (no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-shared", "-fPIC", "-o", tmp, _SRC]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        L.oracle_fp16_values.argtypes = [P, i64, P]
        L.oracle_int4_values.argtypes = [P, i64, P]
        L.oracle_int8_values.argtypes = [P, i64, P]
        L.oracle_int2_values.argtypes = [P, i64, P]
        L.oracle_e2m1_values.argtypes = [P, i64, P]
        L.oracle_e4m3_values.argtypes = [P, i64, P]
        L.oracle_dequant.argtypes = [i32, P, P, ctypes.c_float, i32, i32, P]
        L.oracle_dequant.restype = i32
        L.oracle_route.argtypes = [P, ctypes.c_float, P, i32, P, P, P, P, P, P, P, P, P]
        L.oracle_route.restype = i32
        L.oracle_forward.argtypes = [P, ctypes.c_float, P, P, P, P, P, P, P, P, P, P, i32, P, i32, P, i32]
        L.oracle_forward.restype = i32
        L.oracle_max_threads.restype = i32
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def _np(t):
    """torch tensor or ndarray -> contiguous host ndarray (binary16 kept as uint16 bits)."""
    if t is None:
        return None
    try:
        import torch
        if isinstance(t, torch.Tensor):
            t = t.detach().cpu().contiguous()
            if t.dtype == torch.float16:
                return t.view(torch.int16).numpy().view(np.uint16)
            return t.numpy()
    except ImportError:
        pass
    a = np.ascontiguousarray(t)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    return a


# ---- code tables --------------------------------------------------------
def fp16_values(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.size, dtype=np.float64)
    lib().oracle_fp16_values(_ptr(bits), bits.size, _ptr(out))
    return out.reshape(bits.shape)


def int4_values(q: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint8)
    out = np.empty(2 * q.size, dtype=np.int32)
    lib().oracle_int4_values(_ptr(q), q.size, _ptr(out))
    return out


def int8_values(q: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint8)
    out = np.empty(q.size, dtype=np.int32)
    lib().oracle_int8_values(_ptr(q), q.size, _ptr(out))
    return out


def int2_values(q: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint8)
    out = np.empty(4 * q.size, dtype=np.int32)
    lib().oracle_int2_values(_ptr(q), q.size, _ptr(out))
    return out


def e2m1_values(q: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint8)
    out = np.empty(2 * q.size, dtype=np.float64)
    lib().oracle_e2m1_values(_ptr(q), q.size, _ptr(out))
    return out


def e4m3_values(s: np.ndarray) -> np.ndarray:
    s = np.ascontiguousarray(s, dtype=np.uint8)
    out = np.empty(s.size, dtype=np.float64)
    lib().oracle_e4m3_values(_ptr(s), s.size, _ptr(out))
    return out.reshape(s.shape)


def dequant(fmt: int, q, s, g: float, rows: int, cols: int) -> np.ndarray:
    q, s = _np(q), _np(s)
    out = np.empty((rows, cols), dtype=np.float64)
    rc = lib().oracle_dequant(fmt, _ptr(q), _ptr(s), float(g), rows, cols, _ptr(out))
    if rc != 0:
        raise ValueError("oracle_dequant rejected its arguments")
    return out


# ---- routing and the whole layer ------------------------------------------
class Route:
    def __init__(self, topk_idx, topk_w, z, n_unique, uniq_ids, uniq_off, pairs):
        self.topk_idx, self.topk_w, self.z = topk_idx, topk_w, z
        self.n_unique = int(n_unique)
        self.uniq_ids = uniq_ids[: self.n_unique]
        self.uniq_off = uniq_off[: self.n_unique + 1]
        self.pairs = pairs


def route(dims, x, router_w, router_b, want_z: bool = True, top_p: Optional[float] = None) -> Route:
    """Routing and union; top_p defaults to dims.top_p (0: plain top-k).  The
    threshold is the layer's binary32 parameter (rounded to binary32 here, as
    the C ABI's moe_dims_t.top_p is a float)."""
    if top_p is None:
        top_p = float(getattr(dims, "top_p", 0.0))
    d = np.asarray(dims.as_tuple() if hasattr(dims, "as_tuple") else dims, dtype=np.int32)
    H, I, E, k = int(d[0]), int(d[1]), int(d[2]), int(d[3])
    xb = _np(x)
    T = xb.shape[0] if xb.ndim == 2 else 0
    wr, rb = _np(router_w).astype(np.float32, copy=False), _np(router_b)
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    z = np.empty((T, E), dtype=np.float64) if want_z else None
    nu = np.zeros(1, dtype=np.int32)
    cap = max(1, min(E, T * k))
    ids = np.full(cap, -1, dtype=np.int32)
    off = np.full(cap + 1, -1, dtype=np.int32)
    pairs = np.full(max(1, T * k), -1, dtype=np.int32)
    rc = lib().oracle_route(_ptr(d), float(top_p), _ptr(xb), T, _ptr(wr), _ptr(rb), _ptr(idx), _ptr(w),
                            _ptr(z) if z is not None else None, _ptr(nu), _ptr(ids), _ptr(off), _ptr(pairs))
    if rc != 0:
        raise ValueError("oracle_route rejected its arguments")
    return Route(idx, w, z, nu[0], ids, off, pairs[: T * k])


def forward(layer, x, tokens: Optional[Sequence[int]] = None, threads: int = 0,
            experts_needed: Optional[Sequence[int]] = None) -> np.ndarray:
    """y (float64, [len(tokens) or T][H]) for a synth.Layer and binary16 x.

    Only the experts in ``experts_needed`` (all when None) are copied to the
    host; the shared expert is always included.
    """
    d = layer.dims
    dims = np.asarray(d.as_tuple(), dtype=np.int32)
    xb = _np(x)
    T = xb.shape[0]
    n_store = layer.q_gate.shape[0]
    want = range(n_store) if experts_needed is None else sorted(set(int(e) for e in experts_needed) |
                                                                ({d.n_experts} if d.has_shared else set()))
    keep = []
    arrs = {name: [None] * (d.n_experts + 1) for name in ("qg", "sg", "qu", "su", "qd", "sd")}
    for e in want:
        for name, attr in (("qg", "q_gate"), ("sg", "s_gate"), ("qu", "q_up"), ("su", "s_up"),
                           ("qd", "q_down"), ("sd", "s_down")):
            a = _np(getattr(layer, attr)[e])
            keep.append(a)
            arrs[name][e] = a.ctypes.data
    ptrs = {}
    for name, lst in arrs.items():
        arr = (ctypes.c_void_p * (d.n_experts + 1))(*[p if p is not None else None for p in lst])
        ptrs[name] = arr
    g3 = np.ones((d.n_experts + 1, 3), dtype=np.float32)
    g3_src = _np(layer.g3)
    g3[: g3_src.shape[0]] = g3_src
    wr = _np(layer.router_w).astype(np.float32, copy=False)
    rb = _np(layer.router_b)
    if tokens is None:
        tl = None
        n = T
    else:
        tl = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
        n = tl.size
    y = np.empty((n, d.hidden), dtype=np.float64)
    rc = lib().oracle_forward(_ptr(dims), float(getattr(d, "top_p", 0.0)), ptrs["qg"], ptrs["sg"], ptrs["qu"], ptrs["su"], ptrs["qd"], ptrs["sd"],
                              _ptr(g3), _ptr(wr), _ptr(rb), _ptr(xb), T, _ptr(tl) if tl is not None else None,
                              n, _ptr(y), int(threads))
    if rc == -2:
        raise ValueError("oracle_forward: a selected expert was not supplied")
    if rc != 0:
        raise ValueError("oracle_forward rejected its arguments")
    del keep
    return y


def max_threads() -> int:
    return int(lib().oracle_max_threads())
