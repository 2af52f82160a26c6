"""CPU oracle for the dual-path quantized-base + LoRA linear (ctypes wrapper).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The GPU library
never imports it and shares no code with it; the two meet only through the
seeded inputs of the ``synth`` package.

The arithmetic lives in ``oracle.c`` (plain C, float64, sequential sums,
row-parallel threads); this module only marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None

Q8_0 = 1
Q4_SM = 2
Q4_K = 3

_i64p = ctypes.POINTER(ctypes.c_int64)


class _Lora(ctypes.Structure):
    _fields_ = [("rank", ctypes.c_int32), ("scale", ctypes.c_float),
                ("A", ctypes.c_void_p), ("B", ctypes.c_void_p),
                ("row_ptr", ctypes.c_void_p), ("col", ctypes.c_void_p), ("val", ctypes.c_void_p)]


class _Linear(ctypes.Structure):
    _fields_ = [("qtype", ctypes.c_int32), ("n", ctypes.c_int64), ("k", ctypes.c_int64),
                ("blocks", ctypes.c_void_p), ("ads", ctypes.c_void_p), ("n_ads", ctypes.c_int32)]


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (no FMA contraction)."""
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared", "-Wall",
             "-Wextra", os.path.join(_HERE, "oracle.c"), "-o", tmp, "-lm", "-lpthread"])
        os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build(force=False)
        L = ctypes.CDLL(_SO)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        sig = {
            "or_f16_from_f32": (ctypes.c_uint16, [ctypes.c_float]),
            "or_f32_from_f16": (ctypes.c_float, [ctypes.c_uint16]),
            "or_bf16_from_f32": (ctypes.c_uint16, [ctypes.c_float]),
            "or_bf16_from_f64": (ctypes.c_uint16, [ctypes.c_double]),
            "or_f32_from_bf16": (ctypes.c_float, [ctypes.c_uint16]),
            "or_block_bytes": (i32, [i32]),
            "or_block_weights": (i32, [i32]),
            "or_quantize": (i32, [i32, vp, i64, i64, vp]),
            "or_dequantize": (i32, [i32, vp, i64, i64, vp]),
            "or_linear_dual": (i32, [i32, vp, i64, i64, vp, i32, vp, i32, vp, i64, vp, i32]),
            "or_linear_materialised": (i32, [i32, vp, i64, i64, vp, i32, vp, i32, vp, i64, vp, i32]),
            "or_jit_weff": (i32, [i32, vp, i64, i64, vp, i32, vp, i64, vp, i32]),
            "or_requantize": (i32, [i32, vp, i64, i64, vp, i32, vp, i32]),
            "or_gemm_bf16": (i32, [vp, i64, vp, i64, i64, vp, i32]),
            "or_rms": (None, [vp, i64, ctypes.c_double, vp]),
            "or_block": (i32, [vp, vp, vp, i32]),
            "or_stack": (i32, [vp, i32, vp, i32, vp, i32]),
            "or_f16_from_f32_n": (None, [vp, vp, i64]),
            "or_f32_from_f16_n": (None, [vp, vp, i64]),
            "or_bf16_from_f32_n": (None, [vp, vp, i64]),
            "or_bf16_from_f64_n": (None, [vp, vp, i64]),
            "or_default_threads": (i32, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def default_threads() -> int:
    return int(_load().or_default_threads())


# -- formats -------------------------------------------------------------------
def f16_from_f32(a) -> np.ndarray:
    a = _c(a, np.float32)
    out = np.empty(a.shape, np.uint16)
    _load().or_f16_from_f32_n(a.ctypes.data, out.ctypes.data, a.size)
    return out


def f32_from_f16(a) -> np.ndarray:
    a = _c(a, np.uint16)
    out = np.empty(a.shape, np.float32)
    _load().or_f32_from_f16_n(a.ctypes.data, out.ctypes.data, a.size)
    return out


def bf16_from_f32(a) -> np.ndarray:
    a = _c(a, np.float32)
    out = np.empty(a.shape, np.uint16)
    _load().or_bf16_from_f32_n(a.ctypes.data, out.ctypes.data, a.size)
    return out


def bf16_from_f64(a) -> np.ndarray:
    a = _c(a, np.float64)
    out = np.empty(a.shape, np.uint16)
    _load().or_bf16_from_f64_n(a.ctypes.data, out.ctypes.data, a.size)
    return out


def f32_from_bf16(a) -> np.ndarray:
    a = _c(a, np.uint16)
    return (a.astype(np.uint32) << 16).view(np.float32)


def block_bytes(qtype: int) -> int:
    return int(_load().or_block_bytes(qtype))


def block_weights(qtype: int) -> int:
    return int(_load().or_block_weights(qtype))


def quantize(qtype: int, w) -> np.ndarray:
    """Canonical block bytes (uint8, n x (k/block_weights*block_bytes)) of a float32 matrix."""
    w = _c(w, np.float32)
    n, k = w.shape
    bw = block_weights(qtype)
    if bw == 0:
        raise ValueError(f"unknown quantisation type {qtype}")
    out = np.empty((n, k // bw * block_bytes(qtype)), np.uint8)
    if _load().or_quantize(qtype, w.ctypes.data, n, k, out.ctypes.data) != 0:
        raise ValueError("or_quantize rejected its arguments")
    return out


def dequantize(qtype: int, blocks, n: int, k: int) -> np.ndarray:
    blocks = _c(blocks, np.uint8)
    out = np.empty((n, k), np.float64)
    if _load().or_dequantize(qtype, blocks.ctypes.data, n, k, out.ctypes.data) != 0:
        raise ValueError("or_dequantize rejected its arguments")
    return out


# -- linears -------------------------------------------------------------------
class Lora:
    """One adapter on one linear: A (rank x k), B (n x rank), effective scale."""

    def __init__(self, A, B, scale: float):
        self.A = _c(A, np.float32)
        self.B = _c(B, np.float32)
        self.scale = float(scale)
        assert self.A.shape[0] == self.B.shape[1]

    @property
    def rank(self) -> int:
        return self.A.shape[0]


class Sparse:
    """One sparse delta on one linear, CSR: row_ptr (n+1), col, fp16 value bits, scale."""

    def __init__(self, row_ptr, col, val_f16_bits, scale: float):
        self.row_ptr = _c(row_ptr, np.uint32)
        self.col = _c(col, np.uint32)
        self.val = _c(val_f16_bits, np.uint16)
        self.scale = float(scale)
        assert self.col.size == self.val.size == int(self.row_ptr[-1])
        # non-empty buffers, so that their pointers are never NULL
        self._keep = [np.zeros(1, np.uint32), np.zeros(1, np.uint16)]

    rank = 0


def _lora_array(ads):
    arr = (_Lora * max(1, len(ads)))()
    for i, a in enumerate(ads):
        arr[i].rank, arr[i].scale = a.rank, a.scale
        if a.rank == 0:
            arr[i].row_ptr = a.row_ptr.ctypes.data
            arr[i].col = (a.col if a.col.size else a._keep[0]).ctypes.data
            arr[i].val = (a.val if a.val.size else a._keep[1]).ctypes.data
        else:
            arr[i].A, arr[i].B = a.A.ctypes.data, a.B.ctypes.data
    return arr


def _rows(rows, n):
    if rows is None:
        return None, n
    r = _c(rows, np.int64)
    return r, r.size


def linear_dual(qtype, blocks, n, k, x, ads=(), rows=None, nthreads=0) -> np.ndarray:
    """float64 dual path; x is (batch, k) float; returns (batch, len(rows) or n)."""
    blocks = _c(blocks, np.uint8)
    x = _c(np.atleast_2d(x), np.float64)
    r, nr = _rows(rows, n)
    y = np.empty((x.shape[0], nr), np.float64)
    la = _lora_array(ads)
    rc = _load().or_linear_dual(qtype, blocks.ctypes.data, n, k, x.ctypes.data, x.shape[0],
                                ctypes.addressof(la), len(ads),
                                None if r is None else r.ctypes.data, nr, y.ctypes.data, nthreads)
    if rc != 0:
        raise ValueError("or_linear_dual rejected its arguments")
    return y


def linear_materialised(qtype, blocks, n, k, x, ads=(), rows=None, nthreads=0) -> np.ndarray:
    blocks = _c(blocks, np.uint8)
    x = _c(np.atleast_2d(x), np.float64)
    r, nr = _rows(rows, n)
    y = np.empty((x.shape[0], nr), np.float64)
    la = _lora_array(ads)
    rc = _load().or_linear_materialised(qtype, blocks.ctypes.data, n, k, x.ctypes.data,
                                        x.shape[0], ctypes.addressof(la), len(ads),
                                        None if r is None else r.ctypes.data, nr,
                                        y.ctypes.data, nthreads)
    if rc != 0:
        raise ValueError("or_linear_materialised rejected its arguments")
    return y


def jit_weff(qtype, blocks, n, k, ads=(), rows=None, nthreads=0) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of the JIT-materialised rows."""
    blocks = _c(blocks, np.uint8)
    r, nr = _rows(rows, n)
    out = np.empty((nr, k), np.uint16)
    la = _lora_array(ads)
    rc = _load().or_jit_weff(qtype, blocks.ctypes.data, n, k, ctypes.addressof(la), len(ads),
                             None if r is None else r.ctypes.data, nr, out.ctypes.data, nthreads)
    if rc != 0:
        raise ValueError("or_jit_weff rejected its arguments")
    return out


def requantize(qtype, blocks, n, k, ads=(), nthreads=0) -> np.ndarray:
    """Canonical blocks of Q(deq(W) + sum of the adapters' deltas), the merged
    weight formed by the float32 recipe of or_requantize."""
    blocks = _c(blocks, np.uint8)
    out = np.empty((n, k // block_weights(qtype) * block_bytes(qtype)), np.uint8)
    la = _lora_array(ads)
    if _load().or_requantize(qtype, blocks.ctypes.data, n, k, ctypes.addressof(la), len(ads),
                             out.ctypes.data, nthreads):
        raise ValueError("or_requantize rejected its arguments")
    return out


def gemm_bf16(X_bits, weff_bits, nthreads=0) -> np.ndarray:
    X = _c(X_bits, np.uint16)
    W = _c(weff_bits, np.uint16)
    m, k = X.shape
    nr = W.shape[0]
    assert W.shape[1] == k
    y = np.empty((m, nr), np.float64)
    if _load().or_gemm_bf16(X.ctypes.data, m, W.ctypes.data, nr, k, y.ctypes.data, nthreads):
        raise ValueError("or_gemm_bf16 rejected its arguments")
    return y


def linear_jit(qtype, blocks, n, k, X_bits, ads=(), rows=None, nthreads=0) -> np.ndarray:
    """Prefill through the JIT recipe: (m, len(rows) or n) float64."""
    return gemm_bf16(X_bits, jit_weff(qtype, blocks, n, k, ads, rows, nthreads), nthreads)


def rms(v, eps: float = 1e-6) -> np.ndarray:
    v = _c(v, np.float64)
    out = np.empty_like(v)
    _load().or_rms(v.ctypes.data, v.size, eps, out.ctypes.data)
    return out


class Layer:
    """One linear of a block: quantised blocks plus its adapter list."""

    def __init__(self, qtype, blocks, n, k, ads=()):
        self.qtype, self.n, self.k = qtype, int(n), int(k)
        self.blocks = _c(blocks, np.uint8)
        self.ads = list(ads)


def _layer_array(layers):
    keep = []
    arr = (_Linear * len(layers))()
    for i, L in enumerate(layers):
        la = _lora_array(L.ads)
        keep.append(la)
        arr[i].qtype, arr[i].n, arr[i].k = L.qtype, L.n, L.k
        arr[i].blocks = L.blocks.ctypes.data
        arr[i].ads = ctypes.addressof(la)
        arr[i].n_ads = len(L.ads)
    return arr, keep


def block(layers, h, nthreads=0) -> np.ndarray:
    arr, keep = _layer_array(layers)
    h = _c(h, np.float64).ravel()
    out = np.empty(layers[0].k, np.float64)
    if _load().or_block(ctypes.addressof(arr), h.ctypes.data, out.ctypes.data, nthreads):
        raise ValueError("or_block rejected its arguments")
    del keep
    return out


def stack(layers, x0, n_tokens, nthreads=0) -> np.ndarray:
    assert len(layers) % 7 == 0
    arr, keep = _layer_array(layers)
    x0 = _c(x0, np.float64).ravel()
    y = np.empty((n_tokens, layers[0].k), np.float64)
    if _load().or_stack(ctypes.addressof(arr), len(layers) // 7, x0.ctypes.data, n_tokens,
                        y.ctypes.data, nthreads):
        raise ValueError("or_stack rejected its arguments")
    del keep
    return y
