"""Python binding of libqbl (include/qbl.h): the dual-path quantized-base + LoRA
linear on MI355X.

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  Functions carry the C names; device buffers are torch CUDA tensors
(their data pointers are passed), host buffers are numpy arrays, and the
stream defaults to torch's current stream on the current device.  There is no
CPU fallback: importing this module fails if the library is not built.

The module-level functions call the library built next to this file.  The
`Library` class binds the same functions to another build of the same C ABI
(a path to a shared object), one instance per loaded build.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libqbl.so")

if not os.path.exists(_SO):
    raise ImportError(f"{_SO} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()' "
                      "or python quantized_base_linear_amd/build.py)")

# torch first: the process then holds exactly one HIP runtime (torch's), which
# this library binds to when it is loaded.
import torch  # noqa: E402,F401

QBL_OK = 0
QBL_Q8_0 = 1
QBL_Q4_SM = 2
QBL_Q4_K = 3
QBL_MAX_ADAPTERS = 8
QBL_MAX_RANK = 256
QBL_MAX_TOTAL_RANK = 512
QBL_MAX_BATCH = 8
OP_LINEAR, OP_JIT, OP_BLOCK = 0, 1, 2
QBL_FAULT_DEVICE_ALLOC, QBL_FAULT_CORRUPT, QBL_FAULT_SWAP, QBL_FAULT_HANDOFF = 1, 2, 3, 4

STATUS = {0: "QBL_OK", -1: "QBL_E_ARG", -2: "QBL_E_SHAPE", -3: "QBL_E_FORMAT",
          -4: "QBL_E_NONFINITE", -5: "QBL_E_NOMEM", -6: "QBL_E_BUDGET", -7: "QBL_E_BUSY",
          -8: "QBL_E_DEVICE", -9: "QBL_E_FOREIGN", -10: "QBL_E_DUPLICATE", -11: "QBL_E_LIMIT",
          -12: "QBL_E_CHECKSUM", -13: "QBL_E_INJECTED", -14: "QBL_E_STATE"}
CODE = {name: code for code, name in STATUS.items()}


class QblError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status
        self.name = STATUS.get(status, str(status))
        self.msg = msg


class qbl_linear_desc(ctypes.Structure):
    _fields_ = [("qtype", ctypes.c_int32), ("reserved", ctypes.c_int32), ("n_out", ctypes.c_int64),
                ("k_in", ctypes.c_int64), ("blocks", ctypes.c_void_p), ("nbytes", ctypes.c_int64)]


class qbl_lora_desc(ctypes.Structure):
    _fields_ = [("linear", ctypes.c_int32), ("rank", ctypes.c_int32), ("A", ctypes.c_void_p),
                ("B", ctypes.c_void_p)]


class qbl_sparse_desc(ctypes.Structure):
    _fields_ = [("linear", ctypes.c_int32), ("reserved", ctypes.c_int32), ("nnz", ctypes.c_int64),
                ("row_ptr", ctypes.c_void_p), ("col", ctypes.c_void_p), ("val", ctypes.c_void_p)]


_vp, _i32, _i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
_PP = ctypes.POINTER(ctypes.c_void_p)
EXPORTS = {
    "qbl_last_error": (ctypes.c_char_p, []),
    "qbl_abi_version": (_i32, []),
    "qbl_block_bytes": (_i64, [_i32]),
    "qbl_block_weights": (_i64, [_i32]),
    "qbl_quantize": (_i32, [_i32, _vp, _i64, _i64, _vp, _i32]),
    "qbl_dequantize": (_i32, [_i32, _vp, _i64, _i64, _vp]),
    "qbl_sha256": (_i32, [_vp, _i64, _vp]),
    "qbl_base_load": (_i32, [_vp, _i32, _PP]),
    "qbl_base_digest": (_i32, [_vp, _vp]),
    "qbl_base_hash": (_i32, [_vp, _vp]),
    "qbl_base_count": (_i32, [_vp, _vp]),
    "qbl_base_info": (_i32, [_vp, _i32, _vp, _vp, _vp]),
    "qbl_base_free": (_i32, [_vp]),
    "qbl_base_set_budget": (_i32, [_vp, _i64]),
    "qbl_base_memory": (_i32, [_vp, _vp, _vp]),
    "qbl_adapter_load": (_i32, [_vp, _vp, _i32, _PP]),
    "qbl_adapter_load_sparse": (_i32, [_vp, _vp, _i32, _PP]),
    "qbl_adapter_digest": (_i32, [_vp, _vp]),
    "qbl_adapter_free": (_i32, [_vp]),
    "qbl_comp_create": (_i32, [_vp, _PP]),
    "qbl_comp_attach": (_i32, [_vp, _vp, _vp, _i32]),
    "qbl_comp_clear": (_i32, [_vp]),
    "qbl_comp_rollback": (_i32, [_vp]),
    "qbl_comp_drop_previous": (_i32, [_vp]),
    "qbl_comp_count": (_i32, [_vp, _vp]),
    "qbl_comp_digest": (_i32, [_vp, _vp]),
    "qbl_identity_digest": (_i32, [_vp, _vp, _vp, _i32, _vp]),
    "qbl_comp_free": (_i32, [_vp]),
    "qbl_fault_inject": (_i32, [_i32, _i32]),
    "qbl_device_status": (_i32, []),
    "qbl_workspace_bytes": (_i32, [_vp, _i32, _i32, _i32, _vp]),
    "qbl_linear": (_i32, [_vp, _i32, _vp, _vp, _i32, _vp, _i64, _vp]),
    "qbl_linear_static": (_i32, [_vp, _i32, _vp, _vp, _i32, _vp]),
    "qbl_linear_jit": (_i32, [_vp, _i32, _vp, _vp, _i32, _vp, _i64, _vp]),
    "qbl_block": (_i32, [_vp, _i32, _vp, _vp, _vp, _i64, _vp]),
    "qbl_decode": (_i32, [_vp, _i32, _i32, _vp, _vp, _i32, _vp, _i64, _vp]),
    "qbl_requantize": (_i32, [_vp, _i32, _vp, _i64, _vp]),
    "qbl_hbm_probe": (_i32, [_vp, _i64, _vp, _i32, _vp, _vp]),
    "qbl_profile_enable": (_i32, [_i32]),
    "qbl_profile_read": (_i32, [_i32, _vp, _vp]),
}


def _host(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _dev_ptr(t, dtype=None):
    """Data pointer of a contiguous CUDA tensor (None passes NULL)."""
    if t is None:
        return None
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("device buffers must be contiguous CUDA tensors")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"expected {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _ws(ws):
    if ws is None:
        return None, 0
    return _dev_ptr(ws), ws.numel() * ws.element_size()


def _digest_out():
    return (ctypes.c_uint8 * 32)()


class Library:
    """The functions of include/qbl.h, bound to one loaded build of the library."""

    def __init__(self, path: str):
        self.path = path
        self._lib = ctypes.CDLL(path)
        for name, (res, args) in EXPORTS.items():
            fn = getattr(self._lib, name)
            fn.restype = res
            fn.argtypes = args

    def _check(self, status: int):
        if status != QBL_OK:
            raise QblError(status, self._lib.qbl_last_error().decode(errors="replace"))

    # -- formats -----------------------------------------------------------------
    def qbl_last_error(self) -> str:
        return self._lib.qbl_last_error().decode(errors="replace")

    def qbl_abi_version(self) -> int:
        return int(self._lib.qbl_abi_version())

    def qbl_block_bytes(self, qtype: int) -> int:
        return int(self._lib.qbl_block_bytes(qtype))

    def qbl_block_weights(self, qtype: int) -> int:
        return int(self._lib.qbl_block_weights(qtype))

    def qbl_quantize(self, qtype: int, w, nthreads: int = 0) -> np.ndarray:
        """Canonical blocks (uint8, n x k/block_weights*block_bytes) of a host float32 matrix."""
        w = _host(w, np.float32)
        n, k = w.shape
        bw = max(1, self.qbl_block_weights(qtype))
        out = np.empty((n, max(0, k // bw) * max(1, self.qbl_block_bytes(qtype))), np.uint8)
        self._check(self._lib.qbl_quantize(qtype, w.ctypes.data, n, k, out.ctypes.data, nthreads))
        return out

    def qbl_sha256(self, data: bytes) -> bytes:
        buf = np.frombuffer(bytes(data), np.uint8) if len(data) else np.zeros(1, np.uint8)
        out = _digest_out()
        self._check(self._lib.qbl_sha256(buf.ctypes.data, len(data), ctypes.addressof(out)))
        return bytes(out)

    def qbl_dequantize(self, qtype: int, blocks, n: int, k: int) -> np.ndarray:
        blocks = _host(blocks, np.uint8)
        out = np.empty((n, k), np.float32)
        self._check(self._lib.qbl_dequantize(qtype, blocks.ctypes.data, n, k, out.ctypes.data))
        return out

    # -- base --------------------------------------------------------------------
    def qbl_base_load(self, linears) -> int:
        """linears: sequence of (qtype, n_out, k_in, blocks uint8 array)."""
        keep = [_host(b, np.uint8) for (_, _, _, b) in linears]
        descs = (qbl_linear_desc * max(1, len(linears)))()
        for i, ((qt, n, k, _), b) in enumerate(zip(linears, keep)):
            descs[i].qtype, descs[i].reserved, descs[i].n_out, descs[i].k_in = qt, 0, n, k
            descs[i].blocks, descs[i].nbytes = b.ctypes.data, b.nbytes
        h = ctypes.c_void_p()
        self._check(self._lib.qbl_base_load(ctypes.addressof(descs), len(linears), ctypes.byref(h)))
        return h.value

    def qbl_base_digest(self, base) -> bytes:
        out = _digest_out()
        self._check(self._lib.qbl_base_digest(base, ctypes.addressof(out)))
        return bytes(out)

    def qbl_base_hash(self, base) -> bytes:
        out = _digest_out()
        self._check(self._lib.qbl_base_hash(base, ctypes.addressof(out)))
        return bytes(out)

    def qbl_base_count(self, base) -> int:
        n = ctypes.c_int32()
        self._check(self._lib.qbl_base_count(base, ctypes.addressof(n)))
        return n.value

    def qbl_base_info(self, base, linear: int):
        qt, n, k = ctypes.c_int32(), ctypes.c_int64(), ctypes.c_int64()
        self._check(self._lib.qbl_base_info(base, linear, ctypes.addressof(qt), ctypes.addressof(n),
                                            ctypes.addressof(k)))
        return qt.value, n.value, k.value

    def qbl_base_set_budget(self, base, budget_bytes: int) -> None:
        self._check(self._lib.qbl_base_set_budget(base, budget_bytes))

    def qbl_base_memory(self, base):
        """(bytes held, budget) of a base; budget 0 = no cap."""
        held, budget = ctypes.c_int64(), ctypes.c_int64()
        self._check(self._lib.qbl_base_memory(base, ctypes.addressof(held), ctypes.addressof(budget)))
        return held.value, budget.value

    def qbl_base_free(self, base) -> None:
        self._check(self._lib.qbl_base_free(base))

    # -- adapters ----------------------------------------------------------------
    def qbl_adapter_load(self, base, entries) -> int:
        """entries: sequence of (linear, A (rank x k_in), B (n_out x rank)) host float32."""
        keep = [(_host(A, np.float32), _host(B, np.float32)) for (_, A, B) in entries]
        descs = (qbl_lora_desc * max(1, len(entries)))()
        for i, ((lin, _, _), (A, B)) in enumerate(zip(entries, keep)):
            if A.ndim != 2 or B.ndim != 2 or A.shape[0] != B.shape[1]:
                raise ValueError("A must be rank x k_in and B n_out x rank")
            descs[i].linear, descs[i].rank = lin, A.shape[0]
            descs[i].A, descs[i].B = A.ctypes.data, B.ctypes.data
        h = ctypes.c_void_p()
        self._check(self._lib.qbl_adapter_load(base, ctypes.addressof(descs), len(entries), ctypes.byref(h)))
        return h.value

    def qbl_adapter_load_sparse(self, base, entries) -> int:
        """entries: sequence of (linear, row_ptr uint32 (n_out+1), col uint32, val fp16 bits uint16)."""
        keep = [(_host(rp, np.uint32), _host(c, np.uint32), _host(v, np.uint16)) for (_, rp, c, v) in entries]
        descs = (qbl_sparse_desc * max(1, len(entries)))()
        for i, ((lin, _, _, _), (rp, c, v)) in enumerate(zip(entries, keep)):
            if c.size != v.size:
                raise ValueError("one value per column index")
            descs[i].linear, descs[i].reserved, descs[i].nnz = lin, 0, c.size
            descs[i].row_ptr = rp.ctypes.data
            descs[i].col = c.ctypes.data if c.size else None
            descs[i].val = v.ctypes.data if v.size else None
        h = ctypes.c_void_p()
        self._check(self._lib.qbl_adapter_load_sparse(base, ctypes.addressof(descs), len(entries),
                                                      ctypes.byref(h)))
        return h.value

    def qbl_adapter_digest(self, adapter) -> bytes:
        out = _digest_out()
        self._check(self._lib.qbl_adapter_digest(adapter, ctypes.addressof(out)))
        return bytes(out)

    def qbl_adapter_free(self, adapter) -> None:
        self._check(self._lib.qbl_adapter_free(adapter))

    # -- compositions ------------------------------------------------------------
    def qbl_comp_create(self, base) -> int:
        h = ctypes.c_void_p()
        self._check(self._lib.qbl_comp_create(base, ctypes.byref(h)))
        return h.value

    def qbl_comp_attach(self, comp, adapters, scales) -> None:
        n = len(adapters)
        arr = (ctypes.c_void_p * max(1, n))(*adapters)
        sc = np.ascontiguousarray(scales, np.float32)
        if sc.size != n:
            raise ValueError("one scale per adapter")
        self._check(self._lib.qbl_comp_attach(comp, ctypes.addressof(arr), sc.ctypes.data if n else None, n))

    def qbl_comp_clear(self, comp) -> None:
        self._check(self._lib.qbl_comp_clear(comp))

    def qbl_comp_rollback(self, comp) -> None:
        self._check(self._lib.qbl_comp_rollback(comp))

    def qbl_comp_drop_previous(self, comp) -> None:
        self._check(self._lib.qbl_comp_drop_previous(comp))

    def qbl_comp_count(self, comp) -> int:
        n = ctypes.c_int32()
        self._check(self._lib.qbl_comp_count(comp, ctypes.addressof(n)))
        return n.value

    def qbl_comp_digest(self, comp) -> bytes:
        out = _digest_out()
        self._check(self._lib.qbl_comp_digest(comp, ctypes.addressof(out)))
        return bytes(out)

    def qbl_identity_digest(self, base_digest: bytes, adapter_digests, scales) -> bytes:
        n = len(adapter_digests)
        if len(base_digest) != 32 or any(len(d) != 32 for d in adapter_digests):
            raise ValueError("digests are 32 bytes")
        bd = (ctypes.c_uint8 * 32)(*base_digest)
        ad = (ctypes.c_uint8 * max(32, 32 * n))(*b"".join(adapter_digests))
        sc = np.ascontiguousarray(scales, np.float32)
        if sc.size != n:
            raise ValueError("one scale per adapter")
        out = _digest_out()
        self._check(self._lib.qbl_identity_digest(ctypes.addressof(bd), ctypes.addressof(ad),
                                                  sc.ctypes.data if n else None, n, ctypes.addressof(out)))
        return bytes(out)

    def qbl_comp_free(self, comp) -> None:
        self._check(self._lib.qbl_comp_free(comp))

    def qbl_fault_inject(self, point: int, after: int) -> None:
        self._check(self._lib.qbl_fault_inject(point, after))

    def qbl_device_status(self) -> None:
        """Raises QblError(QBL_E_DEVICE) once per recorded device-side hand-off failure."""
        self._check(self._lib.qbl_device_status())

    # -- runs --------------------------------------------------------------------
    def qbl_workspace_bytes(self, comp, op: int, index: int = 0, m: int = 1) -> int:
        out = ctypes.c_int64()
        self._check(self._lib.qbl_workspace_bytes(comp, op, index, m, ctypes.addressof(out)))
        return out.value

    def workspace(self, comp, op: int, index: int = 0, m: int = 1, device=None):
        """A zeroed device byte buffer of the size qbl_workspace_bytes reports (None if 0)."""
        nb = self.qbl_workspace_bytes(comp, op, index, m)
        if nb == 0:
            return None
        return torch.zeros(nb, dtype=torch.uint8, device=device or "cuda")

    def qbl_linear(self, comp, linear: int, x, y, batch: int, ws=None, stream=None) -> None:
        wp, wb = _ws(ws)
        self._check(self._lib.qbl_linear(comp, linear, _dev_ptr(x, torch.float32), _dev_ptr(y, torch.float32),
                                         batch, wp, wb, _stream(stream)))

    def qbl_linear_static(self, comp, linear: int, x, y, batch: int, stream=None) -> None:
        self._check(self._lib.qbl_linear_static(comp, linear, _dev_ptr(x, torch.float32),
                                                _dev_ptr(y, torch.float32), batch, _stream(stream)))

    def qbl_linear_jit(self, comp, linear: int, x_bf16, y, m: int, ws=None, stream=None) -> None:
        if x_bf16.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
            raise ValueError("x must hold bfloat16 bit patterns")
        wp, wb = _ws(ws)
        self._check(self._lib.qbl_linear_jit(comp, linear, _dev_ptr(x_bf16), _dev_ptr(y, torch.float32), m,
                                             wp, wb, _stream(stream)))

    def qbl_block(self, comp, block: int, x, y, ws=None, stream=None) -> None:
        wp, wb = _ws(ws)
        self._check(self._lib.qbl_block(comp, block, _dev_ptr(x, torch.float32), _dev_ptr(y, torch.float32),
                                        wp, wb, _stream(stream)))

    def qbl_decode(self, comp, first_block: int, n_blocks: int, x0, y_tokens, n_tokens: int, ws=None,
                   stream=None) -> None:
        wp, wb = _ws(ws)
        self._check(self._lib.qbl_decode(comp, first_block, n_blocks, _dev_ptr(x0, torch.float32),
                                         _dev_ptr(y_tokens, torch.float32), n_tokens, wp, wb, _stream(stream)))

    def qbl_requantize(self, comp, linear: int, out, stream=None) -> None:
        """Canonical blocks of the dequantize-add-requantize merge into `out` (a CUDA byte tensor)."""
        self._check(self._lib.qbl_requantize(comp, linear, _dev_ptr(out), out.numel() * out.element_size(),
                                             _stream(stream)))

    # -- timing ------------------------------------------------------------------
    def qbl_hbm_probe(self, buf, sink, stream=None) -> int:
        """Read all of the device tensor buf once (read-only streaming probe); the
        XOR of each workgroup's words goes to sink (device int32/uint32 tensor).
        Returns the number of workgroups (sink words written)."""
        if sink.dtype not in (torch.int32, torch.uint32):
            raise ValueError("sink must hold 32-bit words")
        wg = ctypes.c_int32()
        self._check(self._lib.qbl_hbm_probe(_dev_ptr(buf), buf.numel() * buf.element_size(), _dev_ptr(sink),
                                            sink.numel(), ctypes.addressof(wg), _stream(stream)))
        return wg.value

    def qbl_profile_enable(self, on: bool) -> None:
        self._check(self._lib.qbl_profile_enable(1 if on else 0))

    def qbl_profile_read(self, kind: int):
        """(launches, total_ms) of one kernel kind since timing was enabled."""
        n, ms = ctypes.c_int64(), ctypes.c_double()
        self._check(self._lib.qbl_profile_read(kind, ctypes.addressof(n), ctypes.addressof(ms)))
        return n.value, ms.value


KIND_GEMV, KIND_PREP, KIND_JIT, KIND_DAR, KIND_PROBE = 0, 1, 2, 3, 4

_default = Library(_SO)
_lib = _default._lib
for _name in dir(Library):
    if _name.startswith("qbl_") or _name == "workspace":
        globals()[_name] = getattr(_default, _name)


def library_path() -> str:
    return _SO
