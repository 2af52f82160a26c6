"""Shared set-up for the GPU parity tests: builds library objects and the
matching oracle objects from one synthetic workload.  The library quantises
with its own quantiser, the oracle with its own; the bytes are checked equal."""
from __future__ import annotations

import sys

import numpy as np

import oracle


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


class Built:
    """A workload on both sides: library base/adapters and oracle layers."""

    def __init__(self, wl, check_bytes: bool = True, keep_oracle: bool = True):
        import quantized_base_linear_amd as q
        self.q, self.wl = q, wl
        self.lib_blocks, self.or_blocks = [], []
        descs = []
        for i, L in enumerate(wl.linears):
            w = wl.weight(i)
            lb = q.qbl_quantize(L.qtype, w)
            if check_bytes:
                ob = oracle.quantize(L.qtype, w)
                assert np.array_equal(lb, ob), f"quantiser bytes differ on linear {i}"
            descs.append((L.qtype, L.n_out, L.k_in, lb))
            if keep_oracle:
                self.or_blocks.append(lb if not check_bytes else ob)
            del w
        self.base = q.qbl_base_load(descs)
        del descs
        self.factors = []   # [adapter][linear] -> (A, B), or (row_ptr, col, val) for a sparse delta
        self.adapters = []
        for a, spec in enumerate(wl.adapters):
            if spec.rank == 0:
                fac = [wl.sparse_csr(i, a) for i in range(len(wl.linears))]
                handle = q.qbl_adapter_load_sparse(self.base, [(i, *f) for i, f in enumerate(fac)])
            else:
                fac = [(wl.lora_a(i, a), wl.lora_b(i, a)) for i in range(len(wl.linears))]
                handle = q.qbl_adapter_load(self.base, [(i, A, B) for i, (A, B) in enumerate(fac)])
            self.factors.append(fac if keep_oracle else None)
            self.adapters.append(handle)
        self.comp = q.qbl_comp_create(self.base)

    def attach(self, idx, scales=None):
        scales = [self.wl.adapters[i].scale for i in idx] if scales is None else scales
        self.q.qbl_comp_attach(self.comp, [self.adapters[i] for i in idx], scales)

    def oracle_ads(self, i, idx, scales=None):
        scales = [self.wl.adapters[a].scale for a in idx] if scales is None else scales
        return [(oracle.Sparse if self.wl.adapters[a].rank == 0 else oracle.Lora)(*self.factors[a][i], s)
                for a, s in zip(idx, scales)]

    def oracle_layers(self, idx, scales=None):
        return [oracle.Layer(L.qtype, self.or_blocks[i], L.n_out, L.k_in,
                             self.oracle_ads(i, idx, scales))
                for i, L in enumerate(self.wl.linears)]

    def close(self):
        q = self.q
        q.qbl_comp_free(self.comp)
        for a in self.adapters:
            q.qbl_adapter_free(a)
        q.qbl_base_free(self.base)
