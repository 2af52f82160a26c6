"""The synthetic workloads: shapes, value distributions and per-tensor streams.

Every tensor is drawn from its own stream, named ``"<workload>/<slot>/<tensor>"``.
Distributions (all normal, ``std`` a standard deviation):

* base weights W (out x in): N(0, 0.02)
* LoRA A (r x in): std 1/sqrt(d_in)   (the variance reading of N(0, 1/d_in))
* LoRA B (out x r): N(0, 0.01)
* activations x: N(0, 1)

Workloads (sizes as the pages' LLaMA-7B / 70B-style examples):

* ``single``   one 256x256 q8_0 linear, two rank-8 adapters at scale 2.0, batch 1
* ``block``    one 7B-style block: q,k,v,o 4096x4096, gate/up 11008x4096,
               down 4096x11008, q8_0, one rank-16 adapter per projection at 1.0
* ``stack``    32 such blocks, two adapters per projection in order:
               rank 16 at 1.0, then rank 64 at 0.5; 256 decoded tokens
* ``mlp70b``   gate/up 28672x8192, down 8192x28672, q4_sm, rank 32 at 1.0,
               batch 1 and 8, a fresh x per linear
* ``prefill``  M=512 tokens, K=4096 -> N=14336, q8_0, rank 64 at 1.0, X bf16
* scaled-down variants of each (``small_*``) for the oracle parity cases.

No arithmetic of the method lives here: quantisation, dequantisation and the
linear itself are done separately by the oracle and by the library.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import normal, uniform

BLOCK_LINEARS = ("q", "k", "v", "o", "gate", "up", "down")

Q8_0 = 1
Q4_SM = 2
Q4_K = 3
# canonical bytes and weights of one block, per quantisation type
BLOCK = {Q8_0: (34, 32), Q4_SM: (20, 32), Q4_K: (144, 256)}


@dataclass(frozen=True)
class AdapterSpec:
    name: str          # stream name of this adapter ("A1", "A2", ...)
    rank: int          # 0 for a sparse (DARE) delta
    scale: float
    density: float = 0.0   # sparse deltas: fraction of entries kept


@dataclass(frozen=True)
class LinearSpec:
    tag: str           # stream prefix of this linear
    n_out: int
    k_in: int
    qtype: int = Q8_0


@dataclass
class Workload:
    name: str
    linears: list            # list[LinearSpec], in library linear order
    adapters: list           # list[AdapterSpec] applied (in order) to every linear
    batch: int = 1
    blocks: int = 0          # > 0 when the linears form blocks of 7 (q,k,v,o,gate,up,down)
    tokens: int = 0          # decoded tokens for a stack
    m_tokens: int = 0        # prefill rows
    extra: dict = field(default_factory=dict)

    # -- tensors -------------------------------------------------------------
    def weight(self, i: int) -> np.ndarray:
        L = self.linears[i]
        return normal(L.tag + "/W", (L.n_out, L.k_in), 0.0, 0.02)

    def weight_rows(self, i: int, r0: int, r1: int) -> np.ndarray:
        """Rows [r0, r1) of weight i alone (same values as ``weight(i)[r0:r1]``)."""
        L = self.linears[i]
        return normal(L.tag + "/W", (r1 - r0, L.k_in), 0.0, 0.02, offset=r0 * L.k_in)

    def lora_a(self, i: int, a: int) -> np.ndarray:
        L, ad = self.linears[i], self.adapters[a]
        return normal(L.tag + "/" + ad.name + "/A", (ad.rank, L.k_in), 0.0, 1.0 / np.sqrt(L.k_in))

    def lora_b(self, i: int, a: int) -> np.ndarray:
        L, ad = self.linears[i], self.adapters[a]
        return normal(L.tag + "/" + ad.name + "/B", (L.n_out, ad.rank), 0.0, 0.01)

    def sparse_csr(self, i: int, a: int):
        """A DARE-style sparse delta for linear i: a dense N(0, 0.001) delta, each
        entry kept with probability `density` and rescaled by 1/density, stored as
        CSR (row_ptr uint32 [n+1], col uint32 [nnz], val fp16 bits uint16 [nnz])."""
        L, ad = self.linears[i], self.adapters[a]
        tag = L.tag + "/" + ad.name
        keep = uniform(tag + "/keep", (L.n_out, L.k_in)) < ad.density
        vals = normal(tag + "/delta", (L.n_out, L.k_in), 0.0, 0.001)
        rows, cols = np.nonzero(keep)
        val16 = (vals[rows, cols] / np.float32(ad.density)).astype(np.float16).view(np.uint16)
        row_ptr = np.zeros(L.n_out + 1, np.uint32)
        np.cumsum(np.bincount(rows, minlength=L.n_out), out=row_ptr[1:])
        return row_ptr, cols.astype(np.uint32), val16

    def x(self, i: int = 0, batch: int | None = None) -> np.ndarray:
        """Activations for linear i (fresh per linear), batch x k_in."""
        L = self.linears[i]
        b = self.batch if batch is None else batch
        return normal(self.name + "/" + L.tag + "/x", (b, L.k_in), 0.0, 1.0)

    def x0(self) -> np.ndarray:
        """Input of the first block (block and stack workloads)."""
        return normal(self.name + "/x0", (1, self.linears[0].k_in), 0.0, 1.0)

    def x_prefill_f32(self) -> np.ndarray:
        """Prefill activations before the bf16 cast (the caller casts)."""
        return normal(self.name + "/X", (self.m_tokens, self.linears[0].k_in), 0.0, 1.0)

    # -- accounting (algorithmic bytes) ---------------------------------------
    def base_bytes(self, i: int) -> int:
        L = self.linears[i]
        nbytes, nweights = BLOCK[L.qtype]
        return L.n_out * (L.k_in // nweights) * nbytes

    def lora_bytes(self, i: int) -> int:
        """Bytes of the low-rank adapters of linear i (sparse deltas: sparse_bytes)."""
        L = self.linears[i]
        return sum(4 * ad.rank * (L.n_out + L.k_in) for ad in self.adapters)

    def sparse_bytes(self, i: int, nnz: int) -> int:
        """Bytes of a sparse delta of linear i with nnz entries: row_ptr, 4-byte
        indices and 2-byte values."""
        return 4 * (self.linears[i].n_out + 1) + 6 * nnz


def _block_linears(prefix: str, d: int, h: int, qtype: int = Q8_0) -> list:
    shapes = {"q": (d, d), "k": (d, d), "v": (d, d), "o": (d, d),
              "gate": (h, d), "up": (h, d), "down": (d, h)}
    return [LinearSpec(f"{prefix}/{nm}", *shapes[nm], qtype) for nm in BLOCK_LINEARS]


def single(n: int = 256, k: int = 256) -> Workload:
    return Workload("single", [LinearSpec("single/L0", n, k)],
                    [AdapterSpec("A1", 8, 2.0), AdapterSpec("A2", 8, 2.0)])


def block(d: int = 4096, h: int = 11008, name: str = "block", rank: int = 16) -> Workload:
    return Workload(name, _block_linears(name + "/b0", d, h), [AdapterSpec("A1", rank, 1.0)],
                    blocks=1, tokens=1)


def block_sparse(d: int = 4096, h: int = 11008, name: str = "block_sparse", rank: int = 16,
                 density: float = 0.1) -> Workload:
    """The 7B block with a rank-16 LoRA and, after it in the list, a DARE-style
    sparse delta keeping `density` of each linear's entries, both at scale 1.0."""
    return Workload(name, _block_linears(name + "/b0", d, h),
                    [AdapterSpec("A1", rank, 1.0), AdapterSpec("S1", 0, 1.0, density)], blocks=1, tokens=1)


def stack(d: int = 4096, h: int = 11008, n_blocks: int = 32, tokens: int = 256,
          name: str = "stack", ranks=(16, 64), scales=(1.0, 0.5)) -> Workload:
    lin = []
    for b in range(n_blocks):
        lin += _block_linears(f"{name}/b{b}", d, h)
    ads = [AdapterSpec(f"A{j + 1}", r, s) for j, (r, s) in enumerate(zip(ranks, scales))]
    return Workload(name, lin, ads, blocks=n_blocks, tokens=tokens)


def mlp70b(d: int = 8192, h: int = 28672, batch: int = 1, name: str = "mlp70b",
           rank: int = 32, qtype: int = Q4_SM) -> Workload:
    lin = [LinearSpec(f"{name}/gate", h, d, qtype), LinearSpec(f"{name}/up", h, d, qtype),
           LinearSpec(f"{name}/down", d, h, qtype)]
    return Workload(name, lin, [AdapterSpec("A1", rank, 1.0)], batch=batch)


def prefill(m: int = 512, k: int = 4096, n: int = 14336, name: str = "prefill",
            rank: int = 64) -> Workload:
    return Workload(name, [LinearSpec(f"{name}/L0", n, k)], [AdapterSpec("A1", rank, 1.0)],
                    m_tokens=m)


# Scaled-down variants that the oracle finishes in seconds but that still span
# several kernel tiles and a ragged tail.
def small_block() -> Workload:
    return block(d=544, h=1440, name="small_block")


def small_block_sparse() -> Workload:
    return block_sparse(d=544, h=1440, name="small_block_sparse")


def small_stack() -> Workload:
    return stack(d=256, h=704, n_blocks=4, tokens=48, name="small_stack")


def small_mlp(batch: int = 1) -> Workload:
    return mlp70b(d=640, h=1696, batch=batch, name=f"small_mlp_b{batch}")


# The 70B-style MLP with a q4_K base (k a multiple of the 256-weight super-block).
def mlp70b_q4k(batch: int = 1) -> Workload:
    return mlp70b(batch=batch, name="mlp70b_q4k", qtype=Q4_K)


def small_prefill() -> Workload:
    return prefill(m=96, k=608, n=1184, name="small_prefill")
