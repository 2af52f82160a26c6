"""Pins of the oracle's sparse overlay ("We propose a content-addressed overlay
system", "Runtime Strategy Comparison Matrix", sparse overlay: add stored
values only at their indices, base untouched; "Deep Technical Design",
"Sparse Overlay Bytes": CSR with 4-byte indices and 2-byte f16 values, for
DARE-masked task vectors).

Checked against scipy's CSR product (an independent sparse route), the
closed form of a single entry, the materialised path, and torch for the JIT
recipe's added values.
"""
import numpy as np
import pytest
import scipy.sparse as sp
import torch

import oracle
from oracle import Lora, Sparse
from synth import workloads as W

Q8, Q4, Q4K = oracle.Q8_0, oracle.Q4_SM, oracle.Q4_K


def _base(rng, qtype, n, k):
    return oracle.quantize(qtype, (rng.standard_normal((n, k)) * 0.02).astype(np.float32))


def _dare(n, k, density, tag):
    wl = W.Workload(tag, [W.LinearSpec(tag + "/L", n, k)], [W.AdapterSpec("S", 0, 1.0, density)])
    return wl.sparse_csr(0, 0)


def _scipy(row_ptr, col, val16, n, k):
    v = np.frombuffer(np.ascontiguousarray(val16).tobytes(), np.float16).astype(np.float64)
    return sp.csr_matrix((v, col.astype(np.int64), row_ptr.astype(np.int64)), shape=(n, k))


@pytest.mark.parametrize("qtype,n,k,batch,density", [(Q8, 96, 320, 1, 0.1), (Q4, 64, 256, 3, 0.3),
                                                     (Q4K, 40, 512, 2, 0.02), (Q8, 33, 64, 8, 1.0)])
def test_dual_path_matches_scipy(qtype, n, k, batch, density):
    rng = np.random.default_rng(80 + n)
    blocks = _base(rng, qtype, n, k)
    csr = _dare(n, k, density, f"sp{n}_{k}")
    S = _scipy(*csr, n, k)
    lora = Lora((rng.standard_normal((4, k)) / np.sqrt(k)).astype(np.float32),
                (rng.standard_normal((n, 4)) * 0.01).astype(np.float32), -0.5)
    x = rng.standard_normal((batch, k))
    y = oracle.linear_dual(qtype, blocks, n, k, x, [lora, Sparse(*csr, 1.5)])
    deq = oracle.dequantize(qtype, blocks, n, k)
    ref = x @ deq.T + (-0.5) * (x @ lora.A.astype(np.float64).T) @ lora.B.astype(np.float64).T \
        + 1.5 * (S @ x.T).T
    assert np.max(np.abs(y - ref)) <= 1e-12 * max(1.0, np.abs(ref).max())
    # and the sparse term is really there
    y0 = oracle.linear_dual(qtype, blocks, n, k, x, [lora])
    assert np.abs(y - y0).max() > 1e-3 * np.abs(y0).max()


def test_single_entry_changes_one_output_by_s_v_x():
    rng = np.random.default_rng(81)
    n, k = 48, 128
    blocks = _base(rng, Q8, n, k)
    x = rng.standard_normal((2, k))
    i, j, v = 17, 101, np.float16(0.3125)
    row_ptr = np.zeros(n + 1, np.uint32)
    row_ptr[i + 1:] = 1
    sparse = Sparse(row_ptr, np.array([j], np.uint32), np.array([v]).view(np.uint16), 2.0)
    y0 = oracle.linear_dual(Q8, blocks, n, k, x)
    y1 = oracle.linear_dual(Q8, blocks, n, k, x, [sparse])
    others = np.arange(n) != i
    assert np.array_equal(y1[:, others], y0[:, others])
    assert np.array_equal(y1[:, i], y0[:, i] + 2.0 * (float(v) * x[:, j]))


def test_empty_delta_and_zero_scale_leave_the_base():
    rng = np.random.default_rng(82)
    n, k = 32, 96
    blocks = _base(rng, Q8, n, k)
    x = rng.standard_normal((1, k))
    y0 = oracle.linear_dual(Q8, blocks, n, k, x)
    empty = Sparse(np.zeros(n + 1, np.uint32), np.zeros(0, np.uint32), np.zeros(0, np.uint16), 1.0)
    assert np.array_equal(oracle.linear_dual(Q8, blocks, n, k, x, [empty]), y0)
    csr = _dare(n, k, 0.2, "zs")
    assert np.array_equal(oracle.linear_dual(Q8, blocks, n, k, x, [Sparse(*csr, 0.0)]), y0)


def test_materialised_equals_dual():
    rng = np.random.default_rng(83)
    n, k = 70, 256
    blocks = _base(rng, Q4K, n, k)
    ads = [Sparse(*_dare(n, k, 0.15, "m1"), 0.75), Sparse(*_dare(n, k, 0.05, "m2"), -1.25)]
    x = rng.standard_normal((3, k))
    yd = oracle.linear_dual(Q4K, blocks, n, k, x, ads)
    ym = oracle.linear_materialised(Q4K, blocks, n, k, x, ads)
    assert np.max(np.abs(yd - ym)) <= 1e-12 * np.abs(yd).max()


def test_jit_adds_float32_scaled_values_before_the_one_rounding():
    rng = np.random.default_rng(84)
    n, k = 64, 128
    blocks = _base(rng, Q8, n, k)
    csr = _dare(n, k, 0.25, "jit")
    weff = oracle.jit_weff(Q8, blocks, n, k, [Sparse(*csr, 0.5)])
    deq32 = oracle.dequantize(Q8, blocks, n, k).astype(np.float32)
    S = _scipy(*csr, n, k).toarray()
    add = (np.float32(0.5) * S.astype(np.float32)).astype(np.float64)   # fp16 * 0.5: exact in fp32
    ref = torch.from_numpy(deq32.astype(np.float64) + add).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(weff, ref.view(np.uint16))


def test_malformed_csr_is_rejected():
    rng = np.random.default_rng(85)
    n, k = 16, 64
    blocks = _base(rng, Q8, n, k)
    x = rng.standard_normal((1, k))
    rp = np.arange(n + 1, dtype=np.uint32)
    for bad_rp, bad_col in ((rp, np.full(n, k, np.uint32)),                 # column out of range
                            (rp[::-1].copy(), np.zeros(n, np.uint32))):     # decreasing row_ptr
        s = Sparse.__new__(Sparse)
        s.row_ptr, s.col, s.val, s.scale = bad_rp, bad_col, np.zeros(n, np.uint16), 1.0
        with pytest.raises(ValueError):
            oracle.linear_dual(Q8, blocks, n, k, x, [s])
