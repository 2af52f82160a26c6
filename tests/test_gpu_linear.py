"""GPU parity of the dual-path linear (qbl_linear) against the oracle, and the
pages' invariants on the GPU path itself: zero adapters == base-only bitwise,
base -> A -> base -> B == base -> B bitwise, base bytes unchanged (SHA-256),
determinism, and the closed forms that hold exactly in float32."""
import numpy as np
import pytest

import oracle
from synth import workloads
from tests.gpu_harness import Built, log, rel_l2

pytestmark = pytest.mark.gpu

TOL = 1e-3   # rel-L2 bound for float32 accumulation against the float64 oracle


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return torch


def _run(b, torch, linear, x, batch=None):
    q = b.q
    L = b.wl.linears[linear]
    batch = x.shape[0] if batch is None else batch
    xd = torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()
    yd = torch.empty((batch, L.n_out), dtype=torch.float32, device="cuda")
    ws = q.workspace(b.comp, q.OP_LINEAR, linear, batch)
    q.qbl_linear(b.comp, linear, xd, yd, batch, ws)
    torch.cuda.synchronize()
    return yd.cpu().numpy()


def test_single_linear_parity_and_invariants(torch_cuda):
    torch = torch_cuda
    wl = workloads.single()
    log("single: 256x256 q8_0, adapters r8@2.0 x2")
    b = Built(wl)
    try:
        x = wl.x(0)
        L = wl.linears[0]
        h0 = b.q.qbl_base_hash(b.base)
        y_base = _run(b, torch, 0, x)
        ref_base = oracle.linear_dual(L.qtype, b.or_blocks[0], L.n_out, L.k_in, x)
        assert rel_l2(y_base, ref_base) <= TOL
        # adapter A
        b.attach([0])
        y_a = _run(b, torch, 0, x)
        ref_a = oracle.linear_dual(L.qtype, b.or_blocks[0], L.n_out, L.k_in, x, b.oracle_ads(0, [0]))
        assert rel_l2(y_a, ref_a) <= TOL
        assert rel_l2(y_a - y_base, ref_a - ref_base) <= TOL      # the LoRA delta itself
        assert rel_l2(y_a, y_base) > 1e-2                          # the adapter really acts
        assert np.array_equal(_run(b, torch, 0, x), y_a)           # determinism
        # base -> A -> base -> B  ==  base -> B, bitwise
        b.q.qbl_comp_clear(b.comp)
        assert np.array_equal(_run(b, torch, 0, x), y_base)        # back to base, bitwise
        b.attach([1])
        y_ab = _run(b, torch, 0, x)
        b.q.qbl_comp_clear(b.comp)
        b.attach([1])
        y_b = _run(b, torch, 0, x)
        assert np.array_equal(y_ab, y_b)
        ref_b = oracle.linear_dual(L.qtype, b.or_blocks[0], L.n_out, L.k_in, x, b.oracle_ads(0, [1]))
        assert rel_l2(y_b, ref_b) <= TOL
        # all scales zero == base-only, bitwise; zero-scale entries are dropped
        b.attach([0, 1], [0.0, 0.0])
        assert b.q.qbl_comp_count(b.comp) == 0
        assert np.array_equal(_run(b, torch, 0, x), y_base)
        # both adapters, both orders
        b.attach([0, 1])
        y01 = _run(b, torch, 0, x)
        b.attach([1, 0])
        y10 = _run(b, torch, 0, x)
        ref01 = oracle.linear_dual(L.qtype, b.or_blocks[0], L.n_out, L.k_in, x, b.oracle_ads(0, [0, 1]))
        assert rel_l2(y01, ref01) <= TOL and rel_l2(y10, ref01) <= TOL
        assert rel_l2(y01, y10) <= 1e-4
        # the base bytes never changed
        assert b.q.qbl_base_hash(b.base) == h0
    finally:
        b.close()


def test_one_hot_and_block_indicator_are_exact(torch_cuda):
    torch = torch_cuda
    wl = workloads.single(n=192, k=320)
    b = Built(wl)
    try:
        L = wl.linears[0]
        deq = oracle.dequantize(L.qtype, b.or_blocks[0], L.n_out, L.k_in)
        x = np.zeros((4, L.k_in), np.float32)
        cols = [0, 17, 255, 319]
        for r, c in enumerate(cols):
            x[r, c] = 1.0
        y = _run(b, torch, 0, x)
        for r, c in enumerate(cols):
            assert np.array_equal(y[r].astype(np.float64), deq[:, c])
        xb = np.zeros((1, L.k_in), np.float32)
        xb[0, 64:96] = 1.0
        y = _run(b, torch, 0, xb)
        assert np.array_equal(y[0].astype(np.float64), deq[:, 64:96].sum(1))
    finally:
        b.close()


@pytest.mark.parametrize("qtype,n,k,batch", [
    (1, 1000, 4128, 1), (1, 333, 1056, 3), (1, 96, 12288, 1), (1, 130, 20480, 2),
    (2, 1000, 4160, 1), (2, 257, 1088, 8), (2, 64, 28672, 1), (2, 40, 9216, 5),
    (3, 1000, 4096, 1), (3, 257, 1280, 8), (3, 96, 28672, 1), (3, 130, 11008, 3), (3, 40, 9216, 5),
    (3, 33, 256, 2),
    # tall linears above batch 1: 16-row tiles spread evenly over the compute
    # units, two or three workgroups per unit, ragged last tile
    (1, 24600, 256, 8), (2, 40000, 512, 4), (3, 25000, 256, 7)])
def test_ragged_shapes_and_batches(torch_cuda, qtype, n, k, batch):
    torch = torch_cuda
    wl = workloads.Workload(f"ragged_{qtype}_{n}_{k}_{batch}",
                            [workloads.LinearSpec(f"ragged/{qtype}/{n}/{k}", n, k, qtype)],
                            [workloads.AdapterSpec("A1", 24, 0.75), workloads.AdapterSpec("A2", 8, -1.5)],
                            batch=batch)
    log(f"ragged: qtype={qtype} n={n} k={k} batch={batch}")
    b = Built(wl)
    try:
        x = wl.x(0)
        L = wl.linears[0]
        b.attach([0, 1])
        y = _run(b, torch, 0, x)
        ref = oracle.linear_dual(L.qtype, b.or_blocks[0], n, k, x, b.oracle_ads(0, [0, 1]))
        assert rel_l2(y, ref) <= TOL
        b.q.qbl_comp_clear(b.comp)
        y0 = _run(b, torch, 0, x)
        ref0 = oracle.linear_dual(L.qtype, b.or_blocks[0], n, k, x)
        assert rel_l2(y0, ref0) <= TOL
        assert rel_l2(y - y0, ref - ref0) <= TOL
        # rows of a batch are independent: other rows' values never change a
        # row's bits; a row run alone (the batch-1 kernel) agrees to rounding
        if batch > 1:
            x2 = x.copy()
            x2[1:] = -2.0 * x2[1:] + 0.5
            assert np.array_equal(_run(b, torch, 0, x2)[0], y0[0])
        for r in range(batch):
            assert rel_l2(_run(b, torch, 0, x[r:r + 1]), y0[r:r + 1]) <= 1e-5
    finally:
        b.close()


# One row length per workgroup shape of the batch-1 kernel (waves x chunks per
# lane, chosen from the row's blocks of 64 chunks: 1024 weights for q8_0, 2048
# for the q4 formats), each with a ragged last block of chunk slots.
_B1_SHAPE_KS = ([(1, k) for k in (4096, 6016, 7168, 11008, 12288, 13312, 15360, 17408, 26624, 30720, 40960)] +
                [(qt, k) for qt in (2, 3) for k in (8192, 11264, 14336, 22528, 24576, 28672, 30720, 34816)])


@pytest.mark.parametrize("qtype,k", _B1_SHAPE_KS)
def test_batch1_every_workgroup_shape(torch_cuda, qtype, k):
    torch = torch_cuda
    n = 70
    wl = workloads.Workload(f"b1shape_{qtype}_{k}", [workloads.LinearSpec(f"b1shape/{qtype}/{k}", n, k, qtype)],
                            [workloads.AdapterSpec("A1", 16, 1.0), workloads.AdapterSpec("A2", 8, -0.5)])
    log(f"batch-1 shape: qtype={qtype} n={n} k={k}")
    b = Built(wl)
    try:
        x = wl.x(0, 1)
        b.attach([0, 1])
        y = _run(b, torch, 0, x)
        ref = oracle.linear_dual(qtype, b.or_blocks[0], n, k, x, b.oracle_ads(0, [0, 1]))
        assert rel_l2(y, ref) <= TOL
        b.q.qbl_comp_clear(b.comp)
        y0 = _run(b, torch, 0, x)
        ref0 = oracle.linear_dual(qtype, b.or_blocks[0], n, k, x)
        assert rel_l2(y0, ref0) <= TOL
        assert rel_l2(y - y0, ref - ref0) <= TOL
    finally:
        b.close()


def test_batch1_mixed_ranks_tall_linear(torch_cuda):
    """Batch 1 with four adapters of ranks 16, 64, 6 and 36 on a tall linear
    (16384 rows: 13 or more rows per workgroup): ranks that are and are not
    multiples of 4 (16-byte and 4-byte B loads), small and large, in both list
    orders and alone, against the oracle."""
    torch = torch_cuda
    n, k = 16384, 1024
    wl = workloads.Workload("mixed_ranks", [workloads.LinearSpec("mixed_ranks/q8", n, k, 1)],
                            [workloads.AdapterSpec("A1", 16, 0.5), workloads.AdapterSpec("A2", 64, 1.0),
                             workloads.AdapterSpec("A3", 6, -0.75), workloads.AdapterSpec("A4", 36, 0.25)])
    log(f"mixed ranks: q8_0 {n}x{k}, ranks 16, 64, 6, 36 at batch 1")
    b = Built(wl)
    try:
        x = wl.x(0)
        y0 = _run(b, torch, 0, x)
        ref0 = oracle.linear_dual(1, b.or_blocks[0], n, k, x)
        assert rel_l2(y0, ref0) <= TOL
        for idx in ([0, 1, 2, 3], [3, 2, 1, 0], [1], [3]):
            b.attach(idx)
            y = _run(b, torch, 0, x)
            ref = oracle.linear_dual(1, b.or_blocks[0], n, k, x, b.oracle_ads(0, idx))
            assert rel_l2(y, ref) <= TOL, idx
            assert rel_l2(y - y0, ref - ref0) <= TOL, idx
    finally:
        b.close()


@pytest.mark.parametrize("qtype,n,k", [(1, 300, 1056), (2, 257, 1088), (3, 130, 2304)])
def test_batched_rows_at_extreme_scales(torch_cuda, qtype, n, k):
    """Above batch 1 each input row is scaled by its own power of two before its
    f16 split: rows of 1e-30 and 1e30 magnitude, an all-zero row, a row mixing
    1e20 and 1e-20, and an ordinary row, in one batch, each within the bound of
    the oracle; the zero row gives exact zeros."""
    torch = torch_cuda
    wl = workloads.Workload(f"extreme_{qtype}_{n}_{k}", [workloads.LinearSpec(f"extreme/{qtype}/{n}/{k}", n, k, qtype)],
                            [workloads.AdapterSpec("A1", 16, 0.75), workloads.AdapterSpec("S1", 0, 1.5, 0.05)], batch=5)
    log(f"extreme row scales: qtype={qtype} n={n} k={k}")
    b = Built(wl)
    try:
        rng = np.random.default_rng(1234 + qtype)
        g = rng.standard_normal((5, k))
        x = np.stack([g[0] * 1e-30, g[1] * 1e30, np.zeros(k), g[3],
                      np.where(np.arange(k) % 2 == 0, 1e20, 1e-20) * g[4]]).astype(np.float32)
        b.attach([0, 1])
        y = _run(b, torch, 0, x)
        ref = oracle.linear_dual(qtype, b.or_blocks[0], n, k, x.astype(np.float64), b.oracle_ads(0, [0, 1]))
        for r in (0, 1, 3, 4):
            assert np.all(np.isfinite(y[r])), r
            assert rel_l2(y[r:r + 1], ref[r:r + 1]) <= TOL, r
        assert np.array_equal(y[2], np.zeros(n, np.float32))
    finally:
        b.close()


def test_q4k_one_hot_inputs_give_dequantised_columns(torch_cuda):
    """x = e_c: every product but one is an exact zero, so each output is the
    float32 rounding of D*q - M, the dequantised weight, at batch 1 and 4."""
    torch = torch_cuda
    n, k = 200, 768
    wl = workloads.Workload("onehot_q4k", [workloads.LinearSpec("onehot/q4k", n, k, 3)],
                            [workloads.AdapterSpec("A1", 8, 1.0)])
    b = Built(wl)
    try:
        deq = oracle.dequantize(3, b.or_blocks[0], n, k).astype(np.float32)
        cols = [0, 31, 32, 255, 256, 300, 511, 767]
        for batch in (1, 4):
            for i in range(0, len(cols), batch):
                x = np.zeros((batch, k), np.float32)
                for r, c in enumerate(cols[i:i + batch]):
                    x[r, c] = 1.0
                y = _run(b, torch, 0, x)
                for r, c in enumerate(cols[i:i + batch]):
                    assert np.array_equal(y[r], deq[:, c]), (batch, c)
    finally:
        b.close()


def test_attach_rejections_leave_state_unchanged(torch_cuda):
    torch = torch_cuda
    q = __import__("quantized_base_linear_amd")
    wl = workloads.single()
    b = Built(wl)
    other = Built(workloads.single(n=64, k=64))
    try:
        x = wl.x(0)
        b.attach([0])
        y_a = _run(b, torch, 0, x)
        bad = [
            (lambda: q.qbl_comp_attach(b.comp, [b.adapters[0], b.adapters[0]], [1.0, 1.0]), -10),
            (lambda: q.qbl_comp_attach(b.comp, [b.adapters[1]], [float("nan")]), -4),
            (lambda: q.qbl_comp_attach(b.comp, [b.adapters[1]], [float("inf")]), -4),
            (lambda: q.qbl_comp_attach(b.comp, [other.adapters[0]], [1.0]), -9),
            (lambda: q.qbl_comp_attach(b.comp, [b.adapters[1]] * 9, [1.0] * 9), -11),
        ]
        for fn, status in bad:
            with pytest.raises(q.QblError) as e:
                fn()
            assert e.value.status == status
            assert np.array_equal(_run(b, torch, 0, x), y_a)     # composition untouched
        # adapter load rejections
        A = np.ones((4, 256), np.float32)
        B = np.ones((256, 4), np.float32)
        A[1, 2] = np.inf
        for entries, status in [([(0, A, B)], -4), ([(5, A, B)], -2),
                                ([(0, np.ones((4, 256), np.float32), B)] * 2, -10),
                                ([(0, np.ones((300, 256), np.float32), np.ones((256, 300), np.float32))], -11)]:
            with pytest.raises(q.QblError) as e:
                q.qbl_adapter_load(b.base, entries)
            assert e.value.status == status
        with pytest.raises(q.QblError) as e:       # the base is still referenced
            q.qbl_base_free(b.base)
        assert e.value.status == -7
        # a freed-but-attached adapter keeps working until it is detached
        q.qbl_adapter_free(b.adapters[0])
        b.adapters[0] = q.qbl_adapter_load(b.base, [(0, *b.factors[1][0])])
        assert np.array_equal(_run(b, torch, 0, x), y_a)
        # idempotent attach of the list in place
        b.attach([1])
        y1 = _run(b, torch, 0, x)
        b.attach([1])
        assert np.array_equal(_run(b, torch, 0, x), y1)
    finally:
        other.close()
        b.close()
