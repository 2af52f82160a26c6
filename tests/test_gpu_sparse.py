"""GPU parity of sparse (DARE/CSR) deltas on the decode path against the oracle:
ragged linears of every base type at batch 1..8 with a low-rank adapter and a
sparse delta in one list, the sparse term on its own (delta parity), a single
entry (its row changes by exactly s * v * x_j at batch 1, every other row keeps
its bits), an empty delta, a block through qbl_block at reduced and at full
7B size, and the prefill path's refusal."""
import numpy as np
import pytest

import oracle
from synth import workloads
from tests.gpu_harness import Built, log, rel_l2

pytestmark = pytest.mark.gpu
TOL = 1e-3


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return torch


def _run(b, torch, linear, x):
    q = b.q
    L = b.wl.linears[linear]
    xd = torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()
    yd = torch.empty((x.shape[0], L.n_out), dtype=torch.float32, device="cuda")
    q.qbl_linear(b.comp, linear, xd, yd, x.shape[0], q.workspace(b.comp, q.OP_LINEAR, linear, x.shape[0]))
    torch.cuda.synchronize()
    return yd.cpu().numpy()


def _wl(name, qtype, n, k, batch, density):
    return workloads.Workload(name, [workloads.LinearSpec(f"{name}/L", n, k, qtype)],
                              [workloads.AdapterSpec("A1", 8, 0.75),
                               workloads.AdapterSpec("S1", 0, 1.5, density)], batch=batch)


@pytest.mark.parametrize("qtype,n,k,batch,density", [
    (1, 1000, 4128, 1, 0.1), (1, 96, 12288, 1, 0.02), (1, 64, 2048, 2, 1.0), (2, 257, 1088, 8, 0.3),
    (2, 333, 4160, 1, 0.1), (3, 130, 11008, 3, 0.05), (3, 500, 4096, 1, 0.1)])
def test_sparse_delta_parity(torch_cuda, qtype, n, k, batch, density):
    torch = torch_cuda
    wl = _wl(f"sp_{qtype}_{n}_{k}_{batch}", qtype, n, k, batch, density)
    log(f"sparse: qtype={qtype} n={n} k={k} batch={batch} density={density}")
    b = Built(wl)
    try:
        L = wl.linears[0]
        x = wl.x(0)
        b.attach([0, 1])
        y = _run(b, torch, 0, x)
        ref = oracle.linear_dual(L.qtype, b.or_blocks[0], n, k, x, b.oracle_ads(0, [0, 1]))
        b.attach([0])
        y_l = _run(b, torch, 0, x)
        ref_l = oracle.linear_dual(L.qtype, b.or_blocks[0], n, k, x, b.oracle_ads(0, [0]))
        r, rd = rel_l2(y, ref), rel_l2(y - y_l, ref - ref_l)
        log(f"  rel-L2 {r:.2e}, sparse-delta rel-L2 {rd:.2e}")
        assert r <= TOL and rd <= TOL
        # the sparse delta alone, first in the list, and the same call twice
        b.attach([1, 0], [1.5, 0.75])
        y2 = _run(b, torch, 0, x)
        assert rel_l2(y2, ref) <= TOL
        assert np.array_equal(_run(b, torch, 0, x), y2)
    finally:
        b.close()


def test_single_entry_and_empty_delta(torch_cuda):
    torch = torch_cuda
    n, k = 300, 1024
    wl = workloads.Workload("sp_one", [workloads.LinearSpec("sp_one/L", n, k, 1)],
                            [workloads.AdapterSpec("A1", 8, 1.0)])
    b = Built(wl)
    q = b.q
    try:
        x = wl.x(0)
        y0 = _run(b, torch, 0, x)
        i, j, v, s = 211, 777, np.float16(-0.4375), 2.0
        rp = np.zeros(n + 1, np.uint32)
        rp[i + 1:] = 1
        one = q.qbl_adapter_load_sparse(b.base, [(0, rp, np.array([j], np.uint32), np.array([v]).view(np.uint16))])
        empty = q.qbl_adapter_load_sparse(b.base, [(0, np.zeros(n + 1, np.uint32), np.zeros(0, np.uint32),
                                                    np.zeros(0, np.uint16))])
        b.adapters += [one, empty]
        q.qbl_comp_attach(b.comp, [one], [s])
        y1 = _run(b, torch, 0, x)
        others = np.arange(n) != i
        assert np.array_equal(y1[:, others], y0[:, others])
        expect = np.float32(y0[0, i]) + np.float32(s) * (np.float32(v) * np.float32(x[0, j]))
        assert y1[0, i] == expect
        q.qbl_comp_attach(b.comp, [empty], [1.0])
        assert np.array_equal(_run(b, torch, 0, x), y0)
        # the prefill path refuses a list with a sparse delta
        xb = torch.zeros((4, k), dtype=torch.bfloat16, device="cuda")
        yb = torch.empty((4, n), dtype=torch.float32, device="cuda")
        with pytest.raises(q.QblError) as e:
            q.qbl_linear_jit(b.comp, 0, xb, yb, 4, q.workspace(b.comp, q.OP_JIT, 0, 4))
        assert e.value.name == "QBL_E_FORMAT"
    finally:
        b.close()


def _block(b, torch, x):
    q = b.q
    d = b.wl.linears[0].k_in
    xd = torch.from_numpy(np.ascontiguousarray(x, np.float32).reshape(-1)).cuda()
    yd = torch.empty(d, dtype=torch.float32, device="cuda")
    q.qbl_block(b.comp, 0, xd, yd, q.workspace(b.comp, q.OP_BLOCK))
    torch.cuda.synchronize()
    return yd.cpu().numpy()


@pytest.mark.parametrize("full", [False, True])
def test_block_with_sparse_delta(torch_cuda, full):
    torch = torch_cuda
    wl = workloads.block_sparse() if full else workloads.small_block_sparse()
    log(f"{wl.name}: r16@1.0 then a 10%-dense sparse delta @1.0 on all 7 linears")
    b = Built(wl)
    try:
        x = wl.x0()[0]
        b.attach([0, 1])
        y = _block(b, torch, x)
        ref = oracle.block(b.oracle_layers([0, 1]), x.astype(np.float64))
        b.attach([0])
        y_l = _block(b, torch, x)
        ref_l = oracle.block(b.oracle_layers([0]), x.astype(np.float64))
        r = rel_l2(y, ref)
        log(f"  block rel-L2 {r:.2e} (without the sparse delta {rel_l2(y_l, ref_l):.2e}; "
            f"the delta moves the output by {rel_l2(ref, ref_l):.2e})")
        assert r <= TOL and rel_l2(y_l, ref_l) <= TOL
        assert rel_l2(ref, ref_l) > 10 * TOL          # the sparse delta matters
    finally:
        b.close()


def test_block_with_two_sparse_deltas_around_a_lora():
    """Two sparse deltas and a low-rank adapter in one list (S1, A1, S2): every
    launch group of the block hands over two sparse values per row, added at
    their list positions; parity with the oracle, and the list order matters."""
    import torch
    assert torch.cuda.is_available()
    d, h = 544, 1440
    wl = workloads.Workload("block_two_sparse", workloads._block_linears("block_two_sparse/b0", d, h),
                            [workloads.AdapterSpec("A1", 16, 0.5), workloads.AdapterSpec("S1", 0, 1.0, 0.1),
                             workloads.AdapterSpec("S2", 0, -0.75, 0.3)], blocks=1, tokens=1)
    log("small block with S1, A1, S2")
    b = Built(wl)
    try:
        x = wl.x0()[0]
        b.attach([1, 0, 2])
        y = _block(b, torch, x)
        ref = oracle.block(b.oracle_layers([1, 0, 2]), x.astype(np.float64))
        assert rel_l2(y, ref) <= TOL
        b.attach([0])
        ref_l = oracle.block(b.oracle_layers([0]), x.astype(np.float64))
        assert rel_l2(ref, ref_l) > 10 * TOL                    # the sparse deltas matter
        b.attach([2, 0, 1])
        y2 = _block(b, torch, x)
        assert rel_l2(y2, oracle.block(b.oracle_layers([2, 0, 1]), x.astype(np.float64))) <= TOL
        # one linear at batch 1 (the fused launch) and at batch 3 (the matrix-core path)
        b.attach([1, 0, 2])
        L = wl.linears[4]
        for batch in (1, 3):
            xs = wl.x(4, batch)
            q = b.q
            xd = torch.from_numpy(np.ascontiguousarray(xs, np.float32)).cuda()
            yd = torch.empty((batch, L.n_out), dtype=torch.float32, device="cuda")
            q.qbl_linear(b.comp, 4, xd, yd, batch, q.workspace(b.comp, q.OP_LINEAR, 4, batch))
            torch.cuda.synchronize()
            refl = oracle.linear_dual(L.qtype, b.or_blocks[4], L.n_out, L.k_in, xs, b.oracle_ads(4, [1, 0, 2]))
            assert rel_l2(yd.cpu().numpy(), refl) <= TOL, batch
    finally:
        b.close()



@pytest.mark.parametrize("qtype,n,k,rank", [(1, 1000, 4128, 48), (2, 333, 4160, 80), (1, 4096, 11008, 64)])
def test_sparse_delta_beside_a_high_rank_adapter(torch_cuda, qtype, n, k, rank):
    """At batch 1 a list whose largest rank is above 32 finishes each row in a
    group of lanes (the B row split over them, a fixed xor tree adding the
    parts); the row's first sparse value, fetched before the barrier, reaches
    the group through LDS.  Both orders of the list, against the oracle, and
    the same call twice bitwise."""
    torch = torch_cuda
    wl = workloads.Workload(f"sp_hr_{qtype}_{n}_{k}_{rank}", [workloads.LinearSpec(f"sp_hr/{qtype}/{n}/{k}", n, k, qtype)],
                            [workloads.AdapterSpec("A1", rank, 0.75), workloads.AdapterSpec("S1", 0, 1.5, 0.1)])
    log(f"sparse beside rank {rank}: qtype={qtype} n={n} k={k}")
    b = Built(wl)
    try:
        L = wl.linears[0]
        x = wl.x(0)
        for order, scales in (([0, 1], [0.75, 1.5]), ([1, 0], [1.5, 0.75])):
            b.attach(order, scales)
            y = _run(b, torch, 0, x)
            ref = oracle.linear_dual(L.qtype, b.or_blocks[0], n, k, x, b.oracle_ads(0, order, scales))
            assert rel_l2(y, ref) <= TOL, order
            assert np.array_equal(_run(b, torch, 0, x), y)
    finally:
        b.close()
