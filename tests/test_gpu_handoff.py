"""Batch-1 launches hand values over between their workgroups (the adapter
shrink, sparse row sums).  These tests check what happens when that cannot
work: a wait that gives up is reported as QBL_E_DEVICE (forced from the host by
a test-only fault point: readers wait for a launch number nobody writes, with a
zero time budget, so every kernel still ends normally), and batch-1 runs with
adapters refuse a stream that is capturing a HIP graph.  Also batch-1 inputs of
extreme magnitude through the fused batch-1 kernel ("Explicit Correctness and
Atomicity Invariants": deterministic, hard errors instead of silent wrong
results)."""
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


def _linear(b, torch, x, ws):
    L = b.wl.linears[0]
    xd = torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()
    yd = torch.empty((1, L.n_out), dtype=torch.float32, device="cuda")
    b.q.qbl_linear(b.comp, 0, xd, yd, 1, ws)
    torch.cuda.synchronize()
    return yd.cpu().numpy()


def test_failed_handoff_is_reported(torch_cuda):
    torch = torch_cuda
    wl = workloads.Workload("handoff", [workloads.LinearSpec("handoff/L0", 512, 1024)],
                            [workloads.AdapterSpec("A1", 16, 1.0)])
    b = Built(wl)
    q = b.q
    try:
        b.attach([0])
        L = wl.linears[0]
        x = wl.x(0)
        ws = q.workspace(b.comp, q.OP_LINEAR, 0, 1)
        q.qbl_device_status()                       # nothing recorded
        y_ok = _linear(b, torch, x, ws)
        ref = oracle.linear_dual(L.qtype, b.or_blocks[0], L.n_out, L.k_in, x, b.oracle_ads(0, [0]))
        assert rel_l2(y_ok, ref) <= TOL
        log("arming the hand-off fault point")
        q.qbl_fault_inject(q.QBL_FAULT_HANDOFF, 1)
        _linear(b, torch, x, ws)                    # enqueues fine; its waits give up on the device
        with pytest.raises(q.QblError) as e:        # the next run call refuses
            _linear(b, torch, x, ws)
        assert e.value.status == q.CODE["QBL_E_DEVICE"]
        with pytest.raises(q.QblError) as e:        # the status call reports it once ...
            q.qbl_device_status()
        assert e.value.status == q.CODE["QBL_E_DEVICE"]
        q.qbl_device_status()                       # ... and clears it
        y = _linear(b, torch, x, ws)                # runs work again, with the same bits
        assert np.array_equal(y, y_ok)
    finally:
        q.qbl_fault_inject(q.QBL_FAULT_HANDOFF, 0)
        b.close()


def test_batch1_runs_with_adapters_refuse_graph_capture(torch_cuda):
    torch = torch_cuda
    wl = workloads.small_block()
    b = Built(wl, check_bytes=False, keep_oracle=False)
    q = b.q
    try:
        b.attach([0])
        L = wl.linears[0]
        ws_lin = q.workspace(b.comp, q.OP_LINEAR, 0, 1)
        ws_blk = q.workspace(b.comp, q.OP_BLOCK)
        x = torch.from_numpy(wl.x(0)).cuda()
        y = torch.zeros((1, L.n_out), dtype=torch.float32, device="cuda")
        y_blk = torch.zeros(L.k_in, dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        refused = []
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for call in (lambda: q.qbl_linear(b.comp, 0, x, y, 1, ws_lin),
                         lambda: q.qbl_block(b.comp, 0, x[0], y_blk, ws_blk),
                         lambda: q.qbl_decode(b.comp, 0, 1, x[0], y_blk, 1, ws_blk)):
                try:
                    call()
                except q.QblError as e:
                    refused.append(e.status)
        log(f"refusals under capture: {refused}")
        assert refused == [q.CODE["QBL_E_STATE"]] * 3
        assert float(y.abs().sum()) == 0.0 and float(y_blk.abs().sum()) == 0.0   # nothing ran
        q.qbl_linear(b.comp, 0, x, y, 1, ws_lin)   # outside a capture it runs
        torch.cuda.synchronize()
        assert float(y.abs().sum()) > 0.0
    finally:
        b.close()


@pytest.mark.parametrize("qtype,n,k", [(1, 300, 1056), (2, 257, 1088), (3, 130, 2304),
                                       (1, 4096, 11008)])
def test_batch1_extreme_inputs(torch_cuda, qtype, n, k):
    """One input row per call (the fused batch-1 kernel): magnitudes 1e-30 and
    1e30, an all-zero row (exact zeros out), 1e20 and 1e-20 interleaved, and a
    large common offset (1000 + N(0,1): the q8_0 product subtracts 128 times
    the chunk's input sum, the case where that cancels most), with a low-rank
    adapter and a sparse delta after it."""
    torch = torch_cuda
    wl = workloads.Workload(f"b1extreme_{qtype}_{n}_{k}",
                            [workloads.LinearSpec(f"b1extreme/{qtype}/{n}/{k}", n, k, qtype)],
                            [workloads.AdapterSpec("A1", 16, 0.75), workloads.AdapterSpec("S1", 0, 1.5, 0.05)])
    log(f"batch-1 extreme inputs: qtype={qtype} n={n} k={k}")
    b = Built(wl)
    q = b.q
    try:
        b.attach([0, 1])
        ws = q.workspace(b.comp, q.OP_LINEAR, 0, 1)
        rng = np.random.default_rng(4321 + qtype)
        g = rng.standard_normal((5, k))
        rows = {"1e-30": g[0] * 1e-30, "1e30": g[1] * 1e30, "zero": np.zeros(k),
                "1e20/1e-20": np.where(np.arange(k) % 2 == 0, 1e20, 1e-20) * g[3],
                "offset 1000": 1000.0 + g[4]}
        for name, xr in rows.items():
            x = xr.astype(np.float32)[None, :]
            y = _linear(b, torch, x, ws)
            if name == "zero":
                assert np.array_equal(y, np.zeros((1, n), np.float32))
                continue
            ref = oracle.linear_dual(qtype, b.or_blocks[0], n, k, x.astype(np.float64), b.oracle_ads(0, [0, 1]))
            r = rel_l2(y, ref)
            log(f"  {name}: rel-L2 {r:.2e}")
            assert np.all(np.isfinite(y)) and r <= TOL, name
    finally:
        b.close()
