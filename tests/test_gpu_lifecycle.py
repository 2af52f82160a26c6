"""The transactional lifecycle on the GPU library: device digests against their
byte definitions, verification of real device copies (an injected corruption
is caught), and the pages' state-machine promises observed through the
outputs of the kernels — an aborted change leaves the outputs bit-identical,
rollback restores them bit for bit, and an attach, clear or adapter free made
while a decode is still running on the GPU changes nothing in that decode.
("We propose a content-addressed overlay system": "Explicit Correctness and
Atomicity Invariants", "Proposed Activation/Deactivation State Machine", "TDD
and Fault-Injection Matrix"; "Deep Technical Design", section 6.)"""
import hashlib
import struct

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


def _err(fn, *a):
    import quantized_base_linear_amd as q
    with pytest.raises(q.QblError) as ei:
        fn(*a)
    return ei.value.name


def _run(b, torch, linear, x):
    q = b.q
    L = b.wl.linears[linear]
    xd = torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()
    yd = torch.empty((x.shape[0], L.n_out), dtype=torch.float32, device="cuda")
    q.qbl_linear(b.comp, linear, xd, yd, x.shape[0], q.workspace(b.comp, q.OP_LINEAR, linear, x.shape[0]))
    torch.cuda.synchronize()
    return yd.cpu().numpy()


def test_device_digests_and_injected_faults(torch_cuda):
    torch = torch_cuda
    wl = workloads.single()
    log("lifecycle: 256x256 q8_0, adapters r8@2.0 x2")
    b = Built(wl)
    q = b.q
    try:
        L = wl.linears[0]
        inner = hashlib.sha256(struct.pack("<iiqq", L.qtype, 0, L.n_out, L.k_in)
                               + b.or_blocks[0].tobytes()).digest()
        assert q.qbl_base_digest(b.base) == hashlib.sha256(inner).digest()
        assert q.qbl_base_hash(b.base) == q.qbl_base_digest(b.base)   # device bytes re-read
        for a, fac in zip(b.adapters, b.factors):
            A, B = fac[0]
            e = hashlib.sha256(struct.pack("<ii", 0, A.shape[0]) + A.tobytes() + B.tobytes()).digest()
            assert q.qbl_adapter_digest(a) == hashlib.sha256(e).digest()

        x = wl.x(0)
        b.attach([0])
        yA = _run(b, torch, 0, x)
        ref = oracle.linear_dual(L.qtype, b.or_blocks[0], L.n_out, L.k_in, x, b.oracle_ads(0, [0]))
        assert rel_l2(yA, ref) <= TOL
        held = q.qbl_base_memory(b.base)
        dA = q.qbl_comp_digest(b.comp)

        # staging verification on the real device
        A, B = b.factors[1][0]
        q.qbl_fault_inject(q.QBL_FAULT_CORRUPT, 1)
        assert _err(q.qbl_adapter_load, b.base, [(0, A, B)]) == "QBL_E_CHECKSUM"
        q.qbl_fault_inject(q.QBL_FAULT_DEVICE_ALLOC, 1)
        assert _err(q.qbl_adapter_load, b.base, [(0, A, B)]) == "QBL_E_NOMEM"
        q.qbl_base_set_budget(b.base, held[0] + 1024)
        assert _err(q.qbl_adapter_load, b.base, [(0, A, B)]) == "QBL_E_BUDGET"
        q.qbl_base_set_budget(b.base, 0)
        assert q.qbl_base_memory(b.base) == held
        assert q.qbl_comp_digest(b.comp) == dA
        assert np.array_equal(_run(b, torch, 0, x), yA)

        # a failure between staging and the swap
        q.qbl_fault_inject(q.QBL_FAULT_SWAP, 1)
        assert _err(q.qbl_comp_attach, b.comp, [b.adapters[1], b.adapters[0]], [2.0, 2.0]) == "QBL_E_INJECTED"
        assert q.qbl_comp_digest(b.comp) == dA
        assert np.array_equal(_run(b, torch, 0, x), yA)

        # rollback restores the outputs bit for bit
        y0 = None
        b.attach([1])
        yB = _run(b, torch, 0, x)
        assert not np.array_equal(yB, yA)
        q.qbl_comp_rollback(b.comp)
        assert np.array_equal(_run(b, torch, 0, x), yA)
        q.qbl_comp_rollback(b.comp)
        assert np.array_equal(_run(b, torch, 0, x), yB)
        q.qbl_comp_clear(b.comp)
        y0 = _run(b, torch, 0, x)
        ref0 = oracle.linear_dual(L.qtype, b.or_blocks[0], L.n_out, L.k_in, x)
        assert rel_l2(y0, ref0) <= TOL
        q.qbl_comp_rollback(b.comp)
        assert np.array_equal(_run(b, torch, 0, x), yB)
        assert q.qbl_base_hash(b.base) == q.qbl_base_digest(b.base)
    finally:
        for p in (q.QBL_FAULT_DEVICE_ALLOC, q.QBL_FAULT_CORRUPT, q.QBL_FAULT_SWAP):
            q.qbl_fault_inject(p, 0)
        b.close()


def test_changes_during_a_running_decode_do_not_reach_it(torch_cuda):
    """A decode captures the list at entry; an attach, a clear, and freeing the
    adapter it uses, all done while its kernels may still run, leave its output
    equal to an undisturbed run of the same list."""
    torch = torch_cuda
    wl = workloads.small_stack()
    log("lifecycle during decode: small stack d=256 h=704, 4 blocks, 48 tokens")
    b = Built(wl, check_bytes=False, keep_oracle=False)
    q = b.q
    try:
        d = wl.linears[0].k_in
        x0 = torch.from_numpy(np.ascontiguousarray(wl.x0()[0], np.float32)).cuda()
        b.attach([0, 1])
        ws = q.workspace(b.comp, q.OP_BLOCK)
        y_ref = torch.empty((wl.tokens, d), dtype=torch.float32, device="cuda")
        q.qbl_decode(b.comp, 0, wl.blocks, x0, y_ref, wl.tokens, ws)
        torch.cuda.synchronize()

        # the same decode, with the composition changed right after it is enqueued
        y = torch.empty_like(y_ref)
        q.qbl_decode(b.comp, 0, wl.blocks, x0, y, wl.tokens, ws)
        q.qbl_comp_attach(b.comp, [b.adapters[1]], [-1.0])
        q.qbl_comp_clear(b.comp)
        q.qbl_comp_drop_previous(b.comp)
        q.qbl_adapter_free(b.adapters[0])       # its memory must outlive the running decode
        b.adapters = b.adapters[1:]
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref)
        # the composition itself did change: base-only now
        y_base = torch.empty_like(y_ref)
        q.qbl_decode(b.comp, 0, wl.blocks, x0, y_base, wl.tokens, q.workspace(b.comp, q.OP_BLOCK))
        torch.cuda.synchronize()
        assert not torch.equal(y_base, y_ref)
    finally:
        b.close()


@pytest.mark.parametrize("qtype,n,k,batch", [(1, 4096, 4096, 1), (2, 512, 8192, 8), (3, 640, 4096, 5)])
def test_changes_right_after_a_linear_run_do_not_reach_it(torch_cuda, qtype, n, k, batch):
    """A linear run's last launch carries the list's completion event (at batch
    1 the fused launch; above it the GEMV or, with K split, the reduce launch:
    512 x 8192 splits K).  Attaching, clearing and freeing the adapter right
    after the run is enqueued, before any synchronisation, leaves its output
    equal to an undisturbed run."""
    torch = torch_cuda
    wl = workloads.Workload(f"inflight_{qtype}_{n}_{k}_{batch}",
                            [workloads.LinearSpec(f"inflight/{qtype}/{n}/{k}", n, k, qtype)],
                            [workloads.AdapterSpec("A1", 32, 1.0), workloads.AdapterSpec("A2", 8, -0.5)],
                            batch=batch)
    log(f"lifecycle after a linear run: qtype={qtype} n={n} k={k} batch={batch}")
    b = Built(wl, check_bytes=False, keep_oracle=False)
    q = b.q
    try:
        x = torch.from_numpy(np.ascontiguousarray(wl.x(0), np.float32)).cuda()
        b.attach([0, 1])
        ws = q.workspace(b.comp, q.OP_LINEAR, 0, batch)
        y_ref = torch.empty((batch, n), dtype=torch.float32, device="cuda")
        q.qbl_linear(b.comp, 0, x, y_ref, batch, ws)
        torch.cuda.synchronize()
        y = torch.empty_like(y_ref)
        q.qbl_linear(b.comp, 0, x, y, batch, ws)
        q.qbl_comp_attach(b.comp, [b.adapters[1]], [2.0])
        q.qbl_comp_clear(b.comp)
        q.qbl_comp_drop_previous(b.comp)
        q.qbl_adapter_free(b.adapters[0])       # its memory must outlive the run
        b.adapters = b.adapters[1:]
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref)
    finally:
        b.close()
