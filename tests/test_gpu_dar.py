"""GPU requantise kernel (qbl_requantize, the dequantize-add-requantize merge
used only to measure drift) against the oracle's merge: the canonical bytes are
integer output, so they must be equal bit for bit, for every base type, with
low-rank and sparse terms in one list, at reduced and at full 7B size; the
base itself stays unchanged."""
import numpy as np
import pytest

import oracle
from synth import workloads
from tests.gpu_harness import Built, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return torch


def _requant(b, torch, linear):
    q = b.q
    L = b.wl.linears[linear]
    nbytes = L.n_out * (L.k_in // q.qbl_block_weights(L.qtype)) * q.qbl_block_bytes(L.qtype)
    out = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    q.qbl_requantize(b.comp, linear, out)
    torch.cuda.synchronize()
    return out.cpu().numpy().reshape(L.n_out, -1)


@pytest.mark.parametrize("qtype,n,k", [(1, 300, 1056), (2, 257, 1088), (3, 130, 2304), (1, 64, 11008)])
def test_requantised_bytes_equal_the_oracle(torch_cuda, qtype, n, k):
    torch = torch_cuda
    name = f"dar_{qtype}_{n}_{k}"
    wl = workloads.Workload(name, [workloads.LinearSpec(f"{name}/L", n, k, qtype)],
                            [workloads.AdapterSpec("A1", 8, 0.75), workloads.AdapterSpec("S1", 0, -1.5, 0.1),
                             workloads.AdapterSpec("A2", 4, 1.0)])
    log(f"requantise: qtype={qtype} n={n} k={k}")
    b = Built(wl)
    q = b.q
    try:
        h0 = q.qbl_base_hash(b.base)
        for idx in ([], [0], [1], [0, 1, 2], [2, 1, 0]):
            b.attach(idx)
            got = _requant(b, torch, 0)
            ref = oracle.requantize(qtype, b.or_blocks[0], n, k, b.oracle_ads(0, idx))
            diff = np.nonzero((got != ref).any(1))[0]
            assert diff.size == 0, (idx, diff[:8])
        assert q.qbl_base_hash(b.base) == h0
        small = torch.zeros(16, dtype=torch.uint8, device="cuda")
        with pytest.raises(q.QblError) as e:
            q.qbl_requantize(b.comp, 0, small)
        assert e.value.name == "QBL_E_BUDGET"
    finally:
        b.close()


def test_requantised_bytes_equal_the_oracle_full_size(torch_cuda):
    torch = torch_cuda
    wl = workloads.stack(n_blocks=1, tokens=1, name="dar_full")
    log("requantise full size: 7B gate 11008x4096 and o 4096x4096, r16@1.0 then r64@0.5")
    b = Built(wl)
    try:
        b.attach([0, 1])
        for i in (3, 4):
            L = wl.linears[i]
            got = _requant(b, torch, i)
            ref = oracle.requantize(L.qtype, b.or_blocks[i], L.n_out, L.k_in, b.oracle_ads(i, [0, 1]))
            assert np.array_equal(got, ref), i
    finally:
        b.close()
