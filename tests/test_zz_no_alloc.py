"""qbl_linear_static, the entry point that allocates nothing (its workspace is a
per-GPU file-scope device array), against qbl_linear with a caller-owned
workspace: the same bits on two calls in a row, the second with a smaller
input, at batch 1 (the in-launch hand-off of the adapter shrink goes through
the static array) and above batch 1 (the staged matrix-core operands), and the
size limit refused before anything runs."""
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


def test_static_scratch_matches_workspace_runs(torch_cuda):
    torch = torch_cuda
    wl = workloads.Workload("noalloc", [workloads.LinearSpec("noalloc/big", 4096, 4096),
                                        workloads.LinearSpec("noalloc/small", 300, 1056, 2),
                                        workloads.LinearSpec("noalloc/tall", 66048, 256)],
                            [workloads.AdapterSpec("A1", 16, 1.0), workloads.AdapterSpec("S1", 0, 0.5, 0.05)])
    b = Built(wl)
    q = b.q
    try:
        b.attach([0, 1])
        # (linear, batch): the second call of each pair has a smaller input
        for linear, batch in ((0, 1), (1, 1), (0, 8), (1, 3)):
            L = wl.linears[linear]
            x = wl.x(linear, batch)
            xd = torch.from_numpy(x).cuda()
            y_ws = torch.empty((batch, L.n_out), dtype=torch.float32, device="cuda")
            y_st = torch.full((batch, L.n_out), float("nan"), dtype=torch.float32, device="cuda")
            q.qbl_linear(b.comp, linear, xd, y_ws, batch, q.workspace(b.comp, q.OP_LINEAR, linear, batch))
            q.qbl_linear_static(b.comp, linear, xd, y_st, batch)
            torch.cuda.synchronize()
            a, s = y_ws.cpu().numpy(), y_st.cpu().numpy()
            ref = oracle.linear_dual(L.qtype, b.or_blocks[linear], L.n_out, L.k_in, x, b.oracle_ads(linear, [0, 1]))
            log(f"linear {linear} ({L.n_out}x{L.k_in}) batch {batch}: bitwise equal {np.array_equal(a, s)}, "
                f"rel-L2 vs oracle {rel_l2(s, ref):.2e}")
            assert np.array_equal(a, s)
            assert rel_l2(s, ref) <= TOL
        # above the array's size: refused, nothing enqueued
        need = q.qbl_workspace_bytes(b.comp, q.OP_LINEAR, 2, 8)
        assert need > 32 << 20
        x = torch.zeros((8, 256), dtype=torch.float32, device="cuda")
        y = torch.zeros((8, 66048), dtype=torch.float32, device="cuda")
        with pytest.raises(q.QblError) as e:
            q.qbl_linear_static(b.comp, 2, x, y, 8)
        assert e.value.status == q.CODE["QBL_E_LIMIT"]
        torch.cuda.synchronize()
        assert float(y.abs().sum()) == 0.0
    finally:
        b.close()
