"""GPU parity of the JIT-materialisation prefill path (qbl_linear_jit) against
the oracle's bf16 recipe, its bound against the dual path, and exact cases."""
import numpy as np
import pytest

import oracle
from synth import workloads
from tests.gpu_harness import Built, log, rel_l2

pytestmark = pytest.mark.gpu
TOL = 1e-3
BF16_BOUND = 2.0 ** -8


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available()
    return torch


def _bf16_bits(torch, x32):
    return torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def _jit(b, torch, linear, xbits):
    q = b.q
    L = b.wl.linears[linear]
    m = xbits.shape[0]
    xd = torch.from_numpy(xbits.view(np.int16)).cuda()
    yd = torch.empty((m, L.n_out), dtype=torch.float32, device="cuda")
    ws = q.workspace(b.comp, q.OP_JIT, linear, m)
    q.qbl_linear_jit(b.comp, linear, xd, yd, m, ws)
    torch.cuda.synchronize()
    return yd.cpu().numpy()


# m a multiple of 256 (K of 64) takes the role-split kernel (here also at 512
# and 1024 rows, ragged n, total ranks 8..64, every format), others the
# general one; q8_0 with K a multiple of 256 takes its scales 8 blocks at a
# time (K of 256, 768 and 1280: one group, groups in whole four-step rounds);
# ranks that are all multiples of 8 stage s B eight values per thread, others
# (6 + 36) one
@pytest.mark.parametrize("shape", [(96, 608, 1184, 1, (64,)), (300, 96, 200, 1, (16, 64)),
                                   (257, 1056, 130, 2, (32,)), (40, 640, 384, 1, (8, 8, 8)),
                                   (96, 512, 1184, 3, (64,)), (257, 1280, 130, 3, (16, 32)),
                                   (33, 256, 200, 3, (8,)), (256, 640, 200, 1, (48,)),
                                   (512, 640, 200, 1, (64,)), (1024, 256, 96, 2, (16, 32)),
                                   (512, 512, 130, 3, (8,)), (512, 192, 70, 2, (8, 8, 8)),
                                   (256, 256, 200, 1, (16,)), (512, 768, 96, 1, (8, 8, 8)),
                                   (256, 1280, 130, 1, (64, 8)), (256, 512, 200, 1, (6, 36))])
def test_jit_parity(torch_cuda, shape):
    torch = torch_cuda
    m, k, n, qtype, ranks = shape
    wl = workloads.Workload(f"jit_{m}_{k}_{n}_{qtype}", [workloads.LinearSpec(f"jit/{m}/{k}/{n}/{qtype}", n, k, qtype)],
                            [workloads.AdapterSpec(f"A{i + 1}", r, [1.0, 0.5, -2.0][i % 3]) for i, r in enumerate(ranks)],
                            m_tokens=m)
    log(f"jit m={m} k={k} n={n} qtype={qtype} ranks={ranks}")
    b = Built(wl)
    try:
        xb = _bf16_bits(torch, wl.x_prefill_f32())
        L = wl.linears[0]
        idx = list(range(len(ranks)))
        b.attach(idx)
        y = _jit(b, torch, 0, xb)
        ads = b.oracle_ads(0, idx)
        ref = oracle.linear_jit(L.qtype, b.or_blocks[0], n, k, xb, ads)
        r_recipe = rel_l2(y, ref)
        xd = oracle.f32_from_bf16(xb).astype(np.float64)
        dual = oracle.linear_dual(L.qtype, b.or_blocks[0], n, k, xd, ads)
        r_dual = rel_l2(y, dual)
        log(f"  rel-L2 vs recipe {r_recipe:.2e}, vs dual path {r_dual:.2e}")
        assert r_recipe <= TOL
        assert r_dual <= BF16_BOUND
        assert np.array_equal(_jit(b, torch, 0, xb), y)            # deterministic
        # without adapters the recipe is bf16(dequant) exactly
        b.q.qbl_comp_clear(b.comp)
        y0 = _jit(b, torch, 0, xb)
        assert rel_l2(y0, oracle.linear_jit(L.qtype, b.or_blocks[0], n, k, xb)) <= TOL
    finally:
        b.close()


@pytest.mark.parametrize("qtype", [1, 2, 3])
def test_jit_one_hot_rows_give_bf16_dequant_columns(torch_cuda, qtype):
    torch = torch_cuda
    wl = workloads.Workload(f"jit_onehot_{qtype}", [workloads.LinearSpec(f"jit/onehot/{qtype}", 160, 256, qtype)], [],
                            m_tokens=4)
    b = Built(wl)
    try:
        L = wl.linears[0]
        X = np.zeros((4, 256), np.float32)
        cols = [0, 37, 128, 255]
        for r, c in enumerate(cols):
            X[r, c] = 1.0
        y = _jit(b, torch, 0, _bf16_bits(torch, X))
        weff = oracle.f32_from_bf16(oracle.jit_weff(L.qtype, b.or_blocks[0], 160, 256))
        for r, c in enumerate(cols):
            assert np.array_equal(y[r], weff[:, c])
    finally:
        b.close()
