"""GPU parity of qbl_block / qbl_decode (linears with linear glue) against the
oracle, at sizes the oracle finishes in seconds, plus the stack invariants:
the free-running chain stays within tolerance token by token, swapping the
adapter order changes only rounding, and the base hash never moves."""
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
    assert torch.cuda.is_available()
    return torch


def _block(b, torch, blk, x):
    q = b.q
    d = b.wl.linears[7 * blk].k_in
    xd = torch.from_numpy(np.ascontiguousarray(x, np.float32).reshape(-1)).cuda()
    yd = torch.empty(d, dtype=torch.float32, device="cuda")
    ws = q.workspace(b.comp, q.OP_BLOCK)
    q.qbl_block(b.comp, blk, xd, yd, ws)
    torch.cuda.synchronize()
    return yd.cpu().numpy()


def _decode(b, torch, x0, n_blocks, n_tokens, first=0):
    q = b.q
    d = b.wl.linears[0].k_in
    xd = torch.from_numpy(np.ascontiguousarray(x0, np.float32).reshape(-1)).cuda()
    yd = torch.empty((n_tokens, d), dtype=torch.float32, device="cuda")
    ws = q.workspace(b.comp, q.OP_BLOCK)
    q.qbl_decode(b.comp, first, n_blocks, xd, yd, n_tokens, ws)
    torch.cuda.synchronize()
    return yd.cpu().numpy()


def test_small_block_parity_and_invariants(torch_cuda):
    torch = torch_cuda
    wl = workloads.small_block()
    log("small block d=544 h=1440 r16@1.0")
    b = Built(wl)
    try:
        x = wl.x0()[0]
        h0 = b.q.qbl_base_hash(b.base)
        y0 = _block(b, torch, 0, x)
        ref0 = oracle.block(b.oracle_layers([]), x.astype(np.float64))
        assert rel_l2(y0, ref0) <= TOL
        b.attach([0])
        y1 = _block(b, torch, 0, x)
        ref1 = oracle.block(b.oracle_layers([0]), x.astype(np.float64))
        assert rel_l2(y1, ref1) <= TOL
        assert rel_l2(y1, y0) > 1e-3
        assert np.array_equal(_block(b, torch, 0, x), y1)
        b.q.qbl_comp_clear(b.comp)
        assert np.array_equal(_block(b, torch, 0, x), y0)
        b.attach([0], [0.0])
        assert np.array_equal(_block(b, torch, 0, x), y0)
        # one block, one token of decode is the same computation as qbl_block
        b.attach([0])
        yd = _decode(b, torch, x, 1, 1)
        assert np.array_equal(yd[0], y1)
        assert b.q.qbl_base_hash(b.base) == h0
    finally:
        b.close()


def test_block_with_mixed_ranks(torch_cuda):
    """The block's summed launches (q+k+v, gate+up) with adapters of rank 16,
    64, 6 and 36, side by side across the segments of one launch, in two list
    orders, against the oracle."""
    torch = torch_cuda
    wl = workloads.Workload("mixed_block", workloads.small_block().linears,
                            [workloads.AdapterSpec("A1", 16, 1.0), workloads.AdapterSpec("A2", 64, 0.5),
                             workloads.AdapterSpec("A3", 6, -0.75), workloads.AdapterSpec("A4", 36, 0.25)],
                            blocks=1, tokens=1)
    log("small block d=544 h=1440, ranks 16, 64, 6, 36")
    b = Built(wl)
    try:
        x = wl.x0()[0]
        y0 = _block(b, torch, 0, x)
        for idx in ([0, 1, 2, 3], [2, 3, 0, 1]):
            b.attach(idx)
            y = _block(b, torch, 0, x)
            ref = oracle.block(b.oracle_layers(idx), x.astype(np.float64))
            assert rel_l2(y, ref) <= TOL, idx
            assert rel_l2(y, y0) > 1e-3
    finally:
        b.close()


def test_small_stack_free_running_chain(torch_cuda):
    torch = torch_cuda
    wl = workloads.small_stack()
    nb, nt = wl.blocks, wl.tokens
    log(f"small stack d=256 h=704 blocks={nb} tokens={nt} r16@1.0 + r64@0.5")
    b = Built(wl)
    try:
        x0 = wl.x0()[0]
        h0 = b.q.qbl_base_hash(b.base)
        b.attach([0, 1])
        y = _decode(b, torch, x0, nb, nt)
        ref = oracle.stack(b.oracle_layers([0, 1]), x0.astype(np.float64), nt)
        worst = max(rel_l2(y[t], ref[t]) for t in range(nt))
        log(f"worst per-token rel-L2 {worst:.3e}")
        assert worst <= TOL
        assert rel_l2(y[1], y[0]) > 1e-2          # the chain keeps moving
        # swap the adapter order: only rounding changes
        b.attach([1, 0])
        ys = _decode(b, torch, x0, nb, nt)
        assert not np.array_equal(ys, y)
        assert max(rel_l2(ys[t], ref[t]) for t in range(nt)) <= TOL
        assert b.q.qbl_base_hash(b.base) == h0
        # base -> A -> base -> B == base -> B on the whole chain
        b.q.qbl_comp_clear(b.comp)
        ybase = _decode(b, torch, x0, nb, 4)
        b.attach([0])
        _decode(b, torch, x0, nb, 4)
        b.q.qbl_comp_clear(b.comp)
        assert np.array_equal(_decode(b, torch, x0, nb, 4), ybase)
        b.attach([1])
        yab = _decode(b, torch, x0, nb, 4)
        b.q.qbl_comp_clear(b.comp)
        b.attach([1])
        assert np.array_equal(_decode(b, torch, x0, nb, 4), yab)
        # decode of a sub-range of blocks equals chained single-block calls up to
        # rounding (decode folds the RMS scale of the previous block's output
        # into the next launch instead of writing the scaled vector)
        y2 = _decode(b, torch, x0, 2, 1, first=1)
        assert rel_l2(y2[0], _block(b, torch, 2, _block(b, torch, 1, x0))) <= 1e-5
    finally:
        b.close()
