"""CPU tests of sparse (CSR) adapters through the host-only build of the runtime
(tests/hostsim): the deep checks of "Deep Technical Design" section 11
(strictly monotonic indices, finite f16 payloads, matching dimensions) with
deterministic errors and no side effects, the digest definition, budget
accounting, mixing with low-rank adapters in one list, and the prefill path's
refusal of sparse deltas."""
import hashlib
import struct

import numpy as np
import pytest

import quantized_base_linear_amd as q
from synth import workloads as W
from tests import hostsim
from tests.test_lifecycle_host import World, _err, identity_def


@pytest.fixture(scope="module")
def sim():
    lib, raw = hostsim.load()
    yield lib, raw
    assert raw.qbl_sim_bad_calls() == 0


@pytest.fixture
def world(sim):
    w = World(*sim)
    yield w
    w.close()


def _csr(n, k, density, tag):
    wl = W.Workload(tag, [W.LinearSpec(tag + "/L", n, k)], [W.AdapterSpec("S", 0, 1.0, density)])
    return wl.sparse_csr(0, 0)


def sparse_digest_def(entries, n_of):
    inner = b""
    for lin, rp, col, val in entries:
        hdr = struct.pack("<iiq", lin, -1, col.size)
        inner += hashlib.sha256(hdr + rp.astype("<u4").tobytes() + col.astype("<u4").tobytes()
                                + val.astype("<u2").tobytes()).digest()
    return hashlib.sha256(inner).digest()


def sparse_arena_bytes(entries):
    up = lambda b: -(-b // 256) * 256
    return sum(up(4 * rp.size) + up(4 * col.size) + up(2 * col.size) for _, rp, col, _ in entries)


def test_load_digest_budget_and_attach(world):
    lib = world.lib
    ents = [(0, *_csr(64, 128, 0.1, "h0")), (2, *_csr(32, 96, 0.3, "h2"))]
    held0 = lib.qbl_base_memory(world.base)[0]
    a = lib.qbl_adapter_load_sparse(world.base, ents)
    try:
        assert lib.qbl_adapter_digest(a) == sparse_digest_def(ents, None)
        assert lib.qbl_base_memory(world.base)[0] == held0 + sparse_arena_bytes(ents)
        # in one list with low-rank adapters; the identity covers it like any adapter
        lib.qbl_comp_attach(world.comp, [world.ads[0], a], [1.0, -0.5])
        assert lib.qbl_comp_count(world.comp) == 2
        assert lib.qbl_comp_digest(world.comp) == identity_def(
            lib.qbl_base_digest(world.base), [lib.qbl_adapter_digest(world.ads[0]), lib.qbl_adapter_digest(a)],
            [1.0, -0.5])
        # the prefill path refuses a list with a sparse delta on that linear
        raw = world.raw
        st = raw.qbl_linear_jit(world.comp, 0, 0x1000, 0x2000, 8, None, 0, None)
        assert q.STATUS[st] == "QBL_E_FORMAT"
        assert b"low-rank" in raw.qbl_last_error()
        lib.qbl_comp_clear(world.comp)
        lib.qbl_comp_drop_previous(world.comp)
    finally:
        lib.qbl_adapter_free(a)
    assert lib.qbl_base_memory(world.base)[0] == held0


def test_empty_and_dense_rows(world):
    lib = world.lib
    n, k = 64, 128
    empty = (0, np.zeros(n + 1, np.uint32), np.zeros(0, np.uint32), np.zeros(0, np.uint16))
    rp = np.arange(n + 1, dtype=np.uint32) * k                          # every entry of every row
    full = (0, rp, np.tile(np.arange(k, dtype=np.uint32), n), np.full(n * k, 0x3C00, np.uint16))
    for ents in ([empty], [full]):
        a = lib.qbl_adapter_load_sparse(world.base, ents)
        assert lib.qbl_adapter_digest(a) == sparse_digest_def(ents, None)
        lib.qbl_adapter_free(a)


def test_deep_checks_are_deterministic_and_side_effect_free(world):
    lib = world.lib
    n, k = 96, 64                       # linear 1
    rp, col, val = _csr(n, k, 0.2, "bad")
    assert col.size > 10
    r = int(np.argmax(np.diff(rp.astype(np.int64)) >= 2))               # a row with >= 2 entries
    p = int(rp[r])
    cases = []
    c = col.copy(); c[p], c[p + 1] = c[p + 1], c[p]                     # out of order
    cases.append(("QBL_E_FORMAT", (1, rp, c, val)))
    c = col.copy(); c[p + 1] = c[p]                                     # repeated column
    cases.append(("QBL_E_FORMAT", (1, rp, c, val)))
    c = col.copy(); c[p] = k                                            # column past the row
    cases.append(("QBL_E_SHAPE", (1, rp, c, val)))
    b = rp.copy(); b[0] = 1                                             # row_ptr not from 0
    cases.append(("QBL_E_SHAPE", (1, b, col, val)))
    b = rp.copy(); b[5], b[6] = b[6] + 1, b[5]                          # row_ptr decreasing
    cases.append(("QBL_E_SHAPE", (1, b, col, val)))
    b = rp.copy(); b[n - 1] = b[n] + 50                                 # overshoots nnz, then drops back
    cases.append(("QBL_E_SHAPE", (1, b, col, val)))
    b = rp.copy(); b[n] += 1                                            # ends past the entries given
    cases.append(("QBL_E_SHAPE", (1, b, col, val)))
    for bits in (0x7C00, 0xFC00, 0x7E00, 0x7C01):                       # +Inf, -Inf, NaNs
        v = val.copy(); v[len(v) // 2] = bits
        cases.append(("QBL_E_NONFINITE", (1, rp, col, v)))
    cases.append(("QBL_E_SHAPE", (9, rp, col, val)))                    # unknown linear
    cases.append(("QBL_E_SHAPE", (0, rp, col, val)))                    # shape of another linear
    before = world.state()
    for name, ent in cases:
        e1 = _err(lib.qbl_adapter_load_sparse, world.base, [ent])
        e2 = _err(lib.qbl_adapter_load_sparse, world.base, [ent])
        assert e1.name == name, (name, e1)
        assert e1.msg == e2.msg
        assert world.state() == before
    # the same linear twice in one adapter
    e = _err(lib.qbl_adapter_load_sparse, world.base, [(1, rp, col, val), (1, rp, col, val)])
    assert e.name == "QBL_E_DUPLICATE" and world.state() == before
    # the budget is checked before anything is allocated
    held = lib.qbl_base_memory(world.base)[0]
    lib.qbl_base_set_budget(world.base, held + sparse_arena_bytes([(1, rp, col, val)]) - 1)
    assert _err(lib.qbl_adapter_load_sparse, world.base, [(1, rp, col, val)]).name == "QBL_E_BUDGET"
    lib.qbl_base_set_budget(world.base, 0)
    assert world.state() == before
    # injected corruption of the staged copy is caught
    lib.qbl_fault_inject(q.QBL_FAULT_CORRUPT, 1)
    assert _err(lib.qbl_adapter_load_sparse, world.base, [(1, rp, col, val)]).name == "QBL_E_CHECKSUM"
    assert world.state() == before
