"""CPU tests of the transactional lifecycle, through the C ABI of a host-only
build of the runtime (tests/hostsim: the same runtime source against a HIP
double whose "device" memory is tracked host memory).

What the pages ask of the lifecycle ("We propose a content-addressed overlay
system": "Explicit Correctness and Atomicity Invariants", "Proposed
Activation/Deactivation State Machine", "TDD and Fault-Injection Matrix",
"Composition Identity and Manifest Schema"; "Deep Technical Design", section 6;
"LoRA adapters" blueprint, "Runtime Identity and Cache Safety"):
  - validation before any change, deterministic errors without side effects;
  - a memory budget checked before allocation;
  - staging with verification of the device copy (a forced mismatch aborts);
  - a failure between staging and the swap leaves the old composition active;
  - rollback restores the previous composition; idempotent re-activation;
  - repeated switch cycles leave the base bytes identical and leak nothing;
  - an identity digest over base digest, ordered adapter digests and scales.
The digests are checked against their documented byte definitions computed
here with hashlib.
"""
import ctypes
import hashlib
import struct
import threading

import numpy as np
import pytest

import oracle
import quantized_base_linear_amd as q
from tests import hostsim

ABI = 2


@pytest.fixture(scope="module")
def sim():
    lib, raw = hostsim.load()
    assert lib.qbl_abi_version() == ABI
    yield lib, raw
    assert raw.qbl_sim_bad_calls() == 0, "a copy or free outside the simulated allocations"


def _err(fn, *a):
    with pytest.raises(q.QblError) as ei:
        fn(*a)
    return ei.value


SHAPES = [(q.QBL_Q8_0, 64, 128), (q.QBL_Q4_SM, 96, 64), (q.QBL_Q8_0, 32, 96)]


def _blocks(qtype, n, k, seed):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    return oracle.quantize(qtype, w)


def _linears(seed=0, shapes=SHAPES):
    return [(qt, n, k, _blocks(qt, n, k, seed + i)) for i, (qt, n, k) in enumerate(shapes)]


def _factors(n, k, r, seed):
    rng = np.random.default_rng(seed)
    A = (rng.standard_normal((r, k)) / np.sqrt(k)).astype(np.float32)
    B = (rng.standard_normal((n, r)) * 0.01).astype(np.float32)
    return A, B


def arena_bytes(entries):
    """Device bytes of an adapter: A and B of each entry, each padded to 256 bytes."""
    return sum(-(-4 * A.size // 256) * 256 + -(-4 * B.size // 256) * 256 for _, A, B in entries)


def _adapter_entries(shapes, targets, r, seed):
    return [(i, *_factors(shapes[i][1], shapes[i][2], r, seed + 10 * i)) for i in targets]


# -- documented digest definitions, written out with hashlib ---------------------
def base_digest_def(linears):
    inner = b""
    for qt, n, k, blk in linears:
        hdr = struct.pack("<iiqq", qt, 0, n, k)
        inner += hashlib.sha256(hdr + np.ascontiguousarray(blk).tobytes()).digest()
    return hashlib.sha256(inner).digest()


def adapter_digest_def(entries):
    inner = b""
    for lin, A, B in entries:
        hdr = struct.pack("<ii", lin, A.shape[0])
        inner += hashlib.sha256(hdr + A.astype("<f4").tobytes() + B.astype("<f4").tobytes()).digest()
    return hashlib.sha256(inner).digest()


def identity_def(base_digest, ads, scales):
    eff = [(d, s) for d, s in zip(ads, scales) if s != 0.0]
    msg = struct.pack("<i", ABI) + base_digest + struct.pack("<i", len(eff))
    for d, s in eff:
        msg += d + struct.pack("<f", s)
    return hashlib.sha256(msg).digest()


class World:
    """A base of three linears and three adapters on the host-only library."""

    def __init__(self, lib, raw, seed=0):
        self.lib, self.raw = lib, raw
        self.live0 = raw.qbl_sim_live_bytes()
        self.linears = _linears(seed)
        self.base = lib.qbl_base_load(self.linears)
        self.entries = [_adapter_entries(SHAPES, [0, 1], 4, 100 + seed),
                        _adapter_entries(SHAPES, [1, 2], 8, 200 + seed),
                        _adapter_entries(SHAPES, [0, 2], 2, 300 + seed)]
        self.ads = [lib.qbl_adapter_load(self.base, e) for e in self.entries]
        self.comp = lib.qbl_comp_create(self.base)

    def state(self):
        """Everything an aborted change must leave alone."""
        lib = self.lib
        return (lib.qbl_comp_digest(self.comp), lib.qbl_comp_count(self.comp),
                lib.qbl_base_memory(self.base), self.raw.qbl_sim_live_bytes(),
                self.raw.qbl_sim_live_allocations())

    def digest_of(self, idx, scales):
        return identity_def(self.lib.qbl_base_digest(self.base),
                            [self.lib.qbl_adapter_digest(self.ads[i]) for i in idx], scales)

    def close(self):
        lib = self.lib
        lib.qbl_comp_free(self.comp)
        for a in self.ads:
            lib.qbl_adapter_free(a)
        lib.qbl_base_free(self.base)
        assert self.raw.qbl_sim_live_bytes() == self.live0, "device memory leaked"


@pytest.fixture
def world(sim):
    w = World(*sim)
    yield w
    w.close()


# -- digests -----------------------------------------------------------------------
def test_base_digest_matches_definition_and_device_bytes(world):
    lib = world.lib
    d = lib.qbl_base_digest(world.base)
    assert d == base_digest_def(world.linears)
    assert lib.qbl_base_hash(world.base) == d          # re-read from "device" memory


def test_base_digest_names_bytes_and_format(sim):
    lib, raw = sim
    lins = _linears(5)
    ref = base_digest_def(lins)
    flipped = [list(x) for x in lins]
    blk = flipped[1][3].copy()
    blk[3, 7] ^= 0x10
    flipped[1][3] = blk
    assert base_digest_def([tuple(x) for x in flipped]) != ref
    b1 = lib.qbl_base_load([tuple(x) for x in flipped])
    b0 = lib.qbl_base_load(lins)
    try:
        assert lib.qbl_base_digest(b0) == ref
        assert lib.qbl_base_digest(b1) != ref
        # same bytes, other shape: the header is part of the digest
        qt, n, k, blk = lins[0]
        b2 = lib.qbl_base_load([(qt, n // 2, k * 2, blk)])
        assert lib.qbl_base_digest(b2) != base_digest_def([lins[0]])
        lib.qbl_base_free(b2)
    finally:
        lib.qbl_base_free(b0)
        lib.qbl_base_free(b1)


def test_base_hash_notices_a_changed_device_byte(sim):
    lib, raw = sim
    lins = _linears(9, SHAPES[:1])
    b = lib.qbl_base_load(lins)
    try:
        arena = raw.qbl_sim_last_allocation()
        assert lib.qbl_base_hash(b) == lib.qbl_base_digest(b)
        assert raw.qbl_sim_poke(arena, 0x40) == 0
        assert lib.qbl_base_hash(b) != lib.qbl_base_digest(b)
        assert raw.qbl_sim_poke(arena, 0x40) == 0
        assert lib.qbl_base_hash(b) == lib.qbl_base_digest(b)
    finally:
        lib.qbl_base_free(b)


def test_adapter_digest_matches_definition(world):
    for a, e in zip(world.ads, world.entries):
        assert world.lib.qbl_adapter_digest(a) == adapter_digest_def(e)
    assert len({world.lib.qbl_adapter_digest(a) for a in world.ads}) == 3


def test_identity_digest_definition(sim):
    lib, _ = sim
    rng = np.random.default_rng(1)
    bd = rng.bytes(32)
    ads = [rng.bytes(32) for _ in range(4)]
    for scales in ([1.0, 0.5, -2.0, 3.25], [1.0, 0.0, -0.0, 0.125], [0.0] * 4):
        assert lib.qbl_identity_digest(bd, ads, scales) == identity_def(bd, ads, scales)
    assert lib.qbl_identity_digest(bd, [], []) == identity_def(bd, [], [])
    # zero-scale entries do not count; order, scale and base all do
    assert lib.qbl_identity_digest(bd, ads[:2], [1.0, 0.0]) == lib.qbl_identity_digest(bd, ads[:1], [1.0])
    assert lib.qbl_identity_digest(bd, ads[:2], [1.0, 2.0]) != lib.qbl_identity_digest(bd, ads[1::-1], [2.0, 1.0])
    assert lib.qbl_identity_digest(bd, ads[:1], [1.0]) != lib.qbl_identity_digest(bd, ads[:1], [1.0000001])
    assert lib.qbl_identity_digest(bd, ads[:1], [1.0]) != lib.qbl_identity_digest(ads[3], ads[:1], [1.0])
    assert _err(lib.qbl_identity_digest, bd, ads[:1], [float("nan")]).name == "QBL_E_NONFINITE"
    assert _err(lib.qbl_identity_digest, bd, ads * 3, [1.0] * 12).name == "QBL_E_LIMIT"


def test_composition_digest_follows_the_list(world):
    lib, c = world.lib, world.comp
    assert lib.qbl_comp_digest(c) == world.digest_of([], [])
    for idx, sc in (([0], [1.0]), ([0, 1], [1.0, 0.5]), ([1, 0], [0.5, 1.0]), ([2, 0, 1], [2.0, 0.0, -1.0])):
        lib.qbl_comp_attach(c, [world.ads[i] for i in idx], sc)
        assert lib.qbl_comp_digest(c) == world.digest_of(idx, sc)
    # all-zero scales is the base-only composition
    lib.qbl_comp_attach(c, world.ads[:2], [0.0, 0.0])
    assert lib.qbl_comp_digest(c) == world.digest_of([], [])
    assert lib.qbl_comp_count(c) == 0
    lib.qbl_comp_clear(c)
    assert lib.qbl_comp_digest(c) == world.digest_of([], [])
    # two compositions with the same list have the same identity
    c2 = lib.qbl_comp_create(world.base)
    lib.qbl_comp_attach(c, [world.ads[1]], [0.75])
    lib.qbl_comp_attach(c2, [world.ads[1]], [0.75])
    assert lib.qbl_comp_digest(c) == lib.qbl_comp_digest(c2)
    lib.qbl_comp_free(c2)


# -- validation: deterministic errors, no side effects ---------------------------------
def test_nonfinite_payload_rejected_before_anything_is_allocated(world):
    lib = world.lib
    before = world.state()
    for bad in (np.nan, np.inf, -np.inf):
        e = _adapter_entries(SHAPES, [0, 2], 4, 7)
        e[1][2][5, 1] = bad                               # B of the second entry
        err1 = _err(lib.qbl_adapter_load, world.base, e)
        err2 = _err(lib.qbl_adapter_load, world.base, e)
        assert err1.name == "QBL_E_NONFINITE" and (err1.status, err1.msg) == (err2.status, err2.msg)
        assert world.state() == before
    assert _err(lib.qbl_comp_attach, world.comp, world.ads[:1], [np.nan]).name == "QBL_E_NONFINITE"
    assert world.state() == before


def test_compatibility_checks_leave_the_composition_alone(sim, world):
    lib = world.lib
    lib.qbl_comp_attach(world.comp, [world.ads[0]], [1.0])
    other = World(*sim, seed=3)
    before = world.state()
    try:
        cases = [
            ("QBL_E_FOREIGN", lambda: lib.qbl_comp_attach(world.comp, [world.ads[1], other.ads[0]], [1.0, 1.0])),
            ("QBL_E_DUPLICATE", lambda: lib.qbl_comp_attach(world.comp, [world.ads[1], world.ads[1]], [1.0, 2.0])),
            ("QBL_E_LIMIT", lambda: lib.qbl_comp_attach(world.comp, [world.ads[0]] * 9, [1.0] * 9)),
            ("QBL_E_SHAPE", lambda: lib.qbl_adapter_load(world.base, [(5, *_factors(64, 128, 4, 1))])),
            ("QBL_E_DUPLICATE", lambda: lib.qbl_adapter_load(world.base, _adapter_entries(SHAPES, [0, 0], 4, 1))),
            ("QBL_E_LIMIT", lambda: lib.qbl_adapter_load(world.base, [(0, *_factors(64, 128, 300, 1))])),
            ("QBL_E_ARG", lambda: lib.qbl_adapter_load(world.base, [])),
        ]
        for name, call in cases:
            e1 = _err(call)
            e2 = _err(call)
            assert e1.name == name, (name, e1)
            assert e1.msg == e2.msg
            assert world.state() == before
        # the summed rank per linear is capped over the whole list
        big = [lib.qbl_adapter_load(world.base, [(0, *_factors(64, 128, 256, 50 + i))]) for i in range(3)]
        mid = world.state()
        assert _err(lib.qbl_comp_attach, world.comp, big, [1.0, 1.0, 1.0]).name == "QBL_E_LIMIT"
        assert world.state() == mid
        lib.qbl_comp_attach(world.comp, big, [1.0, 1.0, 0.0])     # a zero scale does not count
        lib.qbl_comp_rollback(world.comp)
        for a in big:
            lib.qbl_adapter_free(a)
        lib.qbl_comp_drop_previous(world.comp)
        assert world.state() == before
    finally:
        other.close()


# -- memory budget -------------------------------------------------------------------
def test_memory_budget_is_checked_before_allocation(world):
    lib, raw, base = world.lib, world.raw, world.base
    held, budget = lib.qbl_base_memory(base)
    assert budget == 0 and held > 0
    e = _adapter_entries(SHAPES, [0, 1, 2], 16, 77)
    need = arena_bytes(e)
    lib.qbl_base_set_budget(base, held + need - 1)
    before = world.state()
    err = _err(lib.qbl_adapter_load, base, e)
    assert err.name == "QBL_E_BUDGET"
    assert world.state() == before
    # a budget below what is held is refused and the old one kept
    assert _err(lib.qbl_base_set_budget, base, held - 1).name == "QBL_E_BUDGET"
    assert lib.qbl_base_memory(base) == (held, held + need - 1)
    lib.qbl_base_set_budget(base, held + need)
    a = lib.qbl_adapter_load(base, e)
    assert lib.qbl_base_memory(base) == (held + need, held + need)
    # attached and freed by the caller: still held until no list refers to it
    lib.qbl_comp_attach(world.comp, [a], [1.0])
    lib.qbl_adapter_free(a)
    lib.qbl_comp_clear(world.comp)
    assert lib.qbl_base_memory(base)[0] == held + need          # kept by the previous list
    lib.qbl_comp_drop_previous(world.comp)
    assert lib.qbl_base_memory(base)[0] == held
    lib.qbl_base_set_budget(base, 0)


def test_device_full_is_reported_without_leaks(world):
    lib, raw = world.lib, world.raw
    before = world.state()
    raw.qbl_sim_set_capacity(raw.qbl_sim_live_bytes() + 1024)
    try:
        err = _err(lib.qbl_adapter_load, world.base, _adapter_entries(SHAPES, [0, 1], 16, 5))
        assert err.name == "QBL_E_NOMEM"
        assert world.state() == before
        assert _err(lib.qbl_base_load, _linears(11)).name == "QBL_E_NOMEM"
        assert world.state() == before
    finally:
        raw.qbl_sim_set_capacity(0)


# -- fault injection at each phase ---------------------------------------------------------
def test_injected_allocation_failure(world):
    lib = world.lib
    before = world.state()
    lins = _linears(21)
    for after in (1, 2, 3):
        lib.qbl_fault_inject(q.QBL_FAULT_DEVICE_ALLOC, after)
        assert _err(lib.qbl_base_load, lins).name == "QBL_E_NOMEM"
        assert world.state() == before
    lib.qbl_fault_inject(q.QBL_FAULT_DEVICE_ALLOC, 1)
    assert _err(lib.qbl_adapter_load, world.base, _adapter_entries(SHAPES, [1], 4, 9)).name == "QBL_E_NOMEM"
    assert world.state() == before
    # fired once: the next load succeeds
    a = lib.qbl_adapter_load(world.base, _adapter_entries(SHAPES, [1], 4, 9))
    lib.qbl_adapter_free(a)
    assert world.state() == before


def test_injected_corruption_is_caught_by_verification(world):
    lib = world.lib
    before = world.state()
    lins = _linears(31)
    for after in (1, 3):
        lib.qbl_fault_inject(q.QBL_FAULT_CORRUPT, after)
        err = _err(lib.qbl_base_load, lins)
        assert err.name == "QBL_E_CHECKSUM", err
        assert world.state() == before
    e = _adapter_entries(SHAPES, [0, 1, 2], 8, 41)
    for after in (1, 2, 3):
        lib.qbl_fault_inject(q.QBL_FAULT_CORRUPT, after)
        assert _err(lib.qbl_adapter_load, world.base, e).name == "QBL_E_CHECKSUM"
        assert world.state() == before
    a = lib.qbl_adapter_load(world.base, e)
    assert lib.qbl_adapter_digest(a) == adapter_digest_def(e)
    lib.qbl_adapter_free(a)
    assert world.state() == before


def test_failure_between_staging_and_swap_keeps_the_active_composition(world):
    lib, c, ads = world.lib, world.comp, world.ads
    lib.qbl_comp_attach(c, [ads[0]], [1.0])
    lib.qbl_comp_attach(c, [ads[1], ads[0]], [0.5, 1.0])
    active = world.state()
    for change in (lambda: lib.qbl_comp_attach(c, [ads[2]], [2.0]),
                   lambda: lib.qbl_comp_clear(c),
                   lambda: lib.qbl_comp_rollback(c)):
        lib.qbl_fault_inject(q.QBL_FAULT_SWAP, 1)
        assert _err(change).name == "QBL_E_INJECTED"
        assert world.state() == active
    # the previous list survived the failures: rollback still returns to [A]
    lib.qbl_comp_rollback(c)
    assert lib.qbl_comp_digest(c) == world.digest_of([0], [1.0])
    # and a retry after the fault succeeds
    lib.qbl_comp_attach(c, [ads[2]], [2.0])
    assert lib.qbl_comp_digest(c) == world.digest_of([2], [2.0])


def test_fault_points_are_validated(sim):
    lib, _ = sim
    assert _err(lib.qbl_fault_inject, 0, 1).name == "QBL_E_ARG"
    assert _err(lib.qbl_fault_inject, 9, 1).name == "QBL_E_ARG"
    assert _err(lib.qbl_fault_inject, q.QBL_FAULT_SWAP, -1).name == "QBL_E_ARG"
    for p in (q.QBL_FAULT_DEVICE_ALLOC, q.QBL_FAULT_CORRUPT, q.QBL_FAULT_SWAP):
        lib.qbl_fault_inject(p, 0)


# -- rollback, idempotency, cycles ----------------------------------------------------------
def test_rollback_exchanges_current_and_previous(world):
    lib, c, ads = world.lib, world.comp, world.ads
    base_only = world.digest_of([], [])
    dA, dB = world.digest_of([0], [1.0]), world.digest_of([1], [0.5])
    assert _err(lib.qbl_comp_rollback, c).name == "QBL_E_STATE"      # nothing to return to
    lib.qbl_comp_attach(c, [ads[0]], [1.0])
    lib.qbl_comp_attach(c, [ads[1]], [0.5])
    lib.qbl_comp_rollback(c)
    assert lib.qbl_comp_digest(c) == dA
    lib.qbl_comp_rollback(c)
    assert lib.qbl_comp_digest(c) == dB
    lib.qbl_comp_clear(c)
    assert lib.qbl_comp_digest(c) == base_only
    lib.qbl_comp_rollback(c)
    assert lib.qbl_comp_digest(c) == dB and lib.qbl_comp_count(c) == 1
    lib.qbl_comp_drop_previous(c)
    assert _err(lib.qbl_comp_rollback, c).name == "QBL_E_STATE"
    assert lib.qbl_comp_digest(c) == dB


def test_repeated_activation_is_a_no_op(world):
    lib, c, ads = world.lib, world.comp, world.ads
    lib.qbl_comp_attach(c, [ads[0]], [1.0])
    after_first = world.state()
    lib.qbl_comp_attach(c, [ads[0]], [1.0])
    assert world.state() == after_first
    lib.qbl_comp_rollback(c)            # the previous list is still base-only
    assert lib.qbl_comp_digest(c) == world.digest_of([], [])
    lib.qbl_comp_clear(c)               # clearing an empty list: no change, previous kept
    lib.qbl_comp_rollback(c)
    assert lib.qbl_comp_digest(c) == world.digest_of([0], [1.0])


def test_switch_cycles_keep_base_bytes_and_memory(world):
    lib, c, ads = world.lib, world.comp, world.ads
    h0 = lib.qbl_base_hash(world.base)
    steady = None
    for cycle in range(20):
        for idx, sc in (([0], [1.0]), ([], []), ([1], [2.0]), ([], []), ([2, 0], [1.0, -1.0])):
            lib.qbl_comp_attach(c, [ads[i] for i in idx], sc)
            assert lib.qbl_comp_digest(c) == world.digest_of(idx, sc)
        lib.qbl_comp_clear(c)
        lib.qbl_comp_drop_previous(c)
        if steady is None:
            steady = world.state()
        assert world.state() == steady
        assert lib.qbl_base_hash(world.base) == h0


def test_references_keep_memory_alive_until_the_last_user(sim):
    lib, raw = sim
    w = World(lib, raw, seed=8)
    c2 = lib.qbl_comp_create(w.base)
    lib.qbl_comp_attach(w.comp, [w.ads[0]], [1.0])
    lib.qbl_comp_attach(c2, [w.ads[0], w.ads[1]], [1.0, 1.0])
    held = lib.qbl_base_memory(w.base)[0]
    lib.qbl_adapter_free(w.ads[0])
    lib.qbl_adapter_free(w.ads[1])
    w.ads = w.ads[2:]
    assert lib.qbl_base_memory(w.base)[0] == held
    assert _err(lib.qbl_base_free, w.base).name == "QBL_E_BUSY"
    lib.qbl_comp_free(c2)              # the last user of ads[1]; w.comp still uses ads[0]
    assert lib.qbl_base_memory(w.base)[0] == held - arena_bytes(w.entries[1])
    lib.qbl_comp_clear(w.comp)
    lib.qbl_comp_drop_previous(w.comp)
    assert lib.qbl_base_memory(w.base)[0] == held - arena_bytes(w.entries[1]) - arena_bytes(w.entries[0])
    w.close()


def test_runs_have_no_cpu_path(world):
    """Run calls need the GPU kernels: the host-only build reports QBL_E_DEVICE."""
    lib, raw = world.lib, world.raw
    x = np.ones((1, 128), np.float32)
    y = np.zeros((1, 64), np.float32)
    st = raw.qbl_linear(world.comp, 0, x.ctypes.data, y.ctypes.data, 1, None, 0, None)
    assert q.STATUS[st] == "QBL_E_DEVICE"
    assert not y.any()


def test_concurrent_changes_serialise(world):
    lib, c, ads = world.lib, world.comp, world.ads
    lists = [([0], [1.0]), ([1, 2], [0.5, 0.25]), ([2], [-1.0]), ([], [])]
    digests = {world.digest_of(i, s) for i, s in lists}
    errors = []

    def worker(t):
        try:
            for j in range(300):
                idx, sc = lists[(t + j) % len(lists)]
                if j % 7 == 3:
                    try:
                        lib.qbl_comp_rollback(c)
                    except q.QblError as e:
                        if e.name != "QBL_E_STATE":
                            raise
                else:
                    lib.qbl_comp_attach(c, [ads[i] for i in idx], sc)
                assert lib.qbl_comp_digest(c) in digests
        except Exception as e:  # noqa: BLE001
            errors.append(e)

    th = [threading.Thread(target=worker, args=(t,)) for t in range(8)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    assert not errors, errors[:3]
    d = lib.qbl_comp_digest(c)
    assert d in digests
    n = lib.qbl_comp_count(c)
    assert n == {world.digest_of(i, s): len([x for x in s if x]) for i, s in lists}[d]
