"""CPU checks of the C-ABI library: it loads, exports every function that
include/qbl.h declares, its host quantiser writes the same bytes as the
oracle's independent one, its SHA-256 matches hashlib, and argument errors
are reported without touching a device."""
import hashlib
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
import quantized_base_linear_amd as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "qbl.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qbl_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert len(names) >= 20
    out = subprocess.run(["nm", "-D", "--defined-only", q.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (qbl_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    assert set(q.EXPORTS) >= set(names)


def test_abi_version_and_block_bytes():
    assert q.qbl_abi_version() == 2
    assert q.qbl_block_bytes(q.QBL_Q8_0) == 34 and q.qbl_block_bytes(q.QBL_Q4_SM) == 20
    assert q.qbl_block_bytes(q.QBL_Q4_K) == 144 and q.qbl_block_weights(q.QBL_Q4_K) == 256
    assert q.qbl_block_weights(q.QBL_Q8_0) == q.qbl_block_weights(q.QBL_Q4_SM) == 32
    assert q.qbl_block_bytes(7) == 0 and q.qbl_block_weights(7) == 0


@pytest.mark.parametrize("qtype", [q.QBL_Q8_0, q.QBL_Q4_SM, q.QBL_Q4_K])
def test_library_quantiser_bytes_equal_oracle(qtype):
    rng = np.random.default_rng(40 + qtype)
    k = 768 if qtype == q.QBL_Q4_K else 640
    w = (rng.standard_normal((300, k)) * 0.02).astype(np.float32)
    w[0, :32] = 0.0                                   # zero block
    w[1, 32:64] = np.float32(0.125)                   # constant block
    w[2, :32] = np.arange(32, dtype=np.float32) - 16  # exact grid
    w[3, :] *= 1e-6                                   # tiny scales (fp16 subnormal range)
    w[4, :] *= 100                                    # large values
    w[5, :256] = 0.0                                  # zero super-block
    w[6, :] = np.abs(w[6, :]) + 0.01                  # all positive (no offset)
    w[7, :] = -np.abs(w[7, :]) - 0.01                 # all negative
    lib = q.qbl_quantize(qtype, w)
    ref = oracle.quantize(qtype, w)
    assert lib.shape == ref.shape and np.array_equal(lib, ref)
    deq = q.qbl_dequantize(qtype, lib, 300, k)
    assert np.array_equal(deq, oracle.dequantize(qtype, ref, 300, k).astype(np.float32))


def test_library_quantiser_on_workload_tensors():
    from synth import workloads
    wl = workloads.small_block()
    for i in (0, 6):
        w = wl.weight(i)
        assert np.array_equal(q.qbl_quantize(q.QBL_Q8_0, w), oracle.quantize(oracle.Q8_0, w))
    wl4 = workloads.small_mlp()
    w = wl4.weight(2)
    assert np.array_equal(q.qbl_quantize(q.QBL_Q4_SM, w), oracle.quantize(oracle.Q4_SM, w))


def test_quantiser_rejections():
    with pytest.raises(q.QblError) as e:
        q.qbl_quantize(q.QBL_Q8_0, np.zeros((2, 48), np.float32))
    assert e.value.status == -3
    w = np.zeros((2, 64), np.float32)
    w[1, 3] = np.nan
    with pytest.raises(q.QblError) as e:
        q.qbl_quantize(q.QBL_Q8_0, w)
    assert e.value.status == -4
    w = np.zeros((2, 64), np.float32)
    w[0, 0] = 1e7                                     # max|w|/127 overflows fp16
    with pytest.raises(q.QblError) as e:
        q.qbl_quantize(q.QBL_Q8_0, w)
    assert e.value.status == -11
    with pytest.raises(q.QblError) as e:
        q.qbl_quantize(9, np.zeros((2, 64), np.float32))
    assert e.value.status == -3


def test_sha256_matches_hashlib_and_fips_examples():
    assert q.qbl_sha256(b"abc").hex() == \
        "ba7816bf8f01cfea414140de5dae2223b00361a396177a9cb410ff61f20015ad"
    assert q.qbl_sha256(b"").hex() == hashlib.sha256(b"").hexdigest()
    rng = np.random.default_rng(0)
    for n in (1, 55, 56, 63, 64, 65, 1000, 123457):
        data = rng.integers(0, 256, n, dtype=np.uint8).tobytes()
        assert q.qbl_sha256(data) == hashlib.sha256(data).digest()


def test_base_load_validates_before_any_device_call():
    good = np.zeros((4, 2 * 34), np.uint8)
    cases = [
        ([(3, 4, 64, good)], -3),                      # unknown type
        ([(1, 4, 48, np.zeros((4, 51), np.uint8))], -3),  # k not a multiple of 32
        ([(1, 4, 64, good[:, :60])], -3),              # byte count mismatch
        ([(1, 0, 64, good)], -2),                      # empty shape
    ]
    for linears, status in cases:
        with pytest.raises(q.QblError) as e:
            q.qbl_base_load(linears)
        assert e.value.status == status, linears
    with pytest.raises(q.QblError):
        q.qbl_base_load([])


def test_errors_leave_a_message():
    with pytest.raises(q.QblError):
        q.qbl_quantize(q.QBL_Q8_0, np.zeros((2, 48), np.float32))
    assert "multiple of 32" in q.qbl_last_error()


def test_hbm_probe_rejects_bad_arguments_before_any_device_call():
    import ctypes
    lib = q._lib
    wg = ctypes.c_int32(-5)
    fake = ctypes.c_void_p(4096)  # never dereferenced: every case fails validation first
    cases = [
        (None, 64, fake, 4),          # null buffer
        (fake, 64, None, 4),          # null sink
        (fake, 0, fake, 4),           # empty
        (fake, 40, fake, 4),          # not a multiple of 16
        (ctypes.c_void_p(4104), 64, fake, 4),  # misaligned
        (fake, 64, fake, 0),          # no sink words
    ]
    for buf, nbytes, sink, words in cases:
        assert lib.qbl_hbm_probe(buf, nbytes, sink, words, ctypes.addressof(wg), None) == -1, (nbytes, words)
        assert q.qbl_last_error()
    assert lib.qbl_hbm_probe(fake, 64, fake, 4, None, None) == -1
    assert wg.value == -5
