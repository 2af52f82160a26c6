"""The shared seeded generator: SplitMix64's published first outputs for seed
0, slice consistency of the counter stream, and the moments of the normals."""
import numpy as np

import synth
from synth import workloads


def test_splitmix64_reference_outputs():
    # first three outputs of SplitMix64 started from state 0
    assert synth.splitmix64_at(0, 0) == 0xE220A8397B1DCDAF
    assert synth.splitmix64_at(0, 1) == 0x6E789E6AA1B965F4
    assert synth.splitmix64_at(0, 2) == 0x06C45D188009454F


def test_offset_slices_and_threads_agree():
    full = synth.normal("slice-test", (300001,), nthreads=1)
    part = synth.normal("slice-test", (1000,), offset=12345)
    assert np.array_equal(part, full[12345:13345])
    mt = synth.normal("slice-test", (300001,), nthreads=7)
    assert np.array_equal(mt, full)


def test_normal_moments():
    x = synth.normal("moments", (2_000_000,), mean=0.0, std=0.02).astype(np.float64)
    assert abs(x.mean()) < 0.02 * 5 / np.sqrt(x.size)
    assert abs(x.std() / 0.02 - 1) < 3e-3
    assert abs(np.mean((x / 0.02) ** 4) - 3.0) < 0.03        # normal kurtosis


def test_workload_rows_match_full_tensor():
    w = workloads.small_block()
    full = w.weight(6)
    assert np.array_equal(w.weight_rows(6, 100, 133), full[100:133])
    assert w.lora_a(0, 0).shape == (16, 544) and w.lora_b(4, 0).shape == (1440, 16)
