"""Pins of the oracle's number formats and quantisers against things other
than the oracle itself: numpy's and torch's IEEE conversions, exact integer
grids, error bounds, and the bit densities the pages print."""
import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# -- binary16 ---------------------------------------------------------------------
def test_f16_to_f32_exhaustive_matches_numpy():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.f32_from_f16(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f16_round_trip_exhaustive():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = h.view(np.float16).astype(np.float32)
    ok = ~np.isnan(f)
    back = oracle.f16_from_f32(f[ok])
    assert np.array_equal(back, h[ok])


def test_f16_rounding_matches_numpy_including_ties():
    rng = np.random.default_rng(1)
    # random binary32 across the whole binary16 range, subnormals and overflow
    e = rng.uniform(-30, 17, 200000)
    v = (rng.choice([-1.0, 1.0], e.size) * 2.0 ** e).astype(np.float32)
    # exact midpoints between neighbouring binary16 values (ties), and +-1 ulp of them
    h = np.arange(0, 0x7BFF, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    mid = ((lo + hi) / 2).astype(np.float32)  # exact: 12 significant bits
    up = np.nextafter(mid, np.float32(np.inf))
    dn = np.nextafter(mid, np.float32(-np.inf))
    special = np.array([65504, 65519.99, 65520, 65536, 1e10, 2.0 ** -24, 2.0 ** -25,
                        2.0 ** -25 * 1.0000001, 2.0 ** -26, 0.0, -0.0, np.inf, -np.inf],
                       dtype=np.float32)
    allv = np.concatenate([v, mid, up, dn, -mid, special])
    ours = oracle.f16_from_f32(allv)
    with np.errstate(over="ignore"):
        ref = allv.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


# -- bfloat16 ---------------------------------------------------------------------
def _torch_bf16_bits(v32):
    return torch.from_numpy(np.ascontiguousarray(v32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def test_bf16_from_f32_matches_torch_including_ties():
    rng = np.random.default_rng(2)
    e = rng.uniform(-140, 128, 200000)
    v = (rng.choice([-1.0, 1.0], e.size) * 2.0 ** e).astype(np.float32)
    bits = rng.integers(0, 2 ** 16, 50000).astype(np.uint32)
    ties = ((bits << 16) | 0x8000).view(np.float32)           # exact half-way cases
    finite = np.isfinite(ties)
    allv = np.concatenate([v, ties[finite], np.array([0.0, -0.0, np.inf, -np.inf,
                                                      3.3895314e38], np.float32)])
    assert np.array_equal(oracle.bf16_from_f32(allv), _torch_bf16_bits(allv))


def test_bf16_from_f64_single_rounding():
    rng = np.random.default_rng(3)
    # doubles that are exactly binary32 must agree with the binary32 route
    v32 = rng.standard_normal(50000).astype(np.float32)
    assert np.array_equal(oracle.bf16_from_f64(v32.astype(np.float64)), _torch_bf16_bits(v32))
    # just above / below an exact tie must round away from the tie, which a
    # double -> float -> bf16 route gets wrong when the offset is below 2^-24
    a = oracle.f32_from_bf16(np.arange(0x3F80, 0x4000, dtype=np.uint16)).astype(np.float64)
    b = oracle.f32_from_bf16(np.arange(0x3F81, 0x4001, dtype=np.uint16)).astype(np.float64)
    mid = (a + b) / 2
    assert np.array_equal(oracle.bf16_from_f64(mid + 2.0 ** -40),
                          np.arange(0x3F81, 0x4001, dtype=np.uint16))
    assert np.array_equal(oracle.bf16_from_f64(mid - 2.0 ** -40),
                          np.arange(0x3F80, 0x4000, dtype=np.uint16))
    # exact ties go to the even neighbour
    even = np.where(np.arange(0x3F80, 0x4000) % 2 == 0, np.arange(0x3F80, 0x4000),
                    np.arange(0x3F81, 0x4001)).astype(np.uint16)
    assert np.array_equal(oracle.bf16_from_f64(mid), even)


# -- q8_0 ----------------------------------------------------------------------------
def _decode_q8(blocks, n, k):
    """Independent decode through numpy's own float16/int8 views."""
    b = blocks.reshape(n, k // 32, 34)
    d = np.ascontiguousarray(b[:, :, :2]).view(np.float16)[..., 0].astype(np.float64)
    q = np.ascontiguousarray(b[:, :, 2:]).view(np.int8).astype(np.float64)
    return d, q


def test_q8_integer_grid_is_exact():
    rng = np.random.default_rng(4)
    n, k = 40, 256
    nb = k // 32
    # fp16-exact normal scales
    d16 = rng.integers(0x1000, 0x2C00, (n, nb)).astype(np.uint16)
    d = d16.view(np.float16).astype(np.float64)
    q = rng.integers(-127, 128, (n, nb, 32))
    q[:, :, 5] = np.where(rng.random((n, nb)) < 0.5, 127, -127)   # force max |q|
    w = (d[:, :, None] * q).reshape(n, k).astype(np.float32)
    assert np.array_equal(w.astype(np.float64), (d[:, :, None] * q).reshape(n, k))
    blocks = oracle.quantize(oracle.Q8_0, w)
    dd, qq = _decode_q8(blocks, n, k)
    assert np.array_equal(np.ascontiguousarray(blocks.reshape(n, nb, 34)[:, :, :2]).view(np.uint16)[..., 0], d16)
    assert np.array_equal(qq, q)
    assert np.array_equal(oracle.dequantize(oracle.Q8_0, blocks, n, k), w.astype(np.float64))


def test_q8_error_bound_and_scale_rule():
    rng = np.random.default_rng(5)
    n, k = 64, 512
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    w[3, 40:72] = 0.0                       # an all-zero block
    blocks = oracle.quantize(oracle.Q8_0, w)
    d, q = _decode_q8(blocks, n, k)
    wb = w.reshape(n, k // 32, 32).astype(np.float64)
    # scale = fp16(max|w| / 127) through numpy's conversion
    amax = np.abs(w.reshape(n, k // 32, 32)).max(-1)
    ref_d = (amax / np.float32(127)).astype(np.float32).astype(np.float16).astype(np.float64)
    assert np.array_equal(d, ref_d)
    err = np.abs(wb - d[..., None] * q)
    assert np.all(err <= d[..., None] / 2 * (1 + 2.0 ** -20))
    nz = amax > 0
    assert np.all(np.abs(q).max(-1)[nz] == 127)
    assert np.all(q[~nz] == 0) and np.all(d[~nz] == 0)
    deq = oracle.dequantize(oracle.Q8_0, blocks, n, k)
    assert np.array_equal(deq, (d[..., None] * q).reshape(n, k))


def test_format_density_golden():
    g = json.load(open(os.path.join(GOLDEN, "format_density.json")))
    assert oracle.block_bytes(oracle.Q8_0) * 8 / g["q8_0"]["weights_per_block"] == \
        g["q8_0"]["bits_per_weight"]
    ex = g["lora_bytes_per_layer"]["example"]
    rng = np.random.default_rng(0)
    A = rng.standard_normal((ex["r"], ex["n"])).astype(np.float32)
    B = rng.standard_normal((ex["m"], ex["r"])).astype(np.float32)
    assert A.nbytes + B.nbytes == ex["bytes"]


# -- q4_sm ---------------------------------------------------------------------------
def _decode_q4(blocks, n, k):
    b = blocks.reshape(n, k // 32, 20)
    d = np.ascontiguousarray(b[:, :, 0:2]).view(np.float16)[..., 0].astype(np.float64)
    m = np.ascontiguousarray(b[:, :, 2:4]).view(np.float16)[..., 0].astype(np.float64)
    nib = b[:, :, 4:]
    q = np.empty((n, k // 32, 32), np.float64)
    q[:, :, 0::2] = nib & 0x0F
    q[:, :, 1::2] = nib >> 4
    return d, m, q


def test_q4_integer_grid_is_exact():
    rng = np.random.default_rng(6)
    n, k = 24, 320
    nb = k // 32
    m = -rng.integers(1, 64, (n, nb)) * 2.0 ** -7          # fp16-exact mins
    d = rng.integers(1, 2048, (n, nb)) * 2.0 ** -14        # fp16-exact scales
    q = rng.integers(0, 16, (n, nb, 32))
    q[:, :, 0], q[:, :, 31] = 0, 15
    w64 = m[..., None] + d[..., None] * q
    w = w64.reshape(n, k).astype(np.float32)
    assert np.array_equal(w.astype(np.float64), w64.reshape(n, k))
    blocks = oracle.quantize(oracle.Q4_SM, w)
    dd, mm, qq = _decode_q4(blocks, n, k)
    assert np.array_equal(dd, d) and np.array_equal(mm, m) and np.array_equal(qq, q)
    assert np.array_equal(oracle.dequantize(oracle.Q4_SM, blocks, n, k), w64.reshape(n, k))


def test_q4_error_bound_and_range():
    rng = np.random.default_rng(7)
    n, k = 48, 640
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    w[5, 64:96] = np.float32(0.0078125)      # constant block: d = 0, w = m exactly
    blocks = oracle.quantize(oracle.Q4_SM, w)
    d, m, q = _decode_q4(blocks, n, k)
    wb = w.reshape(n, k // 32, 32).astype(np.float64)
    lo = wb.min(-1)
    ref_m = lo.astype(np.float32).astype(np.float16).astype(np.float64)
    assert np.array_equal(m, ref_m)
    recon = d[..., None] * q + m[..., None]
    slack = np.abs(lo - m)[..., None]
    assert np.all(np.abs(wb - recon) <= d[..., None] / 2 * (1 + 2.0 ** -20) + slack)
    nonconst = wb.max(-1) > wb.min(-1)
    assert np.all(q.max(-1)[nonconst] == 15) and np.all(q.min(-1)[nonconst] == 0)
    assert d[5, 2] == 0 and np.all(q[5, 2] == 0) and np.all(recon[5, 2] == wb[5, 2])


def test_quantize_rejects_bad_shapes():
    with pytest.raises(ValueError):
        oracle.quantize(oracle.Q8_0, np.zeros((4, 48), np.float32))
    with pytest.raises(ValueError):
        oracle.quantize(7, np.zeros((4, 64), np.float32))
