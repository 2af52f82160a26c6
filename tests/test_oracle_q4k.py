"""Pins of the oracle's q4_K super-block format ("Deep Technical Design",
section 5: 256 weights in 8 sub-blocks of 32, a 6-bit scale and a 6-bit
minimum per sub-block, two fp16 super-scales, 4.5 bits per weight).

The page gives only that sentence; the byte layout and the quantiser are the
reading spelled out in oracle.c.  Each test checks the oracle against
something other than itself: the layout re-packed here with Python integers
(a 96-bit little-endian field of sixteen 6-bit codes), exact integer grids
that a correct quantiser must reproduce code for code, the error bound that
follows from the quantiser's rules, the page's bits per weight, and the dual
path's one-hot closed form.
"""
import json
import os

import numpy as np
import pytest

import oracle

Q4K = oracle.Q4_K
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def pack_superblock(d16: int, dmin16: int, sc, m, q) -> bytes:
    """Canonical 144 bytes from fp16 bit patterns, 8 scale codes, 8 min codes and
    256 nibbles, written from the layout's description."""
    field = 0
    for i, code in enumerate(list(sc) + list(m)):
        assert 0 <= code < 64
        field |= int(code) << (6 * i)
    out = d16.to_bytes(2, "little") + dmin16.to_bytes(2, "little") + field.to_bytes(12, "little")
    q = np.asarray(q, np.uint8).reshape(8, 32)
    for j in range(8):
        out += bytes(int(q[j, 2 * i]) | (int(q[j, 2 * i + 1]) << 4) for i in range(16))
    assert len(out) == 144
    return out


def unpack_superblock(blk: bytes):
    d = float(np.frombuffer(blk[0:2], np.float16)[0])
    dmin = float(np.frombuffer(blk[2:4], np.float16)[0])
    field = int.from_bytes(blk[4:16], "little")
    codes = [(field >> (6 * i)) & 63 for i in range(16)]
    nib = np.frombuffer(blk[16:144], np.uint8).reshape(8, 16)
    q = np.empty((8, 32), np.int64)
    q[:, 0::2] = nib & 0x0F
    q[:, 1::2] = nib >> 4
    return d, dmin, np.array(codes[:8]), np.array(codes[8:]), q


def test_density_matches_the_page():
    g = json.load(open(os.path.join(GOLDEN, "format_density.json")))["q4_K"]
    assert oracle.block_weights(Q4K) == g["weights_per_superblock"] == 256
    assert oracle.block_bytes(Q4K) * 8 / g["weights_per_superblock"] == g["bits_per_weight"]
    assert g["sub_blocks"] * 32 == g["weights_per_superblock"]


def test_dequantisation_follows_the_layout():
    rng = np.random.default_rng(70)
    n, nsb = 6, 3
    blocks = bytearray()
    expect = np.empty((n, nsb * 256), np.float64)
    for r in range(n):
        for s in range(nsb):
            d = np.float16(rng.uniform(1e-4, 3e-3))
            dmin = np.float16(rng.uniform(1e-4, 3e-3))
            sc = rng.integers(0, 64, 8)
            m = rng.integers(0, 64, 8)
            q = rng.integers(0, 16, 256)
            blocks += pack_superblock(int(d.view(np.uint16)), int(dmin.view(np.uint16)), sc, m, q)
            w = (float(d) * sc[:, None] * q.reshape(8, 32)) - float(dmin) * m[:, None]
            expect[r, s * 256:(s + 1) * 256] = w.reshape(-1)
    got = oracle.dequantize(Q4K, np.frombuffer(bytes(blocks), np.uint8), n, nsb * 256)
    assert np.array_equal(got, expect)


def test_code_bit_positions():
    # code i sits in bits 6i..6i+5 of the little-endian field: a single set code
    # lands on a byte and bit that can be written down by hand
    for i, code, byte, val in ((0, 1, 4, 0x01), (1, 1, 4, 0x40), (1, 4, 5, 0x01), (8, 63, 10, 0x3F),
                               (15, 32, 15, 0x80), (5, 3, 7, 0xC0)):
        sc = [0] * 8
        m = [0] * 8
        (sc if i < 8 else m)[i % 8] = code
        blk = pack_superblock(0, 0, sc, m, np.zeros(256))
        nz = {j: b for j, b in enumerate(blk[:16]) if b}
        assert nz == {byte: val}, (i, code, nz)
        d, dmin, sc2, m2, _ = unpack_superblock(blk)
        assert list(sc2) + list(m2) == sc + m


def test_integer_grid_is_reproduced_code_for_code():
    rng = np.random.default_rng(71)
    n, nsb = 10, 4
    d0, dmin0 = 2.0 ** -11, 2.0 ** -10                       # fp16-exact super-scales
    w = np.empty((n, nsb * 256), np.float32)
    expect = bytearray()
    for r in range(n):
        for s in range(nsb):
            sc = rng.integers(1, 64, 8)
            m = rng.integers(0, 64, 8)
            sc[rng.integers(0, 8)] = 63                      # the largest code is 63 ...
            m[rng.integers(0, 8)] = 63                       # ... for both super-scales
            q = rng.integers(0, 16, (8, 32))
            q[:, 3], q[:, 17] = 0, 15                        # each sub-block spans 0..15
            wb = d0 * sc[:, None] * q - dmin0 * m[:, None]   # exact in float32
            w[r, s * 256:(s + 1) * 256] = wb.reshape(-1)
            assert np.array_equal(w[r, s * 256:(s + 1) * 256].astype(np.float64), wb.reshape(-1))
            expect += pack_superblock(int(np.float16(d0).view(np.uint16)),
                                      int(np.float16(dmin0).view(np.uint16)), sc, m, q.reshape(-1))
    blocks = oracle.quantize(Q4K, w)
    assert blocks.tobytes() == bytes(expect)
    assert np.array_equal(oracle.dequantize(Q4K, blocks, n, nsb * 256), w.astype(np.float64))


@pytest.mark.parametrize("kind", ["normal", "positive", "negative", "mixed"])
def test_error_bound(kind):
    rng = np.random.default_rng(72)
    n, k = 16, 1024
    w = rng.standard_normal((n, k)) * 0.02
    if kind == "positive":
        w = np.abs(w) + 0.001
    elif kind == "negative":
        w = -np.abs(w) - 0.001
    elif kind == "mixed":
        w[0, :256] = 0.0                                     # an all-zero super-block
        w[1, 32:64] = 0.05                                   # a constant sub-block
        w[2, :] *= 1000.0                                    # large values
        w[3, :] *= 1e-4                                      # tiny values
    w = w.astype(np.float32)
    blocks = oracle.quantize(Q4K, w).reshape(n, k // 256, 144)
    deq = oracle.dequantize(Q4K, blocks, n, k).reshape(n, k // 256, 8, 32)
    wb = w.astype(np.float64).reshape(n, k // 256, 8, 32)
    for r in range(n):
        for s in range(k // 256):
            d, dmin, sc, m, q = unpack_superblock(blocks[r, s].tobytes())
            lo = np.minimum(0.0, wb[r, s].min(-1))
            span = (wb[r, s].max(-1) - lo) / 15.0
            D = d * sc
            # rounding to the step (D/2) and of the min code (dmin/2); the fp16
            # rounding of the super-scales (dd, dm: it can leave the widest
            # sub-block's step or offset short by 63 of them, which clips the
            # top by up to 15*63*dd); float32 slop
            dd = max(0.0, span.max() / 63 - d)
            dm = abs(-lo.min() / 63 - dmin)
            bound = D / 2 + dmin / 2 + 15 * 63 * dd + 63 * dm + np.abs(wb[r, s]).max(-1) * 2.0 ** -20
            err = np.abs(wb[r, s] - deq[r, s]).max(-1)
            assert np.all(err <= bound), (kind, r, s, err, bound)
            assert np.all(sc <= 63) and np.all(m <= 63)
            if kind == "positive":
                assert dmin == 0.0 and np.all(m == 0)           # min clamps at 0: no offset
    if kind == "mixed":
        assert np.all(deq[0, 0] == 0.0)
        assert not blocks[0, 0, :4].any()                       # d = dmin = 0


def test_one_hot_x_returns_dequantised_column():
    rng = np.random.default_rng(73)
    n, k = 40, 768
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    blocks = oracle.quantize(Q4K, w)
    W = oracle.dequantize(Q4K, blocks, n, k)
    for col in (0, 255, 256, 300, 767):
        x = np.zeros((1, k))
        x[0, col] = 1.0
        assert np.array_equal(oracle.linear_dual(Q4K, blocks, n, k, x)[0], W[:, col])


def test_rejects_k_not_a_multiple_of_256():
    with pytest.raises(ValueError):
        oracle.quantize(Q4K, np.zeros((4, 96), np.float32))
