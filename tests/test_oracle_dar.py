"""Pins of the oracle's dequantize-add-requantize (DAR) merge ("We propose a
content-addressed overlay system", "Quantized-Base Numerical Analysis"; "Deep
Technical Design", "The Pathology of Dequantize-Add-Requantize (DAR) Error"):

* with deltas whose products and sums are exact in float32, the merge equals the
  quantiser applied to the exact merged weight (so the recipe adds the right
  terms, at the right rows and columns, with the right signs and scales);
* requantising an unchanged q8_0 base gives back its bytes wherever a block's
  largest code is 127;
* the page's scale-recomputation shift: one outlier raising a block's maximum
  tenfold collapses the other codes of that block toward zero;
* merging is not associative: Q(Q(W + A) + B) differs from Q(W + A + B), and
  both differ from the exact W + A + B that the dual path computes.
"""
import numpy as np
import pytest

import oracle
from oracle import Lora, Sparse

Q8, Q4, Q4K = oracle.Q8_0, oracle.Q4_SM, oracle.Q4_K


def _grid_factors(rng, n, k, r):
    """LoRA factors on a coarse power-of-two grid: every product and partial sum
    of B A is exact in float32."""
    A = (rng.integers(-2, 3, (r, k)) * 2.0 ** -8).astype(np.float32)
    B = (rng.integers(-2, 3, (n, r)) * 2.0 ** -8).astype(np.float32)
    return A, B


@pytest.mark.parametrize("qtype,n,k", [(Q8, 40, 256), (Q4, 24, 320), (Q4K, 16, 512)])
def test_merge_equals_quantiser_of_exact_merged_weight(qtype, n, k):
    rng = np.random.default_rng(90 + qtype)
    blocks = oracle.quantize(qtype, (rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    A1, B1 = _grid_factors(rng, n, k, 4)
    A2, B2 = _grid_factors(rng, n, k, 3)
    rp = np.zeros(n + 1, np.uint32)
    cols = []
    for r in range(n):
        c = np.sort(rng.choice(k, 5, replace=False)).astype(np.uint32)
        cols.append(c)
        rp[r + 1] = rp[r] + 5
    col = np.concatenate(cols)
    val = (rng.integers(-8, 9, col.size) * 2.0 ** -10).astype(np.float16).view(np.uint16)
    ads = [Lora(A1, B1, 0.5), Sparse(rp, col, val, -2.0), Lora(A2, B2, 1.0)]
    S = np.zeros((n, k))
    S[np.repeat(np.arange(n), 5), col.astype(np.int64)] = val.view(np.float16).astype(np.float64)
    exact = (oracle.dequantize(qtype, blocks, n, k) + 0.5 * (B1.astype(np.float64) @ A1)
             - 2.0 * S + (B2.astype(np.float64) @ A2))
    w32 = exact.astype(np.float32)
    assert np.array_equal(w32.astype(np.float64), exact)          # the merged weight is exact in float32
    got = oracle.requantize(qtype, blocks, n, k, ads)
    assert np.array_equal(got, oracle.quantize(qtype, w32))
    # a transposed or mis-signed delta would give other codes
    assert not np.array_equal(got, oracle.quantize(qtype, (exact + 4.0 * S).astype(np.float32)))


def test_requantising_an_unchanged_q8_base_keeps_its_bytes():
    rng = np.random.default_rng(91)
    n, k = 64, 512
    blocks = oracle.quantize(Q8, (rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    again = oracle.requantize(Q8, blocks, n, k)
    b = blocks.reshape(n, k // 32, 34)
    full = np.abs(b[:, :, 2:].view(np.int8)).max(-1) == 127
    assert full.mean() > 0.9
    assert np.array_equal(again.reshape(n, k // 32, 34)[full], b[full])


def test_scale_recomputation_shift_collapses_the_block():
    """One outlier ten times the block maximum: the new scale is about ten times
    the old, and the block's other codes shrink by the same factor."""
    rng = np.random.default_rng(92)
    k = 64
    w = (rng.standard_normal((1, k)) * 0.02).astype(np.float32)
    blocks = oracle.quantize(Q8, w)
    b0 = blocks.reshape(2, 34)
    d0 = float(b0[0, :2].view(np.float16)[0])
    q0 = b0[0, 2:].view(np.int8).astype(int)
    amax = float(np.abs(oracle.dequantize(Q8, blocks, 1, k)[0, :32]).max())
    j = int(np.argmin(np.abs(q0)))                                   # a small weight gets the outlier
    rp = np.array([0, 1], np.uint32)
    val = np.array([np.float16(10 * amax)]).view(np.uint16)
    merged = oracle.requantize(Q8, blocks, 1, k, [Sparse(rp, np.array([j], np.uint32), val, 1.0)])
    b1 = merged.reshape(2, 34)
    d1 = float(b1[0, :2].view(np.float16)[0])
    q1 = b1[0, 2:].view(np.int8).astype(int)
    assert 9.0 < d1 / d0 < 11.5
    others = np.arange(32) != j
    assert np.all(np.abs(q1[others]) <= np.ceil(np.abs(q0[others]) * d0 / d1) + 1)
    assert (q1[others] == 0).sum() > (q0[others] == 0).sum()         # codes collapse to zero
    assert np.array_equal(b1[1], b0[1])                              # the other block is untouched


def test_chained_merges_are_not_associative():
    rng = np.random.default_rng(93)
    n, k = 128, 512
    W = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    base = oracle.quantize(Q8, W)
    A = Lora((rng.standard_normal((16, k)) / np.sqrt(k)).astype(np.float32),
             (rng.standard_normal((n, 16)) * 0.01).astype(np.float32), 1.0)
    B = Lora((rng.standard_normal((8, k)) / np.sqrt(k)).astype(np.float32),
             (rng.standard_normal((n, 8)) * 0.01).astype(np.float32), 1.0)
    once = oracle.requantize(Q8, base, n, k, [A, B])
    chain = oracle.requantize(Q8, oracle.requantize(Q8, base, n, k, [A]), n, k, [B])
    chain_ba = oracle.requantize(Q8, oracle.requantize(Q8, base, n, k, [B]), n, k, [A])
    assert not np.array_equal(once, chain) and not np.array_equal(chain, chain_ba)
    exact = (oracle.dequantize(Q8, base, n, k) + A.B.astype(np.float64) @ A.A + B.B.astype(np.float64) @ B.A)
    err = lambda blk: np.linalg.norm(oracle.dequantize(Q8, blk, n, k) - exact) / np.linalg.norm(exact)
    assert 0 < err(once) < err(chain)
    # the dual path reaches the exact merged weight's product
    x = rng.standard_normal((1, k))
    y = oracle.linear_dual(Q8, base, n, k, x, [A, B])
    assert np.max(np.abs(y - x @ exact.T)) <= 1e-12 * np.abs(y).max()
