"""Pins of the oracle's dual path, materialised path, JIT recipe and block
glue: closed forms (one-hot inputs, one-hot adapters), library routes (numpy /
torch dense products of the materialised weight), linearity, and the bf16
error bound between the JIT and dual paths."""
import numpy as np
import pytest
import torch

import oracle
from oracle import Lora

Q8, Q4 = oracle.Q8_0, oracle.Q4_SM


def _rand_linear(rng, n, k, qtype=Q8, ranks=(8,), scales=(2.0,)):
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    blocks = oracle.quantize(qtype, w)
    ads = [Lora((rng.standard_normal((r, k)) / np.sqrt(k)).astype(np.float32),
                (rng.standard_normal((n, r)) * 0.01).astype(np.float32), s)
           for r, s in zip(ranks, scales)]
    return blocks, ads


def _dense(qtype, blocks, n, k, ads):
    """Library route: materialise W + sum s B A in float64 with numpy matmul."""
    W = oracle.dequantize(qtype, blocks, n, k)
    for a in ads:
        W = W + a.scale * (a.B.astype(np.float64) @ a.A.astype(np.float64))
    return W


@pytest.mark.parametrize("qtype", [Q8, Q4])
def test_one_hot_x_returns_dequantised_column(qtype):
    rng = np.random.default_rng(10)
    n, k = 96, 160
    blocks, _ = _rand_linear(rng, n, k, qtype)
    W = oracle.dequantize(qtype, blocks, n, k)
    for col in (0, 31, 32, 159):
        x = np.zeros((1, k))
        x[0, col] = 1.0
        y = oracle.linear_dual(qtype, blocks, n, k, x)
        assert np.array_equal(y[0], W[:, col])


def test_block_indicator_x_gives_scale_times_code_sum():
    rng = np.random.default_rng(11)
    n, k = 64, 128
    blocks, _ = _rand_linear(rng, n, k)
    b = blocks.reshape(n, k // 32, 34)
    d = np.ascontiguousarray(b[:, 2, :2]).view(np.float16)[:, 0].astype(np.float64)
    qsum = np.ascontiguousarray(b[:, 2, 2:]).view(np.int8).astype(np.int64).sum(-1)
    x = np.zeros((1, k))
    x[0, 64:96] = 1.0
    y = oracle.linear_dual(Q8, blocks, n, k, x)
    assert np.array_equal(y[0], d * qsum)


@pytest.mark.parametrize("qtype,n,k,batch", [(Q8, 160, 256, 1), (Q8, 33, 96, 3),
                                             (Q4, 96, 320, 2), (Q4, 64, 64, 8)])
def test_dual_matches_dense_library_route(qtype, n, k, batch):
    rng = np.random.default_rng(12 + n)
    blocks, ads = _rand_linear(rng, n, k, qtype, ranks=(8, 3), scales=(2.0, -0.75))
    x = rng.standard_normal((batch, k))
    y = oracle.linear_dual(qtype, blocks, n, k, x, ads)
    ref = x @ _dense(qtype, blocks, n, k, ads).T
    assert np.max(np.abs(y - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))
    ym = oracle.linear_materialised(qtype, blocks, n, k, x, ads)
    assert np.max(np.abs(ym - y)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


def test_one_hot_adapter_changes_one_output_by_s_x():
    rng = np.random.default_rng(13)
    n, k = 64, 96
    blocks, _ = _rand_linear(rng, n, k)
    x = rng.standard_normal((1, k))
    i, j, s = 17, 45, 1.5
    A = np.zeros((1, k), np.float32)
    A[0, j] = 1
    B = np.zeros((n, 1), np.float32)
    B[i, 0] = 1
    y0 = oracle.linear_dual(Q8, blocks, n, k, x)
    y1 = oracle.linear_dual(Q8, blocks, n, k, x, [Lora(A, B, s)])
    diff = y1 - y0
    assert np.all(np.delete(diff[0], i) == 0)
    assert diff[0, i] == pytest.approx(s * x[0, j], rel=1e-15, abs=0)


def test_identity_adapter_adds_scaled_prefix():
    rng = np.random.default_rng(14)
    n, k, r, s = 64, 96, 8, 0.5
    blocks, _ = _rand_linear(rng, n, k)
    A = np.zeros((r, k), np.float32)
    A[:, :r] = np.eye(r)
    B = np.zeros((n, r), np.float32)
    B[:r] = np.eye(r)
    x = rng.standard_normal((1, k))
    d = oracle.linear_dual(Q8, blocks, n, k, x, [Lora(A, B, s)]) - oracle.linear_dual(Q8, blocks, n, k, x)
    np.testing.assert_allclose(d[0, :r], s * x[0, :r], rtol=1e-15, atol=1e-15)
    assert np.all(d[0, r:] == 0)


def test_zero_adapters_and_zero_scale_equal_base():
    rng = np.random.default_rng(15)
    n, k = 48, 128
    blocks, ads = _rand_linear(rng, n, k)
    x = rng.standard_normal((1, k))
    y0 = oracle.linear_dual(Q8, blocks, n, k, x)
    assert np.array_equal(oracle.linear_dual(Q8, blocks, n, k, x, []), y0)
    z = Lora(ads[0].A, ads[0].B, 0.0)
    assert np.array_equal(oracle.linear_dual(Q8, blocks, n, k, x, [z]), y0)


def test_linearity_in_scale_and_order_independence():
    rng = np.random.default_rng(16)
    n, k = 80, 192
    blocks, ads = _rand_linear(rng, n, k, ranks=(16, 64), scales=(1.0, 0.5))
    x = rng.standard_normal((1, k))
    y0 = oracle.linear_dual(Q8, blocks, n, k, x)
    a = ads[0]
    d1 = oracle.linear_dual(Q8, blocks, n, k, x, [Lora(a.A, a.B, 1.0)]) - y0
    d3 = oracle.linear_dual(Q8, blocks, n, k, x, [Lora(a.A, a.B, 3.0)]) - y0
    np.testing.assert_allclose(d3, 3 * d1, rtol=1e-10, atol=1e-13)
    yab = oracle.linear_dual(Q8, blocks, n, k, x, ads)
    yba = oracle.linear_dual(Q8, blocks, n, k, x, ads[::-1])
    np.testing.assert_allclose(yab, yba, rtol=1e-12, atol=1e-14)


def test_row_subset_and_batch_rows_are_independent():
    rng = np.random.default_rng(17)
    n, k = 130, 224
    blocks, ads = _rand_linear(rng, n, k, ranks=(4,), scales=(1.0,))
    x = rng.standard_normal((3, k))
    full = oracle.linear_dual(Q8, blocks, n, k, x, ads)
    rows = np.array([129, 0, 64, 7])
    assert np.array_equal(oracle.linear_dual(Q8, blocks, n, k, x, ads, rows=rows), full[:, rows])
    for b in range(3):
        assert np.array_equal(oracle.linear_dual(Q8, blocks, n, k, x[b:b + 1], ads)[0], full[b])


def test_bad_rows_rejected():
    rng = np.random.default_rng(18)
    blocks, _ = _rand_linear(rng, 8, 32)
    with pytest.raises(ValueError):
        oracle.linear_dual(Q8, blocks, 8, 32, np.zeros((1, 32)), rows=[8])


# -- JIT recipe ----------------------------------------------------------------------
def _bf16_bits_torch(a32):
    return torch.from_numpy(np.ascontiguousarray(a32, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def test_jit_zero_adapters_is_bf16_of_dequant():
    rng = np.random.default_rng(20)
    n, k = 64, 256
    blocks, _ = _rand_linear(rng, n, k)
    W = oracle.dequantize(Q8, blocks, n, k).astype(np.float32)   # exact for q8_0
    weff = oracle.jit_weff(Q8, blocks, n, k, [])
    assert np.array_equal(weff, _bf16_bits_torch(W))
    # one-hot bf16 rows of X pick columns of weff exactly
    X = np.zeros((3, k), np.float32)
    X[0, 5] = X[1, 100] = X[2, 255] = 1.0
    Y = oracle.gemm_bf16(_bf16_bits_torch(X), weff)
    wf = oracle.f32_from_bf16(weff).astype(np.float64)
    assert np.array_equal(Y, np.stack([wf[:, 5], wf[:, 100], wf[:, 255]]))


def test_jit_matches_torch_route():
    rng = np.random.default_rng(21)
    n, k, m = 96, 192, 16
    blocks, ads = _rand_linear(rng, n, k, ranks=(16, 8), scales=(1.0, 0.5))
    W32 = torch.from_numpy(oracle.dequantize(Q8, blocks, n, k)).float()
    acc = W32.double()
    for a in ads:
        sB = (torch.from_numpy(a.B) * a.scale).to(torch.bfloat16).double()
        Ab = torch.from_numpy(a.A).to(torch.bfloat16).double()
        acc = acc + sB @ Ab
    weff = oracle.jit_weff(Q8, blocks, n, k, ads)
    wf = oracle.f32_from_bf16(weff).astype(np.float64)
    # the reference sum has float64 rounding; the two bf16 roundings may differ
    # only where the exact sum sits within a few float64 ulps of a tie
    ulp = np.abs(wf) * 2.0 ** -7
    assert np.all(np.abs(wf - acc.numpy()) <= ulp / 2 * (1 + 1e-9) + 1e-300)
    X = rng.standard_normal((m, k)).astype(np.float32)
    Xb = _bf16_bits_torch(X)
    Y = oracle.gemm_bf16(Xb, weff)
    ref = oracle.f32_from_bf16(Xb).astype(np.float64) @ wf.T
    np.testing.assert_allclose(Y, ref, rtol=1e-12, atol=1e-12)


def test_jit_within_bf16_bound_of_dual_path():
    rng = np.random.default_rng(22)
    n, k, m = 128, 512, 8
    blocks, ads = _rand_linear(rng, n, k, ranks=(64,), scales=(1.0,))
    X = rng.standard_normal((m, k)).astype(np.float32)
    Xb = _bf16_bits_torch(X)
    Yj = oracle.linear_jit(Q8, blocks, n, k, Xb, ads)
    Yd = oracle.linear_dual(Q8, blocks, n, k, oracle.f32_from_bf16(Xb).astype(np.float64), ads)
    rel = np.linalg.norm(Yj - Yd) / np.linalg.norm(Yd)
    assert rel <= 2.0 ** -8
    assert rel > 1e-5    # the bf16 rounding of W_eff is really there


def test_jit_rows_subset():
    rng = np.random.default_rng(23)
    n, k = 70, 96
    blocks, ads = _rand_linear(rng, n, k)
    full = oracle.jit_weff(Q8, blocks, n, k, ads)
    rows = [69, 3, 40]
    assert np.array_equal(oracle.jit_weff(Q8, blocks, n, k, ads, rows=rows), full[rows])


# -- block glue ------------------------------------------------------------------------
def test_rms_closed_forms():
    v = np.full(64, 3.0)
    np.testing.assert_allclose(oracle.rms(v), 3.0 / np.sqrt(9.0 + 1e-6), rtol=1e-15)
    rng = np.random.default_rng(30)
    v = rng.standard_normal(1000) * 7
    out = oracle.rms(v)
    ms = np.mean(v * v)
    assert np.mean(out * out) == pytest.approx(ms / (ms + 1e-6), rel=1e-12)
    assert np.all(np.sign(out) == np.sign(v))


def _block_layers(rng, d, h, ranks=(4,), scales=(1.0,)):
    shapes = [(d, d)] * 4 + [(h, d), (h, d), (d, h)]
    layers = []
    for (n, k) in shapes:
        blocks, ads = _rand_linear(rng, n, k, Q8, ranks, scales)
        layers.append(oracle.Layer(Q8, blocks, n, k, ads))
    return layers


def _np_block(layers, x):
    Ws = [_dense(L.qtype, L.blocks, L.n, L.k, L.ads) for L in layers]

    def r(v):
        return v / np.sqrt(np.mean(v * v) + 1e-6)
    q, k, v = (W @ x for W in Ws[:3])
    a = Ws[3] @ r(q + k + v)
    g, u = Ws[4] @ r(a), Ws[5] @ r(a)
    return r(Ws[6] @ r(g + u))


def test_block_and_stack_match_library_route():
    rng = np.random.default_rng(31)
    d, h = 64, 96
    layers = _block_layers(rng, d, h, ranks=(4, 2), scales=(1.0, 0.5)) + \
        _block_layers(rng, d, h, ranks=(4, 2), scales=(1.0, 0.5))
    x0 = rng.standard_normal(d)
    out = oracle.block(layers[:7], x0)
    np.testing.assert_allclose(out, _np_block(layers[:7], x0), rtol=1e-11, atol=1e-12)
    ys = oracle.stack(layers, x0, 3)
    h_ = x0
    for t in range(3):
        h_ = _np_block(layers[7:], _np_block(layers[:7], h_))
        np.testing.assert_allclose(ys[t], h_, rtol=1e-10, atol=1e-11)


def test_block_rejects_mismatched_shapes():
    rng = np.random.default_rng(32)
    layers = _block_layers(rng, 64, 96)
    bad = list(layers)
    bad[6] = layers[4]
    with pytest.raises(ValueError):
        oracle.block(bad, np.zeros(64))
