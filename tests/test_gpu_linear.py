"""GPU parity of the dense NVFP4 linear layer (nvfp4_linear, nvfp4_linear_w4a16)
against oracle/linear.py, through the C ABI.

Bar: the activation codes and scales are exact (the quantisation is tested
bit for bit elsewhere), so the only error of the FP32 output is the FP32
accumulation of K exact products: |y - y_ref| <= K * 2^-23 * (|x_hat| |W_hat|^T)
elementwise.  The bf16 output must be the round-to-nearest-even of the FP32
output of the same call, bit for bit.
"""
import numpy as np
import pytest
import torch

from nvfp4_block_scaled_03_amd import ops
from oracle import linear as olin
from oracle import nvfp4 as onv

from parity import bf16_bits, device, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return device()


def _weight(dev, N, K, seed):
    g = torch.Generator(device=dev).manual_seed(seed)
    w = 0.02 * torch.randn(N, K, generator=g, device=dev)
    w[0, 0] = 1.0   # the global maximum, known without scanning W
    return w


def _x(dev, M, K, seed):
    g = torch.Generator(device=dev).manual_seed(seed)
    x = torch.randn(M, K, generator=g, device=dev)
    x[:, ::97] *= 20.0   # outlier channels
    return x.to(torch.bfloat16)


def _bound(x_hat, w_hat, K):
    return K * 2.0 ** -23 * (np.abs(x_hat) @ np.abs(w_hat).T) + 1e-30


def _check(dev, x, lw, variant, ref, bound):
    y32 = ops.linear(x, lw, variant, out_dtype=torch.float32)
    y16 = ops.linear(x, lw, variant, out_dtype=torch.bfloat16)
    err = np.abs(to_np(y32).astype(np.float64) - ref)
    assert (err <= bound).all(), f"max excess {float((err - bound).max())}"
    assert np.array_equal(bf16_bits(y16), bf16_bits(y32.to(torch.bfloat16)))


@pytest.mark.parametrize("variant", ["w4a4", "w4a16"])
@pytest.mark.parametrize("M", [1, 5, 13, 16, 17, 64, 256, 300, 1024, 4096])
def test_linear_full(dev, M, variant):
    N, K = 1024, 768
    w = _weight(dev, N, K, 11)
    lw = ops.quantize_linear_weight(w)
    x = _x(dev, M, K, 100 + M)
    xf = to_np(x).astype(np.float64)
    wc, ws, gw = olin.quantize_weight(to_np(w))
    w_hat = onv.dequantize(wc, ws, gw)
    if variant == "w4a4":
        ref = olin.linear_w4a4(xf, wc, ws, gw)
        g = onv.global_scale(xf)
        x_hat = onv.dequantize(*onv.quantize(xf, g), g)
    else:
        ref = olin.linear_w4a16(xf, wc, ws, gw)
        x_hat = xf
    _check(dev, x, lw, variant, ref, _bound(x_hat, w_hat, K))


@pytest.mark.parametrize("variant", ["w4a4", "w4a16"])
@pytest.mark.parametrize("M", [16, 1024])
def test_linear_pages_shape_sampled(dev, M, variant):
    """The pages' per-GEMM shape (gate_up N = 34816, K = 5120): 8 rows x 64
    columns of the output against the oracle, which quantises only those
    weight rows (the weight's global scale is known: its maximum is planted)."""
    N, K = 34816, 5120
    w = _weight(dev, N, K, 12)
    lw = ops.quantize_linear_weight(w)
    x = _x(dev, M, K, 7)
    rng = np.random.default_rng(M)
    rows = np.sort(rng.choice(M, size=min(8, M), replace=False))
    cols = np.sort(np.concatenate([[0], rng.choice(np.arange(1, N), size=63, replace=False)]))
    xf = to_np(x).astype(np.float64)
    gw = np.float32(1.0 / 2688.0)
    w_rows = to_np(w[torch.from_numpy(cols).to(dev)])
    wc, ws = onv.quantize(w_rows, gw)
    w_hat = onv.dequantize(wc, ws, gw)
    if variant == "w4a4":
        g = onv.global_scale(xf)
        x_hat = onv.dequantize(*onv.quantize(xf[rows], g), g)
    else:
        x_hat = xf[rows]
    ref = x_hat @ w_hat.T
    y32 = to_np(ops.linear(x, lw, variant, out_dtype=torch.float32))[np.ix_(rows, cols)]
    err = np.abs(y32.astype(np.float64) - ref)
    assert (err <= _bound(x_hat, w_hat, K)).all()


@pytest.mark.parametrize("variant", ["w4a4", "w4a16"])
@pytest.mark.parametrize("M,K", [(1, 128), (3, 256), (7, 384), (2, 640)])
def test_linear_few_rows_short_k(dev, M, K, variant):
    """Few rows with 1 to 5 chunks of K, so that some wavefronts of the
    split-K kernel get no chunk at all and the others uneven shares."""
    N = 256
    w = _weight(dev, N, K, 13)
    lw = ops.quantize_linear_weight(w)
    x = _x(dev, M, K, 200 + K)
    xf = to_np(x).astype(np.float64)
    wc, ws, gw = olin.quantize_weight(to_np(w))
    w_hat = onv.dequantize(wc, ws, gw)
    if variant == "w4a4":
        ref = olin.linear_w4a4(xf, wc, ws, gw)
        g = onv.global_scale(xf)
        x_hat = onv.dequantize(*onv.quantize(xf, g), g)
    else:
        ref = olin.linear_w4a16(xf, wc, ws, gw)
        x_hat = xf
    _check(dev, x, lw, variant, ref, _bound(x_hat, w_hat, K))
