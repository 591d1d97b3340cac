"""GPU parity of the OCP MXFP4 path (mxfp4_quantize, mxfp4_prep_weights,
mxfp4_linear on the scaled FP4 matrix instruction) against oracle/mxfp4.py,
through the C ABI.

Bar: codes and exponent bytes bit for bit.  The linear map's only error is
the FP32 accumulation of K exact products (E2M1 x E2M1 x 2^k is exact in
FP32 at these magnitudes): |y - y_ref| <= K * 2^-23 * (|x_hat| |W_hat|^T)
elementwise; the bf16 output is the round-to-nearest-even of the FP32 output
of the same call, bit for bit.
"""
import numpy as np
import pytest
import torch

from nvfp4_block_scaled_03_amd import ops
from oracle import mxfp4 as omx
from oracle import nvfp4 as onv

from parity import bf16_bits, device, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return device()


def _special_rows(K):
    """Blocks the rule must get right: zeros, grid values and every rounding
    midpoint (ties), saturation, negative zero, tiny and huge magnitudes."""
    rows = np.zeros((6, K), dtype=np.float32)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 0.1, 7.0])
    rows[1, :32] = np.tile(mids, 2) * np.where(np.arange(32) % 3 == 0, -1, 1)
    rows[1, 32:64] = -0.0
    rows[1, 40] = 6.5
    rows[2, :] = 2.0 ** -130 * (1 + (np.arange(K) % 7))     # subnormal float32
    rows[3, :] = 3.0e38 * np.sin(np.arange(K))              # largest exponents
    rows[4, :] = 2.0 ** np.float32(np.arange(K) % 40 - 20)  # one power of two per element
    rows[5, ::32] = 1.0                                       # one element per block
    return rows


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("rows,K", [(1, 32), (7, 96), (300, 2048), (4099, 640)])
def test_quantize_bit_exact(dev, dtype, rows, K):
    g = torch.Generator(device=dev).manual_seed(rows + K)
    x = torch.randn(rows, K, generator=g, device=dev) * torch.exp(
        4 * torch.randn(rows, 1, generator=g, device=dev))
    if K >= 64:
        sp = torch.from_numpy(_special_rows(K)).to(dev)
        n = min(rows, sp.shape[0])
        x[:n] = sp[:n]
    x = x.to(dtype)
    q, ex = ops.mx_quantize(x)
    codes, exps = omx.quantize(to_np(x).astype(np.float64))
    assert np.array_equal(to_np(ex), exps)
    assert np.array_equal(to_np(q), onv.pack_codes(codes))


def test_quantize_strided(dev):
    g = torch.Generator(device=dev).manual_seed(9)
    base = torch.randn(50, 200, generator=g, device=dev).to(torch.bfloat16)
    x = base[:, 8:168]   # ldx = 200, K = 160
    q, ex = ops.mx_quantize(x)
    codes, exps = omx.quantize(to_np(x).astype(np.float64))
    assert np.array_equal(to_np(ex), exps) and np.array_equal(to_np(q), onv.pack_codes(codes))


def _weight(dev, N, K, seed):
    g = torch.Generator(device=dev).manual_seed(seed)
    w = 0.02 * torch.randn(N, K, generator=g, device=dev)
    w[:, ::131] *= 30.0
    return w


def _x(dev, M, K, seed):
    g = torch.Generator(device=dev).manual_seed(seed)
    x = torch.randn(M, K, generator=g, device=dev)
    x[:, ::97] *= 20.0   # outlier channels
    return x.to(torch.bfloat16)


def _bound(x_hat, w_hat, K):
    return K * 2.0 ** -23 * (np.abs(x_hat) @ np.abs(w_hat).T) + 1e-30


def _check(x, lw, ref, bound):
    y32 = ops.mx_linear(x, lw, out_dtype=torch.float32)
    y16 = ops.mx_linear(x, lw, out_dtype=torch.bfloat16)
    err = np.abs(to_np(y32).astype(np.float64) - ref)
    assert (err <= bound).all(), f"max excess {float((err - bound).max())}"
    assert np.array_equal(bf16_bits(y16), bf16_bits(y32.to(torch.bfloat16)))


@pytest.mark.parametrize("M", [1, 5, 16, 17, 64, 65, 256, 300, 1024])
def test_linear(dev, M):
    """N = 384 leaves the last workgroup half empty; M spans the three row
    tilings (16, 64, 128 rows) with ragged tails."""
    N, K = 384, 1152
    w = _weight(dev, N, K, 21)
    wf = to_np(w).astype(np.float64)
    wc, we = omx.quantize(wf)
    # weight codes from the oracle, through the library's prep
    lw = ops.prepare_mx_weight(torch.from_numpy(onv.pack_codes(wc)).to(dev), torch.from_numpy(we).to(dev))
    x = _x(dev, M, K, 200 + M)
    xf = to_np(x).astype(np.float64)
    ref = omx.linear(xf, wc, we)
    x_hat = omx.dequantize(*omx.quantize(xf))
    _check(x, lw, ref, _bound(x_hat, omx.dequantize(wc, we), K))


@pytest.mark.parametrize("M,N,K", [(3, 128, 128), (20, 256, 384), (40, 128, 640), (100, 128, 256),
                                   (129, 256, 384), (200, 128, 640)])
def test_linear_short_k(dev, M, N, K):
    """K of 1 to 5 chunks of 128 (wavefronts of the split-K kernels with no
    chunk or uneven shares; ring kernels with fewer chunks than ring slots)
    and both row tilings of the ring kernel (128 and 256 rows) with ragged
    tails."""
    w = _weight(dev, N, K, 23)
    wc, we = omx.quantize(to_np(w).astype(np.float64))
    lw = ops.prepare_mx_weight(torch.from_numpy(onv.pack_codes(wc)).to(dev), torch.from_numpy(we).to(dev))
    x = _x(dev, M, K, 4)
    xf = to_np(x).astype(np.float64)
    ref = omx.linear(xf, wc, we)
    _check(x, lw, ref, _bound(omx.dequantize(*omx.quantize(xf)), omx.dequantize(wc, we), K))


def test_linear_gpu_quantised_weight(dev):
    """The weight quantised on the GPU gives the oracle's codes, so the same result."""
    N, K, M = 256, 512, 33
    w = _weight(dev, N, K, 22)
    lw = ops.quantize_mx_weight(w)
    wc, we = omx.quantize(to_np(w).astype(np.float64))
    x = _x(dev, M, K, 3)
    xf = to_np(x).astype(np.float64)
    ref = omx.linear(xf, wc, we)
    _check(x, lw, ref, _bound(omx.dequantize(*omx.quantize(xf)), omx.dequantize(wc, we), K))


@pytest.mark.parametrize("M", [16, 1024])
def test_linear_pages_shape_sampled(dev, M):
    """The per-GEMM shape of the dense sweep (N = 34816, K = 5120): 8 rows x
    64 columns against the oracle, which quantises only those weight rows."""
    N, K = 34816, 5120
    w = _weight(dev, N, K, 12)
    lw = ops.quantize_mx_weight(w)
    x = _x(dev, M, K, 7)
    rng = np.random.default_rng(M)
    rows = np.sort(rng.choice(M, size=min(8, M), replace=False))
    cols = np.sort(np.concatenate([[N - 1], rng.choice(N - 1, size=63, replace=False)]))
    xf = to_np(x).astype(np.float64)
    wc, we = omx.quantize(to_np(w[torch.from_numpy(cols).to(dev)]).astype(np.float64))
    x_hat = omx.dequantize(*omx.quantize(xf[rows]))
    w_hat = omx.dequantize(wc, we)
    ref = x_hat @ w_hat.T
    y32 = to_np(ops.mx_linear(x, lw, out_dtype=torch.float32))[np.ix_(rows, cols)]
    err = np.abs(y32.astype(np.float64) - ref)
    assert (err <= _bound(x_hat, w_hat, K)).all()


def test_linear_zero_rows(dev):
    lw = ops.quantize_mx_weight(_weight(dev, 128, 128, 1))
    y = ops.mx_linear(torch.empty(0, 128, dtype=torch.bfloat16, device=dev), lw)
    assert y.shape == (0, 128)
