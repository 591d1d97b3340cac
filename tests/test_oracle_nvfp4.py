"""Pins for the NVFP4 codec oracle (CPU only).

Each pin checks the oracle against something other than itself: the E2M1 value
grid and E4M3 closed forms, hand-worked blocks (tests/golden/nvfp4_blocks.txt),
an exact-rational nearest-value search, idempotence, and library bfloat16
rounding.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import nvfp4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "nvfp4_blocks.txt")


# ---------------------------------------------------------------- tables
def test_e2m1_grid():
    # The E2M1 value grid {0, 0.5, 1, 1.5, 2, 3, 4, 6} and its negatives.
    assert list(nvfp4.E2M1_MAGS) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    for c in range(16):
        v = nvfp4.e2m1_value(c)
        assert abs(v) == [0, 0.5, 1, 1.5, 2, 3, 4, 6][c & 7]
        assert (np.signbit(v) if c & 8 else not np.signbit(v)) or v == 0


def test_e2m1_grid_roundtrip():
    # A block whose amax is 6 has scale 1.0 at g = 1, so every grid value
    # must encode to its own code.
    for c in range(16):
        x = np.zeros(16)
        x[0] = 6.0
        x[1] = nvfp4.e2m1_value(c)
        if c == 8:
            x[1] = -0.0
        codes, sc = nvfp4.quantize(x[None, :], 1.0)
        assert sc[0, 0] == 0x38
        assert codes[0, 1] == c, c


def test_e4m3_closed_forms():
    assert nvfp4.e4m3_value(0x38) == 1.0
    assert nvfp4.e4m3_value(0x39) == 1.125
    assert nvfp4.e4m3_value(0x7E) == 448.0
    assert nvfp4.e4m3_value(0x08) == 2.0 ** -6
    assert nvfp4.e4m3_value(0x07) == 7 * 2.0 ** -9
    assert nvfp4.e4m3_value(0x01) == 2.0 ** -9
    assert np.isnan(nvfp4.e4m3_value(0x7F))
    assert nvfp4.e4m3_value(0xB8) == -1.0
    t = nvfp4.E4M3_POS
    assert len(t) == 127 and np.all(np.diff(t) > 0)
    # Between 2^-6 and 448 the spacing within a binade is 1/8 of its base.
    for e in range(-6, 9):
        seg = t[(t >= 2.0 ** e) & (t < 2.0 ** (e + 1))]
        assert np.allclose(np.diff(seg), 2.0 ** e / 8)


def test_e4m3_values_round_to_themselves():
    # amax = 6 * v with g = 1 gives amax/(6g) = v exactly.
    x = np.zeros((127, 16))
    x[:, 0] = 6.0 * nvfp4.E4M3_POS
    _, sc = nvfp4.quantize(x, 1.0)
    assert list(sc[:, 0]) == list(range(127))


# ---------------------------------------------------------------- golden blocks
def _golden():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        name, g, vals, sc, packed = [p.strip() for p in line.split("|")]
        rows.append((name, float(g), [float(v) for v in vals.split()],
                     int(sc, 16), [int(b, 16) for b in packed.split()]))
    return rows


@pytest.mark.parametrize("row", _golden(), ids=lambda r: r[0])
def test_golden_block(row):
    name, g, vals, sc, packed = row
    assert len(vals) == 16 and len(packed) == 8
    q, s = nvfp4.quantize_packed(np.array(vals)[None, :], g)
    assert s[0, 0] == sc, name
    assert list(q[0]) == packed, name


def test_golden_blocks_fp32_input():
    # The same blocks given as FP32 (as the weight path sees them).
    for name, g, vals, sc, packed in _golden():
        q, s = nvfp4.quantize_packed(np.array(vals, dtype=np.float32)[None, :], g)
        assert s[0, 0] == sc and list(q[0]) == packed, name


# ---------------------------------------------------------------- exact rational brute force
def _nearest(q: Fraction, grid) -> int:
    best, best_d = None, None
    for c, v in enumerate(grid):
        d = abs(Fraction(v) - q)
        if best is None or d < best_d or (d == best_d and c % 2 == 0):
            best, best_d = c, d
    return best


def _brute_block(x, g):
    g = Fraction(float(np.float32(g)))
    xs = [Fraction(float(v)) for v in x]
    amax = max(abs(v) for v in xs)
    s_code = 0 if amax == 0 else _nearest(amax / (6 * g), nvfp4.E4M3_POS)
    s = Fraction(float(nvfp4.E4M3_POS[s_code]))
    codes = []
    for v, xv in zip(xs, x):
        mag = 0 if (s == 0 or v == 0) else _nearest(abs(v) / (s * g), nvfp4.E2M1_MAGS)
        codes.append(mag | (8 if np.signbit(xv) else 0))
    return codes, s_code


def _tie_blocks(rng, n):
    """Blocks built to sit exactly on rounding midpoints."""
    out = []
    e4_mid = (nvfp4.E4M3_POS[:-1] + nvfp4.E4M3_POS[1:]) / 2
    e2_mid = (nvfp4.E2M1_MAGS[:-1] + nvfp4.E2M1_MAGS[1:]) / 2
    for _ in range(n):
        g = float(np.float32(2.0 ** rng.integers(-8, 4)))
        x = np.zeros(16)
        if rng.random() < 0.5:
            x[0] = 6 * g * rng.choice(e4_mid[8:])      # scale tie
        else:
            x[0] = 6 * g * rng.choice(nvfp4.E4M3_POS[8:])
        _, sc = nvfp4.quantize(x[None, :], g)
        s = nvfp4.E4M3_POS[sc[0, 0]]
        x[1:] = rng.choice(np.concatenate([e2_mid, nvfp4.E2M1_MAGS]), 15) * s * g
        x[1:] *= rng.choice([-1.0, 1.0], 15)
        out.append((x, g))
    return out


def test_bruteforce_random_blocks():
    rng = np.random.default_rng(7)
    cases = []
    for _ in range(300):
        scale = 2.0 ** rng.integers(-12, 10)
        x = (rng.standard_normal(16) * scale).astype(np.float32).astype(np.float64)
        if rng.random() < 0.2:
            x[rng.integers(0, 16)] *= 50
        g = np.float32(np.abs(x).max() / 2688 * rng.choice([0.5, 1.0, 1.0, 3.0, 700.0]))
        cases.append((x, g))
    cases += _tie_blocks(rng, 300)
    for x, g in cases:
        codes, sc = nvfp4.quantize(x[None, :], g)
        bc, bs = _brute_block(x, g)
        assert sc[0, 0] == bs, (x, g)
        assert list(codes[0]) == bc, (x, g)


def test_bruteforce_bf16_inputs():
    # bf16 inputs with the tensor's own global scale, as for activations.
    gen = torch.Generator().manual_seed(3)
    x = (torch.randn(8, 64, generator=gen) * 3).to(torch.bfloat16).float().numpy().astype(np.float64)
    x[0, 5] = 120.0
    g = nvfp4.global_scale(x)
    codes, sc = nvfp4.quantize(x, g)
    for r in range(x.shape[0]):
        for b in range(4):
            bc, bs = _brute_block(x[r, 16 * b:16 * b + 16], g)
            assert sc[r, b] == bs and list(codes[r, 16 * b:16 * b + 16]) == bc


# ---------------------------------------------------------------- global scale
def _nearest_fp32(q: Fraction) -> np.float32:
    c = np.float32(float(q))
    cands = [np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))]
    best = min(cands, key=lambda v: (abs(Fraction(float(v)) - q),
                                     int(np.array(v).view(np.uint32)) & 1))
    return np.float32(best)


def test_global_scale_correctly_rounded():
    rng = np.random.default_rng(11)
    for _ in range(500):
        amax = np.float32(rng.random() * 2.0 ** rng.integers(-20, 20))
        x = np.array([amax, -amax / 3], dtype=np.float32)
        g = nvfp4.global_scale(x)
        assert g == _nearest_fp32(Fraction(float(amax)) / 2688), amax
    assert nvfp4.global_scale(np.zeros(4)) == 0
    assert nvfp4.global_scale(np.array([-2688.0])) == 1.0


# ---------------------------------------------------------------- idempotence
def test_idempotence_normal_scales():
    # quantize(dequantize(q, s, g), g) == (q, s) when every scale is zero or a
    # normal E4M3 value: the block's largest code is then 6 again.
    rng = np.random.default_rng(5)
    g = np.float32(2.0 ** -3)       # power of two: dequantised values stay exact
    x = rng.standard_normal((64, 128)) * 5
    x[3, :16] = 0.0
    codes, sc = nvfp4.quantize(x, g)
    assert np.all((sc == 0) | (sc >= 0x08))
    xh = nvfp4.dequantize(codes, sc, g)
    c2, s2 = nvfp4.quantize(xh, g)
    assert np.array_equal(s2, sc)
    # -0 may turn into +0 on the way back only when the value was a signed zero;
    # compare magnitudes and the sign of non-zero values.
    nz = xh != 0
    assert np.array_equal(c2[nz], codes[nz])
    assert np.array_equal(c2[~nz] & 7, codes[~nz] & 7)


def test_idempotence_fails_for_subnormal_scale():
    # Documented counterexample: amax = 6 * 1.6 * 2^-9, g = 1 gives scale 2^-8
    # (code 0x02) and element 4.8 -> 4 (code 6), i.e. the value 2^-6.  Its
    # block maximum is 4, not 6, so re-encoding picks scale 2^-9 (2^-6/6 is
    # nearest to 1 * 2^-9) and saturates the element at 6 * 2^-9.
    x = np.zeros((1, 16))
    x[0, 0] = 6 * 1.6 * 2.0 ** -9
    codes, sc = nvfp4.quantize(x, 1.0)
    assert sc[0, 0] == 0x02 and codes[0, 0] == 6
    xh = nvfp4.dequantize(codes, sc, 1.0)
    c2, s2 = nvfp4.quantize(xh, 1.0)
    assert s2[0, 0] == 0x01 and c2[0, 0] == 7
    assert nvfp4.dequantize(c2, s2, 1.0)[0, 0] == 6 * 2.0 ** -9 != xh[0, 0]


# ---------------------------------------------------------------- packing
def test_pack_unpack():
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 16, (5, 32)).astype(np.uint8)
    p = nvfp4.pack_codes(codes)
    assert p.shape == (5, 16)
    assert p[0, 0] == (codes[0, 0] | (codes[0, 1] << 4))
    assert np.array_equal(nvfp4.unpack_codes(p), codes)


def test_dequantize_values():
    codes = np.array([[7, 15, 1, 9] + [0] * 12], dtype=np.uint8)
    sc = np.array([[0x39]], dtype=np.uint8)
    v = nvfp4.dequantize(codes, sc, 0.5)
    assert list(v[0, :4]) == [6 * 1.125 * 0.5, -6 * 1.125 * 0.5, 0.5 * 1.125 * 0.5,
                              -0.5 * 1.125 * 0.5]


def test_zero_global_scale_all_zero_tensor():
    x = np.zeros((2, 32))
    x[1, 3] = -0.0
    g = nvfp4.global_scale(x)
    codes, sc = nvfp4.quantize(x, g)
    assert g == 0 and not sc.any()
    assert codes[1, 3] == 8 and codes.sum() == 8


# ---------------------------------------------------------------- bfloat16
def test_round_to_bf16_matches_torch():
    gen = torch.Generator().manual_seed(9)
    v = torch.randn(100000, generator=gen) * torch.exp(torch.randn(100000, generator=gen) * 8)
    v[:10] = torch.tensor([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3e-39, -7e-40, 255.5, 1e30, -1e-30])
    ref = v.to(torch.bfloat16).to(torch.float64).numpy()
    got = nvfp4.round_to_bf16(v.to(torch.float64).numpy())
    assert np.array_equal(got, ref)


def test_near_tie_mask_flags_ties():
    g = 1.0
    x = np.zeros((1, 16))
    x[0, :3] = [6.0, 2.5, 2.3]          # 2.5 is an exact E2M1 midpoint
    ef, bf = nvfp4.near_tie_mask(x, g)
    assert ef[0, 1] and not ef[0, 2] and not bf[0, 0]
    x[0, 0] = 7.125                      # scale tie (see golden B5)
    ef, bf = nvfp4.near_tie_mask(x, g)
    assert bf[0, 0]


# ---------------------------------------------------------------- near ties (exact)
def _near_tie_brute(row, g, rel, abs_tol):
    """Flags of one 16-element block with exact rationals: the block is
    flagged when its amax lies within rel * b + abs_tol of a boundary b = 6 g m
    (m halfway between neighbouring E4M3 values); an element when |x| lies that
    close to a boundary t s g (t halfway between neighbouring E2M1
    magnitudes, s the block's scale)."""
    g = Fraction(float(np.float32(g)))
    rel, abs_tol = Fraction(rel), Fraction(abs_tol)
    vals = [Fraction(float(v)) for v in row]
    amax = max(abs(v) for v in vals)
    e4 = [Fraction(float(v)) for v in nvfp4.E4M3_POS]
    e2 = [Fraction(float(v)) for v in nvfp4.E2M1_MAGS]

    def close(a, b):
        return abs(a - b) <= rel * b + abs_tol

    block = any(close(amax, 6 * g * (e4[i] + e4[i + 1]) / 2) for i in range(len(e4) - 1))
    s = Fraction(float(nvfp4.E4M3_POS[nvfp4.block_scales(np.asarray(row)[None, :], float(g))[0, 0]]))
    elem = [s > 0 and any(close(abs(v), s * g * (e2[i] + e2[i + 1]) / 2) for i in range(7))
            for v in vals]
    return elem, block


def _placed_blocks(rng, g, rel, abs_tol):
    """Blocks with elements and maxima put at chosen distances from their
    rounding boundaries: inside the band (should flag), just outside it (should
    not), exactly on it, and random values in between."""
    out = []
    e4m = nvfp4._midpoints(nvfp4.E4M3_POS)
    e2m = nvfp4._midpoints(nvfp4.E2M1_MAGS)
    for f in (0.0, 0.5, -0.5, 0.9, -0.9, 1.2, -1.2, 3.0, -3.0):
        for _ in range(6):
            s_code = int(rng.integers(0x20, 0x60))
            s = nvfp4.E4M3_POS[s_code]
            row = rng.uniform(-6, 6, 16) * s * g
            row[0] = 6 * s * g                             # amax sits at the scale itself
            t = e2m[int(rng.integers(0, 7))] * s * g
            row[1 + int(rng.integers(0, 15))] = t * (1 + f * rel) + (f * abs_tol if abs_tol else 0.0)
            out.append(row)
            b = 6 * g * e4m[int(rng.integers(0x18, 0x70))]
            row2 = rng.uniform(-1, 1, 16) * b / 2
            row2[int(rng.integers(0, 16))] = b * (1 + f * rel) + (f * abs_tol if abs_tol else 0.0)
            out.append(row2)
    return np.array(out)


@pytest.mark.parametrize("rel,abs_tol", [(2.0 ** -12, 0.0), (2.0 ** -12, 2.0 ** -16), (2.0 ** -8, 0.0)])
def test_near_tie_mask_against_fractions(rel, abs_tol):
    """near_tie_mask equals the exact-rational definition on random blocks
    and on blocks built around the boundaries, so that neither a missed nor an
    over-broad flag (which would quietly loosen the parity bar) gets through."""
    rng = np.random.default_rng(int(1 / rel) + int(abs_tol * 1e6))
    g = np.float32(0.0371)
    rnd = rng.standard_normal((120, 16)) * np.exp(rng.uniform(-3, 3, (120, 1)))
    x = np.concatenate([rnd, _placed_blocks(rng, float(g), rel, abs_tol)])
    ef, bf = nvfp4.near_tie_mask(x, g, rel, abs_tol=abs_tol)
    n_flag = 0
    for r in range(x.shape[0]):
        elem, block = _near_tie_brute(x[r], g, rel, abs_tol)
        assert bool(bf[r, 0]) == block, (r, x[r])
        assert list(ef[r].astype(bool)) == elem, (r, x[r])
        n_flag += sum(elem)
    # the placed values land on both sides of the band
    assert 0 < n_flag < x.size // 4


def test_quantize_at_product_ties_against_fractions():
    """The oracle's decisions next to thresholds g * M that lie exactly
    halfway between two floats, against the exact-rational definition."""
    import ties
    x, gs = ties.product_tie_blocks(np.random.default_rng(31))
    e4 = [Fraction(float(v)) for v in nvfp4.E4M3_POS]
    e2 = [Fraction(float(v)) for v in nvfp4.E2M1_MAGS]

    def nearest(v, grid):          # ties to the even index, saturating
        best = min(range(len(grid)), key=lambda i: (abs(grid[i] - v), i % 2))
        return best

    for r in range(x.shape[0]):
        g = Fraction(float(np.float32(gs[r])))
        codes, sc = nvfp4.quantize(x[r:r + 1], gs[r])
        amax = max(abs(Fraction(float(v))) for v in x[r])
        s_idx = nearest(amax / (6 * g), e4) if amax > 0 else 0
        assert sc[0, 0] == s_idx, r
        s = e4[s_idx]
        for k in range(16):
            v = Fraction(float(x[r, k]))
            m = nearest(abs(v) / (s * g), e2) if s > 0 else 0
            assert codes[0, k] == (m | (8 if x[r, k] < 0 or (x[r, k] == 0 and np.signbit(x[r, k])) else 0)), (r, k)
