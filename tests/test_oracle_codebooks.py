"""Pins of the oracle's codebook and constant variants (oracle/codebooks.py)
against definitions that do not go through it: exact rational arithmetic,
the textbook E2M1 value list, the pinned NF4 oracle, grid round trips, the
storage figures printed on the pages, and the pages' claim that NF4 beats
INT4 and FP4 on normally distributed weights."""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import codebooks as cb

GOLDEN = {}
with open(os.path.join(os.path.dirname(__file__), "golden", "storage_figures.txt")) as f:
    for line in f:
        line = line.split("#")[0].split()
        if line:
            GOLDEN[line[0]] = (float(line[1]), float(line[2]))


def _f32_half_ulp(v: float) -> Fraction:
    x = np.float32(v)
    return Fraction(float(np.spacing(np.abs(x)))) / 2


def test_int4_levels_are_uniform_over_the_unit_interval():
    """Each level is the fp32 nearest to the exact (2k - 15)/15, the ends are
    exactly -1 and +1, and the table is antisymmetric (no zero level)."""
    lv = cb.int4_levels()
    assert lv.dtype == np.float32 and lv.size == 16
    for k in range(16):
        exact = Fraction(2 * k - 15, 15)
        assert abs(Fraction(float(lv[k])) - exact) <= _f32_half_ulp(float(lv[k]))
    assert lv[0] == -1.0 and lv[15] == 1.0
    np.testing.assert_array_equal(lv, -lv[::-1])
    assert np.all(np.diff(lv.astype(np.float64)) > 0)
    assert not np.any(lv == 0)


def test_e2m1_values_are_the_textbook_list():
    """E2M1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 for patterns 0..7, and the
    sign bit negates them."""
    want = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert [cb.e2m1_value(b) for b in range(8)] == want
    assert [cb.e2m1_value(8 + b) for b in range(8)] == [-v for v in want]
    assert np.signbit(cb.e2m1_value(8))


def test_fp4_levels():
    """The E2M1 values over 6, ascending, +0 at code 7 and -0 at code 8."""
    lv = cb.fp4_levels()
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    want = sorted([-m / 6 for m in mags[1:]]) + [0.0, 0.0] + [m / 6 for m in mags[1:]]
    np.testing.assert_array_equal(lv, np.array(want, np.float32))
    assert not np.signbit(lv[7]) and np.signbit(lv[8])
    assert lv[0] == -1.0 and lv[15] == 1.0
    assert np.all(np.diff(lv.astype(np.float64)) >= 0)


def _nearest_exact(x: float, lv) -> int:
    """Nearest level by exact rational distance, ties to the lower index."""
    fx = Fraction(float(x))
    best, bd = 0, None
    for j, l in enumerate(lv):
        d = abs(fx - Fraction(float(l)))
        if bd is None or d < bd:
            best, bd = j, d
    return best


@pytest.mark.parametrize("name", cb.CODEBOOKS)
def test_encode_matches_exact_nearest_level(name):
    """At every midpoint between adjacent levels, its fp32 neighbours, and a
    grid over [-1, 1], the code is the exact nearest level (ties lower)."""
    lv = cb.levels(name)
    xs = list(np.linspace(-1, 1, 401, dtype=np.float32))
    # values next to zero, where INT4's two middle levels compete
    tiny = np.array([1e-45, 1e-38, 1e-30, 2.0 ** -29, 1e-8], np.float32)
    xs += list(tiny) + list(-tiny) + [np.float32(0.0), np.float32(-0.0)]
    for j in range(15):
        mid = (float(lv[j]) + float(lv[j + 1])) / 2
        m32 = np.float32(mid)
        xs += [m32, np.nextafter(m32, np.float32(-2)), np.nextafter(m32, np.float32(2))]
    xs = np.array(xs, np.float32)
    got = cb.encode_levels(xs, lv)
    for x, c in zip(xs, got):
        assert c == _nearest_exact(x, lv), (name, float(x), int(c))


def test_fp4_never_produces_negative_zero():
    """Ties between +0 and -0 go to the lower index: values near zero, of
    either sign, take code 7 (+0)."""
    x = np.array([0.0, -0.0, 1e-30, -1e-30, 0.04, -0.04], np.float32)
    assert list(cb.encode_levels(x, cb.fp4_levels())) == [7] * 6


def test_nf4_variant_is_the_nf4_oracle():
    """With the NF4 table and double quantization, the generic quantizer
    equals the pinned NF4 oracle bit for bit."""
    rng = np.random.default_rng(3)
    W = rng.standard_normal((96, 640)).astype(np.float32)
    W[5, :64] = 0
    a = oracle.quantize(W)
    b = cb.quantize_q4(W, "nf4", True)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    np.testing.assert_array_equal(cb.dequantize_q4(b[0], b[1], b[2], 96, 640, "nf4", True),
                                  oracle.dequantize(a[0], a[1], a[2], 96, 640))
    np.testing.assert_array_equal(cb.encode_levels(W / 4, oracle.nf4_levels()),
                                  oracle.encode(W / 4))


def _grid_weight(name, rng, N, K, scale_pow):
    """Blocks whose values are levels times a power of two, each block holding
    a +-1 level (so its absmax is exactly that power of two)."""
    lv = cb.levels(name)
    allowed = [j for j in range(16) if not (name == "fp4" and j == 8)]
    codes = rng.choice(allowed, size=(N * K // 64, 64))
    codes[:, 0] = rng.choice([0, 15], size=codes.shape[0])
    c = np.float32(2.0) ** rng.integers(-scale_pow, scale_pow, size=codes.shape[0]).astype(np.float32)
    W = (lv[codes] * c[:, None]).astype(np.float32).reshape(N, K)
    return W, codes.reshape(-1), c


@pytest.mark.parametrize("name", cb.CODEBOOKS)
def test_grid_round_trip(name):
    """Weights on the codebook's grid: quantization recovers the codes and the
    exact absmax; without double quantization, dequantization gives back
    bf16(W) exactly."""
    rng = np.random.default_rng(11)
    W, codes, c = _grid_weight(name, rng, 8, 256, 6)
    packed, e, cst, absmax = cb.quantize_q4(W, name, False)
    assert e is None
    np.testing.assert_array_equal(absmax, c)
    np.testing.assert_array_equal(cst, c)
    got = np.empty(packed.size * 2, np.uint8)
    got[0::2], got[1::2] = packed & 15, packed >> 4
    np.testing.assert_array_equal(got, codes)
    np.testing.assert_array_equal(cb.dequantize_q4(packed, None, cst, 8, 256, name, False),
                                  oracle.bf16_rne_bits(W))


@pytest.mark.parametrize("name", cb.CODEBOOKS)
def test_double_quantized_constants_bound(name):
    """With double quantization each constant is within half a step d_g of the
    absmax (the same second level for every codebook), and e, d do not depend
    on the codebook."""
    rng = np.random.default_rng(5)
    W = (rng.standard_normal((64, 1024)) * rng.uniform(0.1, 3, size=(64, 1))).astype(np.float32)
    _, e, d, absmax = cb.quantize_q4(W, name, True)
    c_hat = e.astype(np.float64) * np.repeat(d, 256)[:e.size]
    assert np.all(np.abs(c_hat - absmax) <= np.repeat(d, 256)[:e.size] * (0.5 + 1e-6))
    _, e0, d0, _ = oracle.quantize(W)
    np.testing.assert_array_equal(e, e0)
    np.testing.assert_array_equal(d, d0)


def test_storage_without_double_quantization():
    """Printed figures: 0.5 bits of constants per parameter without double
    quantization, about 0.127 with it (list item (3) of "DL0087 QLoRA")."""
    N, K = 8192, 8192
    no_dq = 8 * cb.storage_bytes_q4(N, K, False) / (N * K) - 4
    dq = 8 * cb.storage_bytes_q4(N, K, True) / (N * K) - 4
    v, tol = GOLDEN["metadata_bits_no_dq"]
    assert abs(no_dq - v) <= tol
    v, tol = GOLDEN["metadata_bits_dq"]
    assert abs(dq - v) <= tol
    assert cb.storage_bytes_q4(N, K, True) == oracle.storage_bytes(N, K)


def test_code_entropy_closed_forms():
    all16 = np.arange(16, dtype=np.uint8)
    assert cb.code_entropy_bits(all16[0::2] | (all16[1::2] << 4)) == pytest.approx(4.0)
    assert cb.code_entropy_bits(np.full(10, 0x77, np.uint8)) == 0.0
    assert cb.code_entropy_bits(np.full(10, 0x70, np.uint8)) == pytest.approx(1.0)


def test_nf4_is_best_on_normal_weights():
    """On Gaussian blocks NF4 uses its codes most evenly (highest entropy) and
    has the lowest squared error of the three types ("4-bit NormalFloat" of
    "QLoRA: Finetuning 65B Models on a Single GPU": optimal for normally
    distributed data, better than INT4 and FP4); double quantization adds
    less than 0.5% to the error of the fp32 constants."""
    rng = np.random.default_rng(0)
    N, K = 256, 4096
    W = rng.standard_normal((N, K)).astype(np.float32)
    H, mse = {}, {}
    for name in cb.CODEBOOKS:
        for dq in (True, False):
            codes, e, d, _ = cb.quantize_q4(W, name, dq)
            Wh = oracle.bf16_bits_to_f64(cb.dequantize_q4(codes, e, d, N, K, name, dq))
            mse[name, dq] = float(((Wh - W) ** 2).mean())
            H[name] = cb.code_entropy_bits(codes)
    assert H["nf4"] > H["fp4"] > H["int4"]
    assert H["nf4"] > 3.85
    for dq in (True, False):
        assert mse["nf4", dq] < mse["int4", dq] and mse["nf4", dq] < mse["fp4", dq]
    for name in cb.CODEBOOKS:
        assert mse[name, False] <= mse[name, True] < 1.005 * mse[name, False]
