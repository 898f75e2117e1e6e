"""Pins of the CPU oracle against things other than itself.

Each test names the fact it checks and where that fact comes from: a figure or
statement on the pages, exact rational arithmetic, an independent library
routine (scipy's normal quantile and CDF, torch's bf16 conversion and linear
layer, torch autograd) or finite differences.  None of these tests needs a GPU.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _next_f32(x, direction):
    return np.nextafter(np.float32(x), np.float32(direction), dtype=np.float32)


# ---------------------------------------------------------------------------
# The level table
# ---------------------------------------------------------------------------

def test_levels_invariants():
    """16 sorted distinct levels in [-1, 1], min -1, max +1, one exact zero."""
    q = oracle.nf4_levels()
    assert q.dtype == np.float32 and q.shape == (16,)
    assert np.all(np.diff(q) > 0)
    assert q[0] == -1.0 and q[15] == 1.0
    assert np.count_nonzero(q == 0) == 1 and q[7] == 0.0
    assert np.all(np.abs(q) <= 1.0)


def test_levels_quantile_inverse_matches_scipy():
    """The bisection inverse CDF agrees with scipy's ndtri (Cephes) to within
    the conditioning of the problem: a few ulps of p divided by the density."""
    for p in [0.5 + (j - 0.5) / 16 for j in range(1, 9)] + \
             [0.5 + (j - 0.5) / 14 for j in range(1, 8)] + [0.01, 0.3, 0.9999]:
        z = scipy.special.ndtri(p)
        tol = 4 * 2.0 ** -53 / scipy.stats.norm.pdf(z) + 4 * 2.0 ** -53 * abs(z)
        assert abs(oracle.normal_quantile(p) - z) <= tol, p


def test_levels_equal_probability_mass():
    """Each level covers an equal probability mass on its side of zero.

    Scaling the positive levels back by the normal quantile of their extreme
    bin centre, the scipy CDF of consecutive levels must step by exactly 1/16,
    and the negative side by 1/14; the innermost level sits half a bin from
    the median (probability-centre of its bin).
    """
    q = oracle.nf4_levels_f64()
    zpos = q[8:] * scipy.special.ndtri(1 - 1 / 32)
    zneg = q[:7] * -scipy.special.ndtri(1 / 28)
    cpos = scipy.stats.norm.cdf(zpos)
    cneg = scipy.stats.norm.cdf(zneg)
    np.testing.assert_allclose(np.diff(cpos), 1 / 16, atol=1e-13)
    np.testing.assert_allclose(np.diff(cneg), 1 / 14, atol=1e-13)
    assert abs(cpos[0] - (0.5 + 1 / 32)) < 1e-13
    assert abs(cneg[-1] - (0.5 - 1 / 28)) < 1e-13


def test_levels_fp32_rounding_is_robust():
    """fp32 rounding of each level is not a near-tie: each fp64 level is more
    than 1e-6 fp32-ulp away from a rounding midpoint, far beyond the ~1e-7 ulp
    error of an fp64 inverse CDF, so any accurate construction gives the same
    fp32 table."""
    q64 = oracle.nf4_levels_f64()
    q32 = oracle.nf4_levels().astype(np.float64)
    for a, b in zip(q64, q32):
        if a == 0.0:
            continue
        ulp = abs(float(np.spacing(np.float32(b))))
        assert abs(a - b) < (0.5 - 1e-6) * ulp


# ---------------------------------------------------------------------------
# bf16 rounding
# ---------------------------------------------------------------------------

def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * np.float32(3.0),
        (rng.integers(0, 1 << 31, 200000, dtype=np.uint32) | 0x8000).view(np.float32),  # exact ties
        (rng.integers(0, 1 << 24, 50000, dtype=np.uint32)).view(np.float32),            # denormals
        np.array([0.0, -0.0, 1.0, -1.0, 3.3895314e38, -3.3895314e38], np.float32),
    ])
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle.bf16_rne_bits(x), ref)


# ---------------------------------------------------------------------------
# Encoding
# ---------------------------------------------------------------------------

def _exact_nearest(x):
    q = [Fraction(float(v)) for v in oracle.nf4_levels()]
    fx = Fraction(float(x))
    dist = [abs(fx - v) for v in q]
    return dist.index(min(dist))   # first minimum: lower index on ties


def _interesting_values():
    q = oracle.nf4_levels()
    vals = [0.0, -0.0, 1.0, -1.0, 1e-45, -1e-45, 1e-38, -3e-39]
    for a, b in zip(q[:-1], q[1:]):
        m = (np.float64(a) + np.float64(b)) / 2       # exact in float64
        m32 = np.float32(m)
        for v in (m32, _next_f32(m32, 2), _next_f32(m32, -2)):
            vals += [v, _next_f32(v, 2), _next_f32(v, -2)]
    vals += list(q) + [_next_f32(v, 2) for v in q] + [_next_f32(v, -2) for v in q]
    return np.clip(np.array(vals, dtype=np.float32), -1, 1)


def test_encode_matches_exact_bruteforce():
    """Nearest level by exact rational distances, first minimum on ties."""
    rng = np.random.default_rng(11)
    x = np.concatenate([_interesting_values(),
                        rng.uniform(-1, 1, 3000).astype(np.float32)])
    got = oracle.encode(x)
    for xi, gi in zip(x, got):
        assert int(gi) == _exact_nearest(xi), (xi, gi)


def test_encode_true_ties_go_to_lower_index():
    q = oracle.nf4_levels()
    ties = 0
    for j in range(15):
        m = (np.float64(q[j]) + np.float64(q[j + 1])) / 2
        if np.float64(np.float32(m)) == m:
            ties += 1
            assert oracle.encode(np.array([m], np.float32))[0] == j
    assert ties >= 1    # the table has exactly representable midpoints


def test_code_boundaries_are_exact_midpoint_crossings():
    """boundary_j is the first float32 strictly above the exact midpoint
    between levels j-1 and j (exact rational check), and encode steps there."""
    q = oracle.nf4_levels()
    b = oracle.code_boundaries()
    assert np.all(np.diff(b) > 0)
    for j in range(1, 16):
        mid = (Fraction(float(q[j - 1])) + Fraction(float(q[j]))) / 2
        bj = b[j - 1]
        assert Fraction(float(bj)) > mid
        assert Fraction(float(_next_f32(bj, -2))) <= mid
        assert oracle.encode(np.array([bj]))[0] == j
        assert oracle.encode(np.array([_next_f32(bj, -2)]))[0] == j - 1


def test_encode_monotone_dense_and_near_boundaries():
    """encode is a non-decreasing step function: dense samples plus every
    float32 within 4096 ulps of each boundary agree with the boundary rule."""
    b = oracle.code_boundaries()
    rng = np.random.default_rng(3)
    xs = [np.sort(rng.uniform(-1, 1, 1 << 20).astype(np.float32))]
    for bj in b:
        u = np.array([bj], np.float32).view(np.int32)[0]
        if bj > 0:
            pats = np.arange(u - 4096, u + 4096, dtype=np.int32)
        else:
            pats = np.arange(u + 4096, u - 4096, -1, dtype=np.int32)
        xs.append(pats.view(np.float32))
    x = np.concatenate(xs)
    expect = np.searchsorted(b, x, side="right")
    np.testing.assert_array_equal(oracle.encode(x), expect)
    srt = np.sort(x)
    assert np.all(np.diff(oracle.encode(srt).astype(int)) >= 0)


# ---------------------------------------------------------------------------
# Quantize / dequantize round trip, double quantization
# ---------------------------------------------------------------------------

def _grid_weight(rng, N, K):
    """A weight whose exact quantization is known by construction.

    Codes are random with one +-1 code per block; d is a float32 with few
    mantissa bits so 255*d and e*d are exact; each group has a block with
    e = 255.  Then quantize must return exactly (codes, e, d) and dequantize
    must return bf16(W).
    """
    q = oracle.nf4_levels()
    nb = N * K // 64
    ng = (nb + 255) // 256
    codes = rng.integers(0, 16, size=(nb, 64)).astype(np.uint8)
    pos = rng.integers(0, 64, nb)
    codes[np.arange(nb), pos] = rng.choice([0, 15], nb)
    e = rng.integers(1, 256, nb).astype(np.uint8)
    for g in range(ng):
        e[g * 256 + rng.integers(0, min(256, nb - g * 256))] = 255
    d = (rng.integers(1, 1 << 12, ng).astype(np.float32)
         * np.float32(2.0) ** rng.integers(-20, -8, ng).astype(np.float32))
    chat = e.astype(np.float32) * np.repeat(d, 256)[:nb]
    W = (q[codes] * chat[:, None]).astype(np.float32).reshape(N, K)
    return W, codes.reshape(-1), e, d


@pytest.mark.parametrize("N,K", [(8, 64), (16, 1024), (5, 64 * 300), (3, 192)])
def test_quantize_dequantize_round_trip(N, K):
    rng = np.random.default_rng(N * 1000 + K)
    W, codes, e, d = _grid_weight(rng, N, K)
    packed, e2, d2, absmax = oracle.quantize(W)
    np.testing.assert_array_equal(oracle.unpack_codes(packed), codes)
    np.testing.assert_array_equal(e2, e)
    np.testing.assert_array_equal(d2.view(np.uint32), d.view(np.uint32))
    deq = oracle.dequantize(packed, e2, d2, N, K)
    np.testing.assert_array_equal(deq, oracle.bf16_rne_bits(W))


def test_nibble_order_low_nibble_is_even_element():
    W = np.zeros((1, 64), np.float32)
    W[0, 0] = 1.0     # code 15 at element 0
    W[0, 1] = -1.0    # code 0 at element 1
    packed, *_ = oracle.quantize(W)
    assert packed[0] == 0x0F
    assert np.all(packed[1:] == 0x77)


def test_zero_block_and_zero_group():
    W = np.zeros((2, 64 * 256), np.float32)
    W[1, 5] = 0.5
    packed, e, d, absmax = oracle.quantize(W)
    assert np.all(oracle.unpack_codes(packed)[:64 * 256] == 7)
    assert d[0] == 0 and d[1] > 0 and e[256] == 255 and np.all(e[:256] == 0)
    assert np.all(e[257:] == 0)
    W0 = np.zeros((1, 128), np.float32)
    packed, e, d, _ = oracle.quantize(W0)
    assert d[0] == 0 and np.all(e == 0) and np.all(packed == 0x77)
    assert np.all(oracle.dequantize(packed, e, d, 1, 128) == 0)


def test_double_quantization_error_bound_and_bruteforce():
    """|c_hat - c| <= d/2 (plus float32 rounding), the group max gets 255, and
    the 8-bit constant is the exact nearest integer to c/d except near ties."""
    rng = np.random.default_rng(5)
    W = workloads.draw_weight(rng, 64, 64 * 300)
    _, e, d, c = oracle.quantize(W)
    nb = c.size
    dg = np.repeat(d, 256)[:nb]
    chat = e.astype(np.float32) * dg
    assert np.all(np.abs(chat.astype(np.float64) - c) <= dg.astype(np.float64) * 0.5001)
    for g in range(d.size):
        sl = slice(g * 256, min(nb, g * 256 + 256))
        assert e[sl].max() == 255
        assert e[sl][np.argmax(c[sl])] == 255
    near_ties = 0
    for i in range(0, nb, 7):
        ratio = Fraction(float(c[i])) / Fraction(float(dg[i]))
        frac_part = ratio - math.floor(ratio)
        if abs(frac_part - Fraction(1, 2)) < Fraction(1, 1 << 15):
            near_ties += 1
            continue
        best = min(range(256), key=lambda k: abs(ratio - k))
        assert e[i] == best, (i, float(ratio), e[i])
    assert near_ties < 5


def test_dequantize_selection_consistent():
    rng = np.random.default_rng(9)
    W = workloads.draw_weight(rng, 12, 640)
    packed, e, d, _ = oracle.quantize(W)
    full = oracle.dequantize(packed, e, d, 12, 640)
    rows, cols = [0, 5, 11], [0, 63, 64, 639]
    np.testing.assert_array_equal(oracle.dequantize(packed, e, d, 12, 640, rows=rows, cols=cols),
                                  full[np.ix_(rows, cols)])


def test_quantization_error_small_for_gaussian_weights():
    """Sanity: NF4 of N(0, 0.02) weights reconstructs to within the level
    spacing (relative Frobenius error of a 4-bit code is a few percent)."""
    rng = np.random.default_rng(1)
    W = workloads.draw_weight(rng, 256, 1024)
    packed, e, d, _ = oracle.quantize(W)
    What = oracle.bf16_bits_to_f64(oracle.dequantize(packed, e, d, 256, 1024))
    rel = np.linalg.norm(What - W) / np.linalg.norm(W)
    assert 0.02 < rel < 0.15


# ---------------------------------------------------------------------------
# Storage cost (closed forms printed on the pages)
# ---------------------------------------------------------------------------

def _golden_storage():
    out = {}
    with open(os.path.join(GOLDEN, "storage_figures.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v, t = line.split()
                out[k] = (float(v), float(t))
    return out


def test_storage_matches_page_figures():
    g = _golden_storage()

    def check(key, value):
        v, tol = g[key]
        assert abs(value - v) <= tol + 1e-12, (key, value, v)

    N, K = 4096, 4096     # any shape with a whole number of DQ groups
    bits = oracle.bits_per_param(N, K)
    assert bits == 4 + 8 / 64 + 32 / (64 * 256) == 4.126953125
    payload = 8 * (N * K // 2) / (N * K)
    check("payload_bits", payload)
    check("dq_constant_bits", 8 * (N * K // 64) / (N * K))
    check("dq_scale_bits", bits - payload - 8 / 64)
    check("total_bits", bits)
    check("metadata_bits_no_dq", 32 / 64)
    check("metadata_bits_dq", bits - payload)
    saving = 32 / 64 - (bits - payload)
    check("dq_saving_bits", saving)
    check("dq_saving_gb_65b", 65e9 * saving / 8 / 1e9)
    check("frozen_gb_7b_bf16", 7e9 * 2 / 1e9)
    check("frozen_gb_7b_nf4", 7e9 * bits / 8 / 1e9)
    check("weights_gb_70b_16bit", 70e9 * 2 / 1e9)
    check("weights_gb_70b_4bit", 70e9 * payload / 8 / 1e9)


def test_storage_bytes_counts_short_last_group():
    assert oracle.storage_bytes(1, 64) == 32 + 1 + 4
    assert oracle.storage_bytes(1, 64 * 257) == 32 * 257 + 257 + 8


# ---------------------------------------------------------------------------
# The linear layer
# ---------------------------------------------------------------------------

def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_fwd_b_zero_is_plain_linear_torch():
    """B = 0 reproduces the quantized base exactly: torch's F.linear(X, W)."""
    rng = np.random.default_rng(2)
    X, W, A = _rand(rng, 5, 64), _rand(rng, 24, 64), _rand(rng, 64, 4)
    B = np.zeros((4, 24))
    Y, _ = oracle.linear_fwd_f64(X, W, A, B, 0.7)
    ref = torch.nn.functional.linear(torch.from_numpy(X), torch.from_numpy(W)).numpy()
    np.testing.assert_allclose(Y, ref, rtol=1e-13, atol=1e-13)
    Y0, _ = oracle.linear_fwd_f64(X, W, np.zeros((64, 0)), np.zeros((0, 24)), 1.0)
    np.testing.assert_allclose(Y0, ref, rtol=1e-13, atol=1e-13)


def test_fwd_equals_merged_weight_linear():
    """LoRA identity: X W^T + s (X A) B = F.linear(X, W + s (A B)^T)."""
    rng = np.random.default_rng(4)
    X, W, A, B = _rand(rng, 7, 128), _rand(rng, 40, 128), _rand(rng, 128, 6), _rand(rng, 6, 40)
    s = 0.375
    Y, T = oracle.linear_fwd_f64(X, W, A, B, s)
    merged = torch.from_numpy(W) + s * (torch.from_numpy(A) @ torch.from_numpy(B)).T
    ref = torch.nn.functional.linear(torch.from_numpy(X), merged).numpy()
    np.testing.assert_allclose(Y, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(T, torch.from_numpy(X).matmul(torch.from_numpy(A)).numpy(),
                               rtol=1e-13, atol=1e-13)


def test_bwd_finite_differences():
    """L = <dY, Y> is affine in each of X, A, B, so central differences are
    exact up to rounding; compare every gradient entry."""
    rng = np.random.default_rng(6)
    M, K, N, r, s = 3, 128, 64, 4, 0.5
    X, W, A, B, dY = (_rand(rng, M, K), _rand(rng, N, K), _rand(rng, K, r),
                      _rand(rng, r, N), _rand(rng, M, N))
    dX, dA, dB = oracle.linear_bwd_f64(dY, X, W, A, B, s)

    def L(X_, A_, B_):
        return float(np.sum(dY * oracle.linear_fwd_f64(X_, W, A_, B_, s)[0]))

    h = 0.5
    for name, P, G in (("X", X, dX), ("A", A, dA), ("B", B, dB)):
        fd = np.empty_like(P)
        for idx in np.ndindex(P.shape):
            Pp, Pm = P.copy(), P.copy()
            Pp[idx] += h
            Pm[idx] -= h
            args_p = {"X": (Pp, A, B), "A": (X, Pp, B), "B": (X, A, Pp)}[name]
            args_m = {"X": (Pm, A, B), "A": (X, Pm, B), "B": (X, A, Pm)}[name]
            fd[idx] = (L(*args_p) - L(*args_m)) / (2 * h)
        err = np.linalg.norm(fd - G) / np.linalg.norm(G)
        assert err < 1e-9, (name, err)


def test_bwd_matches_torch_autograd():
    rng = np.random.default_rng(8)
    M, K, N, r, s = 6, 192, 80, 8, 0.25
    X, W, A, B, dY = (_rand(rng, M, K), _rand(rng, N, K), _rand(rng, K, r),
                      _rand(rng, r, N), _rand(rng, M, N))
    tX, tA, tB = (torch.tensor(a, requires_grad=True) for a in (X, A, B))
    tW = torch.tensor(W, requires_grad=False)
    Y = torch.nn.functional.linear(tX, tW) + s * (tX @ tA) @ tB
    Y.backward(torch.from_numpy(dY))
    dX, dA, dB = oracle.linear_bwd_f64(dY, X, W, A, B, s)
    np.testing.assert_allclose(dX, tX.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dA, tA.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dB, tB.grad.numpy(), rtol=1e-12, atol=1e-12)
    assert tW.grad is None   # the frozen base gets no gradient


def test_bwd_adjoint_identity():
    """<dY, X W^T> = <dY W, X>: dX of the base path is the adjoint."""
    rng = np.random.default_rng(10)
    X, W, dY = _rand(rng, 9, 256), _rand(rng, 33, 256), _rand(rng, 9, 33)
    A0, B0 = np.zeros((256, 0)), np.zeros((0, 33))
    Y, _ = oracle.linear_fwd_f64(X, W, A0, B0, 1.0)
    dX, dA, dB = oracle.linear_bwd_f64(dY, X, W, A0, B0, 1.0)
    assert abs(np.sum(dY * Y) - np.sum(dX * X)) <= 1e-10 * np.sum(np.abs(dY * Y))
    assert dA.shape == (256, 0) and dB.shape == (0, 33)


def test_b_zero_gives_zero_dA():
    rng = np.random.default_rng(12)
    X, W, A, dY = _rand(rng, 4, 64), _rand(rng, 8, 64), _rand(rng, 64, 2), _rand(rng, 4, 8)
    dX, dA, dB = oracle.linear_bwd_f64(dY, X, W, A, np.zeros((2, 8)), 1.0)
    assert np.all(dA == 0)
    assert np.any(dB != 0)


# ---------------------------------------------------------------------------
# Projections that share their input (the fused block)
# ---------------------------------------------------------------------------

def test_block_bwd_finite_differences():
    """L = sum_j <dY_j, Y_j> over three projections of one X: central
    differences of every entry of X, A_j and B_j (exact for this affine loss)
    equal the block's gradients; a dropped or doubled projection in dX fails."""
    rng = np.random.default_rng(14)
    M, K, N, r, s, S = 2, 64, 16, 2, 0.75, 3
    X = _rand(rng, M, K)
    Ws = [_rand(rng, N, K) for _ in range(S)]
    As = [_rand(rng, K, r) for _ in range(S)]
    Bs = [_rand(rng, r, N) for _ in range(S)]
    dYs = [_rand(rng, M, N) for _ in range(S)]
    dX, dAs, dBs = oracle.block_bwd_f64(dYs, X, Ws, As, Bs, s)

    def L(X_, As_, Bs_):
        Ys, _ = oracle.block_fwd_f64(X_, Ws, As_, Bs_, s)
        return float(sum(np.sum(d * y) for d, y in zip(dYs, Ys)))

    h = 0.5

    def fd_of(get, put, shape):
        g = np.empty(shape)
        for idx in np.ndindex(shape):
            v = get()[idx]
            put(idx, v + h)
            lp = L(Xc[0], Ac, Bc)
            put(idx, v - h)
            lm = L(Xc[0], Ac, Bc)
            put(idx, v)
            g[idx] = (lp - lm) / (2 * h)
        return g

    Xc, Ac, Bc = [X.copy()], [a.copy() for a in As], [b.copy() for b in Bs]
    fdX = fd_of(lambda: Xc[0], lambda i, v: Xc[0].__setitem__(i, v), X.shape)
    assert np.linalg.norm(fdX - dX) / np.linalg.norm(dX) < 1e-9
    for j in range(S):
        fdA = fd_of(lambda: Ac[j], lambda i, v: Ac[j].__setitem__(i, v), As[j].shape)
        fdB = fd_of(lambda: Bc[j], lambda i, v: Bc[j].__setitem__(i, v), Bs[j].shape)
        assert np.linalg.norm(fdA - dAs[j]) / np.linalg.norm(dAs[j]) < 1e-9
        assert np.linalg.norm(fdB - dBs[j]) / np.linalg.norm(dBs[j]) < 1e-9


def test_block_matches_torch_autograd_with_shared_input():
    """torch: one X tensor feeding three linear + LoRA branches."""
    rng = np.random.default_rng(15)
    M, K, N, r, s = 4, 96, 40, 8, 0.25
    X = _rand(rng, M, K)
    Ws = [_rand(rng, N, K) for _ in range(3)]
    As = [_rand(rng, K, r) for _ in range(3)]
    Bs = [_rand(rng, r, N) for _ in range(3)]
    dYs = [_rand(rng, M, N) for _ in range(3)]
    tX = torch.tensor(X, requires_grad=True)
    tA = [torch.tensor(a, requires_grad=True) for a in As]
    tB = [torch.tensor(b, requires_grad=True) for b in Bs]
    loss = 0
    for j in range(3):
        Y = torch.nn.functional.linear(tX, torch.from_numpy(Ws[j])) + s * (tX @ tA[j]) @ tB[j]
        loss = loss + (Y * torch.from_numpy(dYs[j])).sum()
    loss.backward()
    dX, dAs, dBs = oracle.block_bwd_f64(dYs, X, Ws, As, Bs, s)
    np.testing.assert_allclose(dX, tX.grad.numpy(), rtol=1e-12, atol=1e-12)
    for j in range(3):
        np.testing.assert_allclose(dAs[j], tA[j].grad.numpy(), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dBs[j], tB[j].grad.numpy(), rtol=1e-12, atol=1e-12)


def test_block_b_zero_is_the_stacked_linear():
    """With every B_j = 0 the projections' outputs side by side are one linear
    layer with the weights stacked along N (torch F.linear)."""
    rng = np.random.default_rng(16)
    X = _rand(rng, 5, 64)
    Ws = [_rand(rng, 24, 64) for _ in range(3)]
    As = [_rand(rng, 64, 8) for _ in range(3)]
    Bs = [np.zeros((8, 24)) for _ in range(3)]
    Ys, _ = oracle.block_fwd_f64(X, Ws, As, Bs, 0.5)
    ref = torch.nn.functional.linear(torch.from_numpy(X),
                                     torch.from_numpy(np.concatenate(Ws, axis=0))).numpy()
    np.testing.assert_allclose(np.concatenate(Ys, axis=1), ref, rtol=1e-13, atol=1e-13)


def test_stacked_weight_quantizes_like_its_parts():
    """Weights whose blocks fill whole groups of 256 constants (N K a multiple
    of 64 * 256) quantize stacked along N exactly as one by one: the codes,
    8-bit constants and group scales are the parts' side by side.  A part
    that does not fill its last group changes the next part's scales."""
    rng = np.random.default_rng(17)
    parts = [workloads.draw_weight(rng, 128, 128) for _ in range(3)]   # 256 blocks each
    whole = oracle.quantize(np.concatenate(parts, axis=0))
    each = [oracle.quantize(p) for p in parts]
    for i in range(3):
        np.testing.assert_array_equal(whole[i], np.concatenate([e[i] for e in each]))
    odd = [workloads.draw_weight(rng, 96, 128) for _ in range(2)]          # 192 blocks each
    whole = oracle.quantize(np.concatenate(odd, axis=0))
    assert not np.array_equal(whole[2], np.concatenate([oracle.quantize(p)[2] for p in odd]))
