"""NF4 storage format: level table, blockwise absmax quantization, double
quantization of the constants, and dequantization to bf16.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Layout conventions (readings; the pages do not fix them):
  * The stored weight is ``W_lin`` of shape [N, K] (the usual out x in layout of
    a linear layer, row-major).  The pages' product X.W uses W = W_lin^T.
  * A block is 64 consecutive elements of the row-major flattening of W_lin;
    K must be a multiple of 64, so a block never crosses a row.
  * A DQ group is 256 consecutive block ids; the last group may be short.
  * Codes are packed two per byte, the even element in the low nibble.
"""
import functools
import math

import numpy as np

BLOCK = 64    # weights per absmax constant: list item (2) of "DL0087 QLoRA"
GROUP = 256   # constants per second-level fp32 scale: list item (3) of "DL0087 QLoRA"


# ---------------------------------------------------------------------------
# The NF4 level table
# ---------------------------------------------------------------------------

def _std_normal_cdf(z: float) -> float:
    return 0.5 * math.erfc(-z / math.sqrt(2.0))


def normal_quantile(p: float) -> float:
    """Phi^{-1}(p) for the standard normal, by bisection over the doubles.

    The interval [lo, hi] is halved until lo and hi are adjacent doubles; the
    end whose CDF lies closer to p is returned.  Slow and plain on purpose.
    """
    if not 0.0 < p < 1.0:
        raise ValueError("p must lie in (0, 1)")
    lo, hi = -40.0, 40.0
    while True:
        mid = 0.5 * (lo + hi)
        if mid <= lo or mid >= hi:
            break
        if _std_normal_cdf(mid) < p:
            lo = mid
        else:
            hi = mid
    return lo if abs(_std_normal_cdf(lo) - p) <= abs(_std_normal_cdf(hi) - p) else hi


@functools.lru_cache(maxsize=None)
def _nf4_levels_tuple():
    pos = [normal_quantile(0.5 + (j - 0.5) / 16.0) for j in range(1, 9)]
    neg = [normal_quantile(0.5 + (j - 0.5) / 14.0) for j in range(1, 8)]
    levels = [-z / neg[-1] for z in neg] + [0.0] + [z / pos[-1] for z in pos]
    return tuple(sorted(levels))


def nf4_levels_f64() -> np.ndarray:
    """The 16 NF4 levels in float64, ascending.

    Pages: "4-bit NormalFloat" section of "QLoRA: Finetuning 65B Models on a
    Single GPU" (levels at quantiles of the standard normal, each level
    covering an equal probability mass), and the Mathematical Formulation of
    "DL0087 QLoRA" (levels from normal quantiles, rescaled to [-1, 1] with an
    exact zero).

    Reading (the construction is not printed): 16 levels with one exact zero
    leave 15 nonzero levels, split 8 positive / 7 negative.  Each half of the
    normal (mass 1/2) is cut into equal-mass bins -- 8 bins of mass 1/16 on the
    positive side, 7 bins of mass 1/14 on the negative side -- and each level
    sits at the quantile of its bin's probability centre:
        z+_j = Phi^{-1}(1/2 + (j - 1/2)/16),  j = 1..8
        z-_j = Phi^{-1}(1/2 + (j - 1/2)/14),  j = 1..7
    Each side is divided by its own extreme quantile so the end levels are
    exactly -1 and +1.
    """
    return np.array(_nf4_levels_tuple(), dtype=np.float64)


def nf4_levels() -> np.ndarray:
    """The NF4 levels as float32 (each fp64 level rounded once, to nearest-even)."""
    return nf4_levels_f64().astype(np.float32)


# ---------------------------------------------------------------------------
# bf16 helpers
# ---------------------------------------------------------------------------

def bf16_rne_bits(x) -> np.ndarray:
    """Round finite float32 values to bfloat16, round-to-nearest-even.

    Returns the 16-bit patterns (uint16).  bf16 keeps the top 16 bits of the
    float32 pattern; adding 0x7FFF plus the lowest kept bit before truncation
    rounds to nearest with ties to the even pattern.  Inputs must be finite.
    """
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact value of bf16 bit patterns, as float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# Blockwise absmax + nearest-level encoding + packing
# ---------------------------------------------------------------------------

def encode(x) -> np.ndarray:
    """Nearest NF4 level index for normalised float32 values x in [-1, 1].

    code = argmin_j |x - q_j| with ties going to the lower index (the pages do
    not state a tie rule; lower index is the reading).  The distances are taken
    in float64 on float32 operands.  This is exact wherever two distances can
    compete: a float32 difference x - q_j loses bits in float64 only when one
    operand is below 2^-29 times the other, and then x lies within 2^-29 of the
    zero level while every other level is at least 0.04 away.
    """
    xs = np.asarray(x, dtype=np.float32).astype(np.float64)
    q = nf4_levels().astype(np.float64)
    out = np.empty(xs.shape, dtype=np.uint8)
    flat_x, flat_o = xs.reshape(-1), out.reshape(-1)
    step = 1 << 20
    for i in range(0, flat_x.size, step):
        d = np.abs(flat_x[i:i + step, None] - q[None, :])
        flat_o[i:i + step] = np.argmin(d, axis=1)   # first minimum on ties
    return out


def quantize(W):
    """Quantize a float32 weight W_lin [N, K] to NF4 with double quantization.

    Pages: list items (2) and (3) of "DL0087 QLoRA" (blocks of 64, one absmax
    per block; the constants quantized to 8 bits with one fp32 scale per 256
    constants) and "Double Quantization and Paged Optimizers" of "QLoRA:
    Finetuning 65B Models" (the 32-bit constants are themselves quantized).

    Per block b:  c_b = max |w|;  x = fl32(w / c_b);  code = encode(x).
    An all-zero block has c_b = 0 and every code 7 (the zero level).
    Per group g of 256 blocks:  s_g = max c_b;  d_g = fl32(s_g / 255);
    e_b = clamp(rint_half_even(fl32(c_b / d_g)), 0, 255), or 0 when d_g = 0.
    Readings: the 8-bit constant format is unsigned linear absmax (constants
    are non-negative); d_g stores s_g / 255 so dequantization is one multiply;
    the 4-bit codes use the unquantized c_b.

    Returns (codes uint8[N*K/2], absmax_q uint8[nb], absmax_scale float32[ng],
    absmax float32[nb]); the last is the transient first-level constant,
    returned for tests only (it is never stored by the format).
    """
    W = np.ascontiguousarray(W, dtype=np.float32)
    if W.ndim != 2 or W.shape[1] % BLOCK != 0:
        raise ValueError("W must be 2-D with K a multiple of 64")
    blocks = W.reshape(-1, BLOCK)
    nb = blocks.shape[0]
    absmax = np.abs(blocks).max(axis=1) if nb else np.zeros(0, np.float32)

    # normalise with an IEEE float32 divide (a zero block divides by 1: its
    # elements are all zero so x = 0 and the code is the zero level)
    safe = np.where(absmax > 0, absmax, np.float32(1.0)).astype(np.float32)
    x = blocks / safe[:, None]
    codes = encode(x).reshape(-1)
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)

    ng = (nb + GROUP - 1) // GROUP
    padded = np.zeros(ng * GROUP, dtype=np.float32)
    padded[:nb] = absmax
    s = padded.reshape(ng, GROUP).max(axis=1) if ng else np.zeros(0, np.float32)
    d = (s / np.float32(255.0)).astype(np.float32)
    d_of_block = np.repeat(d, GROUP)[:nb]
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = (absmax / d_of_block).astype(np.float32)
    e = np.where(d_of_block > 0, np.clip(np.rint(ratio), 0, 255), 0).astype(np.uint8)
    return packed, e, d, absmax


def unpack_codes(codes) -> np.ndarray:
    """Unpack two codes per byte, even element from the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    out = np.empty(c.size * 2, dtype=np.uint8)
    out[0::2] = c & 0x0F
    out[1::2] = c >> 4
    return out


# ---------------------------------------------------------------------------
# Dequantization
# ---------------------------------------------------------------------------

def dequantize_at(codes, absmax_q, absmax_scale, flat_index) -> np.ndarray:
    """Dequantized bf16 bits of W_lin at row-major flat indices n*K + k.

    Pages: Mathematical Formulation and Figure 1 of "DL0087 QLoRA" (the
    dequantization rebuilds a bf16 tile just before the matmul, from the code,
    the level table and the block's constant).
      c_hat_b = fl32(e_b * d_g)
      w_hat   = bf16_rne(fl32(q[code] * c_hat_b))
    Reading: the float32 product is rounded before the bf16 rounding.
    """
    idx = np.asarray(flat_index, dtype=np.int64)
    byte = np.asarray(codes, dtype=np.uint8)[idx >> 1]
    code = np.where((idx & 1) == 0, byte & 0x0F, byte >> 4)
    block = idx >> 6
    c_hat = (np.asarray(absmax_q)[block].astype(np.float32)
             * np.asarray(absmax_scale, dtype=np.float32)[block >> 8])
    w = nf4_levels()[code] * c_hat
    return bf16_rne_bits(w)


def dequantize(codes, absmax_q, absmax_scale, N, K, rows=None, cols=None):
    """bf16 bits of the dequantized W_lin[N, K] (or of its rows x cols submatrix)."""
    r = np.arange(N, dtype=np.int64) if rows is None else np.asarray(rows, np.int64)
    c = np.arange(K, dtype=np.int64) if cols is None else np.asarray(cols, np.int64)
    out = np.empty((r.size, c.size), dtype=np.uint16)
    step = max(1, (1 << 22) // max(1, c.size))
    for i in range(0, r.size, step):
        idx = r[i:i + step, None] * K + c[None, :]
        out[i:i + step] = dequantize_at(codes, absmax_q, absmax_scale, idx)
    return out


# ---------------------------------------------------------------------------
# Code boundaries (for sweeping every float32 through a quantizer)
# ---------------------------------------------------------------------------

def _f32_from_ordinal(o: int) -> np.float32:
    """Map an integer ordinal to a float32 so that ordinals sort like values."""
    if o >= 0:
        return np.array([o], dtype=np.uint32).view(np.float32)[0]
    return -np.array([-o], dtype=np.uint32).view(np.float32)[0]


def code_boundaries() -> np.ndarray:
    """For j = 1..15, the smallest float32 x in [-1, 1] whose code is >= j.

    The nearest-level code is a non-decreasing step function of x (the levels
    are sorted and ties go to the lower index), so these 15 points determine
    encode() on every float32 in [-1, 1].  Found by bisection over the ordered
    float32 values, calling encode() only.
    """
    lo_ord = -int(np.array([1.0], np.float32).view(np.uint32)[0])
    hi_ord = int(np.array([1.0], np.float32).view(np.uint32)[0])
    out = np.empty(15, dtype=np.float32)
    for j in range(1, 16):
        lo, hi = lo_ord, hi_ord          # encode(lo) < j <= encode(hi)
        while hi - lo > 1:
            mid = (lo + hi) // 2
            if int(encode(np.array([_f32_from_ordinal(mid)]))[0]) >= j:
                hi = mid
            else:
                lo = mid
        out[j - 1] = _f32_from_ordinal(hi)
    return out


# ---------------------------------------------------------------------------
# Storage cost
# ---------------------------------------------------------------------------

def storage_bytes(N: int, K: int) -> int:
    """Bytes of the NF4 + double-quantized format for an N x K weight.

    codes N*K/2 bytes + one 8-bit constant per 64 weights + one fp32 scale per
    256 constants (list item (3) and the storage-cost bullet of the
    Mathematical Formulation of "DL0087 QLoRA").
    """
    nb = N * K // BLOCK
    ng = (nb + GROUP - 1) // GROUP
    return N * K // 2 + nb + 4 * ng


def bits_per_param(N: int, K: int) -> float:
    return 8.0 * storage_bytes(N, K) / (N * K)
