"""The 4-bit data types and block-constant formats the pages set NF4 against:
4-bit integers (INT4) and 4-bit floats (FP4) in place of the NF4 levels, and
fp32 block constants without double quantization -- the same blockwise absmax
scheme with another 16-entry codebook or another constant format.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Pages: "4-bit NormalFloat: an information-theoretically optimal quantization
type" of "QLoRA: Finetuning 65B Models on a Single GPU with 4-Bit
Quantization" (NF4 against INT4, whose levels are spaced uniformly, and FP4;
NF4 is optimal for normally distributed weights), and numbered list item (3)
of "DL0087 QLoRA: 4-bit Quantized LoRA" (double quantization takes the
constants' overhead from 0.5 to about 0.127 bits per parameter, so without it
each 64-block keeps a 32-bit constant).

Readings (the pages name the types but print neither table):
  * INT4: sixteen uniformly spaced levels spanning [-1, 1], l_k = (2k - 15)/15
    for k = 0..15 (the fp64 quotient rounded once to fp32).  Absmax scaling
    maps every block onto [-1, 1], and both ends are levels.  There is no zero
    level.
  * FP4: the sixteen values of the E2M1 float (1 sign, 2 exponent bits with
    bias 1, 1 mantissa bit; subnormal when the exponent field is 0), divided
    by its largest magnitude 6 so the range is [-1, 1].  Sorted ascending,
    with +0 before -0: both zeros are codes, and the tie rule below never
    produces the second (-0, code 8); dequantizing code 8 still gives -0 . c.
  * Encoding is the NF4 rule with another table: nearest level, ties to the
    lower index (nf4.encode's reading), evaluated exactly.
  * Without double quantization the constant is the block's fp32 absmax c_b
    itself, and dequantization is bf16_rne(fl32(q[code] . c_b)).  With it, the
    constants are quantized exactly as for NF4 (8-bit e_b, one fp32 d_g per
    256 blocks).
"""
import numpy as np

from .nf4 import BLOCK, GROUP, bf16_rne_bits, nf4_levels

CODEBOOKS = ("nf4", "int4", "fp4")


def int4_levels() -> np.ndarray:
    """INT4 levels (fp32, ascending): l_k = fl32((2k - 15) / 15), k = 0..15."""
    return np.array([(2 * k - 15) / 15.0 for k in range(16)], dtype=np.float64).astype(np.float32)


def e2m1_value(bits: int) -> float:
    """Value of the 4-bit float E2M1 with bit pattern `bits` (s ee m)."""
    s, e, m = (bits >> 3) & 1, (bits >> 1) & 3, bits & 1
    mag = 0.5 * m if e == 0 else 2.0 ** (e - 1) * (1.0 + 0.5 * m)
    return -mag if s else mag


def fp4_levels() -> np.ndarray:
    """FP4 (E2M1) levels over [-1, 1] (fp32): the 16 E2M1 values divided by
    6, negatives first, then +0 and -0, then the positives."""
    vals = [e2m1_value(b) / 6.0 for b in range(16)]
    neg = sorted(v for v in vals if v < 0)
    pos = sorted(v for v in vals if v > 0)
    return np.array(neg + [0.0, -0.0] + pos, dtype=np.float64).astype(np.float32)


def levels(codebook: str) -> np.ndarray:
    """The 16 fp32 levels of a codebook ("nf4", "int4" or "fp4")."""
    if codebook == "nf4":
        return nf4_levels()
    if codebook == "int4":
        return int4_levels()
    if codebook == "fp4":
        return fp4_levels()
    raise ValueError(f"unknown codebook {codebook!r}")


def encode_levels(x, lv) -> np.ndarray:
    """Nearest level of the ascending table `lv` for normalised float32 values
    x, ties to the lower index (the NF4 rule of nf4.encode, any table).

    For sorted levels the nearest level is the first one whose midpoint to the
    next larger distinct level is not below x; a level equal to the one before
    it (FP4's -0 after +0) is never the first.  The midpoints are sums of two
    fp32 halved in float64, so they and the comparisons are exact.  (Distances
    taken in float64 are not exact for tables without a zero level: for
    |x| < 2^-29 the distances to -1/15 and +1/15 round to a tie.)
    """
    q = np.asarray(lv, dtype=np.float32).astype(np.float64)
    upper = np.full(q.size, np.inf)
    for j in range(q.size):
        above = q[j + 1:][q[j + 1:] > q[j]]
        if above.size:
            upper[j] = (q[j] + above[0]) / 2
    xs = np.asarray(x, dtype=np.float32).astype(np.float64)
    return np.searchsorted(upper, xs, side="left").astype(np.uint8)


def quantize_q4(W, codebook: str = "nf4", double_quant: bool = True):
    """Blockwise absmax quantization of W_lin [N, K] with a codebook.

    Per block b: c_b = max |w|;  x = fl32(w / c_b) (an all-zero block divides
    by 1);  code = nearest level.  Codes are packed two per byte, the even
    element in the low nibble.
    double_quant: e_b and d_g as in nf4.quantize (8-bit constants, one fp32
    scale per 256); returns (codes, e uint8[nb], d float32[ng], absmax).
    Without it: returns (codes, None, absmax float32[nb], absmax) -- the
    stored constants are the fp32 absmax values themselves.
    """
    W = np.ascontiguousarray(W, dtype=np.float32)
    if W.ndim != 2 or W.shape[1] % BLOCK != 0:
        raise ValueError("W must be 2-D with K a multiple of 64")
    blocks = W.reshape(-1, BLOCK)
    nb = blocks.shape[0]
    absmax = np.abs(blocks).max(axis=1) if nb else np.zeros(0, np.float32)
    safe = np.where(absmax > 0, absmax, np.float32(1.0)).astype(np.float32)
    x = blocks / safe[:, None]
    codes = encode_levels(x, levels(codebook)).reshape(-1)
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
    if not double_quant:
        return packed, None, absmax.astype(np.float32), absmax
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


def dequantize_q4(codes, absmax_q, absmax_scale, N: int, K: int, codebook: str = "nf4",
                  double_quant: bool = True) -> np.ndarray:
    """bf16 bits of the dequantized W_lin [N, K]:
    bf16_rne(fl32(q[code] . c)) with c = fl32(e_b . d_g) (double
    quantization) or c = the stored fp32 c_b (without)."""
    byte = np.asarray(codes, dtype=np.uint8)
    code = np.empty(byte.size * 2, dtype=np.uint8)
    code[0::2] = byte & 0x0F
    code[1::2] = byte >> 4
    block = np.arange(N * K, dtype=np.int64) >> 6
    if double_quant:
        c = (np.asarray(absmax_q)[block].astype(np.float32)
             * np.asarray(absmax_scale, dtype=np.float32)[block >> 8])
    else:
        c = np.asarray(absmax_scale, dtype=np.float32)[block]
    w = levels(codebook)[code] * c
    return bf16_rne_bits(w).reshape(N, K)


def storage_bytes_q4(N: int, K: int, double_quant: bool = True) -> int:
    """Bytes of a 4-bit weight: N K / 2 of codes, plus one 8-bit constant per
    block and one fp32 scale per 256 blocks (double quantization) or one fp32
    constant per block (without)."""
    nb = N * K // BLOCK
    if double_quant:
        return N * K // 2 + nb + 4 * ((nb + GROUP - 1) // GROUP)
    return N * K // 2 + 4 * nb


def code_entropy_bits(codes) -> float:
    """Shannon entropy (bits) of the empirical distribution of the unpacked
    4-bit codes: 4 bits when all sixteen are used equally often."""
    byte = np.asarray(codes, dtype=np.uint8)
    h = np.bincount(byte & 0x0F, minlength=16) + np.bincount(byte >> 4, minlength=16)
    p = h[h > 0] / h.sum()
    return float(-(p * np.log2(p)).sum())
