"""GPU parity of the NF4 format kernels: bit-exact against the oracle.

Quantize (codes, 8-bit constants, fp32 scales) and dequantize (bf16 bits) are
an encoding, so the GPU must reproduce the oracle exactly: on the seeded
parity weight, on crafted edge blocks (zero blocks, exact ties between
levels, denormals, a short last group, huge and tiny scales) and on every
float32 in [-1, 1] pushed through the real kernel.
"""
import numpy as np
import pytest

import bit_quantized_fine_amd as q
import oracle
import workloads
from gpu_util import bf16, bits, dev, f32, need_gpu, say, torch

pytestmark = pytest.mark.gpu


def _quantize_both(W):
    Wd = f32(W)
    w = q.qlora_nf4_quantize(Wd)
    torch.cuda.synchronize()
    codes, e, d, _ = oracle.quantize(W)
    return w, (codes, e, d)


def _assert_quant_equal(w, ref):
    codes, e, d = ref
    np.testing.assert_array_equal(w.codes.cpu().numpy(), codes)
    np.testing.assert_array_equal(w.absmax_q.cpu().numpy(), e)
    np.testing.assert_array_equal(w.absmax_scale.cpu().numpy().view(np.uint32), d.view(np.uint32))


@pytest.mark.parametrize("N,K", [(1024, 1024), (3, 64), (5, 64 * 300), (257, 192), (64, 11008)])
def test_quantize_dequantize_bit_exact(N, K):
    need_gpu()
    say(f"quantize/dequantize N={N} K={K}")
    rng = np.random.default_rng(N + K)
    W = workloads.draw_weight(rng, N, K)
    w, ref = _quantize_both(W)
    _assert_quant_equal(w, ref)
    deq = q.qlora_nf4_dequantize(w)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(deq), oracle.dequantize(*ref, N, K))


def test_parity_1k_weight_bit_exact():
    need_gpu()
    say("parity_1k weight, seeded recipe")
    (lin, inp), = list(workloads.workload_inputs("parity_1k"))
    w, ref = _quantize_both(inp.W)
    _assert_quant_equal(w, ref)
    np.testing.assert_array_equal(bits(q.qlora_nf4_dequantize(w)),
                                  oracle.dequantize(*ref, lin.N, lin.K))


def _edge_weight():
    qv = oracle.nf4_levels()
    rows = []
    # exact ties between adjacent levels (and their neighbours), with a +1 sentinel
    blk = []
    for a, b in zip(qv[:-1], qv[1:]):
        m = np.float32((np.float64(a) + np.float64(b)) / 2)
        blk += [m, np.nextafter(m, np.float32(2)), np.nextafter(m, np.float32(-2))]
    blk = (blk + [0.0] * 64)[:63] + [1.0]
    rows.append(np.array(blk, np.float32))
    rows.append(np.zeros(64, np.float32))                        # all-zero block
    r = np.linspace(-3, 2, 64).astype(np.float32)                # negative absmax
    rows.append(r)
    rows.append((np.arange(64, dtype=np.float32) - 31) * np.float32(1e-42))  # denormals
    rows.append(np.full(64, -0.0, np.float32))                   # negative zeros
    rows.append(np.array([1e30] + [1e-30] * 63, np.float32))     # huge range
    rows.append(np.array([-5e-39] * 64, np.float32))             # denormal constant
    rng = np.random.default_rng(0)
    rows.append(rng.standard_normal(64).astype(np.float32) * np.float32(1e-20))
    W = np.concatenate([np.stack(rows)] * 40, axis=0)            # 320 blocks: short last group
    return W.reshape(-1, 128)


def test_edge_blocks_bit_exact():
    need_gpu()
    W = _edge_weight()
    say(f"edge blocks {W.shape}")
    w, ref = _quantize_both(W)
    _assert_quant_equal(w, ref)
    np.testing.assert_array_equal(bits(q.qlora_nf4_dequantize(w)),
                                  oracle.dequantize(*ref, *W.shape))


def _codebook_boundaries(codebook):
    """For j = 1..15, the smallest float32 in [-1, 1] whose oracle code (the
    nearest level of the codebook, ties to the lower index) is >= j, found by
    bisection over the ordered float32 values (the code is a non-decreasing
    step function of x)."""
    if codebook == "nf4":
        return oracle.code_boundaries()
    from oracle import codebooks
    lv = codebooks.levels(codebook)
    one = int(np.array([1.0], np.float32).view(np.uint32)[0])

    def f32_of(o):
        u = np.array([abs(o)], dtype=np.uint32).view(np.float32)[0]
        return u if o >= 0 else -u

    def code(o):
        return int(codebooks.encode_levels(np.array([f32_of(o)], np.float32), lv)[0])

    out = np.empty(15, dtype=np.float32)
    for j in range(1, 16):
        lo, hi = -one, one
        if code(lo) >= j:          # code j is reached at -1 already
            out[j - 1] = np.float32(-1.0)
            continue
        while hi - lo > 1:
            mid = (lo + hi) // 2
            if code(mid) >= j:
                hi = mid
            else:
                lo = mid
        out[j - 1] = f32_of(hi)
    return out


@pytest.mark.parametrize("codebook", ["nf4", "int4", "fp4"])
def test_every_float32_in_unit_interval_encodes_like_oracle(codebook):
    """All 2.13e9 float32 values in [-1, 1] go through the quantize kernel in
    blocks whose 64th element is +1.0 (so the block scale is exactly 1 and the
    normalised value equals the input); their codes must equal the oracle's
    nearest-level code of the codebook, given by its 15 boundaries."""
    need_gpu()
    bnd = torch.from_numpy(_codebook_boundaries(codebook)).to(dev())
    one = int(np.array([1.0], np.float32).view(np.uint32)[0])
    per_blk = 63
    chunk_blocks = 1 << 22
    total = 0
    for sign in (0, 1):
        say(f"exhaustive sweep {codebook} sign={sign}")
        start = 0
        while start <= one:
            nvals = min(per_blk * chunk_blocks, one + 1 - start)
            nblk = -(-nvals // per_blk)
            pat = torch.arange(start, start + nblk * per_blk, dtype=torch.int64, device=dev())
            pat = torch.clamp(pat, max=one)                       # pad with +-1.0
            if sign:
                pat = pat + (1 << 31) - (1 << 32)                 # sign bit, as int32
            vals = pat.to(torch.int32).view(torch.float32).view(nblk, per_blk)
            W = torch.ones((nblk, 64), dtype=torch.float32, device=dev())
            W[:, :per_blk] = vals
            w = (q.qlora_nf4_quantize(W) if codebook == "nf4"
                 else q.qlora_q4_quantize(W, codebook, True))
            c = w.codes
            codes = torch.stack([c & 15, c >> 4], dim=1).view(nblk, 64)[:, :per_blk]
            expect = torch.bucketize(vals, bnd, right=True).to(torch.uint8)
            bad = (codes != expect).sum().item()
            assert bad == 0, (sign, start, bad)
            assert torch.all(w.absmax_q == 255)
            total += nvals
            start += nvals
    say(f"swept {total} values")
    assert total == 2 * (one + 1)


# Block constants for the quotient sweep: weight-like scales, values next to
# a power of two, tiny and large ones (2^-100 and 2^126 lie outside the range
# where the kernel forms the quotient from the reciprocal), and, for INT4,
# whose table has a threshold at zero, constants above 1, whose quotients of
# subnormal weights round to zero or not; FP4 at constants of other ranges.
_SWEEP_CASES = [("nf4", c) for c in (
    0.0213, 0.37, float(np.nextafter(np.float32(1), np.float32(0))), 1.5, 3.0, 3.0e-5,
    2.0 ** -60, 2.0 ** 20, 2.0 ** -100, 2.0 ** 126)] + [
    ("int4", 3.0), ("int4", 2.0 ** 20), ("int4", 2.0 ** -100),
    ("fp4", 1.5), ("fp4", 2.0 ** -60), ("fp4", 2.0 ** 126)]


@pytest.mark.parametrize("codebook,cval", _SWEEP_CASES)
def test_every_quotient_by_a_block_constant_encodes_like_oracle(codebook, cval):
    """Every float32 w with |w| <= c goes through the quantize kernel in blocks
    whose 64th element is c, so the block constant is exactly c and every
    code is the oracle's nearest level of fl32(w / c).  The reference quotient
    is taken in float64 and rounded once to float32, which is the correctly
    rounded float32 quotient (53 >= 2 * 24 + 2 bits), then encoded with the
    codebook's 15 boundaries."""
    need_gpu()
    c32 = np.float32(cval)
    cbits = int(np.array([c32], np.float32).view(np.uint32)[0])
    bnd = torch.from_numpy(_codebook_boundaries(codebook)).to(dev())
    per_blk = 63
    chunk_blocks = 1 << 22
    total = 0
    for sign in (0, 1):
        say(f"quotient sweep {codebook} c={float(c32):.6g} sign={sign}")
        start = 0
        while start <= cbits:
            nvals = min(per_blk * chunk_blocks, cbits + 1 - start)
            nblk = -(-nvals // per_blk)
            pat = torch.arange(start, start + nblk * per_blk, dtype=torch.int64, device=dev())
            pat = torch.clamp(pat, max=cbits)                    # pad with +-c
            if sign:
                pat = pat + (1 << 31) - (1 << 32)                # sign bit, as int32
            vals = pat.to(torch.int32).view(torch.float32).view(nblk, per_blk)
            W = torch.full((nblk, 64), float(c32), dtype=torch.float32, device=dev())
            W[:, :per_blk] = vals
            w = (q.qlora_nf4_quantize(W) if codebook == "nf4"
                 else q.qlora_q4_quantize(W, codebook, True))
            cc = w.codes
            codes = torch.stack([cc & 15, cc >> 4], dim=1).view(nblk, 64)[:, :per_blk]
            x = (vals.double() / float(c32)).float()
            expect = torch.bucketize(x, bnd, right=True).to(torch.uint8)
            bad = (codes != expect).sum().item()
            assert bad == 0, (float(c32), sign, start, bad)
            total += nvals
            start += nvals
    assert total == 2 * (cbits + 1)
