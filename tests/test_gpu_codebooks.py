"""GPU parity of the codebook and constant variants (qlora_q4_*): INT4, FP4
and NF4 levels, with double-quantized or fp32 block constants, through the
same quantize, dequantize, streaming and tiled kernels, against the oracle's
definitions in oracle/codebooks.py.

Codes, constants and dequantized weights are compared bit for bit; Y, T,
dX, dA, dB within the layer's tolerance.  The last test measures code
entropy and squared error on Gaussian weights from the GPU's own codes
("4-bit NormalFloat" of "QLoRA: Finetuning 65B Models on a Single GPU":
NF4 is optimal for normally distributed weights and beats INT4 and FP4).
"""
import numpy as np
import pytest

import bit_quantized_fine_amd as q
import oracle
import workloads
from gpu_util import assert_close, bf16, bits, f32, need_gpu, say, torch
from oracle import codebooks as cb

pytestmark = pytest.mark.gpu

FORMATS = [(name, dq) for name in cb.CODEBOOKS for dq in (True, False)]


def _edge_weight(rng, name, N, K):
    """Gaussian rows with edge blocks: an all-zero block, a tiny-valued block,
    blocks whose absmax is 1 holding every threshold of the codebook and the
    float above it, and a scaled row."""
    W = rng.standard_normal((N, K)).astype(np.float32)
    W[0, :64] = 0
    W[0, 64:128] = np.float32(1e-30) * rng.standard_normal(64).astype(np.float32)
    t = np.array(q.qlora_q4_thresholds(name), np.float32)
    probes = np.concatenate([t, np.nextafter(t, np.float32(2), dtype=np.float32)])
    blk = np.zeros(64, np.float32)
    blk[0] = 1.0
    blk[1:1 + 30] = probes
    W[1, :64] = blk
    W[1, 64:128] = -blk
    W[2] *= np.float32(1e4)
    return W


def _unpack(codes):
    c = np.asarray(codes, np.uint8)
    out = np.empty(c.size * 2, np.uint8)
    out[0::2], out[1::2] = c & 15, c >> 4
    return out


@pytest.mark.parametrize("name,dq", FORMATS)
def test_quantize_and_dequantize_bit_exact(name, dq):
    need_gpu()
    N, K = 72, 64 * 300     # 337.5 groups of 256 blocks: a short last group
    say(f"q4 quantize {name} dq={dq} N={N} K={K}")
    rng = np.random.default_rng(10 * cb.CODEBOOKS.index(name) + int(dq))
    W = _edge_weight(rng, name, N, K)
    w = q.qlora_q4_quantize(f32(W), name, dq)
    Wd = q.qlora_q4_dequantize(w)
    torch.cuda.synchronize()
    codes, e, c, _ = cb.quantize_q4(W, name, dq)
    np.testing.assert_array_equal(w.codes.cpu().numpy(), codes)
    if dq:
        np.testing.assert_array_equal(w.absmax_q.cpu().numpy(), e)
    else:
        assert w.absmax_q is None
    np.testing.assert_array_equal(w.absmax_scale.cpu().numpy().view(np.uint32),
                                  c.view(np.uint32))
    np.testing.assert_array_equal(bits(Wd), cb.dequantize_q4(codes, e, c, N, K, name, dq))
    if name == "fp4":   # -0 (code 8) is never produced
        assert not np.any(_unpack(codes) == 8)


def test_nf4_q4_is_the_nf4_layer():
    """The NF4 codebook with double quantization is the qlora_nf4 / qlora_linear
    path: same bytes, same outputs."""
    need_gpu()
    rng = np.random.default_rng(9)
    inp = workloads.draw_linear(rng, 264, 448, 40, 16)
    w4 = q.qlora_q4_quantize(f32(inp.W), "nf4", True)
    w = q.qlora_nf4_quantize(f32(inp.W))
    X, A, B, dY = bf16(inp.X), bf16(inp.A), bf16(inp.B), bf16(inp.dY)
    Y, T = q.qlora_linear_fwd(X, w, A, B, 0.5)
    Y4, T4 = q.qlora_q4_linear_fwd(X, w4, A, B, 0.5)
    g = q.qlora_linear_bwd(dY, X, w, A, B, 0.5, T=T)
    g4 = q.qlora_q4_linear_bwd(dY, X, w4, A, B, 0.5, T=T4)
    torch.cuda.synchronize()
    for a, b in ((w.codes, w4.codes), (w.absmax_q, w4.absmax_q)):
        assert torch.equal(a, b)
    assert torch.equal(w.absmax_scale, w4.absmax_scale)
    np.testing.assert_array_equal(bits(Y), bits(Y4))
    for a, b in zip(g, g4):
        np.testing.assert_array_equal(bits(a), bits(b))


LAYER_CASES = [
    # (M, N, K, r): streaming path (X in LDS whole or in K-slices), tiled path
    (1, 256, 1024, 16),
    (4, 200, 64 * 33, 8),    # half a 128-k chunk past K
    (16, 200, 4096, 64),     # X in 1024-column K-slices
    (9, 72, 64 * 197, 16),   # X in 1024-column K-slices, the last ragged
    (300, 264, 448, 32),
]


@pytest.mark.parametrize("name,dq", FORMATS)
@pytest.mark.parametrize("M,N,K,r", LAYER_CASES)
def test_layer_parity(name, dq, M, N, K, r):
    need_gpu()
    say(f"q4 layer {name} dq={dq} M={M} N={N} K={K} r={r}")
    rng = np.random.default_rng(M * 13 + N + K + r + 10 * cb.CODEBOOKS.index(name) + int(dq))
    inp = workloads.draw_linear(rng, N, K, M, r, x_kind="relu" if M > 1 else "normal")
    w = q.qlora_q4_quantize(f32(inp.W), name, dq)
    X, A, B, dY = bf16(inp.X), bf16(inp.A), bf16(inp.B), bf16(inp.dY)
    s = 0.25
    Y, T = q.qlora_q4_linear_fwd(X, w, A, B, s)
    dX, dA, dB = q.qlora_q4_linear_bwd(dY, X, w, A, B, s, T=T)
    torch.cuda.synchronize()
    codes, e, c, _ = cb.quantize_q4(inp.W, name, dq)
    What = cb.dequantize_q4(codes, e, c, N, K, name, dq)
    Yr, Tr = oracle.linear_fwd(inp.X, What, inp.A, inp.B, s)
    assert_close("Y", Y.float().cpu().numpy(), Yr)
    assert_close("T", T.cpu().numpy(), Tr)
    dXr, dAr, dBr = oracle.linear_bwd(inp.dY, inp.X, What, inp.A, inp.B, s)
    assert_close("dX", dX.float().cpu().numpy(), dXr)
    assert_close("dA", dA.float().cpu().numpy(), dAr)
    assert_close("dB", dB.float().cpu().numpy(), dBr)


@pytest.mark.parametrize("name,dq", [("int4", False), ("fp4", True)])
def test_layer_full_size(name, dq):
    """LLaMA-7B q projection (4096 x 4096) at M = 1 and M = 2048: sampled
    rows of Y against the oracle."""
    need_gpu()
    N = K = 4096
    rng = np.random.default_rng(21)
    W = workloads.draw_weight(rng, N, K)
    w = q.qlora_q4_quantize(f32(W), name, dq)
    codes, e, c, _ = cb.quantize_q4(W, name, dq)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(w.codes.cpu().numpy(), codes)
    What = cb.dequantize_q4(codes, e, c, N, K, name, dq)
    for M in (1, 2048):
        say(f"q4 full size {name} dq={dq} M={M}")
        Xb = workloads.to_bf16_bits(workloads.draw_activations(rng, M, K, "relu"))
        A = workloads.to_bf16_bits(rng.standard_normal((K, 64), dtype=np.float32) / 64)
        B = workloads.to_bf16_bits(rng.standard_normal((64, N), dtype=np.float32) * 0.01)
        Y, _ = q.qlora_q4_linear_fwd(bf16(Xb), w, bf16(A), bf16(B), 0.25)
        torch.cuda.synchronize()
        rows = np.arange(M) if M == 1 else np.random.default_rng(2).choice(M, 64, replace=False)
        Yr, _ = oracle.linear_fwd(Xb[rows], What, A, B, 0.25)
        assert_close(f"Y[rows] M={M}", Y.float().cpu().numpy()[rows], Yr)


def test_nf4_is_best_on_gaussian_weights():
    """Code entropy and mean squared error of the GPU's quantization of a
    Gaussian 1024 x 4096 weight: NF4 has the highest entropy and the lowest
    error of the three codebooks, in both constant formats, and double
    quantization adds less than 0.5% to the error."""
    need_gpu()
    rng = np.random.default_rng(0)
    W = rng.standard_normal((1024, 4096)).astype(np.float32)
    Wg = f32(W)
    H, mse = {}, {}
    for name in cb.CODEBOOKS:
        for dq in (True, False):
            w = q.qlora_q4_quantize(Wg, name, dq)
            Wd = q.qlora_q4_dequantize(w).float()
            c = w.codes
            hist = (torch.bincount((c & 15).long(), minlength=16)
                    + torch.bincount((c >> 4).long(), minlength=16)).double()
            p = hist[hist > 0] / hist.sum()
            H[name] = float(-(p * torch.log2(p)).sum())
            mse[name, dq] = float(((Wd - Wg) ** 2).double().mean())
            if dq:   # the same numbers as the oracle's (the codes are bit-exact)
                assert H[name] == pytest.approx(cb.code_entropy_bits(c.cpu().numpy()), abs=1e-12)
    say(f"  entropy bits {H}")
    say(f"  mse {mse}")
    assert H["nf4"] > H["fp4"] > H["int4"]
    for dq in (True, False):
        assert mse["nf4", dq] < mse["int4", dq] and mse["nf4", dq] < mse["fp4", dq]
    for name in cb.CODEBOOKS:
        assert mse[name, False] <= mse[name, True] < 1.005 * mse[name, False]
