"""GPU parity of the 16-bit LoRA comparator (qlora_lora16_fwd / _bwd: the
layer with a bf16 base weight on the same kernels) against the oracle's
linear layer with that weight, and its identity with the NF4 layer when the
bf16 weight is the NF4 weight's dequantized copy (the GEMM path then stages
the same bf16 tile, so the results agree bit for bit).
"""
import numpy as np
import pytest

import bit_quantized_fine_amd as q
import oracle
import workloads
from gpu_util import assert_close, bf16, bits, f32, need_gpu, say, torch

pytestmark = pytest.mark.gpu


class Dense:
    """One 16-bit LoRA linear: seeded inputs with W rounded to bf16."""

    def __init__(self, M, N, K, r, s, seed, b_zero=False):
        rng = np.random.default_rng(seed)
        inp = workloads.draw_linear(rng, N, K, M, r)
        if b_zero:
            inp.B[:] = 0
        self.M, self.N, self.K, self.r, self.s = M, N, K, r, s
        self.inp = inp
        self.Wb = workloads.to_bf16_bits(inp.W)
        self.W = bf16(self.Wb)
        self.X, self.A, self.B, self.dY = (bf16(inp.X), bf16(inp.A), bf16(inp.B),
                                           bf16(inp.dY))

    def fwd(self):
        if self.r == 0:
            return q.qlora_lora16_fwd(self.X, self.W)
        return q.qlora_lora16_fwd(self.X, self.W, self.A, self.B, self.s)


CASES = [
    # (M, N, K, r, s)
    (1, 256, 256, 8, 1.0),           # one token: split reductions
    (16, 1024, 1024, 16, 1.0),
    (17, 200, 320, 8, 0.5),          # ragged N, K = 5 * 64
    (300, 1000, 64 * 33, 64, 0.25),  # K with a half chunk, ragged M and N
    (520, 264, 192, 40, 0.5),        # rank not a multiple of 32, three token tiles
    (256, 384, 448, 256, 0.0625),    # maximum rank
    (64, 128, 16384, 32, 0.5),       # long reduction, few tiles
    (2048, 8, 64, 8, 1.0),           # one 8-row tile, eight token tiles
    (40, 4104, 128, 16, 0.25),       # N a multiple of 8 only
]


@pytest.mark.parametrize("M,N,K,r,s", CASES)
def test_lora16_parity(M, N, K, r, s):
    need_gpu()
    say(f"lora16 M={M} N={N} K={K} r={r}")
    c = Dense(M, N, K, r, s, seed=M * 11 + N + K + r)
    Y, T = c.fwd()
    dX, dA, dB = q.qlora_lora16_bwd(c.dY, c.X, c.W, c.A, c.B, s, T=T)
    dX2, dA2, dB2 = q.qlora_lora16_bwd(c.dY, c.X, c.W, c.A, c.B, s, T=None)
    torch.cuda.synchronize()
    Yr, Tr = oracle.linear_fwd(c.inp.X, c.Wb, c.inp.A, c.inp.B, s)
    assert_close("Y", Y.float().cpu().numpy(), Yr)
    assert_close("T", T.cpu().numpy(), Tr)
    dXr, dAr, dBr = oracle.linear_bwd(c.inp.dY, c.inp.X, c.Wb, c.inp.A, c.inp.B, s)
    assert_close("dX", dX.float().cpu().numpy(), dXr)
    assert_close("dA", dA.float().cpu().numpy(), dAr)
    assert_close("dB", dB.float().cpu().numpy(), dBr)
    # the recompute form gives the same bits
    for a, b in ((dX, dX2), (dA, dA2), (dB, dB2)):
        np.testing.assert_array_equal(bits(a), bits(b))


def test_lora16_without_adapter():
    """r = 0: Y = X . W^T alone, and dX = dY . W."""
    need_gpu()
    c = Dense(130, 264, 320, 0, 1.0, seed=5)
    Y, _ = c.fwd()
    dX, _, _ = q.qlora_lora16_bwd(c.dY, c.X, c.W)
    torch.cuda.synchronize()
    Xf, Wf = oracle.bf16_bits_to_f64(c.inp.X), oracle.bf16_bits_to_f64(c.Wb)
    assert_close("Y", Y.float().cpu().numpy(), Xf @ Wf.T)
    assert_close("dX", dX.float().cpu().numpy(), oracle.bf16_bits_to_f64(c.inp.dY) @ Wf)


@pytest.mark.parametrize("M,N,K,r", [
    (17, 1024, 1024, 16),     # split reductions
    (300, 520, 448, 64),      # ragged tiles
    (512, 4096, 4096, 64),    # LLaMA-7B q shape
])
def test_lora16_of_dequantized_weight_is_the_nf4_layer(M, N, K, r):
    """Given the NF4 weight's dequantized copy, the 16-bit path computes the
    NF4 layer bit for bit on the tiled GEMMs (M > 16): the two differ only in
    where the bf16 weight tile comes from."""
    need_gpu()
    say(f"lora16 vs nf4, M={M} N={N} K={K}")
    rng = np.random.default_rng(M + N)
    inp = workloads.draw_linear(rng, N, K, M, r)
    w = q.qlora_nf4_quantize(f32(inp.W))
    Wd = q.qlora_nf4_dequantize(w)
    X, A, B, dY = bf16(inp.X), bf16(inp.A), bf16(inp.B), bf16(inp.dY)
    Y4, T4 = q.qlora_linear_fwd(X, w, A, B, 0.25)
    dX4, dA4, dB4 = q.qlora_linear_bwd(dY, X, w, A, B, 0.25, T=T4)
    Y6, T6 = q.qlora_lora16_fwd(X, Wd, A, B, 0.25)
    dX6, dA6, dB6 = q.qlora_lora16_bwd(dY, X, Wd, A, B, 0.25, T=T6)
    torch.cuda.synchronize()
    for name, a, b in (("Y", Y4, Y6), ("dX", dX4, dX6), ("dA", dA4, dA6), ("dB", dB4, dB6)):
        np.testing.assert_array_equal(bits(a), bits(b), err_msg=name)
    assert torch.equal(T4, T6)


def test_lora16_llama7b_gate_full_size():
    """LLaMA-7B gate projection (11008 x 4096) at M = 2048: sampled rows of Y
    and dX, full dA and dB."""
    need_gpu()
    M, N, K, r, s = 2048, 11008, 4096, 64, 0.25
    say(f"lora16 full size M={M} N={N} K={K}")
    c = Dense(M, N, K, r, s, seed=77)
    Y, T = c.fwd()
    dX, dA, dB = q.qlora_lora16_bwd(c.dY, c.X, c.W, c.A, c.B, s, T=T)
    torch.cuda.synchronize()
    rows = np.random.default_rng(4).choice(M, 128, replace=False)
    Yr, _ = oracle.linear_fwd(c.inp.X[rows], c.Wb, c.inp.A, c.inp.B, s)
    assert_close("Y[rows]", Y.float().cpu().numpy()[rows], Yr)
    dXr, _, _ = oracle.linear_bwd(c.inp.dY[rows], c.inp.X[rows], c.Wb, c.inp.A, c.inp.B, s)
    assert_close("dX[rows]", dX.float().cpu().numpy()[rows], dXr)
    _, dAr, dBr = oracle.linear_bwd(c.inp.dY, c.inp.X, c.Wb, c.inp.A, c.inp.B, s, need_dx=False)
    assert_close("dA", dA.float().cpu().numpy(), dAr)
    assert_close("dB", dB.float().cpu().numpy(), dBr)


def test_lora16_refuses_bad_shapes():
    """K % 64, N % 8 and N K <= 2^30 are checked before any launch."""
    need_gpu()
    d = torch.device("cuda:0")
    X = torch.zeros((4, 96), dtype=torch.bfloat16, device=d)
    with pytest.raises(q.QloraError, match="shape"):
        q.qlora_lora16_fwd(X, torch.zeros((64, 96), dtype=torch.bfloat16, device=d))
    X = torch.zeros((4, 64), dtype=torch.bfloat16, device=d)
    with pytest.raises(q.QloraError, match="shape"):
        q.qlora_lora16_fwd(X, torch.zeros((12, 64), dtype=torch.bfloat16, device=d))
