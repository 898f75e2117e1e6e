"""GPU parity of the QLoRA linear forward and backward against the oracle.

The oracle quantizes the same seeded float32 weight itself, dequantizes it,
and computes Y, dX, dA, dB in float64 from the exact bf16 inputs.  The GPU
outputs (bf16, fp32 accumulation) must be within relative Frobenius error
5e-3 and max error 1e-2 * max|ref|.  Cases span both forward paths (M <= 16
streams the weight; larger M runs the MFMA GEMM), several tiles with ragged
tails in every dimension, ranks 8..256, B = 0 and r = 0.
"""
import numpy as np
import pytest

import bit_quantized_fine_amd as q
import oracle
import workloads
from gpu_util import (assert_close, bf16, bits, dev, errors, f32, need_gpu, say,
                      torch)

pytestmark = pytest.mark.gpu


class Case:
    """One linear: seeded inputs, GPU tensors, oracle reference."""

    def __init__(self, M, N, K, r, s, seed, b_std=0.01, b_zero=False, x_kind="normal"):
        rng = np.random.default_rng(seed)
        inp = workloads.draw_linear(rng, N, K, M, r, b_std=b_std, x_kind=x_kind)
        if b_zero:
            inp.B[:] = 0
        self.M, self.N, self.K, self.r, self.s = M, N, K, r, s
        self.inp = inp
        self.w = q.qlora_nf4_quantize(f32(inp.W))
        self.X, self.A, self.B, self.dY = (bf16(inp.X), bf16(inp.A), bf16(inp.B),
                                           bf16(inp.dY))
        codes, e, d, _ = oracle.quantize(inp.W)
        self.What = oracle.dequantize(codes, e, d, N, K)

    def gpu_fwd(self, r=None):
        if (self.r if r is None else r) == 0:
            return q.qlora_linear_fwd(self.X, self.w)
        return q.qlora_linear_fwd(self.X, self.w, self.A, self.B, self.s)

    def ref_fwd(self):
        return oracle.linear_fwd(self.inp.X, self.What, self.inp.A, self.inp.B, self.s)

    def ref_bwd(self):
        return oracle.linear_bwd(self.inp.dY, self.inp.X, self.What, self.inp.A,
                                 self.inp.B, self.s)


FWD_CASES = [
    # (M, N, K, r, s)   decode path M <= 16, GEMM path above
    (1, 1024, 1024, 16, 1.0),
    (4, 1024, 1024, 16, 1.0),
    (16, 1024, 1024, 16, 1.0),
    (7, 200, 320, 8, 0.5),           # ragged N (not a multiple of 16), K = 5 * 64
    (16, 1000, 64 * 33, 64, 0.25),   # X in three K-slices, the last half a chunk
    (1, 232, 64 * 33, 32, 0.5),      # K with a half chunk; X staged in LDS
    (4, 96, 16384, 64, 0.25),        # T folded, X too large for LDS (read from global memory)
    (2, 64, 16384, 8, 0.5),          # X of exactly the LDS staging limit (64 KB); 64 T partials
    (1, 96, 16384 + 64 * 5, 64, 0.25),   # 44 T partial sums, the last of two 128-k slices, one ragged
    (1, 64, 32768, 64, 0.5),         # one token, X from global memory: 64 partials added late
    (8, 264, 64 * 133, 16, 0.5),     # 8 tokens, X from global memory, ragged rows
    (12, 264, 64 * 133, 16, 0.5),    # X in K-slices, the last ragged (half a chunk), ragged rows
    (4, 96, 1024, 256, 0.25),        # M r = 1024: the most T values added after the main loop
    (5, 96, 1024, 256, 0.25),        # M r = 1280: T reduced by a launch of its own
    (8, 96, 16384, 64, 0.25),        # T added after the main loop, X read from global memory
    (2, 64, 32768 + 64, 8, 0.5),     # K beyond the decode kernel: GEMM path at M = 2
    (17, 1024, 1024, 16, 1.0),       # first GEMM size
    (300, 520, 448, 64, 0.25),       # ragged M, N, K over several tiles
    (256, 384, 1024, 256, 0.0625),   # maximum rank
    (129, 136, 64, 8, 2.0),          # single reduction tile
    (520, 264, 192, 40, 0.5),        # rank not a multiple of 32, three token tiles
    (1, 8, 64, 8, 1.0),              # smallest decode: 8 rows, one block (half a 128-k chunk)
    (3, 8, 64, 256, 0.5),            # rank above K, T added after the main loop (M r = 768)
    (2048, 8, 64, 8, 1.0),           # GEMM with one 8-row tile and eight token tiles
    (40, 4104, 128, 16, 0.25),       # N a multiple of 8 only (513 x 8)
]


@pytest.mark.parametrize("M,N,K,r,s", FWD_CASES)
def test_fwd_parity(M, N, K, r, s):
    need_gpu()
    say(f"fwd M={M} N={N} K={K} r={r}")
    c = Case(M, N, K, r, s, seed=M * 7 + N + K + r)
    Y, T = c.gpu_fwd()
    torch.cuda.synchronize()
    Yref, Tref = c.ref_fwd()
    assert_close("Y", Y.float().cpu().numpy(), Yref)
    assert_close("T", T.cpu().numpy(), Tref)


@pytest.mark.parametrize("x_kind", ["relu", "shifted"])
@pytest.mark.parametrize("M,N,K", [
    (1, 256, 8192),       # decode, X in LDS (one 16-byte piece a thread)
    (1, 256, 22016),      # decode, X in LDS (four pieces a thread), 65B FFN width
    (4, 256, 8192),       # decode, X in LDS (four pieces a thread), T folded
    (16, 256, 8192),      # decode, X in K-slices
    (16, 256, 22016),     # the same at the 65B FFN width
    (1, 200, 64 * 33),    # decode, half chunk past K (K % 128 == 64)
    (16, 200, 64 * 33),
    (64, 256, 8192),      # GEMM path
])
def test_fwd_nonzero_mean_activations(M, N, K, x_kind):
    """Activations with a non-zero mean (the positive part of N(0,1), as a
    ReLU-family layer feeds its down projection, and N(1,1)): rounding errors
    of the dequantized weights would add up coherently over K here instead of
    cancelling, so every weight must be the defined bf16_rne(fl32(q . c))."""
    need_gpu()
    say(f"fwd {x_kind} X, M={M} N={N} K={K}")
    c = Case(M, N, K, 64, 0.25, seed=M * 3 + N + K + len(x_kind), x_kind=x_kind)
    Y, T = c.gpu_fwd()
    torch.cuda.synchronize()
    Yref, Tref = c.ref_fwd()
    assert_close("Y", Y.float().cpu().numpy(), Yref)
    assert_close("T", T.cpu().numpy(), Tref)
    # the base product alone (r = 0), where no adapter term can mask an error
    Y0, _ = c.gpu_fwd(r=0)
    torch.cuda.synchronize()
    base = oracle.bf16_bits_to_f64(c.inp.X) @ oracle.bf16_bits_to_f64(c.What).T
    assert_close("Y(r=0)", Y0.float().cpu().numpy(), base)


@pytest.mark.parametrize("M,N,K,r,s", [
    (16, 1024, 1024, 16, 1.0),
    (1, 200, 320, 8, 0.5),
    (300, 520, 448, 64, 0.25),
    (256, 384, 1024, 256, 0.0625),
    (33, 1000, 64 * 33, 64, 0.25),
    (520, 264, 192, 40, 0.5),        # rank not a multiple of 32, three token tiles
    (64, 8, 64, 8, 1.0),             # one 8-row reduction chunk, a half column tile
    (1, 8, 64, 8, 1.0),              # one token
    (3, 4104, 128, 256, 0.5),        # maximum rank, N a multiple of 8 only
])
def test_bwd_parity(M, N, K, r, s):
    need_gpu()
    say(f"bwd M={M} N={N} K={K} r={r}")
    c = Case(M, N, K, r, s, seed=M * 5 + N + K + r)
    Y, T = c.gpu_fwd()
    dX, dA, dB = q.qlora_linear_bwd(c.dY, c.X, c.w, c.A, c.B, c.s, T=T)
    # gradient-checkpointing form: T recomputed inside the backward
    dX2, dA2, dB2 = q.qlora_linear_bwd(c.dY, c.X, c.w, c.A, c.B, c.s, T=None)
    torch.cuda.synchronize()
    dXr, dAr, dBr = c.ref_bwd()
    assert_close("dX", dX.float().cpu().numpy(), dXr)
    assert_close("dA", dA.float().cpu().numpy(), dAr)
    assert_close("dB", dB.float().cpu().numpy(), dBr)
    assert_close("dA(recompute)", dA2.float().cpu().numpy(), dAr)
    assert_close("dB(recompute)", dB2.float().cpu().numpy(), dBr)
    np.testing.assert_array_equal(bits(dX2), bits(dX))


def test_lora_heavy_case():
    """B with standard deviation 1: the adapter term dominates, so a dropped or
    mis-scaled LoRA term (or a wrong hi/lo split) cannot hide in the tolerance."""
    need_gpu()
    for M in (8, 200):
        say(f"lora-heavy M={M}")
        c = Case(M, 256, 512, 32, 0.5, seed=99 + M, b_std=1.0)
        Y, T = c.gpu_fwd()
        dX, dA, dB = q.qlora_linear_bwd(c.dY, c.X, c.w, c.A, c.B, c.s, T=T)
        torch.cuda.synchronize()
        Yr, _ = c.ref_fwd()
        dXr, dAr, dBr = c.ref_bwd()
        assert_close("Y", Y.float().cpu().numpy(), Yr)
        assert_close("dX", dX.float().cpu().numpy(), dXr)
        assert_close("dA", dA.float().cpu().numpy(), dAr)
        assert_close("dB", dB.float().cpu().numpy(), dBr)


@pytest.mark.parametrize("M", [16, 160])
def test_b_zero_reproduces_base(M):
    """B = 0: Y equals the base-only (r = 0) GPU output bit for bit, equals
    the oracle's X . deq(W)^T, and dA is exactly zero (the adapter that starts
    at zero: Mathematical Formulation of "DL0087 QLoRA")."""
    need_gpu()
    say(f"B=0 M={M}")
    c = Case(M, 1024, 1024, 16, 1.0, seed=5 + M, b_zero=True)
    Y, T = c.gpu_fwd()
    Y0, _ = c.gpu_fwd(r=0)
    dX, dA, dB = q.qlora_linear_bwd(c.dY, c.X, c.w, c.A, c.B, c.s, T=T)
    dX0, _, _ = q.qlora_linear_bwd(c.dY, c.X, c.w)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(Y), bits(Y0))
    np.testing.assert_array_equal(bits(dX), bits(dX0))
    assert torch.count_nonzero(dA.float()).item() == 0
    base = oracle.bf16_bits_to_f64(c.inp.X) @ oracle.bf16_bits_to_f64(c.What).T
    assert_close("Y(B=0)", Y.float().cpu().numpy(), base)
    _, _, dBr = c.ref_bwd()
    assert_close("dB(B=0)", dB.float().cpu().numpy(), dBr)


def test_frozen_base_untouched_and_deterministic():
    """The NF4 buffers are bytewise unchanged by fwd and bwd, and repeated
    calls give bitwise-identical outputs."""
    need_gpu()
    for M in (4, 192):
        say(f"frozen/determinism M={M}")
        c = Case(M, 512, 512, 16, 1.0, seed=M)
        before = [t.clone() for t in (c.w.codes, c.w.absmax_q, c.w.absmax_scale)]
        outs = []
        for _ in range(3):
            Y, T = c.gpu_fwd()
            dX, dA, dB = q.qlora_linear_bwd(c.dY, c.X, c.w, c.A, c.B, c.s, T=T)
            torch.cuda.synchronize()
            outs.append([bits(Y), T.cpu().numpy(), bits(dX), bits(dA), bits(dB)])
        for a, b in zip(before, (c.w.codes, c.w.absmax_q, c.w.absmax_scale)):
            assert torch.equal(a, b)
        for o in outs[1:]:
            for x, y in zip(outs[0], o):
                np.testing.assert_array_equal(x, y)


def test_bwd_without_dx():
    need_gpu()
    c = Case(64, 256, 256, 16, 1.0, seed=3)
    Y, T = c.gpu_fwd()
    dX, dA, dB = q.qlora_linear_bwd(c.dY, c.X, c.w, c.A, c.B, c.s, T=T, need_dx=False)
    torch.cuda.synchronize()
    assert dX is None
    _, dAr, dBr = c.ref_bwd()
    assert_close("dA", dA.float().cpu().numpy(), dAr)
    assert_close("dB", dB.float().cpu().numpy(), dBr)


# ---------------------------------------------------------------------------
# Full-size workloads
# ---------------------------------------------------------------------------

def _full_linear_check(key, lin_idx, M=None, rows=None):
    cfg = workloads.WORKLOADS[key]
    (lin, inp), = list(workloads.workload_inputs(key, M=M, linears=[lin_idx]))
    m = inp.X.shape[0]
    say(f"{key} linear {lin.name} N={lin.N} K={lin.K} M={m}")
    w = q.qlora_nf4_quantize(f32(inp.W))
    X, A, B, dY = bf16(inp.X), bf16(inp.A), bf16(inp.B), bf16(inp.dY)
    Y, T = q.qlora_linear_fwd(X, w, A, B, cfg.s)
    dX, dA, dB = q.qlora_linear_bwd(dY, X, w, A, B, cfg.s, T=T)
    torch.cuda.synchronize()
    codes, e, d, _ = oracle.quantize(inp.W)
    np.testing.assert_array_equal(w.codes.cpu().numpy(), codes)
    np.testing.assert_array_equal(w.absmax_q.cpu().numpy(), e)
    What = oracle.dequantize(codes, e, d, lin.N, lin.K)
    sel = slice(None) if rows is None else rows
    Yr, _ = oracle.linear_fwd(inp.X[sel], What, inp.A, inp.B, cfg.s)
    assert_close("Y", Y.float().cpu().numpy()[sel], Yr)
    dXr, dAr, dBr = oracle.linear_bwd(inp.dY, inp.X, What, inp.A, inp.B, cfg.s)
    assert_close("dX", dX.float().cpu().numpy(), dXr)
    assert_close("dA", dA.float().cpu().numpy(), dAr)
    assert_close("dB", dB.float().cpu().numpy(), dBr)


@pytest.mark.parametrize("lin_idx", [0, 4, 6])
def test_llama7b_full_size(lin_idx):
    """LLaMA-7B linears at M=2048 (q, gate, down shapes), compared in full."""
    need_gpu()
    _full_linear_check("llama7b", lin_idx)


@pytest.mark.parametrize("lin_idx", [0, 6])
def test_llama7b_dp8_shard(lin_idx):
    """One GPU's share of 8-way data parallelism (M = 256): the GEMMs have
    too few tiles for the CUs and split their reductions (fp32 partials,
    added up in split order); compared in full."""
    need_gpu()
    _full_linear_check("llama7b", lin_idx, M=256)


@pytest.mark.parametrize("lin_idx", [0, 1, 2])
def test_decode_65b_full_size(lin_idx):
    """65B-shaped decode linears (8192 x 8192, 22016 x 8192, 8192 x 22016),
    each at M = 1, 4 and 16 with the workload's X, and at M = 4 with
    non-negative X too, compared in full (the oracle quantizes the weight
    once per shape)."""
    need_gpu()
    cfg = workloads.WORKLOADS["decode_65b"]
    (lin, inp), = list(workloads.workload_inputs("decode_65b", M=16, linears=[lin_idx],
                                                 with_grad=False))
    say(f"decode_65b {lin.name} N={lin.N} K={lin.K}")
    w = q.qlora_nf4_quantize(f32(inp.W))
    A, B = bf16(inp.A), bf16(inp.B)
    codes, e, d, _ = oracle.quantize(inp.W)
    np.testing.assert_array_equal(w.codes.cpu().numpy(), codes)
    What = oracle.dequantize(codes, e, d, lin.N, lin.K)
    xr = workloads.to_bf16_bits(workloads.draw_activations(np.random.default_rng(lin_idx), 4,
                                                           lin.K, "relu"))
    for M, Xh in ((1, inp.X[:1]), (4, inp.X[:4]), (16, inp.X), (4, xr)):
        say(f"  M={M}")
        Y, T = q.qlora_linear_fwd(bf16(Xh), w, A, B, cfg.s)
        torch.cuda.synchronize()
        Yr, _ = oracle.linear_fwd(Xh, What, inp.A, inp.B, cfg.s)
        assert_close("Y", Y.float().cpu().numpy(), Yr)


@pytest.mark.parametrize("lin_idx", [0, 6])
def test_llama33b_full_size_recompute(lin_idx):
    """33B-shaped linears at M=4096 with the recompute (checkpointing) bwd:
    sampled rows of Y and dX, full dA and dB."""
    need_gpu()
    cfg = workloads.WORKLOADS["llama33b_recompute"]
    (lin, inp), = list(workloads.workload_inputs("llama33b_recompute", linears=[lin_idx]))
    say(f"llama33b_recompute {lin.name} N={lin.N} K={lin.K} M={inp.X.shape[0]}")
    w = q.qlora_nf4_quantize(f32(inp.W))
    X, A, B, dY = bf16(inp.X), bf16(inp.A), bf16(inp.B), bf16(inp.dY)
    Y, _ = q.qlora_linear_fwd(X, w, A, B, cfg.s)
    dX, dA, dB = q.qlora_linear_bwd(dY, X, w, A, B, cfg.s, T=None)
    torch.cuda.synchronize()
    codes, e, d, _ = oracle.quantize(inp.W)
    What = oracle.dequantize(codes, e, d, lin.N, lin.K)
    rows = np.random.default_rng(1).choice(inp.X.shape[0], 256, replace=False)
    Yr, _ = oracle.linear_fwd(inp.X[rows], What, inp.A, inp.B, cfg.s)
    assert_close("Y[rows]", Y.float().cpu().numpy()[rows], Yr)
    dXr, _, _ = oracle.linear_bwd(inp.dY[rows], inp.X[rows], What, inp.A, inp.B, cfg.s)
    assert_close("dX[rows]", dX.float().cpu().numpy()[rows], dXr)
    _, dAr, dBr = oracle.linear_bwd(inp.dY, inp.X, What, inp.A, inp.B, cfg.s, need_dx=False)
    assert_close("dA", dA.float().cpu().numpy(), dAr)
    assert_close("dB", dB.float().cpu().numpy(), dBr)


@pytest.mark.parametrize("fill", [0x00, 0xFF, 0x5A])
def test_workspace_contents_do_not_matter(fill):
    """The forward workspace needs no initialisation: prefilled garbage, and
    reuse across calls of different shapes, give the same bitwise output."""
    need_gpu()
    say(f"workspace fill=0x{fill:02x}")
    c = Case(4, 512, 2048, 64, 0.25, seed=21)
    c2 = Case(16, 256, 1024, 32, 0.5, seed=22)
    need = max(q.lib().qlora_linear_fwd_workspace_bytes(4, 512, 2048, 64),
               q.lib().qlora_linear_fwd_workspace_bytes(16, 256, 1024, 32))
    ws = torch.full((need,), fill, dtype=torch.uint8, device=dev())
    Y1, T1 = q.qlora_linear_fwd(c.X, c.w, c.A, c.B, c.s, workspace=ws)
    Y1, T1 = bits(Y1), T1.cpu().numpy()
    q.qlora_linear_fwd(c2.X, c2.w, c2.A, c2.B, c2.s, workspace=ws)
    Y2, T2 = q.qlora_linear_fwd(c.X, c.w, c.A, c.B, c.s, workspace=ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(Y2), Y1)
    np.testing.assert_array_equal(T2.cpu().numpy(), T1)
    Yr, Tr = c.ref_fwd()
    assert_close("Y", oracle.bf16_bits_to_f64(Y1), Yr)
    assert_close("T", T1, Tr)


def _device_stack_65b_linear(idx, M):
    """Linear idx of the 65B stack, drawn on the device as the stack is
    (seeds 4000 + idx for W, 5000 + idx for A and B), with X and dY drawn on
    the device too; returns device tensors and their host copies (the same
    bytes on both sides)."""
    cfg = workloads.WORKLOADS["stack_65b"]
    lin = cfg.linears[idx]
    W = workloads.device_weight(torch, dev(), lin.N, lin.K, seed=4000 + idx)
    A, B = workloads.device_adapters(torch, dev(), lin.N, lin.K, cfg.r, seed=5000 + idx)
    X = workloads.device_activations(torch, dev(), M, lin.K, seed=6000 + idx)
    dY = workloads.device_activations(torch, dev(), M, lin.N, seed=7000 + idx)
    host = dict(W=W.cpu().numpy(), X=bits(X), A=bits(A), B=bits(B), dY=bits(dY))
    return cfg, lin, W, A, B, X, dY, host


def test_stack_65b_first_linear():
    """65B stack, layer 0's q projection (8192 x 8192, M = 2048) drawn on the
    device: codes and constants in full, sampled rows of Y and dX, full dA
    and dB."""
    need_gpu()
    say("stack_65b linear 0 (q, 8192x8192), M=2048")
    cfg, lin, W, A, B, X, dY, h = _device_stack_65b_linear(0, 2048)
    w = q.qlora_nf4_quantize(W)
    Y, T = q.qlora_linear_fwd(X, w, A, B, cfg.s)
    dX, dA, dB = q.qlora_linear_bwd(dY, X, w, A, B, cfg.s, T=T)
    torch.cuda.synchronize()
    codes, e, d, _ = oracle.quantize(h["W"])
    np.testing.assert_array_equal(w.codes.cpu().numpy(), codes)
    np.testing.assert_array_equal(w.absmax_q.cpu().numpy(), e)
    np.testing.assert_array_equal(w.absmax_scale.cpu().numpy(), d)
    What = oracle.dequantize(codes, e, d, lin.N, lin.K)
    rows = np.random.default_rng(4).choice(2048, 128, replace=False)
    Yr, _ = oracle.linear_fwd(h["X"][rows], What, h["A"], h["B"], cfg.s)
    assert_close("Y[rows]", Y.float().cpu().numpy()[rows], Yr)
    dXr, _, _ = oracle.linear_bwd(h["dY"][rows], h["X"][rows], What, h["A"], h["B"], cfg.s)
    assert_close("dX[rows]", dX.float().cpu().numpy()[rows], dXr)
    _, dAr, dBr = oracle.linear_bwd(h["dY"], h["X"], What, h["A"], h["B"], cfg.s, need_dx=False)
    assert_close("dA", dA.float().cpu().numpy(), dAr)
    assert_close("dB", dB.float().cpu().numpy(), dBr)


def test_stack_65b_last_linear_row_groups():
    """65B stack, layer 79's down projection (8192 x 22016, M = 2048): the
    first and last 32 rows (43 whole groups of 256 block constants each,
    so the oracle can quantize them alone) bit-exact, Y on those rows for
    sampled tokens, full dA, and dB on those rows' columns."""
    need_gpu()
    idx = 559
    say("stack_65b linear 559 (down, 8192x22016), M=2048")
    cfg, lin, W, A, B, X, dY, h = _device_stack_65b_linear(idx, 2048)
    assert lin.name == "down" and (32 * lin.K // 64) % 256 == 0
    w = q.qlora_nf4_quantize(W)
    Y, T = q.qlora_linear_fwd(X, w, A, B, cfg.s)
    _, dA, dB = q.qlora_linear_bwd(dY, X, w, A, B, cfg.s, T=T, need_dx=False)
    torch.cuda.synchronize()
    codes_all = w.codes.cpu().numpy().reshape(lin.N, lin.K // 2)
    e_all = w.absmax_q.cpu().numpy().reshape(lin.N, lin.K // 64)
    d_all = w.absmax_scale.cpu().numpy()
    toks = np.random.default_rng(5).choice(2048, 128, replace=False)
    Yg = Y.float().cpu().numpy()
    for r0 in (0, lin.N - 32):
        rs = slice(r0, r0 + 32)
        codes, e, d, _ = oracle.quantize(h["W"][rs])
        g0 = r0 * (lin.K // 64) // 256
        np.testing.assert_array_equal(codes_all[rs].reshape(-1), codes)
        np.testing.assert_array_equal(e_all[rs].reshape(-1), e)
        np.testing.assert_array_equal(d_all[g0:g0 + len(d)], d)
        What = oracle.dequantize(codes, e, d, 32, lin.K)
        Yr, _ = oracle.linear_fwd(h["X"][toks], What, h["A"], h["B"][:, rs], cfg.s)
        assert_close(f"Y[toks, {r0}:+32]", Yg[toks][:, rs], Yr)
        _, _, dBr = oracle.linear_bwd(h["dY"][:, rs], h["X"], What, h["A"], h["B"][:, rs],
                                      cfg.s, need_dx=False)
        assert_close(f"dB[:, {r0}:+32]", dB.float().cpu().numpy()[:, rs], dBr)
    _, dAr, _ = oracle.linear_bwd(h["dY"], h["X"], None, h["A"], h["B"], cfg.s, need_dx=False)
    assert_close("dA", dA.float().cpu().numpy(), dAr)


def test_largest_weight_sampled_rows():
    """The largest weight the API accepts, N x K = 2^32 (131072 x 32768, 2 GB
    of codes, the largest buffer offsets): codes, constants and Y of the
    decode path (M = 1) and of the GEMM path (M = 256) on the first, last and
    32 random rows, against the oracle on those rows alone (a row holds two
    whole double-quantization groups, so rows quantize independently); then
    the backward at M = 256 with dY nonzero only in those rows' columns."""
    need_gpu()
    N, K, r, s = 131072, 32768, 64, 0.25
    say(f"largest weight {N}x{K}")
    W = workloads.device_weight(torch, dev(), N, K, seed=8000)
    w = q.qlora_nf4_quantize(W)
    rng = np.random.default_rng(8)
    rows = np.concatenate([np.arange(16), np.sort(rng.choice(np.arange(16, N - 16), 32,
                                                             replace=False)),
                           np.arange(N - 16, N)])
    ridx = torch.from_numpy(rows).to(dev())
    Wr = W.index_select(0, ridx).cpu().numpy()
    del W
    torch.cuda.empty_cache()
    A, B = workloads.device_adapters(torch, dev(), N, K, r, seed=8001)
    Ah, Bh = bits(A), bits(B)
    codes, e, d, _ = oracle.quantize(Wr)
    np.testing.assert_array_equal(
        w.codes.view(N, K // 2).index_select(0, ridx).cpu().numpy().reshape(-1), codes)
    np.testing.assert_array_equal(
        w.absmax_q.view(N, K // 64).index_select(0, ridx).cpu().numpy().reshape(-1), e)
    np.testing.assert_array_equal(
        w.absmax_scale.view(N, 2).index_select(0, ridx).cpu().numpy().reshape(-1), d)
    What = oracle.dequantize(codes, e, d, len(rows), K)
    for M in (1, 256):
        X = workloads.device_activations(torch, dev(), M, K, seed=8002 + M)
        Y, T = q.qlora_linear_fwd(X, w, A, B, s)
        torch.cuda.synchronize()
        Yr, _ = oracle.linear_fwd(bits(X), What, Ah, Bh[:, rows], s)
        assert_close(f"Y[M={M}, rows]", Y.float().cpu().numpy()[:, rows], Yr)
    # Backward with dY nonzero only in the sampled rows' columns, so that dX,
    # dA and those columns of dB depend on the sampled rows alone.
    dYh = np.zeros((M, N), np.uint16)
    dYh[:, rows] = workloads.to_bf16_bits(rng.standard_normal((M, len(rows)), dtype=np.float32))
    dX, dA, dB = q.qlora_linear_bwd(bf16(dYh), X, w, A, B, s, T=T)
    torch.cuda.synchronize()
    dXr, dAr, dBr = oracle.linear_bwd(dYh[:, rows], bits(X), What, Ah, Bh[:, rows], s)
    assert_close("dX", dX.float().cpu().numpy(), dXr)
    assert_close("dA", dA.float().cpu().numpy(), dAr)
    dBg = dB.float().cpu().numpy()
    assert_close("dB[:, rows]", dBg[:, rows], dBr)
    others = np.setdiff1d(np.arange(N), rows)
    assert not np.any(dBg[:, others]), "dB nonzero where dY is zero"
