"""GPU checks of qlora_linear_fwd_noalloc, the forward for callers that
cannot allocate device memory: called through the C ABI, it must give the
outputs of qlora_linear_fwd (same kernels, the library's fixed per-GPU
scratch instead of a caller workspace) bit for bit, on consecutive calls
whose second is smaller than the first, and match the oracle."""
import numpy as np
import pytest

import bit_quantized_fine_amd as q
import oracle
import workloads
from gpu_util import assert_close, bf16, bits, f32, need_gpu, say, torch

pytestmark = pytest.mark.gpu


def _case(M, N, K, r, s, seed):
    rng = np.random.default_rng(seed)
    inp = workloads.draw_linear(rng, N, K, M, r, with_grad=False)
    w = q.qlora_nf4_quantize(f32(inp.W))
    A = bf16(inp.A) if r else None
    B = bf16(inp.B) if r else None
    return inp, w, bf16(inp.X), A, B


@pytest.mark.parametrize("shapes", [
    # (M, N, K, r, s): first call larger than the second
    ((256, 4096, 4096, 64, 0.25), (4, 512, 2048, 64, 0.25)),     # GEMM split (32 MiB), then decode
    ((300, 520, 448, 64, 0.25), (16, 256, 1024, 16, 1.0)),       # GEMM + T split, then decode
    ((2048, 1024, 1024, 0, 1.0), (64, 128, 256, 8, 0.5)),        # base only, then a small GEMM
    ((16, 1024, 4096, 64, 0.25), (8, 256, 1024, 64, 0.5)),       # decode, T added after the main loop
])
def test_noalloc_matches_workspace_forward(shapes):
    need_gpu()
    for i, (M, N, K, r, s) in enumerate(shapes):
        say(f"noalloc call {i}: M={M} N={N} K={K} r={r}")
        inp, w, X, A, B = _case(M, N, K, r, s, seed=31 + i + M)
        Y0, T0 = q.qlora_linear_fwd(X, w, A, B, s)
        Y1, T1 = q.qlora_linear_fwd_noalloc(X, w, A, B, s)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits(Y1), bits(Y0))
        if r:
            np.testing.assert_array_equal(T1.cpu().numpy(), T0.cpu().numpy())
        if M * N * K <= 1 << 28:
            codes, e, d, _ = oracle.quantize(inp.W)
            What = oracle.dequantize(codes, e, d, N, K)
            if r:
                Yr, Tr = oracle.linear_fwd(inp.X, What, inp.A, inp.B, s)
                assert_close("T", T1.cpu().numpy(), Tr)
            else:
                Yr = oracle.bf16_bits_to_f64(inp.X) @ oracle.bf16_bits_to_f64(What).T
            assert_close("Y", Y1.float().cpu().numpy(), Yr)


def test_noalloc_repeated_calls_are_deterministic():
    """The scratch keeps the last call's contents; the next call must not
    depend on them (nothing in it needs to start at zero)."""
    need_gpu()
    inp, w, X, A, B = _case(300, 520, 448, 64, 0.25, seed=77)
    outs = []
    for _ in range(3):
        Y, T = q.qlora_linear_fwd_noalloc(X, w, A, B, 0.25)
        torch.cuda.synchronize()
        outs.append((bits(Y), T.cpu().numpy()))
        # another shape in between leaves other values in the scratch
        _, w2, X2, A2, B2 = _case(4, 512, 2048, 64, 0.25, seed=78)
        q.qlora_linear_fwd_noalloc(X2, w2, A2, B2, 0.25)
    torch.cuda.synchronize()
    for y, t in outs[1:]:
        np.testing.assert_array_equal(y, outs[0][0])
        np.testing.assert_array_equal(t, outs[0][1])
