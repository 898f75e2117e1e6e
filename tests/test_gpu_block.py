"""GPU parity of the fused multi-projection block (S projections of one input,
stacked along N in one NF4 weight) against the oracle's per-projection
definition: Y_j and T_j per projection, dX summed over the projections, dA_j
and dB_j per projection.  Cases cover the streaming path (M <= 16, one
launch per projection) and the GEMM path (one launch over all rows), S = 1
to 3, ranks up to S r = 256, and split reductions at small token counts.
"""
import numpy as np
import pytest

import bit_quantized_fine_amd as q
import oracle
import workloads
from gpu_util import assert_close, bf16, bits, f32, need_gpu, say, torch

pytestmark = pytest.mark.gpu


class Block:
    """S projections of one X: seeded inputs, GPU tensors (stacked), oracle."""

    def __init__(self, M, S, nseg, K, r, s, seed, x_kind="normal"):
        rng = np.random.default_rng(seed)
        self.M, self.S, self.nseg, self.K, self.r, self.s = M, S, nseg, K, r, s
        Ws = [workloads.draw_weight(rng, nseg, K) for _ in range(S)]
        self.X = workloads.to_bf16_bits(workloads.draw_activations(rng, M, K, x_kind))
        self.As = [workloads.to_bf16_bits(rng.standard_normal((K, r), dtype=np.float32) / r)
                   for _ in range(S)]
        self.Bs = [workloads.to_bf16_bits(rng.standard_normal((r, nseg), dtype=np.float32) * 0.01)
                   for _ in range(S)]
        self.dYs = [workloads.to_bf16_bits(rng.standard_normal((M, nseg), dtype=np.float32))
                    for _ in range(S)]
        self.w = q.qlora_nf4_quantize(f32(np.concatenate(Ws, axis=0)))
        self.gX = bf16(self.X)
        self.gA = bf16(np.concatenate(self.As, axis=1))
        self.gB = bf16(np.concatenate(self.Bs, axis=1))
        self.gdY = bf16(np.concatenate(self.dYs, axis=1))
        self.What = []
        for W in Ws:
            codes, e, d, _ = oracle.quantize(W)
            self.What.append(oracle.dequantize(codes, e, d, nseg, K))
        self.Wall = Ws

    def check_fwd(self, Y, T):
        Yr, Tr = oracle.block_fwd(self.X, self.What, self.As, self.Bs, self.s)
        Yg, Tg = Y.float().cpu().numpy(), T.cpu().numpy()
        for j in range(self.S):
            cols = slice(j * self.nseg, (j + 1) * self.nseg)
            assert_close(f"Y_{j}", Yg[:, cols], Yr[j])
            assert_close(f"T_{j}", Tg[:, j * self.r:(j + 1) * self.r], Tr[j])

    def check_bwd(self, dX, dA, dB):
        dXr, dAr, dBr = oracle.block_bwd(self.dYs, self.X, self.What, self.As, self.Bs, self.s)
        if dX is not None:
            assert_close("dX (sum over projections)", dX.float().cpu().numpy(), dXr)
        dAg, dBg = dA.float().cpu().numpy(), dB.float().cpu().numpy()
        for j in range(self.S):
            assert_close(f"dA_{j}", dAg[:, j * self.r:(j + 1) * self.r], dAr[j])
            assert_close(f"dB_{j}", dBg[:, j * self.nseg:(j + 1) * self.nseg], dBr[j])


BLOCK_CASES = [
    # (M, S, nseg, K, r, s)
    (1, 3, 128, 128, 8, 1.0),        # streaming path, one projection per launch
    (4, 3, 256, 256, 16, 0.5),
    (16, 2, 128, 512, 64, 0.25),     # streaming path, 16 tokens
    (16, 3, 128, 4096, 16, 0.5),     # streaming path, X in K-slices
    (17, 3, 128, 128, 8, 1.0),       # first GEMM size
    (64, 3, 128, 256, 32, 0.5),      # GEMM with split reductions (few tiles)
    (300, 2, 256, 448, 64, 0.25),    # ragged tokens, K not a multiple of 128
    (520, 3, 128, 128, 80, 0.125),   # S r = 240, three token tiles
    (256, 4, 128, 128, 64, 0.25),    # S r = 256, the largest combined rank
    (1, 1, 128, 128, 8, 1.0),        # S = 1 is the plain layer
]


@pytest.mark.parametrize("M,S,nseg,K,r,s", BLOCK_CASES)
def test_block_parity(M, S, nseg, K, r, s):
    need_gpu()
    say(f"block M={M} S={S} nseg={nseg} K={K} r={r}")
    b = Block(M, S, nseg, K, r, s, seed=M + 3 * S + nseg + K + r)
    Y, T = q.qlora_block_fwd(b.gX, b.w, S, b.gA, b.gB, s)
    dX, dA, dB = q.qlora_block_bwd(b.gdY, b.gX, b.w, S, b.gA, b.gB, s, T=T)
    dX2, dA2, dB2 = q.qlora_block_bwd(b.gdY, b.gX, b.w, S, b.gA, b.gB, s, T=None)
    torch.cuda.synchronize()
    b.check_fwd(Y, T)
    b.check_bwd(dX, dA, dB)
    # the recompute (checkpointing) form gives the same gradients
    b.check_bwd(dX2, dA2, dB2)
    np.testing.assert_array_equal(bits(dX2), bits(dX))


def test_block_matches_the_projections_run_one_by_one():
    """The block's projections equal the plain layer run on each projection's
    own weight and adapters (within the tolerance: T is summed in another
    order), and its dX equals the sum of theirs."""
    need_gpu()
    M, S, nseg, K, r, s = 192, 3, 128, 384, 16, 0.5
    say(f"block vs one by one, M={M}")
    b = Block(M, S, nseg, K, r, s, seed=41, x_kind="relu")
    Y, T = q.qlora_block_fwd(b.gX, b.w, S, b.gA, b.gB, s)
    dX, dA, dB = q.qlora_block_bwd(b.gdY, b.gX, b.w, S, b.gA, b.gB, s, T=T)
    dX_sum = None
    for j in range(S):
        wj = q.qlora_nf4_quantize(f32(b.Wall[j]))
        Yj, Tj = q.qlora_linear_fwd(b.gX, wj, bf16(b.As[j]), bf16(b.Bs[j]), s)
        dXj, dAj, dBj = q.qlora_linear_bwd(bf16(b.dYs[j]), b.gX, wj, bf16(b.As[j]),
                                           bf16(b.Bs[j]), s, T=Tj)
        torch.cuda.synchronize()
        cols = slice(j * nseg, (j + 1) * nseg)
        assert_close(f"Y_{j}", Y.float().cpu().numpy()[:, cols], Yj.float().cpu().numpy())
        assert_close(f"dA_{j}", dA.float().cpu().numpy()[:, j * r:(j + 1) * r],
                     dAj.float().cpu().numpy())
        assert_close(f"dB_{j}", dB.float().cpu().numpy()[:, cols], dBj.float().cpu().numpy())
        dX_sum = dXj.double() if dX_sum is None else dX_sum + dXj.double()
        # the stacked weight's codes are the projection's own
        np.testing.assert_array_equal(
            b.w.codes.view(S, -1)[j].cpu().numpy(), wj.codes.cpu().numpy())
    assert_close("dX", dX.double().cpu().numpy(), dX_sum.cpu().numpy())


@pytest.mark.parametrize("which", ["qkv", "gate_up"])
def test_block_llama7b_full_size(which):
    """LLaMA-7B's q/k/v (3 x 4096 rows) and gate/up (2 x 11008 rows) blocks
    at M = 2048: sampled rows of Y and dX, full dA and dB."""
    need_gpu()
    S, nseg = (3, 4096) if which == "qkv" else (2, 11008)
    K, M, r, s = 4096, 2048, 64, 0.25
    say(f"block {which}: S={S} nseg={nseg} K={K} M={M}")
    b = Block(M, S, nseg, K, r, s, seed=7 if which == "qkv" else 8)
    Y, T = q.qlora_block_fwd(b.gX, b.w, S, b.gA, b.gB, s)
    dX, dA, dB = q.qlora_block_bwd(b.gdY, b.gX, b.w, S, b.gA, b.gB, s, T=T)
    torch.cuda.synchronize()
    rows = np.random.default_rng(3).choice(M, 128, replace=False)
    Yr, _ = oracle.block_fwd(b.X[rows], b.What, b.As, b.Bs, s)
    Yg = Y.float().cpu().numpy()[rows]
    for j in range(S):
        assert_close(f"Y_{j}[rows]", Yg[:, j * nseg:(j + 1) * nseg], Yr[j])
    dXr, _, _ = oracle.block_bwd([d[rows] for d in b.dYs], b.X[rows], b.What, b.As, b.Bs, s)
    assert_close("dX[rows]", dX.float().cpu().numpy()[rows], dXr)
    _, dAr, dBr = oracle.block_bwd(b.dYs, b.X, b.What, b.As, b.Bs, s, need_dx=False)
    for j in range(S):
        assert_close(f"dA_{j}", dA.float().cpu().numpy()[:, j * r:(j + 1) * r], dAr[j])
        assert_close(f"dB_{j}", dB.float().cpu().numpy()[:, j * nseg:(j + 1) * nseg], dBr[j])


def test_block_refuses_misaligned_segments():
    """Segments must start at a 128-row tile and at a group of 256 block
    constants; S r must not exceed 256 (checked before any launch)."""
    need_gpu()
    b = Block(8, 2, 128, 128, 8, 1.0, seed=1)
    with pytest.raises(q.QloraError, match="shape"):
        q.qlora_block_fwd(b.gX, b.w, 4, torch.zeros((128, 32), dtype=torch.bfloat16,
                                                    device=b.gX.device),
                          torch.zeros((8, 256), dtype=torch.bfloat16, device=b.gX.device))
    with pytest.raises(q.QloraError, match="rank"):
        q.qlora_block_fwd(b.gX, b.w, 2, torch.zeros((128, 272), dtype=torch.bfloat16,
                                                    device=b.gX.device),
                          torch.zeros((136, 256), dtype=torch.bfloat16, device=b.gX.device))
