"""End-to-end QLoRA fine-tuning on the library's kernels: an NF4 base layer
with adapters A, B (B starting at zero, so the layer first reproduces the
quantized base model: the rank bullet of the Mathematical Formulation of
"DL0087 QLoRA"), trained with AdamW on paged state to fit a target that
differs from the base by a rank-r update.  The first step's gradients are
checked against the oracle's (its own forward, loss gradient and backward
from the same seeded inputs); the loss must then fall, including across a
step taken with the moments paged out, and the frozen codes never change."""
import numpy as np
import pytest

import bit_quantized_fine_amd as q
import oracle
import workloads
from gpu_util import assert_close, bf16, f32, need_gpu, say, torch

pytestmark = pytest.mark.gpu


def test_qlora_finetuning_loop():
    need_gpu()
    N, K, M, r, s = 256, 512, 64, 16, 1.0
    hp = dict(lr=1e-2, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0)
    rng = np.random.default_rng(12)
    W = workloads.draw_weight(rng, N, K)
    Xb = workloads.to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
    A0 = workloads.to_bf16_bits(rng.standard_normal((K, r), dtype=np.float32) / r)
    B0 = np.zeros((r, N), np.uint16)
    U = rng.standard_normal((K, r)) * 0.05
    V = rng.standard_normal((r, N)) * 0.05
    # the target, from the oracle's dequantized base: X Ŵ^T + X U V
    codes, e, d, _ = oracle.quantize(W)
    What = oracle.dequantize(codes, e, d, N, K)
    Xf = oracle.bf16_bits_to_f64(Xb)
    target = Xf @ oracle.bf16_bits_to_f64(What).T + Xf @ U @ V

    w = q.qlora_nf4_quantize(f32(W))
    codes0 = w.codes.clone()
    X, tgt = bf16(Xb), torch.from_numpy(target.astype(np.float32)).cuda()
    # adapters and their gradients as slices of flat buffers
    n = K * r + r * N
    P = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    G = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    A, B = P[:K * r].view(K, r), P[K * r:].view(r, N)
    dA, dB = G[:K * r].view(K, r), G[K * r:].view(r, N)
    A.copy_(bf16(A0))
    B.copy_(bf16(B0))
    state = q.PagedState(n)
    losses = []
    for step in range(1, 31):
        Y, T = q.qlora_linear_fwd(X, w, A, B, s)
        err = Y.float() - tgt
        losses.append(float(0.5 * (err * err).sum() / M))
        dY = (err / M).to(torch.bfloat16)
        q.qlora_linear_bwd(dY, X, w, A, B, s, T=T, need_dx=False, dA=dA, dB=dB)
        if step == 1:
            # B = 0: the layer is the quantized base model
            assert torch.equal(Y, q.qlora_linear_fwd(X, w)[0])
            # the oracle's step-1 gradients from the same seeded inputs
            # (the loss gradient taken as the loop takes it: from the bf16
            # output, in fp32 against the fp32 target)
            Yr, _ = oracle.linear_fwd(Xb, What, A0, B0, s)
            Y16 = oracle.bf16_bits_to_f64(oracle.bf16_rne_bits(Yr.astype(np.float32)))
            err32 = Y16.astype(np.float32) - target.astype(np.float32)
            dYr = oracle.bf16_rne_bits(err32 / np.float32(M))
            _, dAr, dBr = oracle.linear_bwd(dYr, Xb, What, A0, B0, s, need_dx=False)
            torch.cuda.synchronize()
            assert_close("dA (step 1)", dA.float().cpu().numpy(), dAr)
            assert_close("dB (step 1)", dB.float().cpu().numpy(), dBr)
        if step == 3:   # a step with the moments paged out to host memory
            state.page_out()
        if step == 4:
            state.page_in()
        state.step(P, G, step, **hp)
    torch.cuda.synchronize()
    say(f"  loss: {losses[0]:.4f} -> {losses[9]:.4f} -> {losses[-1]:.4f}")
    assert losses[-1] < 0.5 * losses[0]
    assert all(b < a * 1.05 for a, b in zip(losses, losses[1:]))
    assert torch.equal(w.codes, codes0)   # the base stays frozen
    state.close()
