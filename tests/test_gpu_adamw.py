"""GPU parity of the adapters' AdamW step (qlora_adamw_step) against the
oracle (oracle/adamw.py), and of the paged optimizer state: a step on
paged-out moments (pinned host memory read and written by the GPU) gives the
same bits as a step on resident ones.

The oracle takes the step for the fp32 hyperparameters the kernel receives.
Tolerances: the new parameter within one bf16 step of the oracle's (the
kernel computes in fp32, the oracle in fp64); the new moments within
4 u (|b x| + |(1 - b) y|) of the fp64 values, u = 2^-24, the error bound of
a two-term fp32 sum of rounded products."""
import numpy as np
import pytest

import bit_quantized_fine_amd as q
import oracle
from gpu_util import bf16, bits, need_gpu, say, torch
from oracle import adamw

pytestmark = pytest.mark.gpu

U = 2.0 ** -24
HP = dict(lr=2e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def _draw(rng, n):
    p = oracle.bf16_rne_bits((rng.standard_normal(n) * 0.02).astype(np.float32))
    g = oracle.bf16_rne_bits((rng.standard_normal(n) * 10.0 ** rng.uniform(-4, 0, n))
                             .astype(np.float32))
    m = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    v = (rng.standard_normal(n) ** 2 * 1e-6).astype(np.float32)
    return p, g, m, v


def _ordinal(b):
    b = np.asarray(b, np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def _check_step(p_bits, g_bits, m, v, step, p_gpu, m_gpu, v_gpu, hp=HP):
    # The hyperparameters cross the C ABI as fp32: the oracle takes the step
    # for those values (1 - b is then exact in fp32 too).
    hp = {k: float(np.float32(x)) for k, x in hp.items()}
    pr, mr, vr = adamw.adamw_step(p_bits, g_bits, m, v, step, **hp)
    d = np.abs(_ordinal(p_gpu) - _ordinal(pr))
    say(f"  step {step}: param bf16 steps off: max {d.max()}, {np.count_nonzero(d)} of {d.size}")
    assert d.max() <= 1
    g = oracle.bf16_bits_to_f64(g_bits)
    mb = 4 * U * (hp["beta1"] * np.abs(m) + (1 - hp["beta1"]) * np.abs(g)) + 1e-45
    vb = 4 * U * (hp["beta2"] * np.abs(v) + (1 - hp["beta2"]) * g * g) + 1e-45
    assert np.all(np.abs(m_gpu.astype(np.float64) - mr) <= mb)
    assert np.all(np.abs(v_gpu.astype(np.float64) - vr) <= vb)


@pytest.mark.parametrize("n", [1, 7, 8, 1000003])
def test_adamw_parity(n):
    need_gpu()
    say(f"adamw n={n}")
    rng = np.random.default_rng(n)
    p, g, m, v = _draw(rng, n)
    P, G = bf16(p), bf16(g)
    M = torch.from_numpy(m.copy()).cuda()
    V = torch.from_numpy(v.copy()).cuda()
    for step in (1, 2, 3):
        p0, m0, v0 = bits(P), M.cpu().numpy(), V.cpu().numpy()
        q.qlora_adamw_step(P, G, M, V, step, **HP)
        torch.cuda.synchronize()
        _check_step(p0, g, m0, v0, step, bits(P), M.cpu().numpy(), V.cpu().numpy())


def test_adamw_zero_state_first_step():
    """From zero moments the first step moves each weight by about lr (the
    bias-corrected ratio is g / |g|), after the decay."""
    need_gpu()
    rng = np.random.default_rng(3)
    n = 4096
    p, g, _, _ = _draw(rng, n)
    st = q.PagedState(n)
    P, G = bf16(p), bf16(g)
    st.step(P, G, 1, **HP)
    torch.cuda.synchronize()
    _check_step(p, g, np.zeros(n, np.float32), np.zeros(n, np.float32), 1, bits(P),
                *st.read().cpu().numpy())
    st.close()


def test_paged_state_gives_the_same_bits():
    """Six steps with the moments paged out and in between steps against six
    steps with them resident throughout: parameters and moments agree bit
    for bit, and page-out returns the HBM copy (resident flag)."""
    need_gpu()
    n = 300007
    rng = np.random.default_rng(8)
    p, _, _, _ = _draw(rng, n)
    grads = [bf16(_draw(rng, n)[1]) for _ in range(6)]
    a, b = q.PagedState(n), q.PagedState(n, on_host=True)
    assert a.resident and not b.resident
    Pa, Pb = bf16(p), bf16(p)
    plan = ["host", "host", "in", "out", "host", "in"]   # where b's moments are for each step
    for t, (G, where) in enumerate(zip(grads, plan), start=1):
        if where == "in":
            b.page_in()
            assert b.resident
        elif where == "out":
            b.page_out()
            assert not b.resident
        say(f"  paged step {t}: b {'resident' if b.resident else 'on host'}")
        a.step(Pa, G, t, **HP)
        b.step(Pb, G, t, **HP)
    b.page_out()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(Pa), bits(Pb))
    np.testing.assert_array_equal(a.read().cpu().numpy().view(np.uint32),
                                  b.read().cpu().numpy().view(np.uint32))
    a.close()
    b.close()


def test_paged_state_write_read_round_trip():
    need_gpu()
    n = 1000
    st = q.PagedState(n)
    assert not st.read().any()   # zero at creation
    src = torch.randn(2, n, device="cuda")
    st.write(src)
    st.page_out()
    assert torch.equal(st.read(), src)
    st.page_in()
    assert torch.equal(st.read(), src)
    st.close()


def test_adamw_on_llama7b_adapters_after_backward():
    """The LLaMA-7B layer's seven adapters (5.0 M parameters) as slices of one
    flat buffer: the backward writes dA and dB into slices of one flat
    gradient buffer, and one step updates them all; every parameter checked
    against the oracle."""
    need_gpu()
    import workloads
    M, r = 256, 64
    lins = workloads.WORKLOADS["llama7b"].linears
    sizes = [(l.K * r, r * l.N) for l in lins]
    n = sum(a + b for a, b in sizes)
    say(f"adamw over the 7B layer's adapters: n={n}")
    P = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    G = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    off = 0
    for (lin, inp), (sa, sb) in zip(workloads.workload_inputs("llama7b", M=M), sizes):
        A, B = P[off:off + sa].view(lin.K, r), P[off + sa:off + sa + sb].view(r, lin.N)
        A.copy_(bf16(inp.A))
        B.copy_(bf16(np.ascontiguousarray(inp.B)))
        dA, dB = G[off:off + sa].view(lin.K, r), G[off + sa:off + sa + sb].view(r, lin.N)
        w = q.qlora_nf4_quantize(torch.from_numpy(inp.W).cuda())
        q.qlora_linear_bwd(bf16(inp.dY), bf16(inp.X), w, A, B, 0.25, need_dx=False, dA=dA, dB=dB)
        off += sa + sb
    st = q.PagedState(n)
    p0, g0 = bits(P), bits(G)
    m0, v0 = st.read().cpu().numpy()
    st.step(P, G, 1, **HP)
    torch.cuda.synchronize()
    m1, v1 = st.read().cpu().numpy()
    _check_step(p0, g0, m0, v0, 1, bits(P), m1, v1)
    st.close()


def test_adamw_refuses_bad_arguments():
    need_gpu()
    P = torch.zeros(64, dtype=torch.bfloat16, device="cuda")
    M = torch.zeros(64, dtype=torch.float32, device="cuda")
    with pytest.raises(q.QloraError, match="shape"):
        q.qlora_adamw_step(P, P, M, M, 0)           # steps count from 1
    with pytest.raises(q.QloraError, match="shape"):
        q.qlora_adamw_step(P, P, M, M, 1, beta2=1.0)
    with pytest.raises(q.QloraError, match="aligned"):
        q.qlora_adamw_step(P[1:9], P[1:9], M[:8], M[:8], 1)
