"""Pins of the AdamW oracle (oracle/adamw.py): torch.optim.AdamW run in
float64 on the CPU (an independent implementation of the same rule), the
closed form of the first step, and the zero-gradient case."""
import numpy as np
import pytest

import oracle
from oracle import adamw

torch = pytest.importorskip("torch")


@pytest.mark.parametrize("wd", [0.0, 0.01])
def test_matches_torch_adamw_float64(wd):
    rng = np.random.default_rng(4)
    n, lr, b1, b2, eps = 1000, 2e-4, 0.9, 0.999, 1e-8
    p0 = rng.standard_normal(n) * 0.02
    grads = [rng.standard_normal(n) * 10.0 ** rng.uniform(-3, 0) for _ in range(6)]
    tp = torch.tensor(p0, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.AdamW([tp], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd,
                            foreach=False, fused=False)
    p, m, v = p0.copy(), np.zeros(n), np.zeros(n)
    for t, g in enumerate(grads, start=1):
        tp.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        p, m, v = adamw.adamw_step_f64(p, g, m, v, t, lr, b1, b2, eps, wd)
        st = opt.state[tp]
        np.testing.assert_allclose(p, tp.detach().numpy(), rtol=1e-13, atol=1e-18)
        # (torch forms m by linear interpolation, m + (g - m)(1 - b1): the same
        # value up to rounding, relative to the moment's scale where m crosses 0)
        np.testing.assert_allclose(m, st["exp_avg"].numpy(), rtol=1e-13,
                                   atol=1e-14 * np.abs(m).max())
        np.testing.assert_allclose(v, st["exp_avg_sq"].numpy(), rtol=1e-13, atol=0)


def test_first_step_closed_form():
    """With zero moments the bias-corrected moments are g and g^2, so the
    first step moves every weight by lr g / (|g| + eps) after the decay."""
    rng = np.random.default_rng(1)
    p0, g = rng.standard_normal(64), rng.standard_normal(64)
    lr, wd, eps = 1e-3, 0.1, 1e-8
    p, m, v = adamw.adamw_step_f64(p0, g, 0.0, 0.0, 1, lr, 0.9, 0.999, eps, wd)
    np.testing.assert_allclose(p, p0 * (1 - lr * wd) - lr * g / (np.abs(g) + eps), rtol=1e-14)
    np.testing.assert_allclose(m, 0.1 * g, rtol=1e-15)
    np.testing.assert_allclose(v, 0.001 * g * g, rtol=1e-13)


def test_zero_gradient_only_decays():
    p0 = np.linspace(-1, 1, 9)
    p, m, v = adamw.adamw_step_f64(p0, np.zeros(9), np.zeros(9), np.zeros(9), 3, 0.5, 0.9, 0.999,
                                   1e-8, 0.2)
    np.testing.assert_array_equal(p, p0 * (1 - 0.5 * 0.2))
    assert not m.any() and not v.any()


def test_bits_form_rounds_the_float64_step():
    """The bf16 result is the float64 step rounded (through fp32) to bf16,
    within one bf16 step of torch's float64 parameter."""
    rng = np.random.default_rng(2)
    n = 4096
    p_bits = oracle.bf16_rne_bits(rng.standard_normal(n).astype(np.float32) * 0.05)
    g_bits = oracle.bf16_rne_bits(rng.standard_normal(n).astype(np.float32))
    m = (rng.standard_normal(n) * 0.1).astype(np.float32)
    v = (rng.standard_normal(n) ** 2 * 0.01).astype(np.float32)
    out, m2, v2 = adamw.adamw_step(p_bits, g_bits, m, v, 7, 1e-2, weight_decay=0.01)
    tp = torch.tensor(oracle.bf16_bits_to_f64(p_bits), requires_grad=True)
    opt = torch.optim.AdamW([tp], lr=1e-2, weight_decay=0.01, foreach=False, fused=False)
    tp.grad = torch.tensor(oracle.bf16_bits_to_f64(g_bits))
    opt.state[tp] = {"step": torch.tensor(6.0, dtype=torch.float64),
                     "exp_avg": torch.tensor(m.astype(np.float64)),
                     "exp_avg_sq": torch.tensor(v.astype(np.float64))}
    opt.step()
    ref = tp.detach().numpy()
    got = oracle.bf16_bits_to_f64(out)
    ulp = np.abs(ref) * 2.0 ** -8 + 1e-30
    assert np.all(np.abs(got - ref) <= ulp)
    np.testing.assert_allclose(m2, opt.state[tp]["exp_avg"].numpy(), rtol=1e-13)
    np.testing.assert_allclose(v2, opt.state[tp]["exp_avg_sq"].numpy(), rtol=1e-13)
