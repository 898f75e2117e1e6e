"""Helpers for the GPU parity tests: host <-> device transfer of the seeded
inputs and the tolerance check stated for floating-point outputs."""
import sys

import numpy as np
import pytest

try:
    import torch
except Exception:  # pragma: no cover
    torch = None

# Tolerance for fp outputs (Y, dX, dA, dB): relative Frobenius error <= 5e-3
# and max elementwise error <= 1e-2 * max |ref|.
REL_FRO = 5e-3
REL_MAX = 1e-2


def need_gpu():
    if torch is None or not torch.cuda.is_available():
        pytest.skip("no GPU")


def say(msg):
    """Print and flush a progress line (names the case before GPU work)."""
    print(msg, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev())


def bf16(bits):
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(dev())


def bits(t):
    """bf16 device tensor -> uint16 numpy bit patterns."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def as_f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def errors(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    diff = got - ref
    nref = np.linalg.norm(ref)
    rel = np.linalg.norm(diff) / nref if nref > 0 else np.linalg.norm(diff)
    mref = np.max(np.abs(ref)) if ref.size else 0.0
    mx = np.max(np.abs(diff)) / mref if mref > 0 else (np.max(np.abs(diff)) if diff.size else 0.0)
    return rel, mx


def assert_close(name, got, ref):
    rel, mx = errors(got, ref)
    say(f"  {name}: rel_fro={rel:.3e} rel_max={mx:.3e}")
    assert rel <= REL_FRO and mx <= REL_MAX, (name, rel, mx)
