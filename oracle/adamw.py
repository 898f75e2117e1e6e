"""AdamW step on the LoRA adapters with fp32 moments.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Pages: numbered list items (4) and (5) of "DL0087 QLoRA: 4-bit Quantized LoRA"
(only the adapters train, so optimizer state scales with the adapter rank;
the optimizer states are paged to host RAM during transient memory spikes),
"Double Quantization and Paged Optimizers" of "QLoRA: Finetuning 65B Models
on a Single GPU", and "Memory Management Details" of "QLoRA: Quantized Low
Rank Adaptation at Extreme Scale" (paged optimizers offload their states to
CPU memory when needed).  The pages name the optimizer only as paged; where
its state lives does not change what a step computes.

Readings (the pages print no update rule):
  * The optimizer is AdamW (Adam with decoupled weight decay), step t >= 1:
        p <- p (1 - lr wd)
        m <- b1 m + (1 - b1) g
        v <- b2 v + (1 - b2) g^2
        p <- p - lr (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps)
  * The adapters A and B are bf16 ("16-bit adapters"; updated in place), the
    gradients bf16 (the layer's dA and dB), the moments m and v fp32.  The
    oracle computes in float64 from those exact values; the new parameter is
    rounded to bf16 (through fp32, as a device computing in fp32 stores it),
    the new moments are returned in float64.
"""
import numpy as np

from .nf4 import bf16_bits_to_f64, bf16_rne_bits


def adamw_step_f64(p, g, m, v, step: int, lr: float, beta1: float, beta2: float, eps: float,
                   weight_decay: float):
    """One AdamW step in float64 on float64 arrays; returns (p, m, v)."""
    if step < 1:
        raise ValueError("step counts from 1")
    p = np.asarray(p, np.float64) * (1.0 - lr * weight_decay)
    g = np.asarray(g, np.float64)
    m = beta1 * np.asarray(m, np.float64) + (1.0 - beta1) * g
    v = beta2 * np.asarray(v, np.float64) + (1.0 - beta2) * g * g
    m_hat = m / (1.0 - beta1 ** step)
    v_hat = v / (1.0 - beta2 ** step)
    p = p - lr * m_hat / (np.sqrt(v_hat) + eps)
    return p, m, v


def adamw_step(p_bits, g_bits, m, v, step: int, lr: float, beta1: float = 0.9,
               beta2: float = 0.999, eps: float = 1e-8, weight_decay: float = 0.0):
    """The step on bf16 adapters (bit patterns) and fp32 moments: returns the
    new parameter as bf16 bits and the new moments in float64.  The new
    parameter is stored the way a device computing in fp32 stores it: rounded
    to fp32, then to bf16 (both to nearest even); a result computed in fp32
    throughout lies within one bf16 step of it."""
    p, m2, v2 = adamw_step_f64(bf16_bits_to_f64(p_bits), bf16_bits_to_f64(g_bits),
                               np.asarray(m, np.float32).astype(np.float64),
                               np.asarray(v, np.float32).astype(np.float64),
                               step, lr, beta1, beta2, eps, weight_decay)
    return bf16_rne_bits(p.astype(np.float32)), m2, v2
