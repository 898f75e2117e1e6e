"""The QLoRA linear layer, forward and backward, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Pages: Mathematical Formulation and Figure 1 of "DL0087 QLoRA" (output and
input stay 16-bit; the frozen base is dequantized to a bf16 tile for the
matmul; trainable bf16 adapters of rank r, scaled; the adapter that starts at
zero makes the layer reproduce the quantized base), list item (4) of the same
page and "The Efficient Symphony of the QLoRA Workflow" of "QLoRA (Quantized
Low-Rank Adaptation)" (gradients pass through the frozen 4-bit weights into
the adapters; the base is never updated).

The formula itself was lost from the Mathematical Formulation when the page
was extracted; the reading rebuilt from its bullets is

    Y = X . W_hat_lin^T + s . (X . A) . B

with X [M, K], W_hat_lin [N, K] (the dequantized bf16 base, out x in),
A [K, r], B [r, N], s the LoRA scale (alpha / r), Y [M, N].  The backward of
L with dL/dY = dY is

    G  = dY . B^T                       [M, r]
    dX = dY . W_hat_lin + s . G . A^T   [M, K]
    dA = s . X^T . G                    [K, r]
    dB = s . (X . A)^T . dY             [r, N]

and there is no gradient for the base weight or its constants.
Products are exact-input float64 matmuls; no intermediate is rounded.
"""
import numpy as np

from .nf4 import bf16_bits_to_f64


def linear_fwd_f64(X, W, A, B, s):
    """Forward on float64 operands. Returns (Y, T) with T = X . A."""
    X, W, A, B = (np.asarray(a, dtype=np.float64) for a in (X, W, A, B))
    T = X @ A
    Y = X @ W.T + float(s) * (T @ B)
    return Y, T


def linear_bwd_f64(dY, X, W, A, B, s, need_dx=True):
    """Backward on float64 operands. Returns (dX, dA, dB); dX is None when
    need_dx is False (W is then not read)."""
    dY, X, A, B = (np.asarray(a, dtype=np.float64) for a in (dY, X, A, B))
    s = float(s)
    G = dY @ B.T
    dX = dY @ np.asarray(W, dtype=np.float64) + s * (G @ A.T) if need_dx else None
    dA = s * (X.T @ G)
    dB = s * ((X @ A).T @ dY)
    return dX, dA, dB


def linear_fwd(X_bits, W_bits, A_bits, B_bits, s):
    """Forward from bf16 bit patterns (uint16 arrays); float64 results."""
    return linear_fwd_f64(bf16_bits_to_f64(X_bits), bf16_bits_to_f64(W_bits),
                          bf16_bits_to_f64(A_bits), bf16_bits_to_f64(B_bits), s)


def linear_bwd(dY_bits, X_bits, W_bits, A_bits, B_bits, s, need_dx=True):
    """Backward from bf16 bit patterns (uint16 arrays); float64 results."""
    W = bf16_bits_to_f64(W_bits) if need_dx else None
    return linear_bwd_f64(bf16_bits_to_f64(dY_bits), bf16_bits_to_f64(X_bits), W,
                          bf16_bits_to_f64(A_bits), bf16_bits_to_f64(B_bits), s,
                          need_dx=need_dx)


# ---------------------------------------------------------------------------
# Several projections that read the same input ("LoRA placement: adapters at
# every layer" of "QLoRA: Finetuning 65B Models on a Single GPU": adapters on
# every linear layer -- the query, key and value projections of attention, the
# gate and up projections of the MLP -- which share their input).
# ---------------------------------------------------------------------------

def block_fwd_f64(X, Ws, As, Bs, s):
    """Projections j = 0..S-1 of one input X (float64 operands): lists of Y_j
    and T_j, each the single-layer forward of projection j."""
    outs = [linear_fwd_f64(X, W, A, B, s) for W, A, B in zip(Ws, As, Bs)]
    return [o[0] for o in outs], [o[1] for o in outs]


def block_bwd_f64(dYs, X, Ws, As, Bs, s, need_dx=True):
    """Backward of the projections of one input (float64 operands).  X feeds
    all of them, so its gradient is the sum of the projections' input
    gradients; each adapter pair gets its own projection's gradients.
    Returns (dX or None, list of dA_j, list of dB_j)."""
    dX, dAs, dBs = None, [], []
    for dY, W, A, B in zip(dYs, Ws, As, Bs):
        dXj, dAj, dBj = linear_bwd_f64(dY, X, W, A, B, s, need_dx=need_dx)
        if need_dx:
            dX = dXj if dX is None else dX + dXj
        dAs.append(dAj)
        dBs.append(dBj)
    return dX, dAs, dBs


def block_fwd(X_bits, W_bits_list, A_bits_list, B_bits_list, s):
    """block_fwd_f64 from bf16 bit patterns."""
    return block_fwd_f64(bf16_bits_to_f64(X_bits), [bf16_bits_to_f64(W) for W in W_bits_list],
                         [bf16_bits_to_f64(A) for A in A_bits_list],
                         [bf16_bits_to_f64(B) for B in B_bits_list], s)


def block_bwd(dY_bits_list, X_bits, W_bits_list, A_bits_list, B_bits_list, s, need_dx=True):
    """block_bwd_f64 from bf16 bit patterns."""
    return block_bwd_f64([bf16_bits_to_f64(d) for d in dY_bits_list], bf16_bits_to_f64(X_bits),
                         [bf16_bits_to_f64(W) for W in W_bits_list] if need_dx
                         else [None] * len(dY_bits_list),
                         [bf16_bits_to_f64(A) for A in A_bits_list],
                         [bf16_bits_to_f64(B) for B in B_bits_list], s, need_dx=need_dx)
